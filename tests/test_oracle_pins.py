"""Pins of the fp64 oracle to things other than itself.

Each pin is chosen so that a plausible mistake in the oracle (a dropped term,
a wrong sign or index, a transposed operand, a wrong format bias) fails at
least one of them; `test_planted_mistakes_are_caught` plants such mistakes in
a copy of the oracle's C source and checks exactly that.

Sources of truth used here:
  * the pages' worked example of the block lookup ("9 Decode and KV Cache",
    section 9.5) and its request-A block table (tests/golden/block_lookup.json);
  * closed forms of softmax attention (uniform keys -> mean of V; one token ->
    that value; two tokens -> logistic weights; one dominant key -> its value);
  * invariances: physical block renumbering and prefix-block aliasing (paging
    changes lookup, not the formula, section 9.5), joint token permutation, a
    common shift of all keys, affine maps of V;
  * GQA as MHA over repeated KV heads (GQA teaser on the kv-cache tag page);
  * library routines: torch's bf16 and float8_e4m3fn conversions, torch's
    fp64 scaled_dot_product_attention, numpy's round-half-even;
  * a structurally different brute-force implementation (oracle/brute.py).
"""
from __future__ import annotations

import json
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from oracle import brute
import synth
from synth import F32, BF16, FP8, INT8
from tests.helpers import make_case, permute_physical, unshare

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- lookup
def test_block_lookup_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "block_lookup.json")))
    table = {int(k): v for k, v in g["block_table"].items()}
    for tok, pb, off in g["cases"]:
        assert oracle.locate(table, tok, g["block_size"]) == (pb, off)
    for tok in g["unmapped_tokens"]:
        with pytest.raises(KeyError):
            oracle.locate(table, tok, g["block_size"])
    row = [table[i] for i in range(3)] + [-1]
    for tok, pb, off in g["cases"]:
        assert oracle.slot_of(row, tok, g["block_size"]) == pb * g["block_size"] + off
    with pytest.raises(KeyError):
        oracle.slot_of(row, 48, g["block_size"])


def test_pool_reproduces_request_a():
    """Request A of section 9.5: with physical blocks 7, 2, 15 at the front of
    the free list, a 48-token request maps logical [0, 1, 2] -> [7, 2, 15]."""
    g = json.load(open(os.path.join(GOLDEN, "block_lookup.json")))["request_a"]
    order = [7, 2, 15] + [i for i in range(20) if i not in (7, 2, 15)]
    pool = oracle.OraclePool(20, order)
    table, slots = pool.build_block_table([g["tokens"]], 16, 4)
    assert list(table[0, :3]) == g["physical_blocks"]
    assert table[0, 3] == -1
    assert slots[0] == 15 * 16 + 15          # token 47 -> (15, 15)


# ---------------------------------------------------------------- decoding
def test_bf16_decode_matches_torch():
    import torch
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint16)
    ours = oracle.decode(bits, BF16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_fp8_decode_matches_torch_and_spec_points():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_decode_table()
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9 and ours[0x38] == 1.0
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert np.count_nonzero(np.isfinite(ours)) == 254
    pos = ours[:0x7F]
    assert (np.diff(pos) > 0).all()              # positive codes ascend


def test_int8_decode_identity():
    codes = np.arange(-128, 128, dtype=np.int8)
    assert (oracle.decode(codes, INT8) == codes.astype(np.float64)).all()


# ---------------------------------------------------------------- quantizers
def test_quantize_fp8_matches_torch_cast_in_range():
    import torch
    r = np.random.default_rng(0)
    x = np.concatenate([
        r.standard_normal(20000).astype(np.float32) * 50,
        r.uniform(-448, 448, 20000).astype(np.float32),
        np.float32(2.0 ** -9) * r.uniform(-4, 4, 5000).astype(np.float32),
    ])
    vals = oracle.fp8_decode_table()[:0x7E + 1]
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)   # exact ties
    x = np.concatenate([x, mids, -mids, np.float32([0.0, -0.0, 448.0, -448.0])])
    ours = oracle.quantize_fp8(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ours == ref).all()


def test_quantize_fp8_saturates_and_nan():
    x = np.float32([449.0, 464.0, 470.0, 1e30, np.inf, -1e30, -np.inf, np.nan])
    q = oracle.quantize_fp8(x)
    assert list(q[:5]) == [0x7E] * 5
    assert list(q[5:7]) == [0xFE] * 2
    assert q[7] == 0x7F


def test_quantize_int8_round_half_even_and_clamp():
    x = np.float32([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.49, 127.5, 300, -300,
                    np.inf, -np.inf, np.nan, 3.2, -3.7])
    q = oracle.quantize_int8(x)
    assert list(q) == [0, 2, 2, 0, -2, -2, 126, 127, 127, 127, -127, 127, -127, 0, 3, -4]


def test_quant_input_is_one_fp32_multiply_by_rounded_reciprocal():
    s = np.float32(0.1)
    x = np.float32(3.0)
    inv = np.float32(np.float32(1.0) / s)
    assert oracle.quant_input(x, s) == np.float32(x * inv)
    # differs from dividing directly for some inputs: the definition is the product
    r = np.random.default_rng(1)
    xs = r.standard_normal(10000).astype(np.float32)
    ss = np.abs(r.standard_normal(10000)).astype(np.float32) + np.float32(1e-3)
    prod = oracle.quant_input(xs, ss)
    assert (prod == xs * (np.float32(1) / ss)).all()


# ---------------------------------------------------------------- attention
def _contig_case(seed, n, d_h=64, n_q=2, n_kv=1, dtype=F32):
    return make_case(seed, [n], n_q=n_q, n_kv=n_kv, d_h=d_h, kv_dtype=dtype, q_dtype=dtype)


def pin_closed_forms(paged):
    """Closed forms; `paged(case, **kw)` -> (out, m, z, bad)."""
    fails = []
    # uniform keys -> mean of the values
    c = _contig_case(10, 37)
    kd = oracle.decode(c.k, F32)
    row0 = c.table[0, 0]
    c.k[:] = np.float32(0.0)
    c.k[:] = kd[row0, :, 0:1, :].astype(np.float32)   # every slot holds the same key
    out = paged(c)[0].reshape(c.B, c.n_q, c.d_h)
    vals = brute.gather_contiguous(oracle.decode(c.v, F32), c.table[0], 37, c.bs)
    if not np.allclose(out[0, 0], vals[:, 0, :].mean(axis=0), atol=1e-12, rtol=0):
        fails.append("uniform keys")
    # scale 0 -> mean of the values
    c = _contig_case(11, 53)
    c.scale = 0.0
    out = paged(c)[0].reshape(c.B, c.n_q, c.d_h)
    vals = brute.gather_contiguous(oracle.decode(c.v, F32), c.table[0], 53, c.bs)
    if not np.allclose(out[0, 1], vals[:, 0, :].mean(axis=0), atol=1e-12, rtol=0):
        fails.append("scale 0")
    # one token -> its value, exactly
    c = _contig_case(12, 1)
    out = paged(c)[0].reshape(c.B, c.n_q, c.d_h)
    v0 = oracle.decode(c.v, F32)[c.table[0, 0], 0, 0, :]
    if not (out[0, 0] == v0).all():
        fails.append("one token")
    # two tokens -> logistic weights
    c = _contig_case(13, 2)
    qd = oracle.decode(c.q, F32)[0, 0]
    kd = oracle.decode(c.k, F32)[c.table[0, 0], 0, :2, :]
    vd = oracle.decode(c.v, F32)[c.table[0, 0], 0, :2, :]
    s0, s1 = c.scale * (kd[0] @ qd), c.scale * (kd[1] @ qd)
    w0 = 1.0 / (1.0 + np.exp(s1 - s0))
    ref = w0 * vd[0] + (1 - w0) * vd[1]
    out = paged(c)[0].reshape(c.B, c.n_q, c.d_h)
    if not np.allclose(out[0, 0], ref, atol=1e-12, rtol=0):
        fails.append("two tokens")
    # one dominant key -> its value
    c = _contig_case(14, 40)
    qd = oracle.decode(c.q, F32)[0, 0]
    star = 29
    pb, off = c.table[0, star // 16], star % 16
    c.k[pb, 0, off, :] = (qd * 200.0).astype(np.float32)
    out = paged(c)[0].reshape(c.B, c.n_q, c.d_h)
    vstar = oracle.decode(c.v, F32)[pb, 0, off, :]
    if not np.allclose(out[0, 0], vstar, atol=1e-12, rtol=0):
        fails.append("dominant key")
    return fails


def _paged(case, _lib=None, **kw):
    return oracle.paged_attn(case.q, case.k, case.v, case.table, case.ctx, case.scale,
                             n_q=case.n_q, n_kv=case.n_kv, q_dtype=case.q_dtype,
                             kv_dtype=case.kv_dtype, k_scale=case.k_scale,
                             v_scale=case.v_scale, _lib=_lib, **kw)


def pin_brute_force(paged, seeds=range(6)):
    fails = []
    shapes = [(4, 2, 64, BF16), (8, 2, 32, F32), (6, 3, 16, BF16), (4, 4, 64, F32),
              (16, 2, 32, FP8), (8, 2, 64, INT8)]
    for seed, (n_q, n_kv, d_h, dt) in zip(seeds, shapes):
        r = np.random.default_rng(100 + seed)
        ctx = r.integers(0, 70, size=3)
        c = make_case(200 + seed, ctx, n_q=n_q, n_kv=n_kv, d_h=d_h, kv_dtype=dt,
                      q_dtype=BF16 if dt != F32 else F32)
        ours = paged(c)[0].reshape(c.B, c.n_q, c.d_h)
        ref = brute.attention(c.q, c.k, c.v, c.table, c.ctx, c.scale, n_q=c.n_q, n_kv=c.n_kv,
                              q_dtype=c.q_dtype, kv_dtype=c.kv_dtype, k_scale=c.k_scale,
                              v_scale=c.v_scale)
        if not np.allclose(ours, ref, atol=1e-12, rtol=1e-12):
            fails.append(f"brute force seed {seed}")
    return fails


def pin_gqa_is_repeated_mha(paged):
    fails = []
    c = make_case(31, [45, 17, 64], n_q=8, n_kv=2, d_h=32, kv_dtype=F32, q_dtype=F32)
    gqa = paged(c)[0].reshape(c.B, c.n_q, c.d_h)
    # repeat each KV head g times -> an MHA cache with n_kv = n_q
    mha = make_case(31, [45, 17, 64], n_q=8, n_kv=8, d_h=32, kv_dtype=F32, q_dtype=F32)
    mha.k = np.repeat(c.k, c.g, axis=1)
    mha.v = np.repeat(c.v, c.g, axis=1)
    mha.q, mha.table, mha.ctx = c.q, c.table, c.ctx
    ref = paged(mha)[0].reshape(c.B, c.n_q, c.d_h)
    if not (gqa == ref).all():
        fails.append("gqa vs repeated mha")
    return fails


def pin_invariances(paged):
    fails = []
    c = make_case(41, [70, 33, 1, 48], n_q=4, n_kv=2, d_h=32, kv_dtype=BF16, q_dtype=BF16)
    base = paged(c)[0]
    # physical renumbering -> bit-identical
    if not (paged(permute_physical(c, 5))[0] == base).all():
        fails.append("block permutation")
    # joint token permutation (no positional terms) -> unchanged to 1e-12
    cf = make_case(42, [50], n_q=2, n_kv=1, d_h=32, kv_dtype=F32, q_dtype=F32, extra_blocks=0)
    o1 = paged(cf)[0]
    kd = brute.gather_contiguous(cf.k.astype(np.float64), cf.table[0], 50, 16)
    vd = brute.gather_contiguous(cf.v.astype(np.float64), cf.table[0], 50, 16)
    perm = np.random.default_rng(3).permutation(50)
    for t in range(50):
        pb, off = cf.table[0, t // 16], t % 16
        cf.k[pb, :, off, :] = kd[perm[t]].astype(np.float32)
        cf.v[pb, :, off, :] = vd[perm[t]].astype(np.float32)
    if not np.allclose(paged(cf)[0], o1, atol=1e-12, rtol=0):
        fails.append("token permutation")
    # adding the same vector to every key -> unchanged (keys hold bf16 values,
    # so adding +-0.25 per dimension is exact in fp32)
    cf = make_case(43, [50, 20], n_q=2, n_kv=1, d_h=32, kv_dtype=F32, q_dtype=F32)
    cf.k = synth.bf16_bits_to_f32(synth.bf16_bits_from_f32(cf.k))
    o1 = paged(cf)[0]
    u = np.where(np.random.default_rng(4).random(32) < 0.5, -0.25, 0.25).astype(np.float32)
    cf.k = cf.k + u
    o2 = paged(cf)[0]
    if not np.allclose(o2, o1, atol=1e-12, rtol=1e-12):
        fails.append("key shift")
    # affine map of values: out(aV + c) = a out(V) + c
    cf = make_case(44, [29, 64], n_q=2, n_kv=1, d_h=16, kv_dtype=F32, q_dtype=F32)
    cf.v = synth.bf16_bits_to_f32(synth.bf16_bits_from_f32(cf.v))  # 8 significant bits
    o1 = paged(cf)[0]
    cf.v = cf.v * np.float32(2.0) + np.float32(0.25)               # exact in fp32
    o2 = paged(cf)[0]
    if not np.allclose(o2, 2.0 * o1 + 0.25, atol=1e-12, rtol=1e-12):
        fails.append("affine values")
    return fails


def pin_split_merge(paged):
    fails = []
    c = make_case(51, [100, 37, 16], n_q=4, n_kv=2, d_h=32, kv_dtype=BF16, q_dtype=BF16)
    full = paged(c)[0]
    r = np.random.default_rng(9)
    for trial in range(4):
        n_max = int(c.ctx.max())
        cuts = sorted(set([0, n_max + 5] + list(r.integers(0, n_max + 5, size=trial + 2))))
        if trial == 3:
            cuts = list(range(0, n_max + 2))            # single-token partitions
        parts = [paged(c, t_begin=a, t_end=b) for a, b in zip(cuts[:-1], cuts[1:])]
        for row in range(c.B * c.n_q):
            o = np.stack([p[0][row] for p in parts])
            m = np.array([p[1][row] for p in parts])
            z = np.array([p[2][row] for p in parts])
            got = oracle.merge(o, m, z)
            if not np.allclose(got, full[row], atol=1e-12, rtol=1e-12):
                fails.append(f"merge trial {trial} row {row}")
                break
    return fails


def pin_errors(paged):
    fails = []
    c = make_case(61, [40, 0, 20], n_q=2, n_kv=1, d_h=16, kv_dtype=F32, q_dtype=F32)
    out, m, z, bad = paged(c)
    out = out.reshape(c.B, c.n_q, c.d_h)
    if bad != 0 or not (out[1] == 0).all():
        fails.append("empty row")
    t = c.table.copy()
    t[2, 0] = -1                                          # unmap row 2's first block
    c2 = make_case(61, [40, 0, 20], n_q=2, n_kv=1, d_h=16, kv_dtype=F32, q_dtype=F32)
    c2.table = t
    out2, _, _, bad2 = paged(c2)
    out2 = out2.reshape(c.B, c.n_q, c.d_h)
    if bad2 != 2 or not np.isnan(out2[2]).all() or not (out2[0] == out[0]).all():
        fails.append("unmapped block")
    return fails


def pin_window(paged):
    """Sliding window with attention sinks ("9 Decode and KV Cache", section
    9.7): positions t < S or t >= n - W of each row."""
    fails = []
    c = make_case(81, [100, 37, 200, 1, 16], n_q=4, n_kv=2, d_h=32, kv_dtype=F32, q_dtype=F32)
    full = paged(c)[0]
    # a window covering the whole row, or sinks + window covering it: no change
    if not (paged(c, window=200)[0] == full).all():
        fails.append("window >= n")
    if not (paged(c, window=150, sinks=60)[0] == full).all():
        fails.append("sinks + window >= n")
    # window 1, no sinks: the newest token's value, exactly
    one = paged(c, window=1)[0].reshape(c.B, c.n_q, c.d_h)
    vd = oracle.decode(c.v, F32)
    for b, n in enumerate(c.ctx):
        last = vd[c.table[b, (n - 1) // 16], :, (n - 1) % 16, :]
        if not (one[b] == np.repeat(last, c.g, axis=0)).all():
            fails.append(f"window 1 row {b}")
    # the independent gather-then-softmax reference, windows starting mid-block
    # and sinks crossing a block boundary
    for (w, sk) in [(5, 0), (17, 3), (33, 20), (64, 1), (3, 16)]:
        ours = paged(c, window=w, sinks=sk)[0].reshape(c.B, c.n_q, c.d_h)
        ref = brute.attention(c.q, c.k, c.v, c.table, c.ctx, c.scale, n_q=c.n_q, n_kv=c.n_kv,
                              q_dtype=c.q_dtype, kv_dtype=c.kv_dtype, window=w, sinks=sk)
        if not np.allclose(ours, ref, atol=1e-12, rtol=1e-12):
            fails.append(f"window brute force ({w}, {sk})")
    # unattended positions are never read: NaN there, and an unmapped block
    # that holds only unattended positions, change nothing
    w, sk = 20, 4
    ref = paged(c, window=w, sinks=sk)[0]
    c2 = make_case(81, [100, 37, 200, 1, 16], n_q=4, n_kv=2, d_h=32, kv_dtype=F32, q_dtype=F32)
    for b, n in enumerate(c2.ctx):
        for t in range(n):
            if not (t < sk or t >= n - w):
                pb = c2.table[b, t // 16]
                c2.k[pb, :, t % 16, :] = np.nan
                c2.v[pb, :, t % 16, :] = np.nan
    c2.table = c2.table.copy()
    c2.table[2, 5] = -1          # row 2 (200 tokens): block 5 holds positions 80..95 only
    got, _, _, bad = paged(c2, window=w, sinks=sk)
    if bad != 0 or not (got == ref).all():
        fails.append("unattended positions read")
    return fails


ALL_PINS = [pin_closed_forms, pin_brute_force, pin_gqa_is_repeated_mha, pin_invariances,
            pin_split_merge, pin_errors, pin_window]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_attention_pins(pin):
    assert pin(_paged) == []


def test_prefix_aliasing_bit_identical():
    c = make_case(71, [100, 70, 33, 17], n_q=4, n_kv=2, d_h=32, kv_dtype=BF16, q_dtype=BF16,
                  shared_prefix_blocks=4)
    assert (c.table[:, 0] == c.table[0, 0]).all()       # rows alias the same prefix blocks
    shared = _paged(c)[0]
    private = _paged(unshare(c))[0]
    assert (shared == private).all()


def test_prefix_block_table_worked_case():
    """Shared-prefix table (SoK paper section 2.6; copy on write, section 2.5):
    rows' first prefix_lens[b] logical blocks come from the prefix table,
    using the worked example's physical blocks 7, 2, 15 as the prefix."""
    bt = np.array([[-1, -1, 40, 41, -1],
                   [50, 51, 52, -1, -1],
                   [-1, -1, -1, 60, -1]], dtype=np.int32)
    table, bad = oracle.prefix_block_table(bt, [64, 40, 50], [7, 2, 15], [2, 0, 3])
    assert table.tolist() == [[7, 2, 40, 41, -1], [50, 51, 52, -1, -1], [7, 2, 15, 60, -1]]
    assert not bad.any()
    # validity: the newest token's block is private, the prefix fits its table
    L = oracle.prefix_row_len
    assert L(64, 3, 5, 3) == 3 and L(64, 4, 5, 4) == -1      # 4 blocks: at most 3 shared
    assert L(49, 3, 5, 3) == 3 and L(48, 3, 5, 3) == -1      # 48 tokens fill 3 blocks
    assert L(64, 3, 5, 2) == -1 and L(64, -1, 5, 3) == -1
    assert L(0, 7, 5, 3) == 0                                # empty row: no prefix
    assert L(-1, 0, 5, 3) == -1 and L(81, 0, 5, 3) == -1     # invalid lengths
    _, bad = oracle.prefix_block_table(bt, [64, 32, 50], [7, 2, 15], [2, 2, 3])
    assert bad.tolist() == [False, True, False]


def test_prefix_block_table_matches_the_cow_builder():
    """The copy-on-write builder shares min(n_shared, blocks - 1) leading
    blocks per row; the prefix table with those lengths reproduces its table,
    also where the rows' own entries for the prefix were never filled."""
    pool = oracle.OraclePool(64, list(np.random.default_rng(3).permutation(64)))
    shared = pool.alloc(5)
    ctx = [100, 16, 17, 80, 0, 1, 65]
    table, _ = pool.build_block_table(ctx, 16, 8, shared)
    lens = [min(5, max((n + 15) // 16 - 1, 0)) for n in ctx]
    eff, bad = oracle.prefix_block_table(table, ctx, shared, lens)
    assert (eff == table).all() and not bad.any()
    blank = table.copy()
    for b, pl in enumerate(lens):
        blank[b, :pl] = -1
    eff, bad = oracle.prefix_block_table(blank, ctx, shared, lens)
    assert (eff == table).all() and not bad.any()


def test_matches_torch_sdpa_fp64():
    """torch's fp64 scaled_dot_product_attention (a library routine) on the
    gathered contiguous sequence, with GQA."""
    import torch
    c = make_case(81, [77, 5, 130], n_q=8, n_kv=2, d_h=64, kv_dtype=BF16, q_dtype=BF16)
    ours = _paged(c)[0].reshape(c.B, c.n_q, c.d_h)
    qd = oracle.decode(c.q, BF16)
    kd = oracle.decode(c.k, BF16)
    vd = oracle.decode(c.v, BF16)
    for b in range(c.B):
        n = int(c.ctx[b])
        K = torch.from_numpy(brute.gather_contiguous(kd, c.table[b], n, 16)).permute(1, 0, 2)
        V = torch.from_numpy(brute.gather_contiguous(vd, c.table[b], n, 16)).permute(1, 0, 2)
        Q = torch.from_numpy(qd[b]).unsqueeze(1)                      # [n_q, 1, d]
        K = K.repeat_interleave(c.g, dim=0)
        V = V.repeat_interleave(c.g, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=c.scale)
        assert np.allclose(ours[b], ref[:, 0, :].numpy(), atol=1e-12, rtol=1e-12)


def test_quantized_attention_is_attention_of_dequantized_values():
    for dt in (FP8, INT8):
        c = make_case(91, [60, 33], n_q=4, n_kv=2, d_h=32, kv_dtype=dt, q_dtype=BF16)
        ours = _paged(c)[0]
        # dequantize by hand into an fp32 cache where exact (scale * code fits
        # fp32 only approximately), so compare against the brute force instead
        ref = brute.attention(c.q, c.k, c.v, c.table, c.ctx, c.scale, n_q=c.n_q, n_kv=c.n_kv,
                              q_dtype=c.q_dtype, kv_dtype=dt, k_scale=c.k_scale,
                              v_scale=c.v_scale).reshape(-1, c.d_h)
        assert np.allclose(ours, ref, atol=1e-12, rtol=1e-12)
        # scales equal to 1 reduce to the raw codes as values
        c.k_scale[:] = 1.0
        c.v_scale[:] = 1.0
        ones = _paged(c)[0]
        cf = make_case(91, [60, 33], n_q=4, n_kv=2, d_h=32, kv_dtype=F32, q_dtype=BF16)
        cf.k = oracle.decode(c.k, dt).astype(np.float32)
        cf.v = oracle.decode(c.v, dt).astype(np.float32)
        cf.q, cf.table, cf.ctx = c.q, c.table, c.ctx
        assert np.allclose(ones, _paged(cf)[0], atol=0, rtol=0, equal_nan=True)


# ---------------------------------------------------------------- append
def test_kv_append_places_rows_in_slots():
    g = json.load(open(os.path.join(GOLDEN, "block_lookup.json")))
    table = [g["block_table"][str(i)] for i in range(3)]
    cache = np.zeros((16, 2, 16, 8), dtype=np.uint16)
    tokens = [0, 17, 47]
    slots = np.array([oracle.slot_of(table, t, 16) for t in tokens] + [-1], dtype=np.int64)
    new = np.arange(4 * 2 * 8, dtype=np.uint16).reshape(4, 2, 8) + 1
    out = oracle.kv_append(cache, new, slots)
    for i, (tok, pb, off) in enumerate([(0, 7, 0), (17, 2, 1), (47, 15, 15)]):
        assert (out[pb, :, off, :] == new[i]).all()
    assert np.count_nonzero(out) == 3 * 2 * 8          # padding slot wrote nothing


def test_kv_append_quant_uses_destination_block_scale():
    r = np.random.default_rng(5)
    codes = np.zeros((4, 2, 16, 8), dtype=np.uint8)
    scales = np.float32([[0.5, 2.0], [0.25, 1.0], [1.0, 1.0], [4.0, 0.125]])
    new = r.standard_normal((2, 2, 8)).astype(np.float32) * 3
    slots = np.array([3 * 16 + 5, 1 * 16 + 0], dtype=np.int64)
    out = oracle.kv_append_quant(codes, scales, new, slots, FP8)
    tab = oracle.fp8_decode_table()
    for t, (pb, off) in enumerate([(3, 5), (1, 0)]):
        for h in range(2):
            dec = tab[out[pb, h, off, :]] * scales[pb, h]
            # each reconstructed value is within half a code step of the input
            assert np.all(np.abs(dec - new[t, h]) <= np.abs(new[t, h]) * 2.0 ** -4 + 2.0 ** -10)
    assert np.count_nonzero(out) > 0 and np.count_nonzero(out[0]) == 0


# ---------------------------------------------------------------- planted mistakes
MUTANTS = {
    "gqa head mapping": ("const int j = h / g;", "const int j = h % n_kv;"),
    "dropped scale": ("s[t - lo] = scale * dot;", "s[t - lo] = dot;"),
    "max subtracted with wrong sign": ("const double w = exp(s[t - lo] - m);",
                                       "const double w = exp(m - s[t - lo]);"),
    "keys read from V": ("dot += qd[d] * (ks * dkv(k, base + d));",
                         "dot += qd[d] * (ks * dkv(v, base + d));"),
    "missing normalisation": ("o[d] = acc[d] / z;", "o[d] = acc[d];"),
    "offset off by one": ("* bs + t % bs) * d_h;\n                const double ks",
                          "* bs + (t + 1) % bs) * d_h;\n                const double ks"),
    "block index from remainder": ("block_table[(int64_t)b * max_blocks + t / bs];\n                if (pb < 0",
                                   "block_table[(int64_t)b * max_blocks + t % bs];\n                if (pb < 0"),
    "value scale dropped": ("const double vs = quant ? (double)v_scale[(int64_t)pb * n_kv + j] : 1.0;",
                            "const double vs = 1.0;"),
    "window off by one": ("t >= n - window;", "t > n - window;"),
    "sinks dropped": ("window <= 0 || t < sinks || t >= n - window;",
                      "window <= 0 || t >= n - window;"),
}


def _build_mutant(src_text: str, old: str, new: str, tmp: str):
    assert old in src_text, old
    path_c = os.path.join(tmp, "m.c")
    with open(path_c, "w") as f:
        f.write(src_text.replace(old, new, 1))
    path_so = os.path.join(tmp, "m.so")
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", path_c, "-o",
                    path_so, "-lm"], check=True)
    return oracle.load(path_so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "pda_oracle.c")).read()
    tmp = tempfile.mkdtemp(prefix="oracle_mutant_")
    try:
        L = _build_mutant(src, *MUTANTS[name], tmp)
        paged = lambda case, **kw: _paged(case, _lib=L, **kw)
        fails = []
        for pin in ALL_PINS:
            try:
                fails += pin(paged)
            except (AssertionError, ValueError, KeyError, FloatingPointError):
                fails.append(pin.__name__ + " raised")
            if fails:
                break
        if not fails:   # quantized pins (scales) live in a separate test
            c = make_case(91, [60, 33], n_q=4, n_kv=2, d_h=32, kv_dtype=INT8, q_dtype=BF16)
            ref = brute.attention(c.q, c.k, c.v, c.table, c.ctx, c.scale, n_q=c.n_q,
                                  n_kv=c.n_kv, q_dtype=c.q_dtype, kv_dtype=INT8,
                                  k_scale=c.k_scale, v_scale=c.v_scale).reshape(-1, c.d_h)
            if not np.allclose(paged(c)[0], ref, atol=1e-12, rtol=1e-12):
                fails.append("quantized brute force")
        assert fails, f"planted mistake '{name}' passed every pin"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_planted_fp8_bias_mistake_is_caught():
    src = open(os.path.join(os.path.dirname(oracle.__file__), "pda_oracle.c")).read()
    tmp = tempfile.mkdtemp(prefix="oracle_mutant_")
    try:
        L = _build_mutant(src, "(int)e - 7", "(int)e - 8", tmp)   # FNUZ-style bias
        import torch
        codes = np.arange(256, dtype=np.uint8)
        ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        got = np.array([L.or_dec_fp8_code(int(c)) for c in codes])
        same = (got == ref) | (np.isnan(got) & np.isnan(ref))
        assert not same.all()
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
