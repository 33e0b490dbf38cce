"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small cases (many tiles, ragged tails, every dtype and head-group size) are
compared element by element. Bars: max-abs 5e-3 for bf16 / fp32 caches, 3e-2
for fp8 / int8 caches against the oracle on the dequantized cache, and beside
them a 1e-4 regression bound on the precision the kernels reach; bit-exact
for appends and for invariances that fix the reduction order (physical block
renumbering, prefix aliasing, reruns).
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest

import oracle
from synth import F32, BF16, FP8, INT8
from tests.helpers import make_case, permute_physical, unshare
from tests.gpu_helpers import TOL_16BIT, TOL_8BIT, TOL_REGRESSION, assert_parity, max_err, run_case, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CTX_RAGGED = [1, 15, 16, 17, 100, 257, 513, 1000]


@pytest.mark.parametrize("d_h", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
def test_bf16_cache_ragged(d_h, g):
    n_kv = 2 if g <= 8 else 1
    c = make_case(1000 + g + d_h, CTX_RAGGED, n_q=g * n_kv, n_kv=n_kv, d_h=d_h)
    _say(f"bf16 cache d_h={d_h} g={g}")
    got, _ = run_case(c)
    ref = c.oracle_out()
    assert_parity(max_err(got, ref), TOL_16BIT)


@pytest.mark.parametrize("parts", [1, 2, 3, 7, 0])
def test_split_partitions_agree(parts):
    c = make_case(2000 + parts, [2000, 1, 700, 1999, 64], n_q=16, n_kv=2, d_h=128)
    _say(f"split partitions={parts}")
    got, desc = run_case(c, num_partitions=parts)
    ref = c.oracle_out()
    assert_parity(max_err(got, ref), TOL_16BIT)


@pytest.mark.parametrize("nw", [2, 3, 5, 7, 13, 64, 1000])
@pytest.mark.parametrize("kv_dtype", [BF16, FP8])
def test_stream_ranges_ragged_with_empty_rows(nw, kv_dtype):
    """Wave ranges cut the flattened (sequence, KV head, block) axis at
    arbitrary points: pieces of one segment across several waves, several
    segments in one wave, more ranges than blocks, and sequences with no
    blocks at the start, middle and end of the batch."""
    ctx = [0, 700, 1, 0, 33, 2000, 16, 0]
    c = make_case(2500 + nw + 10 * kv_dtype, ctx, n_q=16, n_kv=2, d_h=128, kv_dtype=kv_dtype)
    _say(f"stream ranges nw={nw} kv={kv_dtype}")
    got, desc = run_case(c, num_partitions=nw)
    ref = c.oracle_out()
    for b in (0, 3, 7):
        assert (got[b] == 0).all()
    assert_parity(max_err(got, ref), (TOL_8BIT if kv_dtype == FP8 else TOL_16BIT))


@pytest.mark.parametrize("d_h", [64, 128])
@pytest.mark.parametrize("g", [1, 3, 16])
def test_stream_default_plan_many_short_rows(d_h, g):
    """A batch of many short, ragged rows on the library's own plan."""
    r = np.random.default_rng(2600 + d_h + g)
    ctx = r.integers(0, 300, size=40).tolist()
    n_kv = 1 if g == 16 else 2
    c = make_case(2600 + d_h + g, ctx, n_q=g * n_kv, n_kv=n_kv, d_h=d_h)
    _say(f"stream default plan d_h={d_h} g={g}")
    got, _ = run_case(c, total_context=int(sum(ctx)))
    assert_parity(max_err(got, c.oracle_out()), TOL_16BIT)
    got2, _ = run_case(c, num_partitions=97)
    assert_parity(max_err(got2, c.oracle_out()), TOL_16BIT)


WINDOWS = [(1, 0), (20, 4), (33, 17), (100, 0), (5, 40), (4096, 4)]


@pytest.mark.parametrize("kv_dtype", [BF16, FP8, F32])
@pytest.mark.parametrize("window,sinks", WINDOWS)
@pytest.mark.parametrize("nw", [0, 1, 7])
def test_window_with_sinks(kv_dtype, window, sinks, nw):
    """Sliding window with attention sinks: positions outside it are NaN-
    poisoned and one block holding only such positions is unmapped; neither
    may reach the output."""
    import synth
    ctx = [0, 700, 1, 33, 2000, 16, 300]
    c = make_case(2700 + window + sinks + kv_dtype, ctx, n_q=8, n_kv=2, d_h=128,
                  kv_dtype=kv_dtype, q_dtype=BF16 if kv_dtype != F32 else F32)
    nan = {F32: np.float32(np.nan), BF16: synth.BF16_NAN, FP8: synth.FP8_NAN}[kv_dtype]
    table = c.table.copy()
    for b, n in enumerate(c.ctx):
        for t in range(n):
            if not (t < sinks or t >= n - window):
                pb = table[b, t // 16]
                c.k[pb, :, t % 16, :] = nan
                c.v[pb, :, t % 16, :] = nan
        # unmap the blocks that hold no attended position (never looked up)
        for blk in range((n + 15) // 16):
            if all(not (t < sinks or t >= n - window) for t in range(16 * blk, min(n, 16 * blk + 16))):
                table[b, blk] = -1
    _say(f"window={window} sinks={sinks} kv={kv_dtype} nw={nw}")
    got, _ = run_case(c, table=table, window=window, sinks=sinks, num_partitions=nw)
    ref = c.oracle_out(window=window, sinks=sinks)
    assert (got[0] == 0).all()
    assert_parity(max_err(got, ref), (TOL_8BIT if kv_dtype == FP8 else TOL_16BIT))


def test_fp32_query_with_bf16_cache():
    c = make_case(3001, CTX_RAGGED, n_q=8, n_kv=2, d_h=128, q_dtype=F32)
    _say("fp32 q, bf16 cache")
    got, _ = run_case(c)
    assert_parity(max_err(got, c.oracle_out()), TOL_16BIT)


@pytest.mark.parametrize("q_dtype", [F32, BF16])
@pytest.mark.parametrize("d_h", [64, 128])
def test_fp32_cache(q_dtype, d_h):
    c = make_case(3100 + d_h + q_dtype, CTX_RAGGED, n_q=8, n_kv=2, d_h=d_h, kv_dtype=F32,
                  q_dtype=q_dtype)
    _say(f"fp32 cache q={q_dtype} d_h={d_h}")
    got, _ = run_case(c)
    assert_parity(max_err(got, c.oracle_out()), TOL_16BIT)
    got2, _ = run_case(c, num_partitions=3)
    assert_parity(max_err(got2, c.oracle_out()), TOL_16BIT)


@pytest.mark.parametrize("g", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("nparts", [0, 1, 4])
def test_fp32_cache_query_groups(g, nparts):
    """fp32 caches: one workgroup per (partition, KV head, row) serves all g
    query heads of the group (head lanes and block lanes of its waves)."""
    c = make_case(3200 + 10 * g + nparts, CTX_RAGGED, n_q=2 * g, n_kv=2, d_h=128,
                  kv_dtype=F32, q_dtype=F32)
    _say(f"fp32 cache g={g} partitions={nparts}")
    got, _ = run_case(c, num_partitions=nparts)
    assert_parity(max_err(got, c.oracle_out()), TOL_16BIT)


@pytest.mark.parametrize("kv_dtype", [FP8, INT8])
@pytest.mark.parametrize("d_h", [64, 128])
@pytest.mark.parametrize("g", [1, 4, 8])
def test_quantized_cache(kv_dtype, d_h, g):
    c = make_case(4000 + 10 * g + d_h + kv_dtype, CTX_RAGGED, n_q=2 * g, n_kv=2, d_h=d_h,
                  kv_dtype=kv_dtype)
    _say(f"quantized cache dtype={kv_dtype} d_h={d_h} g={g}")
    got, _ = run_case(c)
    assert_parity(max_err(got, c.oracle_out()), TOL_8BIT)


def test_bf16_output_is_rne_of_fp32_output():
    import torch
    c = make_case(5001, CTX_RAGGED, n_q=8, n_kv=2, d_h=128)
    _say("bf16 output")
    f32, _ = run_case(c)
    b16, _ = run_case(c, out_dtype=BF16)
    ref = torch.from_numpy(f32).to(torch.bfloat16).float().numpy()
    assert (b16 == ref).all()


def test_physical_permutation_bit_identical():
    c = make_case(6001, CTX_RAGGED, n_q=16, n_kv=2, d_h=128)
    _say("physical block permutation")
    a, _ = run_case(c)
    b, _ = run_case(permute_physical(c, 7))
    assert (a == b).all()
    a2, _ = run_case(c, num_partitions=4)
    b2, _ = run_case(permute_physical(c, 8), num_partitions=4)
    assert (a2 == b2).all()


def test_prefix_aliasing_bit_identical():
    c = make_case(6101, [300, 70, 33, 17, 1], n_q=8, n_kv=2, d_h=128, shared_prefix_blocks=8)
    _say("prefix aliasing")
    a, _ = run_case(c)
    b, _ = run_case(unshare(c))
    assert (a == b).all()
    assert_parity(max_err(a, c.oracle_out()), TOL_16BIT)


@pytest.mark.parametrize("kv_dtype", [BF16, FP8])
def test_reuse_hint_changes_nothing(kv_dtype):
    """The shared-prefix cache hint only picks the load flavour: results are
    bit-identical for any value."""
    c = make_case(6301 + kv_dtype, [300, 70, 33, 17, 1, 0], n_q=8, n_kv=2, d_h=128,
                  shared_prefix_blocks=4, kv_dtype=kv_dtype)
    _say(f"reuse hint kv={kv_dtype}")
    base, _ = run_case(c, num_partitions=5)
    for reuse in (1, 4, 1000):
        got, _ = run_case(c, num_partitions=5, reuse_prefix_blocks=reuse)
        assert (got == base).all()


def test_rerun_deterministic():
    c = make_case(6201, CTX_RAGGED, n_q=16, n_kv=2, d_h=128)
    _say("determinism")
    a, _ = run_case(c)
    b, _ = run_case(c)
    assert (a == b).all()


def test_empty_rows_and_single_token():
    c = make_case(7001, [0, 1, 0, 33], n_q=8, n_kv=2, d_h=128)
    _say("empty rows")
    for parts in (1, 0, 2):
        got, _ = run_case(c, num_partitions=parts)
        assert (got[0] == 0).all() and (got[2] == 0).all()
        # one token: softmax weight exactly 1, output equals that value row
        v = oracle.decode(c.v, BF16)
        pb = c.table[1, 0]
        for h in range(c.n_q):
            assert (got[1, h] == v[pb, h // c.g, 0, :].astype(np.float32)).all()
        assert_parity(max_err(got[3], c.oracle_out()[3]), TOL_16BIT)


@pytest.mark.parametrize("parts", [1, 3])
def test_unmapped_block_poisons_only_its_row(parts):
    c = make_case(7101, [100, 70, 200], n_q=8, n_kv=2, d_h=128)
    t = c.table.copy()
    t[1, 2] = -1                     # unmap a block in the middle of row 1
    t2 = c.table.copy()
    t2[2, 0] = c.num_blocks + 5      # out-of-range physical id in row 2
    _say(f"unmapped block parts={parts}")
    got, _ = run_case(c, table=t, num_partitions=parts)
    ref = c.oracle_out()
    assert np.isnan(got[1]).all()
    assert_parity(max_err(got[[0, 2]], ref[[0, 2]]), TOL_16BIT)
    got, _ = run_case(c, table=t2, num_partitions=parts)
    assert np.isnan(got[2]).all()
    assert_parity(max_err(got[[0, 1]], ref[[0, 1]]), TOL_16BIT)


@pytest.mark.parametrize("bad_id", [-1, 1 << 20])
@pytest.mark.parametrize("kv", [BF16, FP8])
def test_bad_block_in_a_later_metadata_batch(bad_id, kv):
    """Waves of more than 64 blocks read their block ids in batches of 64;
    an unmapped or out-of-range id in the second batch poisons its row only
    (the id is checked where it is used, not where the batch is loaded)."""
    c = make_case(7151, [3000, 2900, 64], n_q=8, n_kv=2, d_h=128, kv_dtype=kv)
    t = c.table.copy()
    t[0, 150] = bad_id              # block 150 of row 0: the second batch of its wave
    _say(f"bad id {bad_id} in a later batch kv={kv}")
    got, _ = run_case(c, table=t, num_partitions=3)
    ref = c.oracle_out()
    assert np.isnan(got[0]).all()
    assert_parity(max_err(got[[1, 2]], ref[[1, 2]]), TOL_16BIT if kv == BF16 else TOL_8BIT)


@pytest.mark.parametrize("parts", [0, 1, 4])
def test_context_beyond_table_is_nan(parts):
    c = make_case(7201, [40, 20], n_q=4, n_kv=2, d_h=64, max_blocks=3)
    bad = c.ctx.copy()
    bad[1] = 3 * 16 + 1              # more tokens than the table can hold
    c2 = make_case(7201, [40, 20], n_q=4, n_kv=2, d_h=64, max_blocks=3)
    c2.ctx = bad
    _say(f"context beyond table parts={parts}")
    got, _ = run_case(c2, max_context=40, num_partitions=parts)
    assert np.isnan(got[1]).all()
    assert_parity(max_err(got[0], c.oracle_out()[0]), TOL_16BIT)


def test_context_above_max_context_still_complete():
    """max_context only sizes the split: a longer row is still attended in full."""
    c = make_case(7301, [900, 50], n_q=8, n_kv=2, d_h=128)
    _say("context above max_context")
    got, _ = run_case(c, max_context=64, num_partitions=4)
    assert_parity(max_err(got, c.oracle_out()), TOL_16BIT)


# ------------------------------------------------------------------- append
def _append_case(seed, dtype, T=37, n_kv=4, d_h=128, nb=40):
    r = np.random.default_rng(seed)
    import synth
    cache_k = synth.gaussian((nb, n_kv, 16, d_h), dtype, r)
    cache_v = synth.gaussian((nb, n_kv, 16, d_h), dtype, r)
    new_k = synth.gaussian((T, n_kv, d_h), dtype, r)
    new_v = synth.gaussian((T, n_kv, d_h), dtype, r)
    slots = r.choice(nb * 16, size=T, replace=False).astype(np.int64)
    slots[3] = -1                    # padding token
    slots[5] = nb * 16 + 3           # beyond the cache: skipped
    return cache_k, cache_v, new_k, new_v, slots


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("d_h", [64, 128])
def test_kv_append_bit_exact(dtype, d_h):
    import torch
    import decode_attention_paged_slot_amd as pda
    ck, cv, nk, nv, slots = _append_case(8000 + dtype + d_h, dtype, d_h=d_h)
    _say(f"kv_append dtype={dtype} d_h={d_h}")
    dk, dv = to_dev(ck, dtype, "cuda"), to_dev(cv, dtype, "cuda")
    pda.kv_append(to_dev(nk, dtype, "cuda"), to_dev(nv, dtype, "cuda"),
                  torch.from_numpy(slots).cuda(), dk, dv)
    torch.cuda.synchronize()
    valid = np.where(slots < ck.shape[0] * 16, slots, -1)
    ref_k = oracle.kv_append(ck, nk, valid)
    ref_v = oracle.kv_append(cv, nv, valid)
    view = np.int16 if dtype == BF16 else np.int32
    gk = dk.view(torch.int16 if dtype == BF16 else torch.int32).cpu().numpy()
    gv = dv.view(torch.int16 if dtype == BF16 else torch.int32).cpu().numpy()
    assert (gk == ref_k.view(view)).all()
    assert (gv == ref_v.view(view)).all()


@pytest.mark.parametrize("cache_dtype", [FP8, INT8])
@pytest.mark.parametrize("src_dtype", [F32, BF16])
def test_kv_append_quant_bit_exact(cache_dtype, src_dtype):
    import torch
    import synth
    import decode_attention_paged_slot_amd as pda
    r = np.random.default_rng(9000 + cache_dtype * 2 + src_dtype)
    nb, n_kv, d_h, T = 30, 4, 128, 25
    codes_k = r.integers(0, 256, size=(nb, n_kv, 16, d_h)).astype(np.uint8)
    codes_v = r.integers(0, 256, size=(nb, n_kv, 16, d_h)).astype(np.uint8)
    if cache_dtype == INT8:
        codes_k, codes_v = codes_k.view(np.int8), codes_v.view(np.int8)
    ks = (np.abs(r.standard_normal((nb, n_kv))) * 0.05 + 1e-3).astype(np.float32)
    vs = (np.abs(r.standard_normal((nb, n_kv))) * 0.05 + 1e-3).astype(np.float32)
    x = (r.standard_normal((T, n_kv, d_h)) * 8).astype(np.float32)
    # special values: saturation, ties at half-code points, zeros, NaN, tiny
    x[0, 0, :8] = [1e9, -1e9, 0.0, -0.0, np.nan, 1e-30, -1e-30, np.inf]
    raw_k = synth.bf16_bits_from_f32(x) if src_dtype == BF16 else x
    raw_v = synth.bf16_bits_from_f32(-x) if src_dtype == BF16 else -x
    xf_k = synth.bf16_bits_to_f32(raw_k) if src_dtype == BF16 else raw_k
    xf_v = synth.bf16_bits_to_f32(raw_v) if src_dtype == BF16 else raw_v
    slots = r.choice(nb * 16, size=T, replace=False).astype(np.int64)
    slots[2] = -1
    _say(f"kv_append_quant cache={cache_dtype} src={src_dtype}")
    dk = torch.from_numpy(codes_k.copy()).cuda()
    dv = torch.from_numpy(codes_v.copy()).cuda()
    pda.kv_append_quant(to_dev(raw_k, src_dtype, "cuda"), to_dev(raw_v, src_dtype, "cuda"),
                        torch.from_numpy(slots).cuda(), dk, dv, torch.from_numpy(ks).cuda(),
                        torch.from_numpy(vs).cuda(), cache_dtype=cache_dtype)
    torch.cuda.synchronize()
    ref_k = oracle.kv_append_quant(codes_k, ks, xf_k, slots, cache_dtype)
    ref_v = oracle.kv_append_quant(codes_v, vs, xf_v, slots, cache_dtype)
    assert (dk.cpu().numpy() == ref_k).all()
    assert (dv.cpu().numpy() == ref_v).all()


def test_kv_append_quant_ties_and_saturation_exact():
    """Inputs placed exactly on fp8 half-code points and beyond +-448 with
    scale 1: the kernel's rounding must pick the same (even) codes."""
    import torch
    import decode_attention_paged_slot_amd as pda
    vals = oracle.fp8_decode_table()[:0x7F]
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    extra = np.float32([448.0, 449.0, 464.0, 465.0, 1e6, 0.0, 2.0 ** -10, 2.0 ** -9 * 0.75])
    x = np.concatenate([mids, -mids, extra, -extra])
    d_h = 128
    T = (x.size + d_h - 1) // d_h
    xx = np.zeros(T * d_h, dtype=np.float32)
    xx[:x.size] = x
    xx = xx.reshape(T, 1, d_h)
    nb = T
    ks = np.ones((nb, 1), dtype=np.float32)
    slots = (np.arange(T) * 16 + 3).astype(np.int64)
    codes = np.zeros((nb, 1, 16, d_h), dtype=np.uint8)
    _say("kv_append_quant ties")
    dk = torch.from_numpy(codes.copy()).cuda()
    dv = torch.from_numpy(codes.copy()).cuda()
    xt = torch.from_numpy(xx).cuda()
    pda.kv_append_quant(xt, xt, torch.from_numpy(slots).cuda(), dk, dv,
                        torch.from_numpy(ks).cuda(), torch.from_numpy(ks).cuda(),
                        cache_dtype=FP8)
    torch.cuda.synchronize()
    ref = oracle.kv_append_quant(codes, ks, xx, slots, FP8)
    assert (dk.cpu().numpy() == ref).all()


# ------------------------------------------------------------------- merge
def test_lse_merge_matches_oracle_merge():
    import torch
    import decode_attention_paged_slot_amd as pda
    c = make_case(9501, [300, 47, 129], n_q=8, n_kv=2, d_h=128)
    cuts = [0, 16, 17, 100, 160, 160, 301]        # includes an empty partition
    parts = [c.oracle(t_begin=a, t_end=b) for a, b in zip(cuts[:-1], cuts[1:])]
    rows = c.B * c.n_q
    P = len(parts)
    po = np.zeros((rows, P, c.d_h), dtype=np.float32)
    pml = np.zeros((rows, P, 2), dtype=np.float32)
    ref = np.zeros((rows, c.d_h))
    for r in range(rows):
        o = np.stack([p[0][r] for p in parts])
        m = np.array([p[1][r] for p in parts])
        z = np.array([p[2][r] for p in parts])
        ref[r] = oracle.merge(o, m, z)
        po[r] = np.where(z[:, None] > 0, o, 0.0)
        pml[r, :, 0] = np.where(z > 0, m * np.log2(np.e), -np.inf)
        pml[r, :, 1] = z
    _say("lse merge")
    out = torch.empty((rows, c.d_h), device="cuda")
    pda.lse_merge(torch.from_numpy(po).cuda(), torch.from_numpy(pml).cuda(), out)
    torch.cuda.synchronize()
    assert max_err(out.cpu().numpy(), ref) < 1e-5
    assert max_err(out.cpu().numpy(), c.oracle_out().reshape(rows, -1)) < 1e-5


# ------------------------------------------------------------------- merge
@pytest.mark.parametrize("d_h", [64, 128])
@pytest.mark.parametrize("out_dtype", [F32, BF16])
def test_merge_many_pieces_per_row(d_h, out_dtype):
    """One long row split into ~1000 pieces: the merge takes its pieces in
    several batches (rescaling between them), over column slices of a row."""
    c = make_case(8100 + d_h + out_dtype, [20000], n_q=4, n_kv=1, d_h=d_h)
    _say(f"merge many pieces d_h={d_h} out={out_dtype}")
    got, _ = run_case(c, num_partitions=1000, out_dtype=out_dtype)
    ref = c.oracle_out()
    tol = TOL_16BIT if out_dtype == F32 else 2e-2   # bf16 output: half an ulp at |x| < 4
    assert_parity(max_err(got, ref), tol, None if out_dtype == BF16 else TOL_REGRESSION)


@pytest.mark.parametrize("d_h", [64, 128])
@pytest.mark.parametrize("nw", [200, 2047])
def test_merge_one_long_row_among_short(d_h, nw):
    """A long row among short ones: its segments take most of the wave ranges
    (far more pieces than the average the merge is laid out for), the short
    rows one or two pieces each."""
    ctx = [100] * 16
    ctx[5] = 30000
    ctx[11] = 3
    c = make_case(8200 + d_h + nw, ctx, n_q=8, n_kv=2, d_h=d_h)
    _say(f"merge long row among short d_h={d_h} nw={nw}")
    got, _ = run_case(c, num_partitions=nw)
    assert_parity(max_err(got, c.oracle_out()), TOL_16BIT)


@pytest.mark.parametrize("nw", [7, 1000])
def test_merge_nan_piece_poisons_row(nw):
    """An unmapped block inside a split row: its piece carries a NaN sum, and
    the merged row must be NaN while the other rows stay exact."""
    c = make_case(8300 + nw, [5000, 4000, 3000], n_q=8, n_kv=2, d_h=128)
    t = c.table.copy()
    t[1, 100] = -1
    _say(f"merge nan piece nw={nw}")
    got, _ = run_case(c, table=t, num_partitions=nw)
    ref = c.oracle_out()
    assert np.isnan(got[1]).all()
    assert_parity(max_err(got[[0, 2]], ref[[0, 2]]), TOL_16BIT)


@pytest.mark.parametrize("kv_dtype", [INT8, FP8, BF16])
@pytest.mark.parametrize("nw", [0, 4])
def test_unattended_slots_are_never_read(kv_dtype, nw):
    """Slots that hold no attended position (the tail of each row's last
    block, and every block no row owns, with its scales) are never read: two
    runs that differ only there give bit-identical output. The synthetic int8
    poison is a finite code (-128), so for int8 only this check shows that no
    stray read happens."""
    c = make_case(9700 + 10 * kv_dtype + nw, CTX_RAGGED, n_q=8, n_kv=2, d_h=128,
                  kv_dtype=kv_dtype)
    _say(f"unattended slots dtype={kv_dtype} nw={nw}")
    a, _ = run_case(c, num_partitions=nw)
    assert_parity(max_err(a, c.oracle_out()), TOL_8BIT if kv_dtype in (FP8, INT8) else TOL_16BIT)
    attended = np.zeros(c.k.shape[:1] + c.k.shape[2:3], dtype=bool)   # [block, offset]
    for b in range(c.B):
        for t in range(int(c.ctx[b])):
            attended[c.table[b, t // c.bs], t % c.bs] = True
    r = np.random.default_rng(98 + kv_dtype)
    k2, v2 = c.k.copy(), c.v.copy()
    for x in (k2, v2):
        raw = x.view(np.uint8 if x.dtype.itemsize == 1 else np.uint16)
        noise = r.integers(0, 1 << (8 * x.dtype.itemsize), size=raw.shape).astype(raw.dtype)
        sel = ~attended[:, None, :, None].repeat(c.n_kv, 1).repeat(c.d_h, 3)
        raw[sel] = noise[sel]
    ks2 = vs2 = None
    if c.k_scale is not None:
        unowned = ~attended.any(axis=1)
        ks2, vs2 = c.k_scale.copy(), c.v_scale.copy()
        ks2[unowned] = r.uniform(0.5, 2.0, size=ks2[unowned].shape).astype(np.float32)
        vs2[unowned] = r.uniform(0.5, 2.0, size=vs2[unowned].shape).astype(np.float32)
    c2 = dataclasses.replace(c, k=k2, v=v2, k_scale=ks2, v_scale=vs2)
    b, _ = run_case(c2, num_partitions=nw)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
