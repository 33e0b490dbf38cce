"""The 4-bit cache with a residual window on the GPU against the oracle
(oracle/int4.py): the append policy bit for bit over consecutive steps that
fill blocks, and attention over encoded blocks plus residual windows.

Cache contents are drawn directly as codes (a centred binomial in [-7, 7],
stored as code + 8 nibbles), per-channel key scales with outlier channels,
per-token value scales and bf16 residual rows; nothing is quantized on the
way in. Blocks not owned by a row and the block behind a row's residual
window carry NaN value scales, and residual slots past a row's length NaN
rows, so any read of them shows up.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from oracle import int4
import synth
from synth import F32, BF16
from tests.gpu_helpers import TOL_8BIT, assert_parity, to_dev

pytestmark = pytest.mark.gpu

INT4 = 4


def _codes(shape, r):
    return (r.binomial(14, 0.5, size=shape) - 7).astype(np.int8)


def _bytes(shape, r):
    """Random packed bytes: two independent codes per byte."""
    lo = _codes(shape, r) + 8
    hi = _codes(shape, r) + 8
    return (lo.astype(np.uint8) | (hi.astype(np.uint8) << 4)).astype(np.uint8)


def _case(seed, ctx, *, n_q, n_kv, d_h, extra=3, poison=True):
    r = np.random.default_rng(seed)
    ctx = np.asarray(ctx, np.int32)
    B = ctx.size
    nblk = (ctx.astype(np.int64) + 15) // 16
    nb = int(nblk.sum()) + extra
    mb = max(int(nblk.max()), 1)
    pool = oracle.OraclePool(nb, list(r.permutation(nb)))
    table, _ = pool.build_block_table(ctx, 16, mb)
    st = {"k": _bytes((nb, n_kv, 16, d_h // 2), r),
          "v": _bytes((nb, n_kv, 16, d_h // 2), r),
          "v_scale": r.uniform(0.1, 0.5, size=(nb, n_kv, 16)).astype(np.float32),
          "k_res": synth.gaussian((B, n_kv, 16, d_h), BF16, r),
          "v_res": synth.gaussian((B, n_kv, 16, d_h), BF16, r)}
    mag = np.where(np.arange(d_h) % 32 == 5, 8.0, 1.0)
    ks = (r.uniform(0.15, 0.3, size=(n_kv, d_h)) * mag).astype(np.float32)
    if poison:
        owned = np.zeros(nb, bool)
        for b, n in enumerate(ctx):
            full = int(n) // 16
            owned[table[b, :full]] = True
        st["v_scale"][~owned] = np.nan
        nan16 = np.uint16(0x7FC0)
        for b, n in enumerate(ctx):
            st["k_res"][b, :, int(n) % 16:, :] = nan16
            st["v_res"][b, :, int(n) % 16:, :] = nan16
    return st, ks, table, ctx, nb, mb


def _dev(st, ks, dev):
    import torch
    return ({"k": torch.from_numpy(st["k"]).to(dev), "v": torch.from_numpy(st["v"]).to(dev),
             "v_scale": torch.from_numpy(st["v_scale"]).to(dev),
             "k_res": to_dev(st["k_res"], BF16, dev), "v_res": to_dev(st["v_res"], BF16, dev)},
            torch.from_numpy(ks).to(dev))


def _desc(B, n_q, n_kv, d_h, mb, nb, q_dtype, out_dtype, ctx, nw):
    import decode_attention_paged_slot_amd as pda
    return pda.AttnDesc(B, n_q, n_kv, d_h, 16, mb, nb, INT4, q_dtype, out_dtype,
                        int(max(ctx.max(), 0)), nw, int(ctx.sum()), 0, 0, 0, BF16, 0)


def _attend(st_d, ks_d, q, table, ctx, scale, desc, out_dtype=F32, dev="cuda"):
    import torch
    import decode_attention_paged_slot_amd as pda
    B, n_q, d_h = q.shape
    out = torch.full((B, n_q, d_h), float("nan"), device=dev,
                     dtype=torch.float32 if out_dtype == F32 else torch.bfloat16)
    ws = pda.workspace_for(desc, dev)
    pda.paged_decode_attn_int4(q, st_d["k"], st_d["v"], ks_d, st_d["v_scale"], st_d["k_res"],
                               st_d["v_res"], torch.from_numpy(table).to(dev),
                               torch.from_numpy(ctx).to(dev), scale, out, desc=desc, workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


CONFIGS = [(128, 8, 1, BF16), (128, 32, 8, BF16), (128, 8, 2, F32), (64, 8, 2, BF16),
           (64, 4, 4, F32)]
CTX = [0, 1, 15, 16, 17, 33, 48, 700, 2063, 4096, 31]


@pytest.mark.parametrize("d_h,n_q,n_kv,qd", CONFIGS)
@pytest.mark.parametrize("nw", [0, 1, 7])
def test_int4_attention_matches_oracle(d_h, n_q, n_kv, qd, nw):
    print(f"int4 attention d_h={d_h} heads={n_q}/{n_kv} q={qd} nw={nw}", flush=True)
    sys.stdout.flush()
    st, ks, table, ctx, nb, mb = _case(5000 + d_h + n_q + nw, CTX, n_q=n_q, n_kv=n_kv, d_h=d_h)
    r = np.random.default_rng(9)
    q_np = synth.gaussian((ctx.size, n_q, d_h), qd, r)
    dev = "cuda"
    st_d, ks_d = _dev(st, ks, dev)
    q = to_dev(q_np, qd, dev)
    scale = 1.0 / np.sqrt(d_h)
    got = _attend(st_d, ks_d, q, table, ctx, scale,
                  _desc(ctx.size, n_q, n_kv, d_h, mb, nb, qd, F32, ctx, nw))
    ref, _, _, bad = oracle.paged_attn_int4(q_np, st, ks, table, ctx, scale, n_q=n_q, n_kv=n_kv,
                                            q_dtype=qd)
    assert bad == 0
    ref = ref.reshape(got.shape)
    assert np.isfinite(got).all()
    assert_parity(float(np.abs(got - ref).max()), TOL_8BIT)
    assert (got[0] == 0).all()   # empty row


@pytest.mark.parametrize("d_h", [128, 64])
@pytest.mark.parametrize("n", [4001, 4015, 4096])
def test_int4_column_split_merge(d_h, n):
    """One long row over 128 waves: the merge splits the row's columns over
    several workgroups, each forming its own share of the residual piece
    (residual windows of 1, 15 and no tokens)."""
    print(f"int4 column-split merge d_h={d_h} n={n}", flush=True)
    sys.stdout.flush()
    st, ks, table, ctx, nb, mb = _case(5400 + d_h + n, [n], n_q=8, n_kv=1, d_h=d_h)
    r = np.random.default_rng(12)
    q_np = synth.gaussian((1, 8, d_h), BF16, r)
    st_d, ks_d = _dev(st, ks, "cuda")
    scale = 1.0 / np.sqrt(d_h)
    desc = _desc(1, 8, 1, d_h, mb, nb, BF16, F32, ctx, 128)
    import decode_attention_paged_slot_amd as pda
    assert pda.attn_plan(desc)[0] == 128   # 128 waves for one (row, head) segment
    got = _attend(st_d, ks_d, to_dev(q_np, BF16, "cuda"), table, ctx, scale, desc)
    ref, _, _, bad = oracle.paged_attn_int4(q_np, st, ks, table, ctx, scale, n_q=8, n_kv=1,
                                            q_dtype=BF16)
    assert bad == 0
    assert np.isfinite(got).all()
    assert_parity(float(np.abs(got - ref.reshape(got.shape)).max()), TOL_8BIT)


def test_int4_bf16_output_and_invalid_rows():
    import torch
    st, ks, table, ctx, nb, mb = _case(5100, [300, 17, 40, 5, 64], n_q=8, n_kv=2, d_h=128)
    r = np.random.default_rng(10)
    q_np = synth.gaussian((ctx.size, 8, 128), BF16, r)
    dev = "cuda"
    st_d, ks_d = _dev(st, ks, dev)
    q = to_dev(q_np, BF16, dev)
    ref, _, _, _ = oracle.paged_attn_int4(q_np, st, ks, table, ctx, 0.1, n_q=8, n_kv=2,
                                          q_dtype=BF16)
    ref = ref.reshape(ctx.size, 8, 128)
    got = _attend(st_d, ks_d, q, table, ctx, 0.1,
                  _desc(ctx.size, 8, 2, 128, mb, nb, BF16, BF16, ctx, 0), out_dtype=BF16)
    assert float(np.abs(got - ref).max()) < 2e-2
    # an unmapped encoded block and an out-of-range length poison only their rows
    bad_table = table.copy()
    bad_table[0, 3] = -1
    bad_ctx = ctx.copy()
    bad_ctx[2] = mb * 16 + 1
    got = _attend(st_d, ks_d, q, bad_table, bad_ctx, 0.1,
                  _desc(ctx.size, 8, 2, 128, mb, nb, BF16, F32, ctx, 0))
    assert np.isnan(got[0]).all() and np.isnan(got[2]).all()
    for b in (1, 3, 4):
        assert_parity(float(np.abs(got[b] - ref[b]).max()), TOL_8BIT)


@pytest.mark.parametrize("d_h", [128, 64])
def test_int4_append_steps_bit_exact(d_h):
    """20 decode steps: every row appends one token per step; blocks fill at
    different steps per row. GPU state equals the oracle's bit for bit."""
    import torch
    import decode_attention_paged_slot_amd as pda
    print(f"int4 append d_h={d_h}", flush=True)
    n_kv, steps = 2, 20
    start = np.array([1, 14, 15, 16, 31, 47, 5], np.int32)   # lengths before the first step
    end = start + steps
    st, ks, table, _, nb, mb = _case(5200 + d_h, end, n_q=4, n_kv=n_kv, d_h=d_h, poison=False)
    r = np.random.default_rng(11)
    dev = "cuda"
    st_d, ks_d = _dev(st, ks, dev)
    bt = torch.from_numpy(table).to(dev)
    for k in range(steps):
        ctx = start + k + 1
        kn = synth.gaussian((ctx.size, n_kv, d_h), BF16, r)
        vn = synth.gaussian((ctx.size, n_kv, d_h), BF16, r)
        desc = _desc(ctx.size, 4, n_kv, d_h, mb, nb, BF16, F32, ctx, 0)
        pda.kv_append_int4(to_dev(kn, BF16, dev), to_dev(vn, BF16, dev), bt,
                           torch.from_numpy(ctx).to(dev), st_d["k"], st_d["v"], ks_d,
                           st_d["v_scale"], st_d["k_res"], st_d["v_res"], desc=desc)
        st = int4.kv_append_int4(st, kn, vn, table, ctx, ks)
    torch.cuda.synchronize()
    assert (st_d["k"].cpu().numpy() == st["k"]).all()
    assert (st_d["v"].cpu().numpy() == st["v"]).all()
    assert (st_d["v_scale"].cpu().numpy().view(np.uint32) == st["v_scale"].view(np.uint32)).all()
    assert (st_d["k_res"].view(torch.int16).cpu().numpy().view(np.uint16) == st["k_res"]).all()
    assert (st_d["v_res"].view(torch.int16).cpu().numpy().view(np.uint16) == st["v_res"]).all()
    # and attention after the steps
    q_np = synth.gaussian((end.size, 4, d_h), BF16, r)
    got = _attend(st_d, ks_d, to_dev(q_np, BF16, dev), table, end, 0.125,
                  _desc(end.size, 4, n_kv, d_h, mb, nb, BF16, F32, end, 0))
    ref, _, _, bad = oracle.paged_attn_int4(q_np, st, ks, table, end, 0.125, n_q=4, n_kv=n_kv,
                                            q_dtype=BF16)
    assert bad == 0
    assert_parity(float(np.abs(got - ref.reshape(got.shape)).max()), TOL_8BIT)


def test_int4_rejects_window_and_prefix():
    import torch
    import decode_attention_paged_slot_amd as pda
    t = torch.zeros(4, device="cuda")
    ctx = np.array([20], np.int32)
    for kw in (dict(window=16), dict(prefix_blocks=1)):
        desc = _desc(1, 4, 2, 64, 2, 4, BF16, F32, ctx, 0)
        for k, v in kw.items():
            setattr(desc, k, v)
        with pytest.raises(pda.PdaError):
            pda.paged_decode_attn_int4(t, t, t, t, t, t, t, t, t, 1.0, t, desc=desc,
                                       workspace=None)


@pytest.mark.parametrize("d_h,n_q,n_kv,nw", [(128, 8, 2, 0), (128, 32, 8, 64), (64, 8, 2, 7),
                                              (128, 8, 1, 1)])
def test_int4_fused_step_matches_two_calls(d_h, n_q, n_kv, nw):
    """decode_step_int4 against kv_append_int4 followed by
    paged_decode_attn_int4, over 20 steps in which blocks fill at different
    steps per row: outputs, codes, value scales and residual buffers
    bit-identical after every step; the outputs also against the oracle at
    the end. Rows include ones shorter than a block, an invalid length and a
    row whose block to encode is unmapped (poisoned in both, append skipped)."""
    import torch
    import decode_attention_paged_slot_amd as pda
    print(f"int4 fused step d_h={d_h} n_q={n_q} n_kv={n_kv} nw={nw}", flush=True)
    steps = 20
    start = np.array([1, 14, 15, 16, 31, 47, 5, 250, 511, 700, 3, 90], np.int32)
    end = start + steps
    st, ks, table, _, nb, mb = _case(5300 + d_h + nw, end, n_q=n_q, n_kv=n_kv, d_h=d_h,
                                     poison=False)
    bad_row, unmapped_row = 10, 11
    table[unmapped_row, 5] = -1   # the block the token at n = 96 completes
    r = np.random.default_rng(12 + nw)
    dev = "cuda"
    a_d, ks_d = _dev(st, ks, dev)
    b_d, _ = _dev(st, ks, dev)
    bt = torch.from_numpy(table).to(dev)

    def bits(x):
        return x.view(torch.int16 if x.element_size() == 2 else
                      (torch.uint8 if x.element_size() == 1 else torch.int32)).cpu().numpy()

    for k in range(steps):
        ctx = start + k + 1
        ctx[bad_row] = mb * 16 + 1
        kn = to_dev(synth.gaussian((ctx.size, n_kv, d_h), BF16, r), BF16, dev)
        vn = to_dev(synth.gaussian((ctx.size, n_kv, d_h), BF16, r), BF16, dev)
        q_np = synth.gaussian((ctx.size, n_q, d_h), BF16, r)
        q = to_dev(q_np, BF16, dev)
        desc = _desc(ctx.size, n_q, n_kv, d_h, mb, nb, BF16, F32, ctx, nw)
        ct = torch.from_numpy(ctx).to(dev)
        out_a = torch.full((ctx.size, n_q, d_h), 7.0, device=dev)
        out_b = torch.full((ctx.size, n_q, d_h), -7.0, device=dev)
        pda.kv_append_int4(kn, vn, bt, ct, a_d["k"], a_d["v"], ks_d, a_d["v_scale"],
                           a_d["k_res"], a_d["v_res"], desc=desc)
        pda.paged_decode_attn_int4(q, a_d["k"], a_d["v"], ks_d, a_d["v_scale"], a_d["k_res"],
                                   a_d["v_res"], bt, ct, 0.1, out_a, desc=desc,
                                   workspace=pda.workspace_for(desc, dev))
        pda.decode_step_int4(q, kn, vn, b_d["k"], b_d["v"], ks_d, b_d["v_scale"], b_d["k_res"],
                             b_d["v_res"], bt, ct, 0.1, out_b, desc=desc,
                             workspace=pda.workspace_for(desc, dev))
        torch.cuda.synchronize()
        assert (bits(out_a) == bits(out_b)).all(), f"output differs at step {k}"
        for key in ("k", "v", "v_scale", "k_res", "v_res"):
            assert (bits(a_d[key]) == bits(b_d[key])).all(), f"{key} differs at step {k}"
        # the oracle follows the rows the kernels serve in full (the two
        # poisoned rows are left out of it)
        good = ctx.copy()
        good[[bad_row, unmapped_row]] = 0
        st = int4.kv_append_int4(st, kn.view(torch.int16).cpu().numpy().view(np.uint16),
                                 vn.view(torch.int16).cpu().numpy().view(np.uint16), table,
                                 good, ks)
    got = out_b.cpu().numpy()
    assert np.isnan(got[bad_row]).all() and np.isnan(got[unmapped_row]).all()
    ref, _, _, _ = oracle.paged_attn_int4(q_np, st, ks, table, good, 0.1, n_q=n_q, n_kv=n_kv,
                                          q_dtype=BF16)
    ref = ref.reshape(got.shape)
    for b in range(ctx.size):
        if b not in (bad_row, unmapped_row):
            assert_parity(float(np.abs(got[b] - ref[b]).max()), TOL_8BIT)


def test_int4_fused_step_takes_bf16_rows_only():
    import torch
    import decode_attention_paged_slot_amd as pda
    t = torch.zeros(4, device="cuda")
    ctx = np.array([20], np.int32)
    desc = _desc(1, 4, 2, 64, 2, 4, BF16, F32, ctx, 0)
    desc.new_dtype = F32
    with pytest.raises(ValueError):
        pda.decode_step_int4(t, t, t, t, t, t, t, t, t, t, t, 1.0, t, desc=desc)
