"""Shared-prefix attention (pda_paged_decode_attn_prefix, pda_decode_step_prefix)
against the fp64 oracle.

The oracle attends through the table the call defines (logical block i of row
b is prefix_table[i] for i < prefix_lens[b]); the rows' own table entries for
their prefix are set to -1 on the GPU side, so a kernel that looked them up
instead of the prefix table would produce NaN rows. Cases span several prefix
chunks (16 blocks each), rows whose prefix ends inside a chunk, rows without a
prefix, a query count that is not a multiple of a 64-query group, every cache
dtype the call takes, and the split plans the tests of the plain call use.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import synth
from synth import F32, BF16, FP8, INT8
from tests.helpers import make_case
from tests.gpu_helpers import TOL_16BIT, TOL_8BIT, assert_parity, to_dev

pytestmark = pytest.mark.gpu

CTX = [5000, 1, 17, 16, 0, 600, 593, 258, 2000, 257, 33, 4100]


def _prefix_lens(c, n_shared):
    nblk = (c.ctx.astype(np.int64) + 15) // 16
    return np.minimum(n_shared, np.maximum(nblk - 1, 0)).astype(np.int32)


def _run(c, prefix_table, prefix_lens, *, out_dtype=F32, nw=0, blank_prefix=True, dev="cuda",
         step=None):
    """The shared-prefix call on the GPU -> (out fp32 numpy [B, n_q, d_h],
    caches after the call)."""
    import torch
    import decode_attention_paged_slot_amd as pda
    quant = c.kv_dtype in (FP8, INT8)
    table = c.table.copy()
    if blank_prefix:
        for b, pl in enumerate(prefix_lens):
            if 0 <= pl <= table.shape[1]:
                table[b, :max(int(pl), 0)] = -1
    q = to_dev(c.q, c.q_dtype, dev)
    k = to_dev(c.k, c.kv_dtype, dev)
    v = to_dev(c.v, c.kv_dtype, dev)
    bt = torch.from_numpy(table).to(dev)
    cl = torch.from_numpy(c.ctx).to(dev)
    pt = torch.from_numpy(np.asarray(prefix_table, dtype=np.int32)).to(dev)
    pls = torch.from_numpy(np.asarray(prefix_lens, dtype=np.int32)).to(dev)
    ks = torch.from_numpy(c.k_scale).to(dev) if quant else None
    vs = torch.from_numpy(c.v_scale).to(dev) if quant else None
    out = torch.full((c.B, c.n_q, c.d_h), float("nan"), device=dev,
                     dtype=torch.float32 if out_dtype == F32 else torch.bfloat16)
    new_dtype = BF16 if quant else c.kv_dtype
    desc = pda.AttnDesc(c.B, c.n_q, c.n_kv, c.d_h, c.bs, bt.shape[1], k.shape[0], c.kv_dtype,
                        c.q_dtype, out_dtype, int(c.ctx.max()), nw, int(c.ctx.sum()), 0, 0, 0,
                        new_dtype, len(prefix_table))
    ws = pda.workspace_for(desc, dev)
    if step is None:
        pda.paged_decode_attn_prefix(q, k, v, ks, vs, bt, cl, pt, pls, c.scale, out, desc=desc,
                                     workspace=ws)
    else:
        kn, vn = step
        pda.decode_step_prefix(q, to_dev(kn, new_dtype, dev), to_dev(vn, new_dtype, dev), k, v,
                               ks, vs, bt, cl, pt, pls, c.scale, out, desc=desc, workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), k, v


def _oracle(c, prefix_table, prefix_lens, k=None, v=None):
    table, invalid = oracle.prefix_block_table(c.table, c.ctx, prefix_table, prefix_lens)
    ref, _, _, bad = oracle.paged_attn(c.q, c.k if k is None else k, c.v if v is None else v,
                                       table, c.ctx, c.scale, n_q=c.n_q, n_kv=c.n_kv,
                                       q_dtype=c.q_dtype, kv_dtype=c.kv_dtype,
                                       k_scale=c.k_scale, v_scale=c.v_scale)
    return ref.reshape(c.B, c.n_q, c.d_h), invalid, bad


CONFIGS = [  # kv, q, d_h, n_q, n_kv
    (BF16, BF16, 128, 8, 2),
    (BF16, F32, 64, 8, 1),
    (FP8, BF16, 128, 32, 8),
    (FP8, F32, 128, 8, 2),
    (INT8, BF16, 128, 8, 2),
    (INT8, BF16, 64, 12, 4),
]


@pytest.mark.parametrize("kv,qd,d_h,n_q,n_kv", CONFIGS)
@pytest.mark.parametrize("nw", [0, 1, 7])
def test_prefix_matches_oracle(kv, qd, d_h, n_q, n_kv, nw):
    print(f"prefix kv={kv} q={qd} d_h={d_h} heads={n_q}/{n_kv} nw={nw}", flush=True)
    sys.stdout.flush()
    n_shared = 37   # chunks of 16, 16 and 5 blocks
    c = make_case(4100 + 7 * kv + d_h + nw, CTX, n_q=n_q, n_kv=n_kv, d_h=d_h, kv_dtype=kv,
                  q_dtype=qd, shared_prefix_blocks=n_shared)
    pl = _prefix_lens(c, n_shared)
    assert pl.max() == n_shared and (pl == 0).any()
    got, _, _ = _run(c, c.shared_ids, pl, nw=nw)
    ref, invalid, bad = _oracle(c, c.shared_ids, pl)
    assert bad == 0 and not invalid.any()
    assert np.isfinite(got).all()
    tol = TOL_8BIT if kv in (FP8, INT8) else TOL_16BIT
    assert_parity(float(np.abs(got - ref).max()), tol)
    assert (got[4] == 0).all()   # the empty row


@pytest.mark.parametrize("kv", [BF16, FP8])
def test_prefix_lengths_below_the_shared_maximum(kv):
    """Rows may use only part of the shared prefix (any length up to their
    last block); where they stop, their own table takes over."""
    r = np.random.default_rng(5 + kv)
    ctx = list(r.integers(1, 1500, size=23))   # B * g = 92: two query groups
    c = make_case(4200 + kv, ctx, n_q=16, n_kv=4, d_h=128, kv_dtype=kv, q_dtype=BF16,
                  shared_prefix_blocks=40)
    top = _prefix_lens(c, 40)
    pl = np.array([int(r.integers(0, t + 1)) for t in top], dtype=np.int32)
    got, _, _ = _run(c, c.shared_ids, pl, nw=0)
    ref, invalid, bad = _oracle(c, c.shared_ids, pl)
    assert bad == 0 and not invalid.any()
    tol = TOL_8BIT if kv == FP8 else TOL_16BIT
    assert_parity(float(np.abs(got - ref).max()), tol)
    got_b, _, _ = _run(c, c.shared_ids, pl, nw=0, out_dtype=BF16)
    assert float(np.abs(got_b - ref).max()) < 2e-2   # bf16 output rounding on top


@pytest.mark.parametrize("kv", [BF16, INT8])
def test_prefix_invalid_rows_are_nan(kv):
    """A prefix reaching the row's newest block, longer than the table, or
    negative makes that row NaN; an unmapped prefix-table entry poisons the
    rows whose prefix covers it. Every other row is unaffected."""
    ctx = [300, 300, 300, 300, 40, 0, 300, 700]
    c = make_case(4300 + kv, ctx, n_q=8, n_kv=2, d_h=128, kv_dtype=kv, q_dtype=BF16,
                  shared_prefix_blocks=18)
    pl = _prefix_lens(c, 18)
    pl[1] = 19          # beyond the prefix table (and its row's last block)
    pl[2] = -3
    pl[4] = 3           # 40 tokens = 3 blocks: the last one is the row's own
    pl[5] = 9           # empty row: ignored
    pl[6] = 17
    pl[7] = 5
    pt = list(c.shared_ids)
    pt[10] = -1         # unmapped: rows 0, 3 (18 blocks of prefix) and 6 (17) -> NaN
    got, _, _ = _run(c, pt, pl, nw=0)
    ref, invalid, _ = _oracle(c, c.shared_ids, pl)
    assert invalid.tolist() == [False, True, True, False, True, False, False, False]
    nan_rows = {0, 1, 2, 3, 4, 6}
    for b in range(c.B):
        if b in nan_rows:
            assert np.isnan(got[b]).all(), b
        else:
            assert np.isfinite(got[b]).all(), b
    tol = TOL_8BIT if kv == INT8 else TOL_16BIT
    assert_parity(float(np.abs(got[7] - ref[7]).max()), tol)
    assert (got[5] == 0).all()


@pytest.mark.parametrize("kv", [BF16, FP8, INT8])
@pytest.mark.parametrize("nw", [0, 5])
def test_decode_step_prefix(kv, nw):
    """The fused step with a shared prefix: caches bit for bit as after the
    append, output as the oracle's attention after its own append."""
    import torch
    print(f"decode_step_prefix kv={kv} nw={nw}", flush=True)
    c = make_case(4400 + kv + nw, CTX, n_q=8, n_kv=2, d_h=128, kv_dtype=kv,
                  q_dtype=BF16 if kv != F32 else F32, shared_prefix_blocks=37)
    quant = kv in (FP8, INT8)
    new_dtype = BF16 if quant else kv
    r = np.random.default_rng(99 + kv)
    kn = synth.gaussian((c.B, c.n_kv, c.d_h), new_dtype, r)
    vn = synth.gaussian((c.B, c.n_kv, c.d_h), new_dtype, r)
    pl = _prefix_lens(c, 37)
    got, k_after, v_after = _run(c, c.shared_ids, pl, nw=nw, step=(kn, vn))
    if quant:
        k2 = oracle.kv_append_quant(c.k, c.k_scale, oracle.decode(kn, new_dtype).astype(np.float32),
                                    c.slots, kv)
        v2 = oracle.kv_append_quant(c.v, c.v_scale, oracle.decode(vn, new_dtype).astype(np.float32),
                                    c.slots, kv)
    else:
        k2 = oracle.kv_append(c.k, kn, c.slots)
        v2 = oracle.kv_append(c.v, vn, c.slots)

    def raw(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()
    assert (raw(k_after) == k2.view(raw(k_after).dtype)).all()
    assert (raw(v_after) == v2.view(raw(v_after).dtype)).all()
    ref, invalid, bad = _oracle(c, c.shared_ids, pl, k=k2, v=v2)
    assert bad == 0 and not invalid.any()
    assert np.isfinite(got).all()
    assert_parity(float(np.abs(got - ref).max()), (TOL_8BIT if quant else TOL_16BIT))


def test_prefix_call_rejects_window_and_f32():
    import torch
    import decode_attention_paged_slot_amd as pda
    c = make_case(4500, [100, 50], n_q=4, n_kv=2, d_h=64, kv_dtype=F32, q_dtype=F32,
                  shared_prefix_blocks=2)
    dev = "cuda"
    desc = pda.AttnDesc(c.B, c.n_q, c.n_kv, c.d_h, c.bs, c.table.shape[1], c.k.shape[0], F32,
                        F32, F32, 100, 0, 150, 0, 0, 0, F32, 2)
    t = torch.zeros(4, device=dev)
    with pytest.raises(pda.PdaError):
        pda.paged_decode_attn_prefix(t, t, t, None, None, t, t, t, t, 1.0, t, desc=desc,
                                     workspace=None)
    desc.kv_dtype, desc.window = BF16, 64
    with pytest.raises(pda.PdaError):
        pda.paged_decode_attn_prefix(t, t, t, None, None, t, t, t, t, 1.0, t, desc=desc,
                                     workspace=None)
