"""Batches whose rows all hold the same number of tokens (the shape of the
70B-layer and long-context workloads), under every combination of the host
hints.

The descriptor's max_context and total_context only size the split: the
kernel recomputes the exact ranges from context_lens. So every hint setting,
consistent or not (max_context one short of the true length, total_context
unknown), must give the oracle's result, and two settings that yield the same
split plan must give the same bits (the same blocks reduced in the same
order). Also covered with uniform rows: sliding windows whose skipped blocks
are unmapped, one odd row among equal ones, unmapped ids early and deep in a
row, and the fused decode step.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import synth
from synth import BF16, FP8, INT8
from tests.helpers import make_case
from tests.gpu_helpers import TOL_16BIT, TOL_8BIT, assert_parity, max_err, run_case, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.int32)


@pytest.mark.parametrize("kv_dtype", [BF16, FP8, INT8])
@pytest.mark.parametrize("d_h,g", [(128, 8), (64, 4), (128, 1)])
@pytest.mark.parametrize("nw", [0, 7, 64])
@pytest.mark.parametrize("n", [16, 1000, 4100])
def test_uniform_rows_hint_settings(kv_dtype, d_h, g, nw, n):
    B, n_kv = 5, 2
    c = make_case(9100 + n + nw + 10 * kv_dtype + d_h + g, [n] * B, n_q=g * n_kv, n_kv=n_kv,
                  d_h=d_h, kv_dtype=kv_dtype)
    _say(f"uniform rows kv={kv_dtype} d_h={d_h} g={g} nw={nw} n={n}")
    # Pairs with the same split plan (with nw = 0 the plan follows the hints;
    # ceil(max_context / 16) is the same for n and n - 1 here): exact hints
    # and max_context one short, with total_context given or unknown.
    assert (n + 15) // 16 == (n + 14) // 16
    exact, _ = run_case(c, max_context=n, total_context=B * n, num_partitions=nw)
    short, _ = run_case(c, max_context=n - 1, total_context=B * n, num_partitions=nw)
    unknown, _ = run_case(c, max_context=n, total_context=0, num_partitions=nw)
    unknown_short, _ = run_case(c, max_context=n - 1, total_context=0, num_partitions=nw)
    tol = TOL_8BIT if kv_dtype in (FP8, INT8) else TOL_16BIT
    ref = c.oracle_out()
    for got in (exact, short, unknown, unknown_short):
        assert_parity(max_err(got, ref), tol)
    assert (_bits(exact) == _bits(short)).all()
    assert (_bits(unknown) == _bits(unknown_short)).all()


@pytest.mark.parametrize("kv_dtype", [BF16, FP8])
@pytest.mark.parametrize("nw", [7, 64, 200])
def test_full_row_hint_that_does_not_hold(kv_dtype, nw):
    """total_context = B * max_context claims that every row is full; here
    the rows are ragged (an empty row, a one-token row, a row longer than
    max_context among them). With the wave count fixed, the claim must not
    change a bit against no hint at all. nw = 200 (>= 64 pieces per segment
    on average) takes the column-split merge."""
    ctx = [3000, 0, 1, 2990, 17, 3100]
    B, n_kv = len(ctx), 1
    c = make_case(9200 + nw + kv_dtype, ctx, n_q=4, n_kv=n_kv, d_h=128, kv_dtype=kv_dtype,
                  max_blocks=(3100 + 15) // 16)
    _say(f"full-row hint that does not hold kv={kv_dtype} nw={nw}")
    claimed, _ = run_case(c, max_context=3000, total_context=B * 3000, num_partitions=nw)
    none, _ = run_case(c, max_context=3000, total_context=0, num_partitions=nw)
    assert (_bits(claimed) == _bits(none)).all()
    ref = c.oracle_out()
    keep = [0, 2, 3, 4, 5]
    assert (claimed[1] == 0).all()
    assert_parity(max_err(claimed[keep], ref[keep]), (TOL_8BIT if kv_dtype == FP8 else TOL_16BIT))


@pytest.mark.parametrize("kv_dtype", [BF16, INT8])
@pytest.mark.parametrize("n", [16, 2000, 40000])
def test_full_rows_column_split_merge(kv_dtype, n):
    """Full rows split finely enough for the column-split merge (many pieces
    per segment), with exact hints and with max_context one token short:
    same bits, and the oracle's result."""
    B, n_kv = 2, 2
    nw = 64 * B * n_kv + 3
    c = make_case(9250 + n + kv_dtype, [n] * B, n_q=8, n_kv=n_kv, d_h=128, kv_dtype=kv_dtype)
    _say(f"full rows column-split merge kv={kv_dtype} n={n}")
    exact, _ = run_case(c, max_context=n, total_context=B * n, num_partitions=nw)
    short, _ = run_case(c, max_context=n - 1, total_context=B * n, num_partitions=nw)
    assert (_bits(exact) == _bits(short)).all()
    tol = TOL_8BIT if kv_dtype == INT8 else TOL_16BIT
    assert_parity(max_err(exact, c.oracle_out()), tol)


@pytest.mark.parametrize("window,sinks", [(100, 4), (33, 0), (4000, 20)])
@pytest.mark.parametrize("nw", [0, 9])
def test_uniform_rows_with_window(window, sinks, nw):
    """Sliding window over equal rows: a segment lists the sink blocks, then
    the window blocks; blocks outside both are unmapped and NaN-poisoned."""
    B, n = 4, 3000
    c = make_case(9300 + window + sinks + nw, [n] * B, n_q=16, n_kv=2, d_h=128)
    table = c.table.copy()
    for b in range(B):
        for blk in range((n + 15) // 16):
            ts = range(16 * blk, min(n, 16 * blk + 16))
            if all(not (t < sinks or t >= n - window) for t in ts):
                pb = table[b, blk]
                c.k[pb] = synth.BF16_NAN
                c.v[pb] = synth.BF16_NAN
                table[b, blk] = -1
    _say(f"uniform rows window={window} sinks={sinks} nw={nw}")
    exact, _ = run_case(c, table=table, max_context=n, total_context=B * n, window=window,
                        sinks=sinks, num_partitions=nw)
    short, _ = run_case(c, table=table, max_context=n - 1, total_context=B * n,
                        window=window, sinks=sinks, num_partitions=nw)
    assert_parity(max_err(exact, c.oracle_out(window=window, sinks=sinks)), TOL_16BIT)
    assert (_bits(exact) == _bits(short)).all()


@pytest.mark.parametrize("odd", ["shorter", "empty", "one_token", "longer"])
def test_one_odd_row_among_equal_rows(odd):
    """One row differs from the others (shorter, empty, a single token, or
    longer than max_context, which is still attended in full)."""
    n = 2000
    ctx = [n] * 6
    ctx[3] = {"shorter": n - 1, "empty": 0, "one_token": 1, "longer": n + 40}[odd]
    c = make_case(9500 + len(odd), ctx, n_q=8, n_kv=2, d_h=128, max_blocks=(n + 40 + 15) // 16)
    _say(f"one odd row: {odd}")
    for nw in (0, 5):
        got, _ = run_case(c, max_context=n, total_context=0, num_partitions=nw)
        ref = c.oracle_out()
        if odd == "empty":
            assert (got[3] == 0).all()
            keep = [0, 1, 2, 4, 5]
            assert_parity(max_err(got[keep], ref[keep]), TOL_16BIT)
        else:
            assert_parity(max_err(got, ref), TOL_16BIT)


@pytest.mark.parametrize("nw", [0, 3])
def test_uniform_rows_unmapped_entries(nw):
    """An unmapped first block and an out-of-range id deep in a row poison
    only their own rows."""
    n, B = 1500, 4
    c = make_case(9700 + nw, [n] * B, n_q=8, n_kv=2, d_h=128)
    t = c.table.copy()
    t[1, 0] = -1                        # first block of row 1 (first batch of a wave)
    t[2, 70] = c.num_blocks + 3         # deep inside row 2
    _say(f"uniform rows unmapped nw={nw}")
    got, _ = run_case(c, table=t, max_context=n, total_context=B * n, num_partitions=nw)
    ref = c.oracle_out()
    assert np.isnan(got[1]).all() and np.isnan(got[2]).all()
    assert_parity(max_err(got[[0, 3]], ref[[0, 3]]), TOL_16BIT)


@pytest.mark.parametrize("kv_dtype", [BF16, FP8])
def test_uniform_rows_fused_step(kv_dtype):
    """The fused decode step with uniform lengths: caches and output bit for
    bit as the two calls, and the oracle's append-then-attend."""
    import torch
    import decode_attention_paged_slot_amd as pda

    n, B = 1234, 6
    c = make_case(9900 + kv_dtype, [n] * B, n_q=16, n_kv=2, d_h=128, kv_dtype=kv_dtype)
    r = np.random.default_rng(99 + kv_dtype)
    kn = synth.gaussian((B, c.n_kv, c.d_h), BF16, r)
    vn = synth.gaussian((B, c.n_kv, c.d_h), BF16, r)
    dev = "cuda"
    quant = kv_dtype == FP8
    q = to_dev(c.q, c.q_dtype, dev)
    bt = torch.from_numpy(c.table).to(dev)
    cl = torch.from_numpy(c.ctx).to(dev)
    sl = torch.from_numpy(c.slots).to(dev)
    dkn, dvn = to_dev(kn, BF16, dev), to_dev(vn, BF16, dev)
    ks = torch.from_numpy(c.k_scale).to(dev) if quant else None
    vs = torch.from_numpy(c.v_scale).to(dev) if quant else None
    desc = pda.AttnDesc(c.B, c.n_q, c.n_kv, c.d_h, c.bs, bt.shape[1], c.k.shape[0], kv_dtype,
                        c.q_dtype, synth.F32, n, 0, B * n, 0, 0, 0, BF16)
    ws = pda.workspace_for(desc, dev)
    _say(f"uniform rows fused step kv={kv_dtype}")
    ka, va = to_dev(c.k, kv_dtype, dev), to_dev(c.v, kv_dtype, dev)
    out_a = torch.full((B, c.n_q, c.d_h), float("nan"), device=dev)
    kb, vb = to_dev(c.k, kv_dtype, dev), to_dev(c.v, kv_dtype, dev)
    out_b = torch.full((B, c.n_q, c.d_h), float("nan"), device=dev)
    if quant:
        pda.kv_append_quant(dkn, dvn, sl, ka, va, ks, vs, cache_dtype=kv_dtype)
        pda.paged_decode_attn_quant(q, ka, va, ks, vs, bt, cl, c.scale, out_a, desc=desc,
                                    workspace=ws)
        pda.decode_step_quant(q, dkn, dvn, kb, vb, ks, vs, bt, cl, c.scale, out_b, desc=desc,
                              workspace=ws)
    else:
        pda.kv_append(dkn, dvn, sl, ka, va)
        pda.paged_decode_attn(q, ka, va, bt, cl, c.scale, out_a, desc=desc, workspace=ws)
        pda.decode_step(q, dkn, dvn, kb, vb, bt, cl, c.scale, out_b, desc=desc, workspace=ws)
    torch.cuda.synchronize()
    assert (kb.view(torch.uint8).cpu().numpy() == ka.view(torch.uint8).cpu().numpy()).all()
    assert (vb.view(torch.uint8).cpu().numpy() == va.view(torch.uint8).cpu().numpy()).all()
    a, b = out_a.cpu().numpy(), out_b.cpu().numpy()
    assert (_bits(a) == _bits(b)).all()
    if quant:
        k2 = oracle.kv_append_quant(c.k, c.k_scale, oracle.decode(kn, BF16).astype(np.float32),
                                    c.slots, kv_dtype)
        v2 = oracle.kv_append_quant(c.v, c.v_scale, oracle.decode(vn, BF16).astype(np.float32),
                                    c.slots, kv_dtype)
    else:
        k2 = oracle.kv_append(c.k, kn, c.slots)
        v2 = oracle.kv_append(c.v, vn, c.slots)
    ref, _, _, bad = oracle.paged_attn(c.q, k2, v2, c.table, c.ctx, c.scale, n_q=c.n_q,
                                       n_kv=c.n_kv, q_dtype=c.q_dtype, kv_dtype=kv_dtype,
                                       k_scale=c.k_scale, v_scale=c.v_scale)
    assert bad == 0
    assert_parity(max_err(b.reshape(-1, c.d_h), ref), (TOL_8BIT if quant else TOL_16BIT))
