"""The fused decode step (append of each row's new token + paged attention in
one launch) against the two separate calls, and against the oracle.

pda_decode_step must leave the caches and the output bit for bit as
pda_kv_append (slot of position n - 1 of each row) followed by
pda_paged_decode_attn; the quantized variant must encode the new rows exactly
as pda_kv_append_quant does.
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

CASES = [(BF16, BF16), (F32, F32), (FP8, BF16), (FP8, F32), (INT8, BF16), (INT8, F32)]


def _bits(t):
    import torch
    if t.dtype in (torch.float32,):
        return t.view(torch.int32).cpu().numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.cpu().numpy()


@pytest.mark.parametrize("kv_dtype,new_dtype", CASES)
@pytest.mark.parametrize("nw", [0, 1, 5])
@pytest.mark.parametrize("window", [0, 20])
def test_decode_step_equals_append_then_attend(kv_dtype, new_dtype, nw, window):
    import torch
    import decode_attention_paged_slot_amd as pda

    print(f"decode step kv={kv_dtype} new={new_dtype} nw={nw} window={window}", flush=True)
    sys.stdout.flush()
    ctx = [0, 700, 1, 33, 2000, 16, 300]
    c = make_case(3300 + 10 * kv_dtype + new_dtype + nw + window, ctx, n_q=8, n_kv=2, d_h=128,
                  kv_dtype=kv_dtype, q_dtype=BF16 if kv_dtype != F32 else F32)
    r = np.random.default_rng(77 + kv_dtype)
    kn = synth.gaussian((c.B, c.n_kv, c.d_h), new_dtype, r)
    vn = synth.gaussian((c.B, c.n_kv, c.d_h), new_dtype, r)
    dev = "cuda"
    quant = kv_dtype in (FP8, INT8)
    q = to_dev(c.q, c.q_dtype, dev)
    bt = torch.from_numpy(c.table).to(dev)
    cl = torch.from_numpy(c.ctx).to(dev)
    sl = torch.from_numpy(c.slots).to(dev)
    dkn, dvn = to_dev(kn, new_dtype, dev), to_dev(vn, new_dtype, dev)
    ks = torch.from_numpy(c.k_scale).to(dev) if quant else None
    vs = torch.from_numpy(c.v_scale).to(dev) if quant else None
    desc = pda.AttnDesc(c.B, c.n_q, c.n_kv, c.d_h, c.bs, bt.shape[1], c.k.shape[0], kv_dtype,
                        c.q_dtype, F32, int(c.ctx.max()), nw, int(c.ctx.sum()), 0, window, 4,
                        new_dtype)
    ws = pda.workspace_for(desc, dev)

    # two calls
    ka, va = to_dev(c.k, kv_dtype, dev), to_dev(c.v, kv_dtype, dev)
    out_a = torch.full((c.B, c.n_q, c.d_h), float("nan"), device=dev)
    if quant:
        pda.kv_append_quant(dkn, dvn, sl, ka, va, ks, vs, cache_dtype=kv_dtype)
        pda.paged_decode_attn_quant(q, ka, va, ks, vs, bt, cl, c.scale, out_a, desc=desc,
                                    workspace=ws)
    else:
        pda.kv_append(dkn, dvn, sl, ka, va)
        pda.paged_decode_attn(q, ka, va, bt, cl, c.scale, out_a, desc=desc, workspace=ws)
    # one fused call
    kb, vb = to_dev(c.k, kv_dtype, dev), to_dev(c.v, kv_dtype, dev)
    out_b = torch.full((c.B, c.n_q, c.d_h), float("nan"), device=dev)
    if quant:
        pda.decode_step_quant(q, dkn, dvn, kb, vb, ks, vs, bt, cl, c.scale, out_b, desc=desc,
                              workspace=ws)
    else:
        pda.decode_step(q, dkn, dvn, kb, vb, bt, cl, c.scale, out_b, desc=desc, workspace=ws)
    torch.cuda.synchronize()

    assert (_bits(kb) == _bits(ka)).all() and (_bits(vb) == _bits(va)).all()
    assert (_bits(out_b) == _bits(out_a)).all()

    # and the oracle: its own append, then its attention
    if quant:
        k2 = oracle.kv_append_quant(c.k, c.k_scale, oracle.decode(kn, new_dtype).astype(np.float32),
                                    c.slots, kv_dtype)
        v2 = oracle.kv_append_quant(c.v, c.v_scale, oracle.decode(vn, new_dtype).astype(np.float32),
                                    c.slots, kv_dtype)
    else:
        k2 = oracle.kv_append(c.k, kn, c.slots)
        v2 = oracle.kv_append(c.v, vn, c.slots)
    ref, _, _, bad = oracle.paged_attn(c.q, k2, v2, c.table, c.ctx, c.scale, n_q=c.n_q,
                                       n_kv=c.n_kv, q_dtype=c.q_dtype, kv_dtype=kv_dtype,
                                       k_scale=c.k_scale, v_scale=c.v_scale, window=window,
                                       sinks=4 if window else 0)
    assert bad == 0
    got = out_b.cpu().numpy().reshape(-1, c.d_h).astype(np.float64)
    assert np.isfinite(got).all()
    assert_parity(float(np.abs(got - ref).max()), (TOL_8BIT if quant else TOL_16BIT))
    assert (got.reshape(c.B, c.n_q, c.d_h)[0] == 0).all()
