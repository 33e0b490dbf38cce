"""Calls on two streams at once, each with its own workspace and output, must
give the same bits as the same calls run one after the other: the library
keeps no device state of its own between or across calls, and every kernel
of a call runs on the stream it is given. Both streams have the default
priority.
"""
from __future__ import annotations

import numpy as np
import pytest

from synth import BF16, FP8
from tests.helpers import make_case
from tests.gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


def _call_factory(c, dev, nw):
    import torch
    import decode_attention_paged_slot_amd as pda
    q = to_dev(c.q, c.q_dtype, dev)
    k = to_dev(c.k, c.kv_dtype, dev)
    v = to_dev(c.v, c.kv_dtype, dev)
    bt = torch.from_numpy(c.table).to(dev)
    cl = torch.from_numpy(c.ctx).to(dev)
    desc = pda.attn_desc(q, k, bt, max_context=int(c.ctx.max()), kv_dtype=c.kv_dtype,
                         num_partitions=nw)
    ws = pda.workspace_for(desc, dev)
    out = torch.full((c.B, c.n_q, c.d_h), float("nan"), device=dev)
    quant = c.kv_dtype == FP8
    ks = torch.from_numpy(c.k_scale).to(dev) if quant else None
    vs = torch.from_numpy(c.v_scale).to(dev) if quant else None

    def call():
        if quant:
            pda.paged_decode_attn_quant(q, k, v, ks, vs, bt, cl, c.scale, out, desc=desc,
                                        workspace=ws)
        else:
            pda.paged_decode_attn(q, k, v, bt, cl, c.scale, out, desc=desc, workspace=ws)
    return call, out


@pytest.mark.parametrize("nw", [0, 37])
def test_two_streams_match_serial(nw):
    import torch
    print(f"two streams nw={nw}", flush=True)
    dev = "cuda"
    ca = make_case(64_000 + nw, [3000, 17, 900, 4100], n_q=16, n_kv=2, d_h=128)
    cb = make_case(64_100 + nw, [50, 2500, 1, 0, 700, 3333], n_q=8, n_kv=8, d_h=64,
                   kv_dtype=FP8)
    call_a, out_a = _call_factory(ca, dev, nw)
    call_b, out_b = _call_factory(cb, dev, nw)
    call_a()
    call_b()
    torch.cuda.synchronize()
    ref_a, ref_b = out_a.clone(), out_b.clone()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(5):
        out_a.fill_(float("nan"))
        out_b.fill_(float("nan"))
        torch.cuda.synchronize()
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s1):
            for _ in range(3):
                call_a()
        with torch.cuda.stream(s2):
            for _ in range(3):
                call_b()
        torch.cuda.synchronize()
        assert torch.equal(out_a, ref_a), f"stream A differs on repetition {rep}"
        assert torch.equal(out_b, ref_b), f"stream B differs on repetition {rep}"
    assert np.isfinite(ref_a.cpu().numpy()).all()
