"""The decode step (append + attention + split-KV merge) captured in a HIP
graph must reproduce the eager result on every replay.

Each replay is separated by eager work on the same buffers (an eager step
that overwrites the output with different inputs, and a host
synchronisation), so a replay that silently reused stale state or skipped a
node would show up as a mismatch. The kernels are deterministic, so the
comparison is bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

from synth import BF16, FP8
from tests.helpers import make_case
from tests.gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv_dtype", [BF16, FP8])
def test_graph_replay_matches_eager(kv_dtype):
    import torch
    import decode_attention_paged_slot_amd as pda

    print(f"graph replay kv_dtype={kv_dtype}", flush=True)
    c = make_case(9901 + kv_dtype, [700, 33, 1, 2000, 129], n_q=16, n_kv=2, d_h=128,
                  kv_dtype=kv_dtype)
    dev = "cuda"
    q = to_dev(c.q, c.q_dtype, dev)
    q_other = torch.randn_like(q.float()).to(q.dtype)
    k = to_dev(c.k, c.kv_dtype, dev)
    v = to_dev(c.v, c.kv_dtype, dev)
    bt = torch.from_numpy(c.table).to(dev)
    cl = torch.from_numpy(c.ctx).to(dev)
    sl = torch.from_numpy(c.slots).to(dev)
    kn = torch.randn((c.B, c.n_kv, c.d_h), device=dev).to(torch.bfloat16)
    vn = torch.randn((c.B, c.n_kv, c.d_h), device=dev).to(torch.bfloat16)
    out = torch.empty((c.B, c.n_q, c.d_h), device=dev)
    desc = pda.attn_desc(q, k, bt, max_context=int(c.ctx.max()), kv_dtype=c.kv_dtype,
                         num_partitions=3)
    assert pda.attn_plan(desc)[0] > 1          # the merge kernel is part of the graph
    ws = pda.workspace_for(desc, dev)
    quant = kv_dtype == FP8
    if quant:
        ks = torch.from_numpy(c.k_scale).to(dev)
        vs = torch.from_numpy(c.v_scale).to(dev)

    def step(query):
        if quant:
            pda.kv_append_quant(kn, vn, sl, k, v, ks, vs, cache_dtype=FP8)
            pda.paged_decode_attn_quant(query, k, v, ks, vs, bt, cl, c.scale, out, desc=desc,
                                        workspace=ws)
        else:
            pda.kv_append(kn, vn, sl, k, v)
            pda.paged_decode_attn(query, k, v, bt, cl, c.scale, out, desc=desc, workspace=ws)

    step(q)
    torch.cuda.synchronize()
    eager = out.clone()
    step(q_other)
    torch.cuda.synchronize()
    other = out.clone()
    assert not torch.equal(eager, other)

    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_cap):
        step(q)
    torch.cuda.current_stream().wait_stream(s_cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(q)
    torch.cuda.synchronize()
    for rep in range(4):
        step(q_other)                            # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, other)
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        assert torch.equal(got, eager), f"replay {rep} differs from the eager step"
    assert np.isfinite(eager.cpu().numpy()).all()
