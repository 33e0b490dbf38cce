"""Calls captured in a HIP graph must reproduce the eager result on every
replay: the two-call decode step (append + attention + split-KV merge), the
fused step, a row split finely enough for the column-split merge, the
shared-prefix call (prefix pass, suffix pass, merge) and the 4-bit call
(streaming kernel, merge forming the residual-window piece).

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


def _check_replays(call, call_other, out, reps=4):
    """Capture `call` in a graph; every replay, after eager `call_other` work
    on the same output, must reproduce the eager `call` bit for bit."""
    import torch
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    call_other()
    torch.cuda.synchronize()
    other = out.clone()
    assert not torch.equal(eager, other)
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_cap):
        call()
    torch.cuda.current_stream().wait_stream(s_cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(reps):
        call_other()
        torch.cuda.synchronize()
        assert torch.equal(out, other)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
    assert torch.isfinite(eager).all()


@pytest.mark.parametrize("case", ["fused_step", "wide_merge"])
def test_graph_fused_step_and_wide_merge(case):
    """The fused decode step (one launch + the one-wave merge), and a long row
    split into enough pieces to take the column-split block merge."""
    import torch
    import decode_attention_paged_slot_amd as pda

    print(f"graph replay {case}", flush=True)
    ctx = [700, 33, 1, 2000, 129] if case == "fused_step" else [6000]
    n_kv = 2
    c = make_case(9950 + len(case), ctx, n_q=16, n_kv=n_kv, d_h=128)
    dev = "cuda"
    q = to_dev(c.q, c.q_dtype, dev)
    q_other = torch.randn_like(q.float()).to(q.dtype)
    k = to_dev(c.k, c.kv_dtype, dev)
    v = to_dev(c.v, c.kv_dtype, dev)
    bt = torch.from_numpy(c.table).to(dev)
    cl = torch.from_numpy(c.ctx).to(dev)
    kn = torch.randn((c.B, c.n_kv, c.d_h), device=dev).to(torch.bfloat16)
    vn = torch.randn((c.B, c.n_kv, c.d_h), device=dev).to(torch.bfloat16)
    out = torch.empty((c.B, c.n_q, c.d_h), device=dev)
    nw = 3 if case == "fused_step" else 64 * c.B * n_kv + 8    # >= 64 pieces per segment
    desc = pda.attn_desc(q, k, bt, max_context=int(c.ctx.max()), num_partitions=nw,
                         new_dtype=BF16)
    assert pda.attn_plan(desc)[0] > 1
    ws = pda.workspace_for(desc, dev)

    if case == "fused_step":
        def run(query):
            pda.decode_step(query, kn, vn, k, v, bt, cl, c.scale, out, desc=desc, workspace=ws)
    else:
        def run(query):
            pda.paged_decode_attn(query, k, v, bt, cl, c.scale, out, desc=desc, workspace=ws)
    _check_replays(lambda: run(q), lambda: run(q_other), out)


def test_graph_shared_prefix_call():
    """Prefix pass, suffix pass and the merge of both kinds of pieces."""
    import torch
    import decode_attention_paged_slot_amd as pda
    from tests import test_gpu_prefix as pfx

    print("graph replay shared prefix", flush=True)
    n_shared = 21
    c = make_case(9960, pfx.CTX, n_q=8, n_kv=2, d_h=128, kv_dtype=FP8,
                  shared_prefix_blocks=n_shared)
    pl = pfx._prefix_lens(c, n_shared)
    table = c.table.copy()
    for b, p in enumerate(pl):
        table[b, :int(p)] = -1
    dev = "cuda"
    q = to_dev(c.q, c.q_dtype, dev)
    q_other = torch.randn_like(q.float()).to(q.dtype)
    k = to_dev(c.k, FP8, dev)
    v = to_dev(c.v, FP8, dev)
    ks = torch.from_numpy(c.k_scale).to(dev)
    vs = torch.from_numpy(c.v_scale).to(dev)
    bt = torch.from_numpy(table).to(dev)
    cl = torch.from_numpy(c.ctx).to(dev)
    pt = torch.from_numpy(np.asarray(c.shared_ids, dtype=np.int32)).to(dev)
    pls = torch.from_numpy(pl).to(dev)
    out = torch.empty((c.B, c.n_q, c.d_h), device=dev)
    desc = pda.AttnDesc(c.B, c.n_q, c.n_kv, c.d_h, c.bs, bt.shape[1], k.shape[0], FP8, c.q_dtype,
                        0, int(c.ctx.max()), 7, int(c.ctx.sum()), 0, 0, 0, BF16, n_shared)
    ws = pda.workspace_for(desc, dev)

    def run(query):
        pda.paged_decode_attn_prefix(query, k, v, ks, vs, bt, cl, pt, pls, c.scale, out,
                                     desc=desc, workspace=ws)
    _check_replays(lambda: run(q), lambda: run(q_other), out)


def test_graph_int4_call():
    """4-bit attention: the streaming kernel and the merge that forms each
    row's residual-window piece."""
    import torch
    import synth
    from synth import F32
    from tests import test_gpu_int4 as i4
    import decode_attention_paged_slot_amd as pda

    print("graph replay 4-bit", flush=True)
    st, ks, table, ctx, nb, mb = i4._case(9970, [300, 17, 40, 5, 64, 2063], n_q=8, n_kv=2,
                                          d_h=128)
    dev = "cuda"
    st_d, ks_d = i4._dev(st, ks, dev)
    r = np.random.default_rng(12)
    q = to_dev(synth.gaussian((ctx.size, 8, 128), BF16, r), BF16, dev)
    q_other = torch.randn_like(q.float()).to(q.dtype)
    bt = torch.from_numpy(table).to(dev)
    cl = torch.from_numpy(ctx).to(dev)
    out = torch.empty((ctx.size, 8, 128), device=dev)
    desc = i4._desc(ctx.size, 8, 2, 128, mb, nb, BF16, F32, ctx, 5)
    ws = pda.workspace_for(desc, dev)

    def run(query):
        pda.paged_decode_attn_int4(query, st_d["k"], st_d["v"], ks_d, st_d["v_scale"],
                                   st_d["k_res"], st_d["v_res"], bt, cl, 0.1, out, desc=desc,
                                   workspace=ws)
    _check_replays(lambda: run(q), lambda: run(q_other), out)
