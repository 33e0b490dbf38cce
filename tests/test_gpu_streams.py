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


def _int4_call(dev):
    """4-bit attention: the streaming kernel, then the merge that adds each
    row's residual-window piece."""
    import torch
    import synth
    from synth import F32
    from tests import test_gpu_int4 as i4
    import decode_attention_paged_slot_amd as pda
    st, ks, table, ctx, nb, mb = i4._case(64_200, [300, 17, 40, 5, 64, 2063, 0, 4111], n_q=8,
                                          n_kv=2, d_h=128)
    st_d, ks_d = i4._dev(st, ks, dev)
    r = np.random.default_rng(13)
    q = to_dev(synth.gaussian((ctx.size, 8, 128), BF16, r), BF16, dev)
    bt = torch.from_numpy(table).to(dev)
    cl = torch.from_numpy(ctx).to(dev)
    out = torch.full((ctx.size, 8, 128), float("nan"), device=dev)
    desc = i4._desc(ctx.size, 8, 2, 128, mb, nb, BF16, F32, ctx, 0)
    ws = pda.workspace_for(desc, dev)

    def call():
        pda.paged_decode_attn_int4(q, st_d["k"], st_d["v"], ks_d, st_d["v_scale"],
                                   st_d["k_res"], st_d["v_res"], bt, cl, 0.1, out, desc=desc,
                                   workspace=ws)
    return call, out


def _prefix_call(dev):
    """fp8 shared-prefix call: the prefix pass, the suffix pass and the merge
    of both kinds of pieces."""
    import torch
    import decode_attention_paged_slot_amd as pda
    from tests import test_gpu_prefix as pfx
    n_shared = 21
    c = make_case(64_300, pfx.CTX, n_q=8, n_kv=2, d_h=128, kv_dtype=FP8,
                  shared_prefix_blocks=n_shared)
    pl = pfx._prefix_lens(c, n_shared)
    table = c.table.copy()
    for b, p in enumerate(pl):
        table[b, :int(p)] = -1
    q = to_dev(c.q, c.q_dtype, dev)
    k = to_dev(c.k, FP8, dev)
    v = to_dev(c.v, FP8, dev)
    ks = torch.from_numpy(c.k_scale).to(dev)
    vs = torch.from_numpy(c.v_scale).to(dev)
    bt = torch.from_numpy(table).to(dev)
    cl = torch.from_numpy(c.ctx).to(dev)
    pt = torch.from_numpy(np.asarray(c.shared_ids, dtype=np.int32)).to(dev)
    pls = torch.from_numpy(pl).to(dev)
    out = torch.full((c.B, c.n_q, c.d_h), float("nan"), device=dev)
    desc = pda.AttnDesc(c.B, c.n_q, c.n_kv, c.d_h, c.bs, bt.shape[1], k.shape[0], FP8, c.q_dtype,
                        0, int(c.ctx.max()), 0, int(c.ctx.sum()), 0, 0, 0, BF16, n_shared)
    ws = pda.workspace_for(desc, dev)

    def call():
        pda.paged_decode_attn_prefix(q, k, v, ks, vs, bt, cl, pt, pls, c.scale, out, desc=desc,
                                     workspace=ws)
    return call, out


def test_two_streams_int4_and_prefix():
    """The same, for the calls with more than one kernel and stored pieces of
    their own: the 4-bit call on one stream, the shared-prefix call on the
    other."""
    import torch
    print("two streams: 4-bit and shared prefix", flush=True)
    dev = "cuda"
    call_a, out_a = _int4_call(dev)
    call_b, out_b = _prefix_call(dev)
    call_a()
    call_b()
    torch.cuda.synchronize()
    ref_a, ref_b = out_a.clone(), out_b.clone()
    assert np.isfinite(ref_b.cpu().numpy()).all()
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
        assert torch.equal(out_a, ref_a), f"4-bit stream differs on repetition {rep}"
        assert torch.equal(out_b, ref_b), f"prefix stream differs on repetition {rep}"
