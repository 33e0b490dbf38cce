"""pda_paged_decode_attn_noalloc: the call that takes its split-KV workspace
from the library's fixed device scratch instead of the caller. Through the C
ABI it must give exactly what pda_paged_decode_attn gives with a caller
workspace (same kernels, same split), on consecutive calls of different
sizes, and stay within the bf16 bar of the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest

from synth import BF16, F32
from tests.gpu_helpers import TOL_16BIT, assert_parity, max_err, to_dev
from tests.helpers import make_case

pytestmark = pytest.mark.gpu


def _run_both(case, num_partitions=0, out_dtype=F32):
    """(noalloc output, caller-workspace output, descriptor) as fp32 numpy."""
    import torch
    import decode_attention_paged_slot_amd as pda
    dev = "cuda"
    q = to_dev(case.q, case.q_dtype, dev)
    k = to_dev(case.k, case.kv_dtype, dev)
    v = to_dev(case.v, case.kv_dtype, dev)
    bt = torch.from_numpy(np.ascontiguousarray(case.table)).to(dev)
    cl = torch.from_numpy(np.ascontiguousarray(case.ctx)).to(dev)
    odt = torch.float32 if out_dtype == F32 else torch.bfloat16
    desc = pda.AttnDesc(case.B, case.n_q, case.n_kv, case.d_h, case.bs, bt.shape[1],
                        k.shape[0], case.kv_dtype, case.q_dtype, out_dtype,
                        int(case.ctx.max()), num_partitions, int(case.ctx.sum()), 0, 0, 0,
                        case.kv_dtype, 0)
    out_na = torch.full((case.B, case.n_q, case.d_h), float("nan"), device=dev, dtype=odt)
    out_ws = torch.full((case.B, case.n_q, case.d_h), float("nan"), device=dev, dtype=odt)
    print(f"noalloc case B={case.B} n_q={case.n_q} n_kv={case.n_kv} d_h={case.d_h} "
          f"ctx={case.ctx.tolist()} P={pda.attn_plan(desc)[0]}", flush=True)
    pda.paged_decode_attn_noalloc(q, k, v, bt, cl, case.scale, out_na, desc=desc)
    pda.paged_decode_attn(q, k, v, bt, cl, case.scale, out_ws, desc=desc,
                          workspace=pda.workspace_for(desc, dev))
    torch.cuda.synchronize()
    return out_na.float().cpu().numpy(), out_ws.float().cpu().numpy(), desc


def test_noalloc_matches_caller_workspace_on_consecutive_calls():
    import decode_attention_paged_slot_amd as pda
    big = make_case(91_000, [3000, 1500, 4096, 77, 2049], n_q=32, n_kv=8, d_h=128)
    small = make_case(91_001, [900, 33], n_q=8, n_kv=2, d_h=64)
    for case in (big, small):   # the second call is smaller: stale scratch must not leak
        got, want, desc = _run_both(case)
        assert pda.attn_workspace_size(desc) > 0          # the split path uses the scratch
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        assert_parity(max_err(got, case.oracle_out()), TOL_16BIT)


def test_noalloc_fp32_cache_and_bf16_output():
    import decode_attention_paged_slot_amd as pda
    c32 = make_case(91_002, [700, 260, 1], n_q=8, n_kv=2, d_h=64, kv_dtype=F32, q_dtype=F32)
    got, want, desc = _run_both(c32, num_partitions=4)
    assert pda.attn_workspace_size(desc) > 0
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert_parity(max_err(got, c32.oracle_out()), TOL_16BIT)
    cb = make_case(91_003, [1800, 640], n_q=16, n_kv=4, d_h=128, kv_dtype=BF16)
    got, want, _ = _run_both(cb, out_dtype=BF16)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_noalloc_rejects_workspace_above_the_limit():
    import torch
    import decode_attention_paged_slot_amd as pda
    # 4096 rows x 64 KV heads at g = 16, split: the workspace exceeds 16 MiB
    d = pda.AttnDesc(4096, 1024, 64, 128, 16, 64, 1 << 20, BF16, BF16, F32, 1024, 2048,
                     4096 * 1024, 0, 0, 0, BF16, 0)
    assert pda.attn_workspace_size(d) > pda.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(16, device="cuda")
    rc = pda.binding._lib.pda_paged_decode_attn_noalloc(
        t.data_ptr(), t.data_ptr(), t.data_ptr(), t.data_ptr(), t.data_ptr(), 1.0, t.data_ptr(),
        pda.binding.ctypes.byref(d), None)
    assert rc == pda.binding.EWORKSPACE
    assert "limit" in pda.last_error()
