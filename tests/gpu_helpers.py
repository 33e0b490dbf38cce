"""Move oracle-side test cases to the GPU and run them through the C ABI."""
from __future__ import annotations

import numpy as np

from synth import F32, BF16, FP8, INT8

TOL_16BIT = 5e-3     # bf16 / fp32 caches: max-abs error vs the fp64 oracle
TOL_8BIT = 3e-2      # fp8 / int8 / 4-bit caches: vs the oracle on the dequantized cache
# Regression bound beside the contract bars: the kernels keep ~16 bits of
# every weight and fp32 query (bf16 hi + lo parts) and accumulate in fp32, so
# they reach 1e-7 .. 1e-5 of the oracle on every cache type; a lost precision
# step (a dropped lo part, a bf16-only scaled query) lands far above 1e-4
# while still inside the bars.
TOL_REGRESSION = 1e-4


def assert_parity(err: float, bar: float, regression=TOL_REGRESSION) -> None:
    """max-abs error within the contract bar and within the regression bound
    (regression=None where the output itself is rounded, e.g. bf16 out)."""
    assert err < bar, f"max-abs error {err:.3g} over the contract bar {bar}"
    if regression is not None:
        assert err < regression, (f"max-abs error {err:.3g} over the regression bound "
                                  f"{regression} (contract bar {bar})")


def torch_dtype(code: int):
    import torch
    return {F32: torch.float32, BF16: torch.bfloat16, FP8: torch.uint8, INT8: torch.int8}[code]


def to_dev(a: np.ndarray, code: int, dev):
    """Raw numpy storage -> device tensor of the matching dtype (bit copy)."""
    import torch
    if code == BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    if code == FP8:
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def run_case(case, *, out_dtype=F32, num_partitions=0, max_context=None, total_context=0,
             table=None, reuse_prefix_blocks=0, window=0, sinks=0, dev="cuda"):
    """Paged decode attention of a tests.helpers.Case on the GPU -> fp32 numpy
    [B, n_q, d_h] (or the raw bf16 tensor's fp32 values for out_dtype=BF16)."""
    import torch
    import decode_attention_paged_slot_amd as pda
    q = to_dev(case.q, case.q_dtype, dev)
    k = to_dev(case.k, case.kv_dtype, dev)
    v = to_dev(case.v, case.kv_dtype, dev)
    bt = torch.from_numpy(np.ascontiguousarray(case.table if table is None else table)).to(dev)
    cl = torch.from_numpy(np.ascontiguousarray(case.ctx)).to(dev)
    out = torch.full((case.B, case.n_q, case.d_h), float("nan"), device=dev,
                     dtype=torch.float32 if out_dtype == F32 else torch.bfloat16)
    mc = int(case.ctx.max()) if (max_context is None and case.B) else (max_context or 0)
    desc = pda.AttnDesc(case.B, case.n_q, case.n_kv, case.d_h, case.bs, bt.shape[1],
                        k.shape[0], case.kv_dtype, case.q_dtype, out_dtype, mc,
                        num_partitions, total_context, reuse_prefix_blocks, window, sinks,
                        case.kv_dtype)
    ws = pda.workspace_for(desc, dev)
    if case.kv_dtype in (FP8, INT8):
        ks = torch.from_numpy(case.k_scale).to(dev)
        vs = torch.from_numpy(case.v_scale).to(dev)
        pda.paged_decode_attn_quant(q, k, v, ks, vs, bt, cl, case.scale, out, desc=desc,
                                    workspace=ws)
    else:
        pda.paged_decode_attn(q, k, v, bt, cl, case.scale, out, desc=desc, workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), desc


def max_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if np.isnan(gpu).any() or np.isnan(ref).any():
        return float("inf")
    return float(np.abs(gpu - ref).max()) if gpu.size else 0.0
