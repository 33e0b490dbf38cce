"""Seeded synthetic inputs for paged decode attention.

This module is shared by the oracle side and the GPU side of every test and by
the benchmark. It holds no part of the method's arithmetic: no dot products, no
softmax, no slot or block lookups, no quantization of the kind the kernels do.
It only draws random numbers and lays them out with the shapes, distributions
and structure of the workloads:

  * per-sequence context lengths (fixed or uniform in a range),
  * a random order of physical block ids (the pool's initial free list; the
    allocation itself is the block manager's job, see the block-table builders),
  * Gaussian queries / keys / values rounded to bf16 by round-to-nearest-even
    (numpy on the host, or torch on a device for the large workloads),
  * NaN poison for memory that no sequence owns, so any stray read shows up,
  * for quantized caches, codes drawn by torch's own fp8/int8 casts of scaled
    Gaussians (a library routine independent of both the oracle's and the
    kernels' quantizers) together with per-(block, head) fp32 scales.

Workload recipes follow the five configurations of the decode-attention study
(tiny MHA, Llama-3-8B layer, Llama-3-70B layer, long-context with sinks, and
quantized KV with a shared prefix); the shapes come from the pages'
KV-layout discussion ("9 Decode and KV Cache", sections 9.3-9.5) and the SoK
paper's Llama-3-70B running example (section 1.2).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

# dtype tags used across the repository's Python code (kept in sync with the
# C headers by value, not by import: 0 f32, 1 bf16, 2 fp8 e4m3 (OCP), 3 int8)
F32, BF16, FP8, INT8, INT4 = 0, 1, 2, 3, 4
DTYPE_NAMES = {F32: "f32", BF16: "bf16", FP8: "fp8_e4m3", INT8: "int8", INT4: "int4"}
ELEM_BYTES = {F32: 4, BF16: 2, FP8: 1, INT8: 1, INT4: 0.5}
BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and structure of one decode-attention workload."""
    name: str
    seed: int
    B: int
    n_q: int
    n_kv: int
    d_h: int
    block_size: int
    kv_dtype: int
    q_dtype: int
    ctx_lo: int            # context lengths (incl. the token appended this step)
    ctx_hi: int            # uniform integer in [ctx_lo, ctx_hi]
    pool_blocks: Optional[int] = None  # None: exactly the blocks needed
    free_fraction: float = 0.0         # extra free (poisoned) blocks in the pool
    sink_tokens: int = 0               # K rows at logical positions < sink_tokens ...
    sink_factor: float = 1.0           # ... are multiplied by this (exact in bf16)
    shared_prefix_tokens: int = 0      # first tokens' blocks shared by all rows
    scale: Optional[float] = None      # softmax scale; None -> 1/sqrt(d_h)
    attn_window: int = 0               # sliding window of the attention call (0 = none)
    attn_sinks: int = 0                # attention-sink tokens kept with the window

    @property
    def g(self) -> int:
        return self.n_q // self.n_kv

    @property
    def softmax_scale(self) -> float:
        return float(self.scale) if self.scale is not None else 1.0 / math.sqrt(self.d_h)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the study (shapes from the pages), and three variants of
# the 70B layer (sliding window with sinks, 4-bit cache) defined below.
TINY_MHA = Workload("tiny_mha", 1, B=1, n_q=4, n_kv=4, d_h=64, block_size=16,
                    kv_dtype=F32, q_dtype=F32, ctx_lo=256, ctx_hi=256, pool_blocks=32)
LLAMA8B_LAYER = Workload("llama3_8b_layer", 2, B=32, n_q=32, n_kv=8, d_h=128, block_size=16,
                         kv_dtype=BF16, q_dtype=BF16, ctx_lo=512, ctx_hi=4096,
                         scale=1.0 / math.sqrt(128))
LLAMA70B_LAYER = Workload("llama3_70b_layer_b8_32k", 3, B=8, n_q=64, n_kv=8, d_h=128,
                          block_size=16, kv_dtype=BF16, q_dtype=BF16, ctx_lo=32768,
                          ctx_hi=32768, free_fraction=0.10)
LONG_SINKS = Workload("long_context_131k_sinks", 4, B=1, n_q=64, n_kv=8, d_h=128,
                      block_size=16, kv_dtype=BF16, q_dtype=BF16, ctx_lo=131072,
                      ctx_hi=131072, sink_tokens=4, sink_factor=8.0)
QUANT_PREFIX_FP8 = Workload("quant_prefix_fp8", 5, B=64, n_q=32, n_kv=8, d_h=128,
                            block_size=16, kv_dtype=FP8, q_dtype=BF16, ctx_lo=1024,
                            ctx_hi=16384, shared_prefix_tokens=2048)
QUANT_PREFIX_INT8 = QUANT_PREFIX_FP8.with_(name="quant_prefix_int8", seed=6, kv_dtype=INT8)
# the 70B layer with a Mistral-style 4096-token sliding window plus the first
# 4 tokens kept as attention sinks ("9 Decode and KV Cache", section 9.7)
LLAMA70B_WINDOW = LLAMA70B_LAYER.with_(name="llama3_70b_layer_b8_32k_window4k_sinks4", seed=7,
                                       attn_window=4096, attn_sinks=4)

# The 70B layer on a 4-bit cache with a residual window: contexts end at
# every residual length, so some rows fill a block in this step.
LLAMA70B_INT4 = LLAMA70B_LAYER.with_(name="llama3_70b_layer_b8_32k_int4", seed=8, kv_dtype=INT4,
                                     ctx_lo=32753, ctx_hi=32768)

WORKLOADS = {w.name: w for w in (TINY_MHA, LLAMA8B_LAYER, LLAMA70B_LAYER, LONG_SINKS,
                                 QUANT_PREFIX_FP8, QUANT_PREFIX_INT8, LLAMA70B_WINDOW,
                                 LLAMA70B_INT4)}


# ---------------------------------------------------------------- primitives
def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns by round-to-nearest-even (input dtype conversion,
    done the standard way: add 0x7FFF plus the kept LSB, keep the high half).
    NaN inputs map to the canonical bf16 NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r[np.isnan(x)] = BF16_NAN
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def context_lengths(w: Workload, r: np.random.Generator) -> np.ndarray:
    if w.ctx_lo == w.ctx_hi:
        return np.full(w.B, w.ctx_lo, dtype=np.int32)
    return r.integers(w.ctx_lo, w.ctx_hi + 1, size=w.B).astype(np.int32)


def blocks_needed(ctx: np.ndarray, block_size: int) -> np.ndarray:
    """Number of logical blocks each row occupies (ceil division of its length)."""
    return (np.asarray(ctx, dtype=np.int64) + block_size - 1) // block_size


def pool_size(w: Workload, ctx: np.ndarray) -> int:
    need = int(blocks_needed(ctx, w.block_size).sum())
    if w.shared_prefix_tokens:
        # shared blocks are stored once; every row's private blocks are extra
        sp = w.shared_prefix_tokens // w.block_size
        nb = blocks_needed(ctx, w.block_size)
        need = sp + int(np.sum(nb - np.minimum(sp, nb - 1)))
    if w.pool_blocks is not None:
        return max(int(w.pool_blocks), need)
    if w.free_fraction > 0:
        return int(math.ceil(need / (1.0 - w.free_fraction)))
    return need


def free_order(num_blocks: int, r: np.random.Generator) -> np.ndarray:
    """A random permutation of physical block ids: the pool's initial free list.
    Drawing it here (rather than inside the pool) keeps the allocator's
    placement reproducible on both sides from one seeded input."""
    return r.permutation(num_blocks).astype(np.int32)


@dataclasses.dataclass
class HostInputs:
    """Host (numpy) inputs of one decode step."""
    w: Workload
    ctx: np.ndarray             # [B] int32, context lengths incl. the new token
    num_blocks: int
    free_order: np.ndarray      # [num_blocks] int32 permutation
    shared_ids_count: int       # number of shared prefix blocks (0 if none)
    q: np.ndarray               # [B, n_q, d_h] raw (float32 or uint16 bf16 bits)
    k_cache: np.ndarray         # [NB, n_kv, bs, d_h] raw (float32 / uint16 / uint8 / int8)
    v_cache: np.ndarray
    k_scale: Optional[np.ndarray] = None   # [NB, n_kv] float32 (quantized only)
    v_scale: Optional[np.ndarray] = None
    k_new: Optional[np.ndarray] = None     # [B, n_kv, d_h] raw, the step's new K
    v_new: Optional[np.ndarray] = None


def gaussian(shape, dtype: int, r: np.random.Generator) -> np.ndarray:
    """N(0,1) samples in the storage form of `dtype` (fp32, or bf16 bits)."""
    x = r.standard_normal(size=shape, dtype=np.float32)
    if dtype == F32:
        return x
    if dtype == BF16:
        return bf16_bits_from_f32(x)
    raise ValueError("gaussian(): only f32 / bf16 storage")


def raw_dtype(dtype: int):
    return {F32: np.float32, BF16: np.uint16, FP8: np.uint8, INT8: np.int8}[dtype]


def make_host_inputs(w: Workload, seed: Optional[int] = None, with_new: bool = True) -> HostInputs:
    """Draw every random input of one decode step of workload `w` on the host.

    The cache is filled with N(0,1) everywhere; which blocks and slots end up
    owned by a sequence is decided by the block-table builder from
    `free_order`, after which `poison_unowned` marks the rest as NaN.
    """
    if w.kv_dtype == INT4:
        raise ValueError("4-bit cache inputs are drawn on the device (make_device_inputs)")
    r = rng(w.seed if seed is None else seed)
    ctx = context_lengths(w, r)
    nb = pool_size(w, ctx)
    order = free_order(nb, r)
    q = gaussian((w.B, w.n_q, w.d_h), w.q_dtype, r)
    shape = (nb, w.n_kv, w.block_size, w.d_h)
    ks = vs = None
    if w.kv_dtype in (F32, BF16):
        kc = gaussian(shape, w.kv_dtype, r)
        vc = gaussian(shape, w.kv_dtype, r)
    else:
        kc, ks = quantized_gaussian(shape, w.kv_dtype, r)
        vc, vs = quantized_gaussian(shape, w.kv_dtype, r)
    kn = vn = None
    if with_new:
        src = BF16 if w.kv_dtype != F32 else F32
        kn = gaussian((w.B, w.n_kv, w.d_h), src, r)
        vn = gaussian((w.B, w.n_kv, w.d_h), src, r)
    sp = w.shared_prefix_tokens // w.block_size if w.shared_prefix_tokens else 0
    return HostInputs(w, ctx, nb, order, sp, q, kc, vc, ks, vs, kn, vn)


def quantized_gaussian(shape, dtype: int, r: np.random.Generator):
    """Codes + per-(block, head) scales for N(0,1) data stored 8-bit.

    scale = amax over the (block, head) tile / qmax (448 for fp8 e4m3, 127 for
    int8); codes come from torch's own casts of x/scale (float8_e4m3fn cast,
    or round + clamp for int8), a library path that neither the oracle nor the
    kernels use.
    """
    import torch
    x = r.standard_normal(size=shape, dtype=np.float32)
    amax = np.abs(x).max(axis=(2, 3))
    qmax = 448.0 if dtype == FP8 else 127.0
    scale = np.where(amax > 0, amax / qmax, 1.0).astype(np.float32)
    y = torch.from_numpy(x / scale[:, :, None, None])
    y = y.clamp(-qmax, qmax)
    if dtype == FP8:
        codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    else:
        codes = torch.round(y).clamp(-127, 127).to(torch.int8).numpy().copy()
    return codes, scale


def apply_sinks(w: Workload, k_cache: np.ndarray, block_table: np.ndarray) -> None:
    """Multiply the K rows of logical positions < w.sink_tokens by w.sink_factor
    (in place, all KV heads). Positions are located through the given table;
    a power-of-two factor is exact in bf16/fp32."""
    if not w.sink_tokens:
        return
    for b in range(block_table.shape[0]):
        for t in range(w.sink_tokens):
            pb = int(block_table[b, t // w.block_size])
            off = t % w.block_size
            if w.kv_dtype == BF16:
                vals = bf16_bits_to_f32(k_cache[pb, :, off, :]) * np.float32(w.sink_factor)
                k_cache[pb, :, off, :] = bf16_bits_from_f32(vals)
            elif w.kv_dtype == F32:
                k_cache[pb, :, off, :] *= np.float32(w.sink_factor)
            else:
                raise ValueError("sinks are defined for f32/bf16 caches")


def poison_unowned(w: Workload, k_cache, v_cache, block_table: np.ndarray, ctx: np.ndarray,
                   k_scale=None, v_scale=None) -> None:
    """Fill blocks no row references, and slots past each row's length in its
    last block, with NaN (fp32/bf16/fp8) so a stray read poisons the output.
    int8 has no NaN: unowned blocks get NaN scales and tail slots code -128."""
    nb = k_cache.shape[0]
    owned = np.zeros(nb, dtype=bool)
    bs = w.block_size
    for b in range(block_table.shape[0]):
        n = int(ctx[b])
        nblk = (n + bs - 1) // bs
        ids = block_table[b, :nblk]
        owned[ids] = True
    free = ~owned
    nan = {F32: np.float32(np.nan), BF16: BF16_NAN, FP8: FP8_NAN, INT8: np.int8(-128)}[w.kv_dtype]
    k_cache[free] = nan
    v_cache[free] = nan
    if k_scale is not None:
        k_scale[free] = np.float32(np.nan)
        v_scale[free] = np.float32(np.nan)
    for b in range(block_table.shape[0]):
        n = int(ctx[b])
        if n % bs:
            pb = int(block_table[b, (n - 1) // bs])
            # a shared block is never a row's last block, so this cannot
            # clobber another row's data
            k_cache[pb, :, n % bs:, :] = nan
            v_cache[pb, :, n % bs:, :] = nan


# ----------------------------------------------------- device (torch) inputs
def device_gaussian_bf16(shape, gen, device):
    """N(0,1) bf16 tensor drawn on `device` with a seeded torch generator; the
    fp32 -> bf16 cast is torch's round-to-nearest-even."""
    import torch
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


@dataclasses.dataclass
class DeviceInputs:
    """Device (torch) inputs of one decode step; block tables are built by the
    caller (the oracle's pool model in tests, the library's pool in the
    benchmark) from `free_order`."""
    w: Workload
    ctx: np.ndarray
    num_blocks: int
    free_order: np.ndarray
    shared_ids_count: int
    q: "object"
    k_cache: "object"
    v_cache: "object"
    k_scale: "object" = None
    v_scale: "object" = None
    k_new: "object" = None
    v_new: "object" = None
    k_res: "object" = None     # 4-bit cache: residual buffers [B][n_kv][16][d_h] bf16
    v_res: "object" = None


def _device_int4(shape, gen, device):
    """4-bit cache bytes drawn as codes: two independent codes per byte, each
    round(2 N(0,1)) clamped to [-7, 7] and stored as code + 8."""
    import torch
    def nib():
        c = torch.randn(shape, generator=gen, device=device).mul_(2.0).round_().clamp_(-7, 7)
        return (c + 8).to(torch.uint8)
    return nib() | (nib() << 4)


def _device_quantized(shape, dtype: int, gen, device):
    """Codes and per-(block, head) scales of N(0,1) data, with torch's casts."""
    import torch
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    amax = x.abs().amax(dim=(2, 3))
    qmax = 448.0 if dtype == FP8 else 127.0
    scale = torch.where(amax > 0, amax / qmax, torch.ones_like(amax)).float()
    y = (x / scale[:, :, None, None]).clamp_(-qmax, qmax)
    del x
    if dtype == FP8:
        codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    else:
        codes = torch.round(y).clamp_(-127, 127).to(torch.int8)
    return codes, scale


def make_device_inputs(w: Workload, device, seed: Optional[int] = None,
                       with_new: bool = True) -> DeviceInputs:
    """Draw one decode step's inputs of workload `w` directly in device memory
    (torch's seeded Philox generator; bf16 by torch's round-to-nearest-even
    cast). Lengths and the free-list order come from numpy as on the host."""
    import torch
    s = w.seed if seed is None else seed
    r = rng(s)
    ctx = context_lengths(w, r)
    nb = pool_size(w, ctx)
    order = free_order(nb, r)
    gen = torch.Generator(device=device)
    gen.manual_seed(s)
    qdt = torch.bfloat16 if w.q_dtype == BF16 else torch.float32
    q = torch.randn((w.B, w.n_q, w.d_h), generator=gen, device=device).to(qdt)
    shape = (nb, w.n_kv, w.block_size, w.d_h)
    ks = vs = kres = vres = None
    if w.kv_dtype == INT4:
        # codes, per-channel key scales (every 32nd channel an 8x outlier),
        # per-token value scales, bf16 residual windows
        cshape = (nb, w.n_kv, w.block_size, w.d_h // 2)
        k = _device_int4(cshape, gen, device)
        v = _device_int4(cshape, gen, device)
        mag = torch.where(torch.arange(w.d_h, device=device) % 32 == 5, 8.0, 1.0)
        ks = (0.15 + 0.15 * torch.rand((w.n_kv, w.d_h), generator=gen, device=device)) * mag
        vs = 0.1 + 0.4 * torch.rand((nb, w.n_kv, w.block_size), generator=gen, device=device)
        rshape = (w.B, w.n_kv, w.block_size, w.d_h)
        kres = torch.randn(rshape, generator=gen, device=device).to(torch.bfloat16)
        vres = torch.randn(rshape, generator=gen, device=device).to(torch.bfloat16)
    elif w.kv_dtype in (F32, BF16):
        kdt = torch.bfloat16 if w.kv_dtype == BF16 else torch.float32
        k = torch.randn(shape, generator=gen, device=device).to(kdt)
        v = torch.randn(shape, generator=gen, device=device).to(kdt)
    else:
        k, ks = _device_quantized(shape, w.kv_dtype, gen, device)
        v, vs = _device_quantized(shape, w.kv_dtype, gen, device)
    kn = vn = None
    if with_new:
        ndt = torch.float32 if w.kv_dtype == F32 else torch.bfloat16
        kn = torch.randn((w.B, w.n_kv, w.d_h), generator=gen, device=device).to(ndt)
        vn = torch.randn((w.B, w.n_kv, w.d_h), generator=gen, device=device).to(ndt)
    sp = w.shared_prefix_tokens // w.block_size if w.shared_prefix_tokens else 0
    return DeviceInputs(w, ctx, nb, order, sp, q, k, v, ks, vs, kn, vn, kres, vres)


def poison_unowned_device(w: Workload, inp: DeviceInputs, block_table: np.ndarray) -> None:
    """Device counterpart of `poison_unowned` (NaN in unowned blocks and in the
    tail slots of each row's last block; int8: NaN scales / code -128)."""
    import torch
    dev = inp.k_cache.device
    bs = w.block_size
    owned = np.zeros(inp.num_blocks, dtype=bool)
    for b in range(block_table.shape[0]):
        nblk = (int(inp.ctx[b]) + bs - 1) // bs
        owned[block_table[b, :nblk]] = True
    if w.kv_dtype == INT4:
        # blocks not yet encoded (free, or behind a residual window) get NaN
        # value scales; residual slots past the newest token get NaN rows
        # (the slots a filling append encodes from stay intact)
        full = np.zeros(inp.num_blocks, dtype=bool)
        for b in range(block_table.shape[0]):
            full[block_table[b, :int(inp.ctx[b]) // bs]] = True
        idx = torch.from_numpy(np.nonzero(~full)[0]).to(dev)
        if idx.numel():
            inp.v_scale[idx] = float("nan")
        for b in range(block_table.shape[0]):
            n = int(inp.ctx[b])
            first = (n - 1) % bs + 1 if n > 0 else 0
            inp.k_res[b, :, first:, :] = float("nan")
            inp.v_res[b, :, first:, :] = float("nan")
        return
    free = torch.from_numpy(np.nonzero(~owned)[0]).to(dev)
    if w.kv_dtype == F32:
        nan = float("nan")
    elif w.kv_dtype == BF16:
        nan = float("nan")
    elif w.kv_dtype == FP8:
        nan = 0x7F
    else:
        nan = -128
    if free.numel():
        inp.k_cache[free] = nan
        inp.v_cache[free] = nan
        if inp.k_scale is not None:
            inp.k_scale[free] = float("nan")
            inp.v_scale[free] = float("nan")
    for b in range(block_table.shape[0]):
        n = int(inp.ctx[b])
        if n % bs:
            pb = int(block_table[b, (n - 1) // bs])
            inp.k_cache[pb, :, n % bs:, :] = nan
            inp.v_cache[pb, :, n % bs:, :] = nan


def apply_sinks_device(w: Workload, inp: DeviceInputs, block_table: np.ndarray) -> None:
    """Device counterpart of `apply_sinks` (power-of-two factor: exact)."""
    if not w.sink_tokens:
        return
    for b in range(block_table.shape[0]):
        for t in range(w.sink_tokens):
            pb = int(block_table[b, t // w.block_size])
            inp.k_cache[pb, :, t % w.block_size, :] *= w.sink_factor
