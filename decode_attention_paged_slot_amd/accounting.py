"""Algorithmic byte and FLOP accounting for paged decode attention.

Counts what the method must move, not what a kernel happens to move:

* KV bytes of a sequence: 2 * T * L * H_kv * d_h * b (keys and values, T
  tokens, L layers, H_kv KV heads, head dim d_h, b bytes per element) -- the
  formula in "9 Decode and KV Cache", section 9.7 (worked example "One
  128k-token sequence"), which is also Eq. (1) of the SoK paper (section 1.2;
  the display equation is lost in extraction, the text keeps its factors).
* Attention FLOPs: 4 * s * d_h per query head over s cached tokens (one
  score and one weighted-sum multiply-add per element), read against
  2 * s * d_h * w_kv bytes per KV head: 2 / w_kv FLOP/B, times the group
  factor g with grouped-query attention (SoK section 1.1). The worked 8B
  layer gives 4 FLOP/B (section 9.3). Softmax adds a 3 / (4 d_h) fraction of
  the contraction count (SoK appendix A.1).
* Per step, the cache is read exactly once with no score spill; the write of
  the new token's K/V is a 1/s correction (SoK appendix A.1 and C.4).

Units are decimal (GB = 1e9 bytes, TB/s = 1e12 bytes/s), as in the SoK
paper's appendix C.2.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

ELEM_BYTES = {0: 4, 1: 2, 2: 1, 3: 1}   # f32, bf16, fp8 e4m3, int8


def kv_bytes_per_token(layers: int, n_kv: int, d_h: int, elem_bytes: float) -> int:
    """Bytes of keys plus values one token adds to the cache, all layers."""
    return int(2 * layers * n_kv * d_h * elem_bytes)


def kv_bytes_sequence(tokens: int, layers: int, n_kv: int, d_h: int, elem_bytes: float) -> int:
    """2 * T * L * H_kv * d_h * b."""
    return int(2 * tokens * layers * n_kv * d_h * elem_bytes)


def mla_bytes_per_token(latent_dims: int, layers: int, elem_bytes: int) -> int:
    """A latent-compressed cache stores one latent vector per token per layer."""
    return latent_dims * layers * elem_bytes


def attention_flops(n_q: int, d_h: int, tokens: int) -> int:
    """4 * s * d_h per query head (score + weighted sum), softmax excluded."""
    return 4 * n_q * d_h * tokens


def attention_intensity(g: int, elem_bytes: float) -> float:
    """FLOP per KV byte read: 2 g / w_kv."""
    return 2.0 * g / elem_bytes


def softmax_fraction(d_h: int) -> float:
    return 3.0 / (4.0 * d_h)


def rate_ceiling(bandwidth_bytes_per_s: float, bytes_per_token: int) -> float:
    """Long-context token-rate ceiling R_inf = beta / (KV bytes per token)."""
    return bandwidth_bytes_per_s / bytes_per_token


def ridge_point(flops_per_s: float, bytes_per_s: float) -> float:
    return flops_per_s / bytes_per_s


@dataclasses.dataclass
class StepBytes:
    """Algorithmic bytes of one decode step of one layer."""
    kv_read: int          # every valid (token, KV head) K and V row once
    kv_read_unique: int   # shared physical blocks counted once
    q_read: int
    table_read: int       # block-table entries in use, 4 B each
    lens_read: int
    scales_read: int      # per-(block, KV head) K and V scales of touched blocks
    out_write: int        # fp32 (or bf16) outputs
    append_read: int      # the new K/V rows and their slot indices
    append_write: int     # the new K/V rows landing in the cache

    @property
    def attention(self) -> int:
        """Bytes the attention (+ merge) must move."""
        return (self.kv_read + self.q_read + self.table_read + self.lens_read +
                self.scales_read + self.out_write)

    @property
    def attention_unique(self) -> int:
        return self.attention - self.kv_read + self.kv_read_unique

    @property
    def step(self) -> int:
        """Append + attention."""
        return self.attention + self.append_read + self.append_write


def attended_tokens(n: int, window: int = 0, sinks: int = 0) -> int:
    """Positions of an n-token row that attention reads: all of them, or with
    a sliding window the last `window` plus the first `sinks`."""
    if window <= 0 or n <= sinks + window:
        return n
    return sinks + window


def attended_blocks(n: int, block_size: int, window: int = 0, sinks: int = 0) -> int:
    """Blocks holding at least one attended position of an n-token row."""
    nblk = -(-n // block_size)
    if window <= 0 or n <= sinks + window:
        return nblk
    sb = -(-sinks // block_size)
    return sb + nblk - max((n - window) // block_size, sb)


def step_bytes(context_lens: Sequence[int], *, n_q: int, n_kv: int, d_h: int, block_size: int,
               kv_dtype: int, q_dtype: int, out_bytes: int = 4, new_dtype: Optional[int] = None,
               appended_tokens: Optional[int] = None, shared_prefix_blocks: int = 0,
               window: int = 0, sinks: int = 0) -> StepBytes:
    """Bytes one decode step must move (SoK appendix A.1 accounting); with a
    sliding window only the attended positions count."""
    w_q = ELEM_BYTES[q_dtype]
    B = len(context_lens)
    if kv_dtype == 4:
        return _step_bytes_int4(context_lens, n_q=n_q, n_kv=n_kv, d_h=d_h, w_q=w_q,
                                out_bytes=out_bytes, appended_tokens=appended_tokens)
    w_kv = ELEM_BYTES[kv_dtype]
    tokens = sum(attended_tokens(int(n), window, sinks) for n in context_lens)
    blocks = [attended_blocks(int(n), block_size, window, sinks) for n in context_lens]
    kv = 2 * tokens * n_kv * d_h * w_kv
    if shared_prefix_blocks:
        shared = [min(shared_prefix_blocks, max(nb - 1, 0)) for nb in blocks]
        used_shared = max(shared) if shared else 0
        dup_tokens = sum(s * block_size for s in shared) - used_shared * block_size
        kv_unique = kv - 2 * dup_tokens * n_kv * d_h * w_kv
    else:
        kv_unique = kv
    quant = kv_dtype in (2, 3)
    scales = 2 * sum(blocks) * n_kv * 4 if quant else 0
    T = B if appended_tokens is None else appended_tokens
    w_new = ELEM_BYTES[new_dtype if new_dtype is not None else (kv_dtype if not quant else 1)]
    return StepBytes(
        kv_read=kv, kv_read_unique=kv_unique, q_read=B * n_q * d_h * w_q,
        table_read=4 * sum(blocks), lens_read=4 * B, scales_read=scales,
        out_write=B * n_q * d_h * out_bytes,
        append_read=2 * T * n_kv * d_h * w_new + 8 * T,
        append_write=2 * T * n_kv * d_h * w_kv)


def _step_bytes_int4(context_lens, *, n_q, n_kv, d_h, w_q, out_bytes, appended_tokens):
    """4-bit cache with a residual window: each row's floor(n / 16) encoded
    blocks (half a byte per K and V element, a 4-B value scale per token and
    KV head) plus its n % 16 residual tokens in bf16; the per-channel key
    scales once; the block-table entries of the encoded blocks. The append
    writes the new rows into the residual buffers."""
    B = len(context_lens)
    full = sum((int(n) // 16) * 16 for n in context_lens)
    res = sum(int(n) % 16 for n in context_lens)
    kv = n_kv * d_h * (full + 4 * res)            # 2 (K, V) * (0.5 * full + 2 * res)
    T = B if appended_tokens is None else appended_tokens
    return StepBytes(
        kv_read=kv, kv_read_unique=kv, q_read=B * n_q * d_h * w_q,
        table_read=4 * (full // 16), lens_read=4 * B,
        scales_read=4 * n_kv * full + 4 * n_kv * d_h,
        out_write=B * n_q * d_h * out_bytes,
        append_read=2 * T * n_kv * d_h * 2 + 4 * T,
        append_write=2 * T * n_kv * d_h * 2)


def step_flops(context_lens: Sequence[int], n_q: int, d_h: int) -> int:
    return attention_flops(n_q, d_h, sum(int(n) for n in context_lens))


def decode_floor_seconds(weight_bytes: float, kv_bytes: float, bandwidth: float) -> float:
    """Ideal step-time floor: every weight and KV byte read once at full
    bandwidth (section 9.3, Table 9.1)."""
    return (weight_bytes + kv_bytes) / bandwidth


def gib(x: float) -> float:
    return x / float(1 << 30)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("dataclasses", "math")]
