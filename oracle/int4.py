"""4-bit KV cache with a full-precision residual window (fp64 oracle side).

TEST INFRASTRUCTURE, like the rest of this package.

What the pages fix: a quantized KV cache stores older entries with fewer bits
and reconstructs them when attention consumes them, with scale metadata
(kv-cache tag page, KV-cache quantization teaser); keys carry outlier
channels, so they are quantized per channel and values per token, and the
most recent tokens stay at full precision until a group of them is
quantized (SoK paper section 2.3, KIVI; section 4.3: 4-bit storage is
near-free with per-channel keys, low-bit storage needs a full-precision
residual window).

Readings (where the pages leave the step open):
* the quantization group is one paged block of 16 tokens: each row's newest,
  partially filled block is held in a bf16 residual buffer
  ``[B][n_kv][16][d_h]`` at slot ``t % 16``; the append that fills a block
  (position ``t`` with ``t % 16 == 15``) encodes all 16 tokens into the
  block's physical slot;
* keys: one fixed fp32 scale per (KV head, channel), ``k_scale [n_kv][d_h]``
  (calibrated per-channel key scaling, chosen by the caller);
* values: one fp32 scale per token, ``v_scale [NB][n_kv][16]``, set when the
  block is encoded: ``amax / 7`` over the token's ``d_h`` values (1 when the
  row is all zero or not finite);
* codes: symmetric, ``code = RNE(fp32(x) * fp32(1 / scale))`` clamped to
  ``[-7, 7]``, value ``scale * code``; stored as the nibble ``code + 8``;
* packing: each group of 8 channels ``8k .. 8k+7`` takes 4 bytes; byte
  ``4k + i`` holds channel ``8k + i`` in its low nibble and ``8k + 4 + i`` in
  its high nibble (a layout chosen so one 16-byte load feeds the matrix
  cores).
"""
from __future__ import annotations

import numpy as np

BLOCK = 16
INT4 = 4           # cache dtype code of the 4-bit cache
F64 = 5            # oracle-internal: a cache already decoded to fp64
CODE_MAX = 7


def quantize_int4(y: np.ndarray) -> np.ndarray:
    """fp32 value -> symmetric 4-bit code: round half to even, clamp to
    [-7, 7]; NaN -> 0. Returned as int8."""
    y = np.asarray(y, dtype=np.float32)
    r = np.rint(y.astype(np.float64))
    r = np.where(np.isnan(r), 0.0, np.clip(r, -CODE_MAX, CODE_MAX))
    return r.astype(np.int8)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """codes [..., d_h] in [-7, 7] -> bytes [..., d_h / 2] in the packing
    above."""
    c = np.asarray(codes, dtype=np.int16)
    d_h = c.shape[-1]
    assert d_h % 8 == 0
    nib = (c + 8).astype(np.uint8)                      # 1 .. 15
    g = nib.reshape(c.shape[:-1] + (d_h // 8, 8))
    lo, hi = g[..., :4], g[..., 4:]
    return (lo | (hi << 4)).reshape(c.shape[:-1] + (d_h // 2,)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """bytes [..., d_h / 2] -> codes [..., d_h] (int8), inverse of pack_int4."""
    p = np.asarray(packed, dtype=np.uint8)
    nb = p.shape[-1]
    g = p.reshape(p.shape[:-1] + (nb // 4, 4))
    lo = (g & 0x0F).astype(np.int16) - 8
    hi = (g >> 4).astype(np.int16) - 8
    return np.concatenate([lo, hi], axis=-1).reshape(p.shape[:-1] + (2 * nb,)).astype(np.int8)


def _bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def token_scale(v: np.ndarray) -> np.ndarray:
    """Per-token value scale: fp32(amax / 7) over the last axis; 1 where the
    amax is 0 or not finite."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.max(np.abs(v), axis=-1)
    s = (amax / np.float32(CODE_MAX)).astype(np.float32)
    return np.where((amax > 0) & np.isfinite(amax), s, np.float32(1.0)).astype(np.float32)


def encode_block(k_vals: np.ndarray, v_vals: np.ndarray, k_scale: np.ndarray):
    """One full block's 16 tokens -> its stored form.
    k_vals, v_vals [n_kv][16][d_h] fp32 values; k_scale [n_kv][d_h] fp32.
    Returns (k packed [n_kv][16][d_h/2], v packed, v_scale [n_kv][16])."""
    k_vals = np.asarray(k_vals, dtype=np.float32)
    v_vals = np.asarray(v_vals, dtype=np.float32)
    kinv = np.float32(1.0) / np.asarray(k_scale, dtype=np.float32)
    kc = quantize_int4(k_vals * kinv[:, None, :])
    vs = token_scale(v_vals)
    vinv = np.float32(1.0) / vs
    vc = quantize_int4(v_vals * vinv[..., None])
    return pack_int4(kc), pack_int4(vc), vs


def kv_append_int4(state: dict, k_new: np.ndarray, v_new: np.ndarray, block_table: np.ndarray,
                   context_lens: np.ndarray, k_scale: np.ndarray) -> dict:
    """The append of each row's newest token (position n - 1) under the
    residual-window policy. state: 'k', 'v' packed caches [NB][n_kv][16][d_h/2]
    uint8, 'v_scale' [NB][n_kv][16] fp32, 'k_res', 'v_res' residual buffers
    [B][n_kv][16][d_h] bf16 bits. k_new, v_new [B][n_kv][d_h] bf16 bits.
    Returns a new state; rows with n <= 0 append nothing."""
    out = {k: np.array(v, copy=True) for k, v in state.items()}
    for b, n in enumerate(np.asarray(context_lens, dtype=np.int64)):
        if n <= 0:
            continue
        t = int(n) - 1
        r = t % BLOCK
        out["k_res"][b, :, r, :] = k_new[b]
        out["v_res"][b, :, r, :] = v_new[b]
        if r == BLOCK - 1:
            pb = int(block_table[b][t // BLOCK])
            kq, vq, vs = encode_block(_bf16_bits_to_f32(out["k_res"][b]),
                                      _bf16_bits_to_f32(out["v_res"][b]), k_scale)
            out["k"][pb] = kq
            out["v"][pb] = vq
            out["v_scale"][pb] = vs
    return out


def decoded_cache(state: dict, k_scale: np.ndarray, block_table: np.ndarray,
                  context_lens: np.ndarray):
    """The cache attention reads, in fp64: every full block decoded
    (k = k_scale[j][d] * code, v = v_scale[pb][j][t] * code), and each row's
    open block taken from its residual buffer as logical block n // 16,
    placed at physical index NB + b. Returns (k64, v64, table) with table the
    block table extended to point at those residual blocks."""
    kq, vq, vs = state["k"], state["v"], state["v_scale"]
    NB, n_kv = kq.shape[0], kq.shape[1]
    B = len(context_lens)
    kc = unpack_int4(kq).astype(np.float64) * np.asarray(k_scale, np.float64)[None, :, None, :]
    vc = unpack_int4(vq).astype(np.float64) * np.asarray(vs, np.float64)[..., None]
    kres = _bf16_bits_to_f32(state["k_res"]).astype(np.float64)
    vres = _bf16_bits_to_f32(state["v_res"]).astype(np.float64)
    k64 = np.concatenate([kc, kres], axis=0)
    v64 = np.concatenate([vc, vres], axis=0)
    table = np.array(block_table, dtype=np.int32, copy=True)
    for b, n in enumerate(np.asarray(context_lens, dtype=np.int64)):
        if n > 0 and n % BLOCK:
            table[b, n // BLOCK] = NB + b
    return k64, v64, table
