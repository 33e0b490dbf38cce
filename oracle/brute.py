"""Brute-force contiguous attention in NumPy fp64 (test infrastructure).

A second, structurally different route to the same definition as the C
oracle: first walk every logical position through the block table to gather a
contiguous K and V per sequence, then apply softmax(q K^T * scale) V with
matrix products. Paging only decides where each position's rows are stored
and how they are found, so the result must equal plain attention over the
gathered rows ("9 Decode and KV Cache", section 9.5): the two must agree.
Intended for tiny inputs only.
"""
from __future__ import annotations

import numpy as np

from . import decode, FP8, INT8


def gather_contiguous(cache_f64: np.ndarray, table_row: np.ndarray, n: int, block_size: int):
    """[n, n_kv, d_h] rows of logical positions 0..n-1 of one sequence."""
    rows = []
    for t in range(n):
        pb = int(table_row[t // block_size])
        if pb < 0 or pb >= cache_f64.shape[0]:
            raise KeyError(t // block_size)
        rows.append(cache_f64[pb, :, t % block_size, :])
    return np.stack(rows) if rows else np.zeros((0,) + cache_f64.shape[1:2] + cache_f64.shape[3:])


def gather_positions(cache_f64: np.ndarray, table_row: np.ndarray, positions, block_size: int):
    """Rows of the listed logical positions only (the others are never looked up)."""
    rows = []
    for t in positions:
        pb = int(table_row[t // block_size])
        if pb < 0 or pb >= cache_f64.shape[0]:
            raise KeyError(t // block_size)
        rows.append(cache_f64[pb, :, t % block_size, :])
    return np.stack(rows)


def attended_positions(n: int, window: int = 0, sinks: int = 0):
    """Logical positions of an n-token row that enter the softmax: all of
    them, or with a sliding window of `window` tokens the last `window` plus
    the first `sinks` (attention sinks)."""
    if window <= 0 or n <= sinks + window:
        return list(range(n))
    return list(range(min(sinks, n))) + list(range(n - window, n))


def attention(q, k_cache, v_cache, block_table, context_lens, scale, *, n_q, n_kv, q_dtype,
              kv_dtype, k_scale=None, v_scale=None, window=0, sinks=0):
    """[B, n_q, d_h] fp64 outputs for every row."""
    qd = decode(q, q_dtype)
    kd = decode(k_cache, kv_dtype)
    vd = decode(v_cache, kv_dtype)
    if kv_dtype in (FP8, INT8):
        kd = kd * np.asarray(k_scale, dtype=np.float64)[:, :, None, None]
        vd = vd * np.asarray(v_scale, dtype=np.float64)[:, :, None, None]
    B, _, d_h = qd.shape
    g = n_q // n_kv
    bs = k_cache.shape[2]
    out = np.zeros((B, n_q, d_h))
    for b in range(B):
        n = int(context_lens[b])
        if n == 0:
            continue
        idx = attended_positions(n, window, sinks)
        K = gather_positions(kd, block_table[b], idx, bs)   # [len(idx), n_kv, d_h]
        V = gather_positions(vd, block_table[b], idx, bs)
        for h in range(n_q):
            j = h // g
            s = (K[:, j, :] @ qd[b, h]) * scale
            p = np.exp(s - s.max())
            out[b, h] = (p @ V[:, j, :]) / p.sum()
    return out
