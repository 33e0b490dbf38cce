"""fp64 CPU oracle for paged single-token decode attention.

TEST INFRASTRUCTURE. Only the test suite, the smoke check of the repository's
entry module and the benchmark's CPU-baseline leg may import this package. The
product library never loads it, and it imports nothing from the product: the
two sides share only the seeded input generators (the separate `synth`
module), which hold none of the method's arithmetic.

Contents, each written from the pages' statement of the method:

* `paged_attn`      -- decode attention through a block table, fp64, two-pass
                       softmax (C, `pda_oracle.c`). Paging only decides where
                       each position's rows are stored and how they are found;
                       the arithmetic is plain attention ("9 Decode and KV
                       Cache", section 9.5); GQA maps query head
                       h to KV head h // g (kv-cache tag page, GQA teaser; SoK
                       paper section 1.1). Optional sliding window with
                       attention sinks (section 9.7; sink and sliding-window
                       teasers on the tag page).
* `locate`, `slot_of` -- logical position -> (physical block, offset), the
                       translation that section 9.5's block-lookup example
                       performs, and the flat slot index pb * bs + off used to
                       address a cache row.
* `kv_append`       -- the append path (section 9.4, "Append path"): each new
                       token's K/V row lands in its mapped slot, bit for bit.
* `fp8_decode`, `quantize_fp8`, `quantize_int8`, `kv_append_quant` -- an
                       8-bit cache is encoded with fewer bits and reconstructed
                       when attention consumes it, with scale metadata (KV-cache
                       quantization teasers on the tag page; SoK section 2.3).
                       fp8 is OCP E4M3; the quantizer picks the nearest finite
                       code by brute force with ties to the even code.
* `merge`           -- log-sum-exp merge of split-KV partial results.
* `prefix_block_table`, `prefix_row_len` -- a prompt prefix stored once and
                       shared by many rows (SoK paper section 2.6): the block
                       table a shared-prefix call attends through, and which
                       rows are valid (copy on write, section 2.5).
* `int4` (module)   -- 4-bit cache with per-channel key scales, per-token
                       value scales and a full-precision residual window
                       (SoK paper sections 2.3 and 4.3): format, quantizer,
                       append policy, decoded cache; `paged_attn_int4`
                       attends through it.
* `OraclePool`      -- fixed-size blocks allocated on demand from a free list,
                       per-request block tables, reference-counted sharing
                       with copy-on-write (section 9.5; SoK section 2.5, tau=16).

Parity unpinned: none of the functions above (every one has a pin in
tests/test_oracle_*.py).
"""
from __future__ import annotations

import collections
import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from . import build as _build

F32, BF16, FP8, INT8 = 0, 1, 2, 3

_lib = None


def load(path: str) -> ctypes.CDLL:
    """Open a compiled oracle library and declare its C signatures."""
    L = ctypes.CDLL(path)
    L.or_paged_attn.restype = ctypes.c_int64
    L.or_paged_attn.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_double, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    L.or_decode.restype = ctypes.c_int
    L.or_decode.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]
    L.or_dec_fp8_code.restype = ctypes.c_double
    L.or_dec_fp8_code.argtypes = [ctypes.c_uint]
    L.or_num_threads.restype = ctypes.c_int
    return L


def lib() -> ctypes.CDLL:
    """The compiled oracle (PDA_ORACLE_LIB names another build of it, such as
    the test suite's sanitizer build)."""
    global _lib
    if _lib is None:
        other = os.environ.get("PDA_ORACLE_LIB")
        _lib = load(other if other else _build.ensure_built())
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def num_threads() -> int:
    return int(lib().or_num_threads())


# ------------------------------------------------------------------ decoding
def decode(raw: np.ndarray, dtype: int) -> np.ndarray:
    """Raw storage (fp32 / bf16 bits / fp8 codes / int8) -> fp64."""
    raw = np.ascontiguousarray(raw)
    out = np.empty(raw.size, dtype=np.float64)
    rc = lib().or_decode(raw.ctypes.data, dtype, raw.size, out.ctypes.data)
    if rc != 0:
        raise ValueError("unknown dtype")
    return out.reshape(raw.shape)


def fp8_decode(code: int) -> float:
    """OCP E4M3 value of one 8-bit code (NaN for S.1111.111)."""
    return float(lib().or_dec_fp8_code(int(code) & 0xFF))


def fp8_decode_table() -> np.ndarray:
    return np.array([fp8_decode(c) for c in range(256)], dtype=np.float64)


# ------------------------------------------------------------------ attention
def paged_attn(q, k_cache, v_cache, block_table, context_lens, scale, *, n_q, n_kv,
               q_dtype, kv_dtype, k_scale=None, v_scale=None, rows=None, t_begin=-1,
               t_end=-1, window=0, sinks=0, nthreads=0, _lib=None):
    """fp64 paged decode attention (see pda_oracle.c for the definition).

    Returns (out [n_rows, d_h], m [n_rows], z [n_rows], n_bad). `rows` lists
    flat (b * n_q + h) indices; None computes all. m is the max scaled score
    (natural-log units), z = sum_t exp(s_t - m). With window > 0 only the
    positions t < sinks or t >= n - window of each row are attended (sliding
    window with attention sinks, "9 Decode and KV Cache", section 9.7)."""
    q = np.ascontiguousarray(q)
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    B, nq_, d_h = q.shape
    assert nq_ == n_q
    num_blocks, nkv_, bs, dh2 = k_cache.shape
    assert nkv_ == n_kv and dh2 == d_h and v_cache.shape == k_cache.shape
    ks = vs = None
    if kv_dtype in (FP8, INT8):
        ks = np.ascontiguousarray(k_scale, dtype=np.float32)
        vs = np.ascontiguousarray(v_scale, dtype=np.float32)
    r = None
    n_rows = B * n_q
    if rows is not None:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = r.size
    out = np.empty((n_rows, d_h), dtype=np.float64)
    m = np.empty(n_rows, dtype=np.float64)
    z = np.empty(n_rows, dtype=np.float64)
    L = lib() if _lib is None else _lib
    bad = L.or_paged_attn(B, n_q, n_kv, d_h, bs, num_blocks, bt.shape[1], _ptr(q), q_dtype,
                          _ptr(k_cache), _ptr(v_cache), kv_dtype, _ptr(ks), _ptr(vs),
                          _ptr(bt), _ptr(cl), float(scale), _ptr(r), n_rows, int(t_begin),
                          int(t_end), int(window), int(sinks), _ptr(out), _ptr(m), _ptr(z),
                          int(nthreads))
    if bad < 0:
        raise ValueError("oracle: bad arguments")
    return out, m, z, int(bad)


def paged_attn_int4(q, state: dict, k_scale, block_table, context_lens, scale, *, n_q, n_kv,
                    q_dtype, rows=None, nthreads=0):
    """Decode attention over a 4-bit cache with a residual window: the
    definition of paged_attn applied to the cache as stored (full blocks
    decoded, each row's open block from its residual buffer; see int4)."""
    from . import int4
    k64, v64, table = int4.decoded_cache(state, k_scale, block_table, context_lens)
    return paged_attn(q, k64, v64, table, context_lens, scale, n_q=n_q, n_kv=n_kv,
                      q_dtype=q_dtype, kv_dtype=int4.F64, rows=rows, nthreads=nthreads)


def merge(o: np.ndarray, m: np.ndarray, z: np.ndarray) -> np.ndarray:
    """Merge split-KV partials of one row: o [P, d] (each normalised over its
    partition), m [P] max scores (natural log units), z [P] = sum exp(s - m).
    Partitions with z == 0 are empty and skipped; all empty -> zero row."""
    o = np.asarray(o, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    live = z > 0
    if not live.any():
        return np.zeros(o.shape[1])
    M = m[live].max()
    w = np.where(live, z * np.exp(np.where(live, m, M) - M), 0.0)
    return (w[:, None] * np.where(live[:, None], o, 0.0)).sum(axis=0) / w.sum()


# ------------------------------------------------------------ shared prefix
def prefix_row_len(n: int, pl: int, max_blocks: int, prefix_blocks: int) -> int:
    """Shared-prefix length of one row, or -1 for an invalid row. A row's first
    pl logical blocks are the shared prefix's blocks (SoK paper section 2.6,
    prefix sharing); the block that receives the row's newest token is never
    shared (section 2.5, copy on write), so pl <= ceil(n / bs) - 1, and pl
    cannot exceed the prefix table. An empty row has no prefix; a row whose
    length is itself invalid is invalid."""
    if n < 0 or n > max_blocks * 16:
        return -1
    if n == 0:
        return 0
    if pl < 0 or pl > prefix_blocks or pl >= (n + 15) // 16:
        return -1
    return pl


def prefix_block_table(block_table, context_lens, prefix_table, prefix_lens):
    """The block table a shared-prefix call attends through: logical block i
    of row b is prefix_table[i] for i < prefix_lens[b], else block_table[b][i].
    Returns (table [B, max_blocks] int32, invalid [B] bool); an invalid row
    (see prefix_row_len) keeps its entries and must come out NaN."""
    table = np.array(block_table, dtype=np.int32, copy=True)
    B, max_blocks = table.shape
    pt = [int(x) for x in prefix_table]
    invalid = np.zeros(B, dtype=bool)
    for b in range(B):
        pl = prefix_row_len(int(context_lens[b]), int(prefix_lens[b]), max_blocks, len(pt))
        if pl < 0:
            invalid[b] = True
            continue
        for i in range(pl):
            table[b, i] = pt[i]
    return table, invalid


# ---------------------------------------------------------- lookup and append
def locate(table, pos: int, block_size: int = 16):
    """(physical block, offset in it) of logical position `pos`.

    `table` maps logical block numbers to physical ones: a dict, or a
    sequence indexed by logical block in which a negative entry means
    "unmapped". divmod splits the position into its logical block and the
    offset; a logical block the table does not map raises KeyError (a row
    cannot be read there)."""
    lb, off = divmod(int(pos), int(block_size))
    if isinstance(table, dict):
        pb = table.get(lb, -1)
    else:
        pb = int(table[lb]) if 0 <= lb < len(table) else -1
    if pb < 0:
        raise KeyError(lb)
    return int(pb), off


def slot_of(block_table_row: Sequence[int], token_index: int, block_size: int) -> int:
    """Flat cache-row index of a logical position: physical block * bs + offset."""
    pb, off = locate(block_table_row, token_index, block_size)
    return pb * block_size + off


def kv_append(cache: np.ndarray, new: np.ndarray, slots: np.ndarray) -> np.ndarray:
    """cache [NB, n_kv, bs, d_h] raw; new [T, n_kv, d_h] raw; slots [T] int64.
    Returns a copy where row `slot` of every head holds the new bits; a
    negative slot is a padding token and writes nothing."""
    out = cache.copy()
    bs = cache.shape[2]
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        out[s // bs, :, s % bs, :] = new[t]
    return out


def _fp8_positive_values() -> np.ndarray:
    # codes 0x00 .. 0x7E are the non-negative finite values, ascending
    return np.array([fp8_decode(c) for c in range(0x7F)], dtype=np.float64)


def quantize_fp8(y: np.ndarray) -> np.ndarray:
    """fp32 -> OCP E4M3 code: the finite code nearest to y (brute force over
    all of them), ties to the even code; |y| beyond 448 therefore saturates to
    +-448. NaN -> 0x7F. The sign bit of y is kept (so -0.0 -> 0x80)."""
    y = np.asarray(y, dtype=np.float32)
    flat = y.reshape(-1)
    vals = _fp8_positive_values()
    # anything at or beyond the largest finite value is nearest to it; clamping
    # first keeps the distance comparison exact for huge or infinite inputs
    a = np.minimum(np.abs(flat.astype(np.float64)), vals[-1])
    out = np.empty(flat.size, dtype=np.uint8)
    chunk = 1 << 16
    for s in range(0, flat.size, chunk):
        aa = a[s:s + chunk]
        diff = np.abs(aa[:, None] - vals[None, :])
        first = np.argmin(diff, axis=1)                # lowest code among the ties
        best = diff[np.arange(aa.size), first]
        nxt = np.minimum(first + 1, vals.size - 1)
        tie = (nxt != first) & (diff[np.arange(aa.size), nxt] == best)
        code = np.where(tie & (first % 2 == 1), nxt, first)
        out[s:s + chunk] = code.astype(np.uint8)
    out |= np.where(np.signbit(flat), 0x80, 0).astype(np.uint8)
    out[np.isnan(flat)] = 0x7F
    return out.reshape(y.shape)


def quantize_int8(y: np.ndarray) -> np.ndarray:
    """fp32 -> symmetric int8 code: round half to even, clamp to [-127, 127];
    NaN -> 0."""
    y = np.asarray(y, dtype=np.float32)
    r = np.rint(y.astype(np.float64))
    r = np.where(np.isnan(r), 0.0, np.clip(r, -127.0, 127.0))
    return r.astype(np.int8)


def quant_input(x: np.ndarray, scale) -> np.ndarray:
    """The value the quantizer rounds: fp32(x) * fp32(1 / scale), each step
    one IEEE fp32 operation."""
    inv = np.float32(1.0) / np.asarray(scale, dtype=np.float32)
    return np.asarray(x, dtype=np.float32) * inv


def kv_append_quant(codes: np.ndarray, scales: np.ndarray, new_f32: np.ndarray,
                    slots: np.ndarray, dtype: int) -> np.ndarray:
    """Quantize each new row with its destination block's (per KV head) scale
    and store the codes in its slot. codes [NB, n_kv, bs, d_h] uint8/int8,
    scales [NB, n_kv] fp32, new_f32 [T, n_kv, d_h] fp32 values."""
    out = codes.copy()
    bs = codes.shape[2]
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        pb, off = s // bs, s % bs
        y = quant_input(new_f32[t], scales[pb][:, None])
        c = quantize_fp8(y) if dtype == FP8 else quantize_int8(y)
        out[pb, :, off, :] = c.view(out.dtype)
    return out


# ------------------------------------------------------------------ the pool
class NoSpace(Exception):
    """The pool cannot satisfy an allocation: the preemption signal."""


class OraclePool:
    """Reference model of the block manager: a FIFO free list (initial order
    given), all-or-nothing allocation from its front, reference counts for
    shared blocks, and a block returns to the back of the list when its last
    reference goes."""

    def __init__(self, num_blocks: int, free_order: Optional[Sequence[int]] = None):
        self.num_blocks = int(num_blocks)
        order = range(num_blocks) if free_order is None else [int(x) for x in free_order]
        assert sorted(order) == list(range(num_blocks)), "free_order must be a permutation"
        self.free = collections.deque(order)
        self.ref = [0] * num_blocks

    def num_free(self) -> int:
        return len(self.free)

    def alloc(self, n: int):
        if n < 0:
            raise ValueError("negative count")
        if n > len(self.free):
            raise NoSpace(n)
        ids = [self.free.popleft() for _ in range(n)]
        for i in ids:
            self.ref[i] = 1
        return ids

    def share(self, ids):
        for i in ids:
            if not (0 <= i < self.num_blocks) or self.ref[i] == 0:
                raise ValueError(f"share of unallocated block {i}")
        for i in ids:
            self.ref[i] += 1

    def release(self, ids):
        need = collections.Counter(int(i) for i in ids)
        for i, c in need.items():
            if not (0 <= i < self.num_blocks) or self.ref[i] < c:
                raise ValueError(f"free of unallocated block {i}")
        for i in ids:
            self.ref[i] -= 1
            if self.ref[i] == 0:
                self.free.append(i)

    def build_block_table(self, context_lens, block_size: int, max_blocks: int,
                          shared_ids: Sequence[int] = ()):
        """Per row b with n tokens: ceil(n / bs) logical blocks; the first
        min(len(shared_ids), blocks - 1) reuse the shared blocks (one more
        reference each), the rest are fresh blocks taken in order; the block
        that receives the row's newest token is always private (copy on
        write). Unused entries are -1. Returns (table [B, max_blocks] int32,
        slots [B] int64 of the newest token, -1 for an empty row).
        All-or-nothing: raises NoSpace / ValueError with no state change."""
        ctx = [int(x) for x in context_lens]
        plan = []
        fresh_total = 0
        for n in ctx:
            if n < 0:
                raise ValueError("negative context length")
            nblk = (n + block_size - 1) // block_size
            if nblk > max_blocks:
                raise ValueError("row needs more blocks than the table holds")
            sh = min(len(shared_ids), max(nblk - 1, 0))
            plan.append((n, nblk, sh))
            fresh_total += nblk - sh
        for sid in shared_ids:
            if not (0 <= sid < self.num_blocks) or self.ref[sid] == 0:
                raise ValueError("shared block is not allocated")
        if fresh_total > len(self.free):
            raise NoSpace(fresh_total)
        table = np.full((len(ctx), max_blocks), -1, dtype=np.int32)
        slots = np.full(len(ctx), -1, dtype=np.int64)
        for b, (n, nblk, sh) in enumerate(plan):
            ids = list(shared_ids[:sh])
            self.share(ids)
            ids += self.alloc(nblk - sh)
            table[b, :nblk] = ids
            if n > 0:
                slots[b] = slot_of(table[b], n - 1, block_size)
        return table, slots
