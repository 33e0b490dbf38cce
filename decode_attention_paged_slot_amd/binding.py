"""ctypes binding of libpda (include/pda.h): argument marshalling only.

Each function carries the C name without the `pda_` prefix. Device buffers
are torch tensors (their data pointers are passed; torch only provides device
memory and streams); host buffers of the block pool are numpy arrays. Every
piece of the decode step runs in the library's HIP kernels. Importing this
module fails loudly when libpda.so has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpda.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m decode_attention_paged_slot_amd.build` "
        "(or __graft_entry__.build()); there is no fallback implementation")

# One HIP runtime per process: torch ships its own libamdhip64.so.7. Loading
# torch first makes libpda's dependency (same soname) resolve to that copy, so
# torch's device pointers and streams are valid in the library's calls.
try:
    import torch as _torch_preload  # noqa: F401
except ImportError:
    pass

_lib = ctypes.CDLL(LIB_PATH)

OK, EINVAL, ENOSPC, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
F32, BF16, FP8_E4M3, INT8, INT4 = 0, 1, 2, 3, 4
_STATUS = {EINVAL: "EINVAL", ENOSPC: "ENOSPC", EWORKSPACE: "EWORKSPACE", EHIP: "EHIP"}


class PdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)}: {last_error()}")


class NoSpace(PdaError):
    """The block pool is exhausted (the engine's preemption signal)."""


class KvDesc(ctypes.Structure):
    _fields_ = [("n_kv", ctypes.c_int32), ("d_h", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("cache_dtype", ctypes.c_int32), ("src_dtype", ctypes.c_int32)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32),
                ("d_h", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("max_context", ctypes.c_int32),
                ("num_partitions", ctypes.c_int32), ("total_context", ctypes.c_int64),
                ("reuse_prefix_blocks", ctypes.c_int32), ("window", ctypes.c_int32),
                ("sink_tokens", ctypes.c_int32), ("new_dtype", ctypes.c_int32),
                ("prefix_blocks", ctypes.c_int32)]


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_p32 = ctypes.POINTER(ctypes.c_int32)
_SIGS = {
    "pda_version": (ctypes.c_char_p, []),
    "pda_last_error": (ctypes.c_char_p, []),
    "pda_pool_create": (_i32, [_i32, _vp, ctypes.POINTER(_vp)]),
    "pda_pool_destroy": (_i32, [_vp]),
    "pda_pool_alloc": (_i32, [_vp, _i32, _vp]),
    "pda_pool_share": (_i32, [_vp, _i32, _vp]),
    "pda_pool_free": (_i32, [_vp, _i32, _vp]),
    "pda_pool_num_free": (_i32, [_vp, _p32]),
    "pda_pool_refcount": (_i32, [_vp, _i32, _p32]),
    "pda_build_block_table": (_i32, [_vp, _i32, _vp, _i32, _i32, _vp, _i32, _vp, _vp]),
    "pda_kv_append": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, ctypes.POINTER(KvDesc), _vp]),
    "pda_kv_append_quant": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp,
                                   ctypes.POINTER(KvDesc), _vp]),
    "pda_attn_workspace_size": (_i32, [ctypes.POINTER(AttnDesc), ctypes.POINTER(_sz)]),
    "pda_attn_plan": (_i32, [ctypes.POINTER(AttnDesc), _p32, _p32]),
    "pda_paged_decode_attn": (_i32, [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                                     ctypes.POINTER(AttnDesc), _vp, _sz, _vp]),
    "pda_paged_decode_attn_quant": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float,
                                           _vp, ctypes.POINTER(AttnDesc), _vp, _sz, _vp]),
    "pda_lse_merge": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "pda_decode_step": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                               ctypes.POINTER(AttnDesc), _vp, _sz, _vp]),
    "pda_decode_step_quant": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float,
                                     _vp, ctypes.POINTER(AttnDesc), _vp, _sz, _vp]),
    "pda_paged_decode_attn_prefix": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                            ctypes.c_float, _vp, ctypes.POINTER(AttnDesc), _vp,
                                            _sz, _vp]),
    "pda_decode_step_prefix": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      ctypes.c_float, _vp, ctypes.POINTER(AttnDesc), _vp, _sz,
                                      _vp]),
    "pda_kv_append_int4": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  ctypes.POINTER(AttnDesc), _vp]),
    "pda_paged_decode_attn_int4": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          ctypes.c_float, _vp, ctypes.POINTER(AttnDesc), _vp,
                                          _sz, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTS = tuple(_SIGS)


def version() -> str:
    return _lib.pda_version().decode()


def last_error() -> str:
    return _lib.pda_last_error().decode()


def _check(rc: int, where: str) -> None:
    if rc == OK:
        return
    if rc == ENOSPC:
        raise NoSpace(rc, where)
    raise PdaError(rc, where)


# ------------------------------------------------------------ torch helpers
def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3,
         torch.int8: INT8}
    if t.dtype not in m:
        raise TypeError(f"unsupported tensor dtype {t.dtype}; pass uint8 codes with an explicit dtype")
    return m[t.dtype]


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


# ------------------------------------------------------------------ append
def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, *, stream=None) -> None:
    """pda_kv_append: k_new/v_new [T, n_kv, d_h]; caches [NB, n_kv, bs, d_h]
    (same dtype, f32 or bf16); slot_mapping [T] int64."""
    nb, n_kv, bs, d_h = k_cache.shape
    dt = dtype_code(k_cache)
    d = KvDesc(n_kv, d_h, bs, nb, dt, dtype_code(k_new))
    _check(_lib.pda_kv_append(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), int(k_new.shape[0]),
                              _ptr(k_cache), _ptr(v_cache), ctypes.byref(d), _stream(stream)),
           "pda_kv_append")


def kv_append_quant(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, *,
                    cache_dtype: Optional[int] = None, stream=None) -> None:
    """pda_kv_append_quant: caches hold 8-bit codes (torch.float8_e4m3fn,
    torch.int8, or uint8 with `cache_dtype`); scales [NB, n_kv] fp32."""
    nb, n_kv, bs, d_h = k_cache.shape
    dt = cache_dtype if cache_dtype is not None else dtype_code(k_cache)
    d = KvDesc(n_kv, d_h, bs, nb, dt, dtype_code(k_new))
    _check(_lib.pda_kv_append_quant(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
                                    int(k_new.shape[0]), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(k_scale), _ptr(v_scale), ctypes.byref(d),
                                    _stream(stream)), "pda_kv_append_quant")


# --------------------------------------------------------------- attention
def attn_desc(q, k_cache, block_table, *, max_context: int, out_dtype: int = F32,
              kv_dtype: Optional[int] = None, num_partitions: int = 0,
              total_context: int = 0, reuse_prefix_blocks: int = 0, window: int = 0,
              sink_tokens: int = 0, new_dtype: Optional[int] = None,
              prefix_blocks: int = 0) -> AttnDesc:
    B, n_q, d_h = q.shape
    nb, n_kv, bs, d2 = k_cache.shape
    kvd = kv_dtype if kv_dtype is not None else dtype_code(k_cache)
    assert d2 == d_h or (kvd == INT4 and 2 * d2 == d_h)   # 4-bit: two codes per byte
    return AttnDesc(B, n_q, n_kv, d_h, bs, int(block_table.shape[1]), nb, kvd, dtype_code(q),
                    out_dtype, int(max_context), int(num_partitions), int(total_context),
                    int(reuse_prefix_blocks), int(window), int(sink_tokens),
                    kvd if new_dtype is None else int(new_dtype), int(prefix_blocks))


def attn_workspace_size(desc: AttnDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.pda_attn_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "pda_attn_workspace_size")
    return int(n.value)


def attn_plan(desc: AttnDesc):
    p, b = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(_lib.pda_attn_plan(ctypes.byref(desc), ctypes.byref(p), ctypes.byref(b)),
           "pda_attn_plan")
    return int(p.value), int(b.value)


def workspace_for(desc: AttnDesc, device):
    """Allocate a workspace tensor of the size the descriptor needs (or None)."""
    n = attn_workspace_size(desc)
    if n == 0:
        return None
    torch = _torch()
    return torch.empty(n, dtype=torch.uint8, device=device)


def paged_decode_attn(q, k_cache, v_cache, block_table, context_lens, scale: float, out, *,
                      desc: Optional[AttnDesc] = None, workspace=None, max_context: int = 0,
                      num_partitions: int = 0, total_context: int = 0,
                      reuse_prefix_blocks: int = 0, window: int = 0, sink_tokens: int = 0,
                      stream=None) -> None:
    """pda_paged_decode_attn (f32 / bf16 caches). `out` [B, n_q, d_h] f32 or bf16."""
    if desc is None:
        desc = attn_desc(q, k_cache, block_table, max_context=max_context,
                         out_dtype=dtype_code(out), num_partitions=num_partitions,
                         total_context=total_context, reuse_prefix_blocks=reuse_prefix_blocks,
                         window=window, sink_tokens=sink_tokens)
    if workspace is None:
        workspace = workspace_for(desc, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pda_paged_decode_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                      _ptr(context_lens), float(scale), _ptr(out),
                                      ctypes.byref(desc), _ptr(workspace), ws_bytes,
                                      _stream(stream)), "pda_paged_decode_attn")


def paged_decode_attn_quant(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                            scale: float, out, *, kv_dtype: Optional[int] = None,
                            desc: Optional[AttnDesc] = None, workspace=None,
                            max_context: int = 0, num_partitions: int = 0,
                            total_context: int = 0, reuse_prefix_blocks: int = 0,
                            window: int = 0, sink_tokens: int = 0, stream=None) -> None:
    """pda_paged_decode_attn_quant (fp8 e4m3 / int8 caches with per-(block, head)
    fp32 scales [NB, n_kv])."""
    if desc is None:
        desc = attn_desc(q, k_cache, block_table, max_context=max_context,
                         out_dtype=dtype_code(out), kv_dtype=kv_dtype,
                         num_partitions=num_partitions, total_context=total_context,
                         reuse_prefix_blocks=reuse_prefix_blocks, window=window,
                         sink_tokens=sink_tokens)
    if workspace is None:
        workspace = workspace_for(desc, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pda_paged_decode_attn_quant(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                            _ptr(v_scale), _ptr(block_table), _ptr(context_lens),
                                            float(scale), _ptr(out), ctypes.byref(desc),
                                            _ptr(workspace), ws_bytes, _stream(stream)),
           "pda_paged_decode_attn_quant")


def decode_step(q, k_new, v_new, k_cache, v_cache, block_table, context_lens, scale: float,
                out, *, desc: AttnDesc, workspace=None, stream=None) -> None:
    """pda_decode_step: append each row's new K/V at position n - 1 and
    attend, in one launch (f32 / bf16 caches; k_new, v_new [B, n_kv, d_h])."""
    if workspace is None:
        workspace = workspace_for(desc, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pda_decode_step(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                _ptr(block_table), _ptr(context_lens), float(scale), _ptr(out),
                                ctypes.byref(desc), _ptr(workspace), ws_bytes, _stream(stream)),
           "pda_decode_step")


def decode_step_quant(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table,
                      context_lens, scale: float, out, *, desc: AttnDesc, workspace=None,
                      stream=None) -> None:
    """pda_decode_step_quant: as decode_step on an 8-bit cache; the new rows
    (desc.new_dtype f32 / bf16) are encoded with their blocks' scales."""
    if workspace is None:
        workspace = workspace_for(desc, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pda_decode_step_quant(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                      _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                      _ptr(block_table), _ptr(context_lens), float(scale),
                                      _ptr(out), ctypes.byref(desc), _ptr(workspace), ws_bytes,
                                      _stream(stream)), "pda_decode_step_quant")


def paged_decode_attn_prefix(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                             prefix_table, prefix_lens, scale: float, out, *, desc: AttnDesc,
                             workspace=None, stream=None) -> None:
    """pda_paged_decode_attn_prefix: attention with a shared prefix read once.
    prefix_table [desc.prefix_blocks] int32, prefix_lens [B] int32; k_scale /
    v_scale [NB, n_kv] f32 for 8-bit caches, None for bf16."""
    if workspace is None:
        workspace = workspace_for(desc, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pda_paged_decode_attn_prefix(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                             _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
                                             _ptr(context_lens), _ptr(prefix_table),
                                             _ptr(prefix_lens), float(scale), _ptr(out),
                                             ctypes.byref(desc), _ptr(workspace), ws_bytes,
                                             _stream(stream)), "pda_paged_decode_attn_prefix")


def decode_step_prefix(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table,
                       context_lens, prefix_table, prefix_lens, scale: float, out, *,
                       desc: AttnDesc, workspace=None, stream=None) -> None:
    """pda_decode_step_prefix: the fused decode step with a shared prefix read once."""
    if workspace is None:
        workspace = workspace_for(desc, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pda_decode_step_prefix(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                       _ptr(block_table), _ptr(context_lens), _ptr(prefix_table),
                                       _ptr(prefix_lens), float(scale), _ptr(out),
                                       ctypes.byref(desc), _ptr(workspace), ws_bytes,
                                       _stream(stream)), "pda_decode_step_prefix")


def kv_append_int4(k_new, v_new, block_table, context_lens, k_q, v_q, k_scale, v_scale, k_res,
                   v_res, *, desc: AttnDesc, stream=None) -> None:
    """pda_kv_append_int4: each row's newest token into its residual slot;
    a filled block is encoded into the 4-bit cache. k_new, v_new [B, n_kv,
    d_h] bf16; k_q, v_q [NB, n_kv, 16, d_h / 2] uint8; k_scale [n_kv, d_h]
    f32; v_scale [NB, n_kv, 16] f32; k_res, v_res [B, n_kv, 16, d_h] bf16."""
    _check(_lib.pda_kv_append_int4(_ptr(k_new), _ptr(v_new), _ptr(block_table),
                                   _ptr(context_lens), _ptr(k_q), _ptr(v_q), _ptr(k_scale),
                                   _ptr(v_scale), _ptr(k_res), _ptr(v_res), ctypes.byref(desc),
                                   _stream(stream)), "pda_kv_append_int4")


def paged_decode_attn_int4(q, k_q, v_q, k_scale, v_scale, k_res, v_res, block_table,
                           context_lens, scale: float, out, *, desc: AttnDesc, workspace=None,
                           stream=None) -> None:
    """pda_paged_decode_attn_int4: attention over the 4-bit cache and the
    rows' residual windows (desc.kv_dtype = INT4)."""
    if workspace is None:
        workspace = workspace_for(desc, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pda_paged_decode_attn_int4(_ptr(q), _ptr(k_q), _ptr(v_q), _ptr(k_scale),
                                           _ptr(v_scale), _ptr(k_res), _ptr(v_res),
                                           _ptr(block_table), _ptr(context_lens), float(scale),
                                           _ptr(out), ctypes.byref(desc), _ptr(workspace),
                                           ws_bytes, _stream(stream)),
           "pda_paged_decode_attn_int4")


def lse_merge(part_o, part_ml, out, *, stream=None) -> None:
    """pda_lse_merge: part_o [rows, P, d_h], part_ml [rows, P, 2] -> out [rows, d_h]."""
    rows, P, d_h = part_o.shape
    _check(_lib.pda_lse_merge(_ptr(part_o), _ptr(part_ml), rows, P, d_h, _ptr(out),
                              _stream(stream)), "pda_lse_merge")


# -------------------------------------------------------------------- pool
def _i32arr(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


class Pool:
    """Host block pool (pda_pool_*): FIFO free list from `free_order`."""

    def __init__(self, num_blocks: int, free_order: Optional[Sequence[int]] = None):
        self._h = ctypes.c_void_p()
        fo = None if free_order is None else _i32arr(free_order)
        if fo is not None and fo.size != num_blocks:
            raise ValueError("free_order must list every block once")
        _check(_lib.pda_pool_create(int(num_blocks), None if fo is None else fo.ctypes.data,
                                    ctypes.byref(self._h)), "pda_pool_create")
        self.num_blocks = int(num_blocks)

    def close(self) -> None:
        if self._h:
            _lib.pda_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc(self, n: int) -> np.ndarray:
        ids = np.empty(max(n, 0), dtype=np.int32)
        _check(_lib.pda_pool_alloc(self._h, int(n), ids.ctypes.data if n > 0 else None),
               "pda_pool_alloc")
        return ids

    def share(self, ids) -> None:
        a = _i32arr(ids)
        _check(_lib.pda_pool_share(self._h, a.size, a.ctypes.data if a.size else None),
               "pda_pool_share")

    def free(self, ids) -> None:
        a = _i32arr(ids)
        _check(_lib.pda_pool_free(self._h, a.size, a.ctypes.data if a.size else None),
               "pda_pool_free")

    def num_free(self) -> int:
        n = ctypes.c_int32(0)
        _check(_lib.pda_pool_num_free(self._h, ctypes.byref(n)), "pda_pool_num_free")
        return int(n.value)

    def refcount(self, block: int) -> int:
        n = ctypes.c_int32(0)
        _check(_lib.pda_pool_refcount(self._h, int(block), ctypes.byref(n)), "pda_pool_refcount")
        return int(n.value)

    def build_block_table(self, context_lens, block_size: int, max_blocks: int,
                          shared_ids=()):
        """-> (block_table [B, max_blocks] int32, slot_mapping [B] int64)."""
        cl = _i32arr(context_lens)
        sh = _i32arr(shared_ids)
        table = np.empty((cl.size, max_blocks), dtype=np.int32)
        slots = np.empty(cl.size, dtype=np.int64)
        _check(_lib.pda_build_block_table(self._h, cl.size, cl.ctypes.data if cl.size else None,
                                          int(block_size), sh.size,
                                          sh.ctypes.data if sh.size else None, int(max_blocks),
                                          table.ctypes.data if cl.size else None,
                                          slots.ctypes.data if cl.size else None),
               "pda_build_block_table")
        return table, slots
