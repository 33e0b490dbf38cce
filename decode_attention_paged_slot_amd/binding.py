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
# PDA_LIB names another build of the library to load instead (the test suite
# loads a host-only sanitizer build this way)
LIB_PATH = os.environ.get("PDA_LIB") or os.path.join(_HERE, "libpda.so")

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
    "pda_decode_step_int4": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    ctypes.c_float, _vp, ctypes.POINTER(AttnDesc), _vp, _sz,
                                    _vp]),
    "pda_hbm_read_probe": (_i32, [_vp, _sz, _vp, _i64, _i32, _i32, _vp, _vp]),
    "pda_paged_decode_attn_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                                             ctypes.POINTER(AttnDesc), _vp]),
}
NOALLOC_SCRATCH_BYTES = 16 << 20   # PDA_NOALLOC_SCRATCH_BYTES
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


# ------------------------------------------------------- argument checking
# Every device buffer is checked for dtype, device and contiguity before its
# pointer is handed over: the library sees raw pointers only, so a wrong
# element size (say an int32 slot_mapping) would otherwise be read as if it
# were right.
def _storage_dtypes(code: int):
    torch = _torch()
    return {F32: (torch.float32,), BF16: (torch.bfloat16,),
            FP8_E4M3: (torch.uint8, torch.float8_e4m3fn), INT8: (torch.int8, torch.uint8),
            INT4: (torch.uint8,)}[code]


def _need(t, name: str, dtypes, dev=None, shape=None, numel=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    return t


def _f32():
    return (_torch().float32,)


def _i32():
    return (_torch().int32,)


class BoundCall:
    """One library call with its arguments marshalled once.

    The argument block (device pointers, sizes, a private copy of the
    descriptor, the stream handle) is converted to C types when the call is
    bound; each call() then only re-enters the library with the same block,
    so the host cost per launch is the ctypes call itself. The bound tensors
    are kept alive by this object; writing new data into them between calls
    is how a caller feeds the next step."""

    __slots__ = ("_fn", "_args", "_keep", "name")

    def __init__(self, fn, args, keep, name):
        conv = []
        for a, t in zip(args, fn.argtypes):
            conv.append(a if isinstance(a, (ctypes._SimpleCData, ctypes.Structure))
                        or type(a).__name__ == "CArgObject" else t(a) if a is not None else None)
        self._fn = fn
        self._args = tuple(conv)
        self._keep = keep
        self.name = name

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc:
            _check(rc, self.name)


def _launch(name: str, args, keep, bind: bool, descs=()):
    fn = getattr(_lib, name)
    if bind:
        # private descriptor copies: a later change to the caller's struct
        # must not change what the bound call launches
        args = list(args)
        for i, a in enumerate(args):
            if isinstance(a, (AttnDesc, KvDesc)):
                cp = type(a).from_buffer_copy(a)
                keep = tuple(keep) + (cp,)
                args[i] = ctypes.byref(cp)
        return BoundCall(fn, args, keep, name)
    args = [ctypes.byref(a) if isinstance(a, (AttnDesc, KvDesc)) else a for a in args]
    _check(fn(*args), name)
    return None


# ------------------------------------------------------------------ append
def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, *, stream=None, bind=False):
    """pda_kv_append: k_new/v_new [T, n_kv, d_h]; caches [NB, n_kv, bs, d_h]
    (same dtype, f32 or bf16); slot_mapping [T] int64. bind=True returns a
    BoundCall instead of launching."""
    torch = _torch()
    dt = dtype_code(k_cache)
    nb, n_kv, bs, d_h = k_cache.shape
    dev = k_cache.device
    _need(k_cache, "k_cache", _storage_dtypes(dt), dev)
    _need(v_cache, "v_cache", _storage_dtypes(dt), dev, shape=k_cache.shape)
    T = int(k_new.shape[0])
    _need(k_new, "k_new", _storage_dtypes(dtype_code(k_new)), dev, shape=(T, n_kv, d_h))
    _need(v_new, "v_new", (k_new.dtype,), dev, shape=(T, n_kv, d_h))
    _need(slot_mapping, "slot_mapping", (torch.int64,), dev, numel=T)
    d = KvDesc(n_kv, d_h, bs, nb, dt, dtype_code(k_new))
    return _launch("pda_kv_append", (_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), T,
                                     _ptr(k_cache), _ptr(v_cache), d, _stream(stream)),
                   (k_new, v_new, slot_mapping, k_cache, v_cache), bind)


def kv_append_quant(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, *,
                    cache_dtype: Optional[int] = None, stream=None, bind=False):
    """pda_kv_append_quant: caches hold 8-bit codes (torch.float8_e4m3fn,
    torch.int8, or uint8 with `cache_dtype`); scales [NB, n_kv] fp32."""
    torch = _torch()
    nb, n_kv, bs, d_h = k_cache.shape
    dt = cache_dtype if cache_dtype is not None else dtype_code(k_cache)
    dev = k_cache.device
    _need(k_cache, "k_cache", _storage_dtypes(dt), dev)
    _need(v_cache, "v_cache", _storage_dtypes(dt), dev, shape=k_cache.shape)
    T = int(k_new.shape[0])
    _need(k_new, "k_new", (torch.float32, torch.bfloat16), dev, shape=(T, n_kv, d_h))
    _need(v_new, "v_new", (k_new.dtype,), dev, shape=(T, n_kv, d_h))
    _need(slot_mapping, "slot_mapping", (torch.int64,), dev, numel=T)
    _need(k_scale, "k_scale", _f32(), dev, numel=nb * n_kv)
    _need(v_scale, "v_scale", _f32(), dev, numel=nb * n_kv)
    d = KvDesc(n_kv, d_h, bs, nb, dt, dtype_code(k_new))
    return _launch("pda_kv_append_quant",
                   (_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), T, _ptr(k_cache),
                    _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), d, _stream(stream)),
                   (k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale), bind)


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
    """A workspace tensor of the size the descriptor needs (or None),
    zero-filled so that its contents are the same on every run."""
    n = attn_workspace_size(desc)
    if n == 0:
        return None
    torch = _torch()
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _check_attn(desc: AttnDesc, q, k_cache, v_cache, block_table, context_lens, out,
                k_scale=None, v_scale=None, workspace=None, quant=False):
    """Shapes and dtypes of the attention tensors against the descriptor."""
    d = desc
    dev = q.device
    _need(q, "q", _storage_dtypes(d.q_dtype), dev, shape=(d.B, d.n_q, d.d_h))
    codes = INT4 if d.kv_dtype == INT4 else d.kv_dtype
    cols = d.d_h // 2 if d.kv_dtype == INT4 else d.d_h
    cshape = (d.num_blocks, d.n_kv, d.block_size, cols)
    _need(k_cache, "k_cache", _storage_dtypes(codes), dev, shape=cshape)
    _need(v_cache, "v_cache", _storage_dtypes(codes), dev, shape=cshape)
    _need(block_table, "block_table", _i32(), dev, shape=(d.B, d.max_blocks_per_seq))
    _need(context_lens, "context_lens", _i32(), dev, numel=d.B)
    _need(out, "out", _storage_dtypes(d.out_dtype), dev, shape=(d.B, d.n_q, d.d_h))
    if quant:
        n_sc = d.n_kv * d.d_h if d.kv_dtype == INT4 else d.num_blocks * d.n_kv
        _need(k_scale, "k_scale", _f32(), dev, numel=n_sc)
        n_vs = d.num_blocks * d.n_kv * d.block_size if d.kv_dtype == INT4 else d.num_blocks * d.n_kv
        _need(v_scale, "v_scale", _f32(), dev, numel=n_vs)
    _need(workspace, "workspace", (_torch().uint8,), dev, optional=True)


def _ws(desc, q, workspace):
    if workspace is None:
        workspace = workspace_for(desc, q.device)
    return workspace, (0 if workspace is None else workspace.numel() * workspace.element_size())


def _new_rows(desc: AttnDesc, k_new, v_new):
    shape = (desc.B, desc.n_kv, desc.d_h)
    _need(k_new, "k_new", _storage_dtypes(desc.new_dtype), k_new.device, shape=shape)
    _need(v_new, "v_new", _storage_dtypes(desc.new_dtype), k_new.device, shape=shape)


def paged_decode_attn(q, k_cache, v_cache, block_table, context_lens, scale: float, out, *,
                      desc: Optional[AttnDesc] = None, workspace=None, max_context: int = 0,
                      num_partitions: int = 0, total_context: int = 0,
                      reuse_prefix_blocks: int = 0, window: int = 0, sink_tokens: int = 0,
                      stream=None, bind=False):
    """pda_paged_decode_attn (f32 / bf16 caches). `out` [B, n_q, d_h] f32 or bf16."""
    if desc is None:
        desc = attn_desc(q, k_cache, block_table, max_context=max_context,
                         out_dtype=dtype_code(out), num_partitions=num_partitions,
                         total_context=total_context, reuse_prefix_blocks=reuse_prefix_blocks,
                         window=window, sink_tokens=sink_tokens)
    workspace, ws_bytes = _ws(desc, q, workspace)
    _check_attn(desc, q, k_cache, v_cache, block_table, context_lens, out, workspace=workspace)
    return _launch("pda_paged_decode_attn",
                   (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(context_lens),
                    float(scale), _ptr(out), desc, _ptr(workspace), ws_bytes, _stream(stream)),
                   (q, k_cache, v_cache, block_table, context_lens, out, workspace), bind)


def paged_decode_attn_noalloc(q, k_cache, v_cache, block_table, context_lens, scale: float,
                              out, *, desc: Optional[AttnDesc] = None, max_context: int = 0,
                              num_partitions: int = 0, total_context: int = 0,
                              reuse_prefix_blocks: int = 0, window: int = 0, sink_tokens: int = 0,
                              stream=None, bind=False):
    """pda_paged_decode_attn_noalloc: as paged_decode_attn, with the workspace
    taken from the library's fixed device scratch (no allocation anywhere)."""
    if desc is None:
        desc = attn_desc(q, k_cache, block_table, max_context=max_context,
                         out_dtype=dtype_code(out), num_partitions=num_partitions,
                         total_context=total_context, reuse_prefix_blocks=reuse_prefix_blocks,
                         window=window, sink_tokens=sink_tokens)
    _check_attn(desc, q, k_cache, v_cache, block_table, context_lens, out)
    return _launch("pda_paged_decode_attn_noalloc",
                   (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(context_lens),
                    float(scale), _ptr(out), desc, _stream(stream)),
                   (q, k_cache, v_cache, block_table, context_lens, out), bind)


def paged_decode_attn_quant(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                            scale: float, out, *, kv_dtype: Optional[int] = None,
                            desc: Optional[AttnDesc] = None, workspace=None,
                            max_context: int = 0, num_partitions: int = 0,
                            total_context: int = 0, reuse_prefix_blocks: int = 0,
                            window: int = 0, sink_tokens: int = 0, stream=None, bind=False):
    """pda_paged_decode_attn_quant (fp8 e4m3 / int8 caches with per-(block, head)
    fp32 scales [NB, n_kv])."""
    if desc is None:
        desc = attn_desc(q, k_cache, block_table, max_context=max_context,
                         out_dtype=dtype_code(out), kv_dtype=kv_dtype,
                         num_partitions=num_partitions, total_context=total_context,
                         reuse_prefix_blocks=reuse_prefix_blocks, window=window,
                         sink_tokens=sink_tokens)
    workspace, ws_bytes = _ws(desc, q, workspace)
    _check_attn(desc, q, k_cache, v_cache, block_table, context_lens, out, k_scale, v_scale,
                workspace, quant=True)
    return _launch("pda_paged_decode_attn_quant",
                   (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                    _ptr(block_table), _ptr(context_lens), float(scale), _ptr(out), desc,
                    _ptr(workspace), ws_bytes, _stream(stream)),
                   (q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, out,
                    workspace), bind)


def decode_step(q, k_new, v_new, k_cache, v_cache, block_table, context_lens, scale: float,
                out, *, desc: AttnDesc, workspace=None, stream=None, bind=False):
    """pda_decode_step: append each row's new K/V at position n - 1 and
    attend, in one launch (f32 / bf16 caches; k_new, v_new [B, n_kv, d_h])."""
    workspace, ws_bytes = _ws(desc, q, workspace)
    _check_attn(desc, q, k_cache, v_cache, block_table, context_lens, out, workspace=workspace)
    _new_rows(desc, k_new, v_new)
    return _launch("pda_decode_step",
                   (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                    _ptr(block_table), _ptr(context_lens), float(scale), _ptr(out), desc,
                    _ptr(workspace), ws_bytes, _stream(stream)),
                   (q, k_new, v_new, k_cache, v_cache, block_table, context_lens, out,
                    workspace), bind)


def decode_step_quant(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table,
                      context_lens, scale: float, out, *, desc: AttnDesc, workspace=None,
                      stream=None, bind=False):
    """pda_decode_step_quant: as decode_step on an 8-bit cache; the new rows
    (desc.new_dtype f32 / bf16) are encoded with their blocks' scales."""
    workspace, ws_bytes = _ws(desc, q, workspace)
    _check_attn(desc, q, k_cache, v_cache, block_table, context_lens, out, k_scale, v_scale,
                workspace, quant=True)
    _new_rows(desc, k_new, v_new)
    return _launch("pda_decode_step_quant",
                   (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                    _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(context_lens),
                    float(scale), _ptr(out), desc, _ptr(workspace), ws_bytes, _stream(stream)),
                   (q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table,
                    context_lens, out, workspace), bind)


def _prefix_args(desc, prefix_table, prefix_lens, dev):
    _need(prefix_table, "prefix_table", _i32(), dev, numel=desc.prefix_blocks)
    _need(prefix_lens, "prefix_lens", _i32(), dev, numel=desc.B)


def paged_decode_attn_prefix(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                             prefix_table, prefix_lens, scale: float, out, *, desc: AttnDesc,
                             workspace=None, stream=None, bind=False):
    """pda_paged_decode_attn_prefix: attention with a shared prefix read once.
    prefix_table [desc.prefix_blocks] int32, prefix_lens [B] int32; k_scale /
    v_scale [NB, n_kv] f32 for 8-bit caches, None for bf16."""
    workspace, ws_bytes = _ws(desc, q, workspace)
    quant = desc.kv_dtype in (FP8_E4M3, INT8)
    _check_attn(desc, q, k_cache, v_cache, block_table, context_lens, out, k_scale, v_scale,
                workspace, quant=quant)
    _prefix_args(desc, prefix_table, prefix_lens, q.device)
    return _launch("pda_paged_decode_attn_prefix",
                   (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                    _ptr(block_table), _ptr(context_lens), _ptr(prefix_table),
                    _ptr(prefix_lens), float(scale), _ptr(out), desc, _ptr(workspace),
                    ws_bytes, _stream(stream)),
                   (q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                    prefix_table, prefix_lens, out, workspace), bind)


def decode_step_prefix(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table,
                       context_lens, prefix_table, prefix_lens, scale: float, out, *,
                       desc: AttnDesc, workspace=None, stream=None, bind=False):
    """pda_decode_step_prefix: the fused decode step with a shared prefix read once."""
    workspace, ws_bytes = _ws(desc, q, workspace)
    quant = desc.kv_dtype in (FP8_E4M3, INT8)
    _check_attn(desc, q, k_cache, v_cache, block_table, context_lens, out, k_scale, v_scale,
                workspace, quant=quant)
    _new_rows(desc, k_new, v_new)
    _prefix_args(desc, prefix_table, prefix_lens, q.device)
    return _launch("pda_decode_step_prefix",
                   (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                    _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(context_lens),
                    _ptr(prefix_table), _ptr(prefix_lens), float(scale), _ptr(out), desc,
                    _ptr(workspace), ws_bytes, _stream(stream)),
                   (q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table,
                    context_lens, prefix_table, prefix_lens, out, workspace), bind)


def _int4_state(desc, k_res, v_res, dev):
    torch = _torch()
    res = (desc.B, desc.n_kv, desc.block_size, desc.d_h)
    _need(k_res, "k_res", (torch.bfloat16,), dev, shape=res)
    _need(v_res, "v_res", (torch.bfloat16,), dev, shape=res)


def kv_append_int4(k_new, v_new, block_table, context_lens, k_q, v_q, k_scale, v_scale, k_res,
                   v_res, *, desc: AttnDesc, stream=None, bind=False):
    """pda_kv_append_int4: each row's newest token into its residual slot;
    a filled block is encoded into the 4-bit cache. k_new, v_new [B, n_kv,
    d_h] bf16; k_q, v_q [NB, n_kv, 16, d_h / 2] uint8; k_scale [n_kv, d_h]
    f32; v_scale [NB, n_kv, 16] f32; k_res, v_res [B, n_kv, 16, d_h] bf16."""
    torch = _torch()
    dev = k_q.device
    d = desc
    shape = (d.B, d.n_kv, d.d_h)
    _need(k_new, "k_new", (torch.bfloat16,), dev, shape=shape)
    _need(v_new, "v_new", (torch.bfloat16,), dev, shape=shape)
    _need(block_table, "block_table", _i32(), dev, shape=(d.B, d.max_blocks_per_seq))
    _need(context_lens, "context_lens", _i32(), dev, numel=d.B)
    cshape = (d.num_blocks, d.n_kv, d.block_size, d.d_h // 2)
    _need(k_q, "k_q", (torch.uint8,), dev, shape=cshape)
    _need(v_q, "v_q", (torch.uint8,), dev, shape=cshape)
    _need(k_scale, "k_scale", _f32(), dev, numel=d.n_kv * d.d_h)
    _need(v_scale, "v_scale", _f32(), dev, numel=d.num_blocks * d.n_kv * d.block_size)
    _int4_state(d, k_res, v_res, dev)
    return _launch("pda_kv_append_int4",
                   (_ptr(k_new), _ptr(v_new), _ptr(block_table), _ptr(context_lens), _ptr(k_q),
                    _ptr(v_q), _ptr(k_scale), _ptr(v_scale), _ptr(k_res), _ptr(v_res), desc,
                    _stream(stream)),
                   (k_new, v_new, block_table, context_lens, k_q, v_q, k_scale, v_scale, k_res,
                    v_res), bind)


def paged_decode_attn_int4(q, k_q, v_q, k_scale, v_scale, k_res, v_res, block_table,
                           context_lens, scale: float, out, *, desc: AttnDesc, workspace=None,
                           stream=None, bind=False):
    """pda_paged_decode_attn_int4: attention over the 4-bit cache and the
    rows' residual windows (desc.kv_dtype = INT4)."""
    workspace, ws_bytes = _ws(desc, q, workspace)
    _check_attn(desc, q, k_q, v_q, block_table, context_lens, out, k_scale, v_scale, workspace,
                quant=True)
    _int4_state(desc, k_res, v_res, q.device)
    return _launch("pda_paged_decode_attn_int4",
                   (_ptr(q), _ptr(k_q), _ptr(v_q), _ptr(k_scale), _ptr(v_scale), _ptr(k_res),
                    _ptr(v_res), _ptr(block_table), _ptr(context_lens), float(scale), _ptr(out),
                    desc, _ptr(workspace), ws_bytes, _stream(stream)),
                   (q, k_q, v_q, k_scale, v_scale, k_res, v_res, block_table, context_lens, out,
                    workspace), bind)


def decode_step_int4(q, k_new, v_new, k_q, v_q, k_scale, v_scale, k_res, v_res, block_table,
                     context_lens, scale: float, out, *, desc: AttnDesc, workspace=None,
                     stream=None, bind=False):
    """pda_decode_step_int4: kv_append_int4 and paged_decode_attn_int4 in
    one launch pair (context_lens count the new token; k_new, v_new [B, n_kv,
    d_h] bf16, desc.new_dtype = BF16). Same bits as the two calls."""
    torch = _torch()
    if desc.new_dtype != BF16:
        raise ValueError("a fused 4-bit step takes bf16 k_new / v_new (desc.new_dtype = BF16)")
    workspace, ws_bytes = _ws(desc, q, workspace)
    _check_attn(desc, q, k_q, v_q, block_table, context_lens, out, k_scale, v_scale, workspace,
                quant=True)
    _int4_state(desc, k_res, v_res, q.device)
    shape = (desc.B, desc.n_kv, desc.d_h)
    _need(k_new, "k_new", (torch.bfloat16,), q.device, shape=shape)
    _need(v_new, "v_new", (torch.bfloat16,), q.device, shape=shape)
    return _launch("pda_decode_step_int4",
                   (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_q), _ptr(v_q), _ptr(k_scale),
                    _ptr(v_scale), _ptr(k_res), _ptr(v_res), _ptr(block_table),
                    _ptr(context_lens), float(scale), _ptr(out), desc, _ptr(workspace),
                    ws_bytes, _stream(stream)),
                   (q, k_new, v_new, k_q, v_q, k_scale, v_scale, k_res, v_res, block_table,
                    context_lens, out, workspace), bind)


def lse_merge(part_o, part_ml, out, *, stream=None, bind=False):
    """pda_lse_merge: part_o [rows, P, d_h], part_ml [rows, P, 2] -> out [rows, d_h]."""
    rows, P, d_h = part_o.shape
    dev = part_o.device
    _need(part_o, "part_o", _f32(), dev)
    _need(part_ml, "part_ml", _f32(), dev, shape=(rows, P, 2))
    _need(out, "out", _f32(), dev, shape=(rows, d_h))
    return _launch("pda_lse_merge", (_ptr(part_o), _ptr(part_ml), rows, P, d_h, _ptr(out),
                                     _stream(stream)), (part_o, part_ml, out), bind)


def hbm_read_probe(buf, sink, *, tile_offsets=None, tile_bytes: int = 4096, waves: int = 1024,
                   stream=None, bind=False):
    """pda_hbm_read_probe: read `buf` (a device tensor) sequentially, or the
    tiles at `tile_offsets` (device int64 byte offsets, checked here on the
    host against the buffer), folding every dword into `sink` (device uint32
    [waves * 64])."""
    torch = _torch()
    dev = buf.device
    nbytes = buf.numel() * buf.element_size()
    _need(buf, "buf", (buf.dtype,), dev)
    _need(sink, "sink", (torch.uint32, torch.int32), dev, numel=waves * 64)
    n_tiles = 0
    if tile_offsets is not None:
        _need(tile_offsets, "tile_offsets", (torch.int64,), dev)
        n_tiles = tile_offsets.numel()
        if n_tiles:
            lo, hi = int(tile_offsets.min()), int(tile_offsets.max())
            bad = int((tile_offsets % 16 != 0).sum())
            if lo < 0 or hi + tile_bytes > nbytes or bad:
                raise ValueError("tile offsets must be 16-byte aligned and inside the buffer")
    return _launch("pda_hbm_read_probe", (_ptr(buf), nbytes, _ptr(tile_offsets), n_tiles,
                                          int(tile_bytes), int(waves), _ptr(sink),
                                          _stream(stream)),
                   (buf, sink, tile_offsets), bind)


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
