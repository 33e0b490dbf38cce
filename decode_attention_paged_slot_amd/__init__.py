"""Paged single-token decode attention for AMD MI355X (gfx950).

The C library libpda (include/pda.h) holds the block pool, the block-table
builder and the HIP kernels (KV append, quantized append, paged decode
attention over bf16 / fp32 / fp8 / int8 caches, split-KV log-sum-exp merge).
This package is its thin ctypes binding; see `binding` for the calls.

The binding is loaded on first use of any of its names, so that the build
module (`decode_attention_paged_slot_amd.build`) can be imported before the
library exists. Using the binding without a built libpda.so raises ImportError:
there is no fallback implementation.
"""
import importlib

_BINDING_NAMES = (
    "AttnDesc", "KvDesc", "NoSpace", "PdaError", "Pool", "EXPORTS", "LIB_PATH",
    "F32", "BF16", "FP8_E4M3", "INT8", "INT4",
    "version", "last_error", "dtype_code",
    "kv_append", "kv_append_quant",
    "attn_desc", "attn_workspace_size", "attn_plan", "workspace_for",
    "paged_decode_attn", "paged_decode_attn_quant", "lse_merge",
    "decode_step", "decode_step_quant", "paged_decode_attn_prefix", "decode_step_prefix",
    "kv_append_int4", "paged_decode_attn_int4", "decode_step_int4", "hbm_read_probe", "BoundCall",
    "paged_decode_attn_noalloc", "NOALLOC_SCRATCH_BYTES",
)

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        binding = importlib.import_module(".binding", __name__)
        return getattr(binding, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
