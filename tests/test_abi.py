"""The C ABI: libpda loads without a GPU, exports every function the header
declares, and its host-only calls validate arguments."""
from __future__ import annotations

import os
import re
import subprocess

import pytest

import decode_attention_paged_slot_amd as pda
from decode_attention_paged_slot_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pda_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("pda_kv_append", "pda_kv_append_quant", "pda_paged_decode_attn",
                 "pda_paged_decode_attn_quant", "pda_lse_merge", "pda_attn_workspace_size",
                 "pda_pool_create", "pda_build_block_table", "pda_version", "pda_last_error"):
        assert must in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (pda_[a-z0-9_]+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    assert set(binding.EXPORTS) == set(declared_functions())


def test_version_and_error_text():
    assert "gfx950" in pda.version()
    with pytest.raises(pda.PdaError) as e:
        pda.Pool(0)
    assert "num_blocks" in str(e.value)


def _desc(**kw):
    base = dict(B=2, n_q=8, n_kv=2, d_h=128, block_size=16, max_blocks_per_seq=64,
                num_blocks=200, kv_dtype=pda.BF16, q_dtype=pda.BF16, out_dtype=pda.F32,
                max_context=1000, num_partitions=0, total_context=0, reuse_prefix_blocks=0,
                window=0, sink_tokens=0, new_dtype=pda.BF16, prefix_blocks=0)
    base.update(kw)
    return pda.AttnDesc(*[base[f] for f, _ in pda.AttnDesc._fields_])


@pytest.mark.parametrize("bad", [dict(d_h=96), dict(block_size=32), dict(n_q=9),
                                 dict(n_q=34, n_kv=2), dict(kv_dtype=7),
                                 dict(q_dtype=pda.INT8), dict(out_dtype=pda.FP8_E4M3),
                                 dict(max_blocks_per_seq=0), dict(num_blocks=0),
                                 dict(max_context=-1), dict(B=-1),
                                 dict(reuse_prefix_blocks=-1),
                                 dict(window=-1), dict(sink_tokens=-1),
                                 dict(prefix_blocks=-1), dict(prefix_blocks=65),
                                 dict(prefix_blocks=4, window=64),
                                 dict(prefix_blocks=4, kv_dtype=pda.F32)])
def test_attention_descriptor_validation(bad):
    with pytest.raises(pda.PdaError):
        pda.attn_workspace_size(_desc(**bad))


def test_workspace_and_plan():
    # 16-bit cache (stream plan): 1 = one wave per (sequence, KV head), no workspace
    d = _desc(num_partitions=1)
    assert pda.attn_workspace_size(d) == 0
    assert pda.attn_plan(d)[0] == 1
    # k > 1: k equal wave ranges over the flattened (sequence, head, block) axis;
    # workspace = partials of (segments + k) slots x g rows, then segment info
    d = _desc(num_partitions=4)
    P, bpp = pda.attn_plan(d)
    assert P == 4 and bpp >= 1
    g, S = 4, 2 * 2
    ws = pda.attn_workspace_size(d)
    assert ws >= (S + 4) * g * (128 + 2) * 4 + S * 8
    # 70B layer shape: B=8, n_kv=8, 32k context -> 1024 wave ranges (256 workgroups)
    d = _desc(B=8, n_q=64, n_kv=8, max_blocks_per_seq=2048, num_blocks=18205,
              max_context=32768, total_context=8 * 32768)
    P, bpp = pda.attn_plan(d)
    assert P == 1024 and 128 <= bpp <= 129
    assert pda.attn_workspace_size(d) < 0.01 * 8 * 8 * 32768 * 512
    # a batch of short contexts is not split (under 8 blocks per range)
    d = _desc(B=64, n_q=32, n_kv=8, max_blocks_per_seq=4, max_context=40, total_context=64 * 40)
    assert pda.attn_plan(d)[0] == 1 and pda.attn_workspace_size(d) == 0
    # fp32 cache (partition plan): P partitions of bpp blocks per sequence
    d = _desc(kv_dtype=pda.F32, num_partitions=1)
    assert pda.attn_workspace_size(d) == 0
    assert pda.attn_plan(d) == (1, 63)
    d = _desc(kv_dtype=pda.F32, num_partitions=4)
    assert pda.attn_plan(d) == (4, 16)
    assert pda.attn_workspace_size(d) >= 2 * 8 * 4 * (128 + 2) * 4


def test_workgroup_override(monkeypatch):
    # the environment override is read at each call, by the size query and
    # the plan alike; without a device the default assumes 256 compute units
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count \
        if torch.cuda.is_available() else 256
    d = _desc(B=8, n_q=64, n_kv=8, max_blocks_per_seq=2048, num_blocks=18205,
              max_context=32768, total_context=8 * 32768)
    assert pda.attn_plan(d)[0] == 4 * cus
    q = _desc(B=8, n_q=64, n_kv=8, max_blocks_per_seq=2048, num_blocks=18205,
              max_context=32768, total_context=8 * 32768, kv_dtype=pda.FP8_E4M3)
    assert pda.attn_plan(q)[0] == 8 * cus
    ws_default = pda.attn_workspace_size(d)
    monkeypatch.setenv("PDA_ATTN_WORKGROUPS", "100")
    assert pda.attn_plan(d)[0] == 400 and pda.attn_plan(q)[0] == 400
    assert pda.attn_workspace_size(d) < ws_default
    monkeypatch.delenv("PDA_ATTN_WORKGROUPS")
    assert pda.attn_plan(d)[0] == 4 * cus


def test_stream_plan_limits():
    # more than 4096 sequences, or a flattened block axis of 2^31, in one call
    with pytest.raises(pda.PdaError):
        pda.attn_workspace_size(_desc(B=4097, max_blocks_per_seq=4))
    with pytest.raises(pda.PdaError):
        pda.attn_workspace_size(_desc(B=4096, n_q=64, n_kv=64, max_blocks_per_seq=8192))


def test_cache_dtype_must_match_the_call():
    d16 = _desc(kv_dtype=pda.BF16)
    d8 = _desc(kv_dtype=pda.FP8_E4M3)
    assert pda.attn_workspace_size(d8) >= 0
    rc = binding._lib.pda_paged_decode_attn_quant(None, None, None, None, None, None, None, 1.0,
                                                  None, binding.ctypes.byref(d16), None, 0, None)
    assert rc == binding.EINVAL
    rc = binding._lib.pda_paged_decode_attn(None, None, None, None, None, 1.0, None,
                                            binding.ctypes.byref(d8), None, 0, None)
    assert rc == binding.EINVAL


def test_null_pointers_rejected_without_gpu():
    d = _desc()
    rc = binding._lib.pda_paged_decode_attn(None, None, None, None, None, 1.0, None,
                                            binding.ctypes.byref(d), None, 0, None)
    assert rc == pda.binding.EINVAL
    kd = pda.KvDesc(2, 128, 16, 10, pda.BF16, pda.BF16)
    assert binding._lib.pda_kv_append(None, None, None, 0, None, None,
                                      binding.ctypes.byref(kd), None) == binding.OK
    assert binding._lib.pda_kv_append(None, None, None, 3, None, None,
                                      binding.ctypes.byref(kd), None) == binding.EINVAL
    kd_bad = pda.KvDesc(2, 128, 16, 10, pda.BF16, pda.F32)
    assert binding._lib.pda_kv_append(None, None, None, 3, None, None,
                                      binding.ctypes.byref(kd_bad), None) == binding.EINVAL
    assert binding._lib.pda_lse_merge(None, None, 4, 0, 128, None, None) == binding.EINVAL
    assert binding._lib.pda_lse_merge(None, None, 4, 2049, 128, None, None) == binding.EINVAL
    assert binding._lib.pda_lse_merge(None, None, 0, 4, 128, None, None) == binding.OK


def _ws_parts(d):
    """Expected stream-plan workspace bytes: partial slots, their statistics,
    segment info, and (with a shared prefix) the prefix pass's partials."""
    def a256(x):
        return (x + 255) // 256 * 256
    P, _ = pda.attn_plan(d)
    S, g, rows = d.B * d.n_kv, d.n_q // d.n_kv, d.B * d.n_q
    n = a256((S + P) * g * d.d_h * 4) + a256((S + P) * g * 2 * 4) + a256(S * 8)
    if d.prefix_blocks:
        chunks = -(-d.prefix_blocks // 16)
        n += a256(chunks * rows * d.d_h * 4) + a256(chunks * rows * 2 * 4)
    return n


def test_prefix_plan_and_workspace():
    # a shared prefix always takes the split plan (the suffix pieces go through
    # the merge), even where the plain call would run unsplit
    d = _desc(B=64, n_q=32, n_kv=8, max_blocks_per_seq=4, max_context=40, total_context=64 * 40)
    assert pda.attn_plan(d)[0] == 1 and pda.attn_workspace_size(d) == 0
    d.prefix_blocks = 2
    P, _ = pda.attn_plan(d)
    assert P == 64 * 8   # "unsplit": one range per (sequence, KV head)
    assert pda.attn_workspace_size(d) == _ws_parts(d)
    # shared-prefix workload shape: 128 prefix blocks -> 8 chunks of 16
    d = _desc(B=64, n_q=32, n_kv=8, max_blocks_per_seq=1024, num_blocks=40000,
              max_context=16384, total_context=64 * 8704, kv_dtype=pda.FP8_E4M3,
              prefix_blocks=128)
    assert pda.attn_workspace_size(d) == _ws_parts(d)
    plain = _desc(B=64, n_q=32, n_kv=8, max_blocks_per_seq=1024, num_blocks=40000,
                  max_context=16384, total_context=64 * 8704, kv_dtype=pda.FP8_E4M3)
    assert pda.attn_plan(plain) == pda.attn_plan(d)
    assert pda.attn_workspace_size(d) - pda.attn_workspace_size(plain) == \
        8 * 64 * 32 * 128 * 4 + 8 * 64 * 32 * 2 * 4
    with pytest.raises(pda.PdaError):   # beyond the per-call prefix limit
        pda.attn_workspace_size(_desc(max_blocks_per_seq=40000, prefix_blocks=32769))


def test_prefix_calls_check_the_descriptor_first():
    null13 = (None,) * 9
    d0 = _desc()                       # prefix_blocks == 0: not a shared-prefix call
    rc = binding._lib.pda_paged_decode_attn_prefix(*null13, 1.0, None,
                                                   binding.ctypes.byref(d0), None, 0, None)
    assert rc == binding.EINVAL and "prefix_blocks" in pda.last_error()
    d4 = _desc(prefix_blocks=4)        # the plain calls refuse a prefix descriptor
    rc = binding._lib.pda_paged_decode_attn(None, None, None, None, None, 1.0, None,
                                            binding.ctypes.byref(d4), None, 0, None)
    assert rc == binding.EINVAL and "prefix" in pda.last_error()
    rc = binding._lib.pda_decode_step_prefix(*((None,) * 11), 1.0, None,
                                             binding.ctypes.byref(_desc(prefix_blocks=4,
                                                                        kv_dtype=pda.F32)),
                                             None, 0, None)
    assert rc == binding.EINVAL
    # valid descriptor, NULL prefix pointers
    rc = binding._lib.pda_paged_decode_attn_prefix(*null13, 1.0, None,
                                                   binding.ctypes.byref(d4), None, 0, None)
    assert rc == binding.EINVAL and "NULL" in pda.last_error()


def test_int4_descriptor_rules():
    d = _desc(kv_dtype=pda.INT4, num_partitions=1)
    # a 4-bit cache always takes the split bookkeeping (rows with a residual
    # window go through the merge, which forms that piece itself): no extra
    # workspace beyond the stream plan's
    assert pda.attn_plan(d)[0] > 1 or pda.attn_workspace_size(d) > 0
    assert pda.attn_workspace_size(d) == _ws_parts(d)
    null = (None,) * 9
    # only the int4 calls take it, and no window or shared prefix with it
    rc = binding._lib.pda_paged_decode_attn(None, None, None, None, None, 1.0, None,
                                            binding.ctypes.byref(d), None, 0, None)
    assert rc == binding.EINVAL
    rc = binding._lib.pda_paged_decode_attn_quant(*(None,) * 7, 1.0, None,
                                                  binding.ctypes.byref(d), None, 0, None)
    assert rc == binding.EINVAL
    for bad in (dict(window=16), dict(prefix_blocks=1)):
        rc = binding._lib.pda_paged_decode_attn_int4(*null, 1.0, None,
                                                     binding.ctypes.byref(_desc(kv_dtype=pda.INT4,
                                                                                **bad)),
                                                     None, 0, None)
        assert rc == binding.EINVAL
    rc = binding._lib.pda_paged_decode_attn_int4(*null, 1.0, None, binding.ctypes.byref(
        _desc(kv_dtype=pda.BF16)), None, 0, None)
    assert rc == binding.EINVAL
    rc = binding._lib.pda_kv_append_int4(*(None,) * 10, binding.ctypes.byref(d), None)
    assert rc == binding.EINVAL and "NULL" in pda.last_error()


# entry points taking an attention descriptor: (name, kv dtype, prefix blocks,
# fused new-row dtype); every pointer is NULL below
_ZERO_WORK_CALLS = [
    ("pda_paged_decode_attn", pda.BF16, 0), ("pda_paged_decode_attn_noalloc", pda.BF16, 0),
    ("pda_paged_decode_attn_quant", pda.FP8_E4M3, 0), ("pda_decode_step", pda.BF16, 0),
    ("pda_decode_step_quant", pda.INT8, 0), ("pda_paged_decode_attn_prefix", pda.FP8_E4M3, 4),
    ("pda_decode_step_prefix", pda.FP8_E4M3, 4), ("pda_kv_append_int4", pda.INT4, 0),
    ("pda_paged_decode_attn_int4", pda.INT4, 0), ("pda_decode_step_int4", pda.INT4, 0),
]


@pytest.mark.parametrize("name,kv,prefix", _ZERO_WORK_CALLS)
def test_zero_work_returns_ok_and_runs_nothing(name, kv, prefix):
    """A request with no work (B = 0, or no tokens to append) returns OK with
    every pointer NULL. Without a GPU here, any HIP call would have failed the
    call, so OK also shows that nothing was launched. With B > 0 the same
    call fails (the NULL pointers, or for the allocation-free call the
    missing device, whose scratch it resolves first)."""
    fn = getattr(binding._lib, name)
    for B in (0, 2):
        d = _desc(B=B, kv_dtype=kv, prefix_blocks=prefix,
                  new_dtype=pda.BF16 if kv in (pda.BF16, pda.INT4) else pda.F32)
        args = []
        for t in fn.argtypes:
            if t is binding.ctypes.c_float:
                args.append(1.0)
            elif t is binding.ctypes.c_size_t:
                args.append(0)
            elif t is binding.ctypes.POINTER(pda.AttnDesc):
                args.append(binding.ctypes.byref(d))
            else:
                args.append(None)
        rc = fn(*args)
        assert (rc == binding.OK) == (B == 0), (name, B, rc, pda.last_error())


def test_zero_tokens_quantized_append():
    kd = pda.KvDesc(2, 128, 16, 10, pda.FP8_E4M3, pda.BF16)
    assert binding._lib.pda_kv_append_quant(None, None, None, 0, None, None, None, None,
                                            binding.ctypes.byref(kd), None) == binding.OK
    assert binding._lib.pda_kv_append_quant(None, None, None, 1, None, None, None, None,
                                            binding.ctypes.byref(kd), None) == binding.EINVAL


def test_block_axis_limit_leaves_room_for_pad_and_segment_units():
    """The stream kernel indexes its block axis in 32 bits: B * n_kv segments
    of up to max_blocks_per_seq blocks, plus one pad block (4-bit cache) and
    up to 64 split units per segment. A descriptor whose bare block count
    fits under 2^31 but whose axis with that margin does not is refused."""
    B, n_kv = 4096, 8
    ok = (1 << 31) // (B * n_kv) - 65 - 1          # the largest max_blocks_per_seq accepted
    d = _desc(B=B, n_q=n_kv, n_kv=n_kv, max_blocks_per_seq=ok, num_blocks=1000)
    size = binding.ctypes.c_size_t()
    assert binding._lib.pda_attn_workspace_size(binding.ctypes.byref(d),
                                                binding.ctypes.byref(size)) == binding.OK
    for mb in (ok + 1, (1 << 31) // (B * n_kv) - 1):   # the second fits without the margin
        d = _desc(B=B, n_q=n_kv, n_kv=n_kv, max_blocks_per_seq=mb, num_blocks=1000)
        assert B * n_kv * mb < (1 << 31)
        assert binding._lib.pda_attn_workspace_size(binding.ctypes.byref(d),
                                                    binding.ctypes.byref(size)) == binding.EINVAL
        assert "2^31" in pda.last_error()


@pytest.mark.parametrize("name,kv,prefix", [
    ("pda_paged_decode_attn", pda.BF16, 0), ("pda_paged_decode_attn_quant", pda.FP8_E4M3, 0),
    ("pda_paged_decode_attn_int4", pda.INT4, 0), ("pda_paged_decode_attn_prefix", pda.INT8, 4)])
def test_short_workspace_is_refused_before_any_launch(name, kv, prefix):
    """A split plan needs a workspace of pda_attn_workspace_size bytes: one
    byte less, none, or a misaligned one is EWORKSPACE, decided on the host
    before anything is launched (the device pointers are never touched, so
    placeholder addresses do here)."""
    d = _desc(B=8, n_q=64, n_kv=8, max_blocks_per_seq=2048, num_blocks=20000, kv_dtype=kv,
              max_context=32768, total_context=8 * 32768, prefix_blocks=prefix)
    need = binding.ctypes.c_size_t()
    assert binding._lib.pda_attn_workspace_size(binding.ctypes.byref(d),
                                                binding.ctypes.byref(need)) == binding.OK
    assert need.value > 0
    fn = getattr(binding._lib, name)
    fake = 1 << 20                                  # 16-byte aligned, never dereferenced
    for ws, nbytes in ((fake, need.value - 1), (None, need.value), (fake + 8, need.value)):
        args = []
        for t in fn.argtypes:
            if t is binding.ctypes.c_float:
                args.append(0.125)
            elif t is binding.ctypes.POINTER(pda.AttnDesc):
                args.append(binding.ctypes.byref(d))
            else:
                args.append(None)
        # pointers in order; the workspace, its size and the stream are the last three
        ptrs = [i for i, t in enumerate(fn.argtypes[:-3])
                if t not in (binding.ctypes.c_float, binding.ctypes.POINTER(pda.AttnDesc))]
        for i in ptrs:
            args[i] = fake
        args[-3], args[-2], args[-1] = ws, nbytes, None
        assert fn(*args) == binding.EWORKSPACE, (name, ws, nbytes, pda.last_error())
        assert "workspace" in pda.last_error()


def _call_with(fn, d, ptr, scale, override=None):
    """Arguments for an attention / step entry point: every pointer `ptr`,
    the float `scale`, descriptor `d`, no workspace; `override` maps a
    parameter index to a value."""
    args = []
    for t in fn.argtypes:
        if t is binding.ctypes.c_float:
            args.append(scale)
        elif t is binding.ctypes.c_size_t:
            args.append(0)
        elif t is binding.ctypes.POINTER(pda.AttnDesc):
            args.append(binding.ctypes.byref(d))
        else:
            args.append(ptr)
    args[-1] = None   # stream
    args[-3] = None   # workspace
    for i, v in (override or {}).items():
        args[i] = v
    return fn(*args)


def test_bad_scale_alignment_and_new_row_dtype_are_refused_before_any_launch():
    """The other host-side refusals of the attention calls, with placeholder
    device addresses that are never touched: a non-finite scale, a buffer not
    16-byte aligned, and a fused step whose new rows are not in the cache's
    dtype (16-bit caches) or in F32 / BF16 (8-bit caches)."""
    fake = 1 << 20
    d = _desc(B=2, max_context=100)   # short rows: an unsplit plan, no workspace
    fn = binding._lib.pda_paged_decode_attn
    for bad in (float("nan"), float("inf"), float("-inf")):
        assert _call_with(fn, d, fake, bad) == binding.EINVAL
        assert "scale" in pda.last_error()
    for i in (0, 1, 2, 6):                        # q, k_cache, v_cache, out
        assert _call_with(fn, d, fake, 0.1, {i: fake + 8}) == binding.EINVAL
        assert "aligned" in pda.last_error()
    step = binding._lib.pda_decode_step
    assert _call_with(step, _desc(B=2, max_context=100, new_dtype=pda.F32), fake,
                      0.1) == binding.EINVAL
    assert "new_dtype" in pda.last_error()
    step_q = binding._lib.pda_decode_step_quant
    assert _call_with(step_q, _desc(B=2, max_context=100, kv_dtype=pda.FP8_E4M3,
                                    new_dtype=pda.INT8), fake, 0.1) == binding.EINVAL
    assert "new_dtype" in pda.last_error()
    # k_new / v_new of a fused step must be aligned as well
    assert _call_with(step, _desc(B=2, max_context=100), fake, 0.1,
                      {1: fake + 4}) == binding.EINVAL
    assert "k_new" in pda.last_error()


def test_binding_refuses_host_tensors():
    """The Python binding checks every tensor before the C call; a host
    tensor's address is not a device pointer, so the call is refused (the
    dtype, shape and contiguity checks are run on the GPU)."""
    import torch
    k = torch.zeros((4, 2, 16, 64), dtype=torch.bfloat16)
    kn = torch.zeros((3, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        pda.kv_append(kn, kn.clone(), torch.zeros(3, dtype=torch.int64), k, k.clone())
