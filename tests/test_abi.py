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
                max_context=1000, num_partitions=0, total_context=0)
    base.update(kw)
    return pda.AttnDesc(*[base[f] for f, _ in pda.AttnDesc._fields_])


@pytest.mark.parametrize("bad", [dict(d_h=96), dict(block_size=32), dict(n_q=9),
                                 dict(n_q=34, n_kv=2), dict(kv_dtype=7),
                                 dict(q_dtype=pda.INT8), dict(out_dtype=pda.FP8_E4M3),
                                 dict(max_blocks_per_seq=0), dict(num_blocks=0),
                                 dict(max_context=-1), dict(B=-1)])
def test_attention_descriptor_validation(bad):
    with pytest.raises(pda.PdaError):
        pda.attn_workspace_size(_desc(**bad))


def test_workspace_and_plan():
    d = _desc(num_partitions=1)
    assert pda.attn_workspace_size(d) == 0
    assert pda.attn_plan(d) == (1, 63)
    d = _desc(num_partitions=4)
    P, bpp = pda.attn_plan(d)
    assert (P, bpp) == (4, 16)
    ws = pda.attn_workspace_size(d)
    assert ws >= 2 * 8 * 4 * (128 + 2) * 4
    # 70B layer shape: B=8, n_kv=8, 32k context -> split with <= 2048 partitions
    d = _desc(B=8, n_q=64, n_kv=8, max_blocks_per_seq=2048, num_blocks=18205,
              max_context=32768, total_context=8 * 32768)
    P, bpp = pda.attn_plan(d)
    assert P * bpp >= 2048 and 1 < P <= 2048 and bpp % 4 == 0
    assert pda.attn_workspace_size(d) < 0.02 * 8 * 8 * 32768 * 512


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
