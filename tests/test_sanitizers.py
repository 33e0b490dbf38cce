"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The block pool, the descriptor checks, the split plan and workspace layout,
and the argument validation of every call (csrc/pool.cpp, csrc/api.cpp) are
built with the host compiler and -fsanitize=address,undefined, with the
device launches replaced by stubs (tests/sanitize/host_stubs.cpp); the fp64
oracle (oracle/pda_oracle.c) is built the same way. The CPU suites that
drive them -- the pool against its oracle model, the boundary checks, the
oracle pins -- then run in a child process with the sanitizer runtimes
preloaded, and any report fails the test.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_paged_slot_amd", "csrc")
ROCM = "/opt/rocm"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _build(tmp):
    pda = os.path.join(tmp, "libpda_host_san.so")
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__",
                    f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}",
                    os.path.join(CSRC, "pool.cpp"), os.path.join(CSRC, "api.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"),
                    f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", pda],
                   check=True, capture_output=True, text=True)
    orc = os.path.join(tmp, "liboracle_san.so")
    subprocess.run(["gcc", "-std=c11", "-fPIC", "-shared", "-fopenmp", *SAN, "-fno-fast-math",
                    "-ffp-contract=off", os.path.join(ROOT, "oracle", "pda_oracle.c"), "-lm",
                    "-o", orc], check=True, capture_output=True, text=True)
    return pda, orc


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(f"{ROCM}/include/hip"),
                    reason="needs g++ and the HIP headers")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not found")
    pda, orc = _build(str(tmp_path))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": f"{asan}:{ubsan}",
        # Python itself is not instrumented: no leak report at its exit, and
        # the preloaded runtime stands in for the link-order check
        "ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "PDA_LIB": pda,
        "PDA_ORACLE_LIB": orc,
        "OMP_NUM_THREADS": "2",
    })
    # the instrumentation is live: a free order shorter than the pool, passed
    # straight through the C ABI, is an out-of-bounds read the build reports
    probe = ("import ctypes, numpy as np, decode_attention_paged_slot_amd.binding as b\n"
             "h = ctypes.c_void_p()\n"
             "short = np.arange(5, dtype=np.int32)\n"
             "b._lib.pda_pool_create(10, short.ctypes.data, ctypes.byref(h))\n")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
    suites = ["tests/test_pool.py", "tests/test_abi.py", "tests/test_oracle_pins.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *suites], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
