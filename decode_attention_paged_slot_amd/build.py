"""Build libpda.so (HIP for gfx950) in the package directory.

    python -m decode_attention_paged_slot_amd.build

compiles every source under csrc/ with hipcc into objects (in parallel) and
links them into decode_attention_paged_slot_amd/libpda.so. All device code is
compiled without packed-fp32 instructions (-packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpda.so")
ARCH = os.environ.get("PDA_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON = ["-std=c++17", "-O3", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}",
          f"-I{CSRC}"] + os.environ.get("PDA_EXTRA_FLAGS", "").split()
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE, "-x", "hip", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise and verbose:
        print("\n".join(noise), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile and link libpda.so; always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = sources() + glob.glob(os.path.join(CSRC, "*.h")) + [os.path.join(INCLUDE, "pda.h")]
    return any(os.path.getmtime(p) > t for p in deps)


def ensure_built() -> str:
    return build() if stale() else LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
