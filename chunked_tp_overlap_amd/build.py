"""Build the C-ABI library ``lib/libub.so`` from ``csrc/`` with hipcc for gfx950.

Usage: ``python -m chunked_tp_overlap_amd.build`` (or ``__graft_entry__.build()``).
Objects go to ``_build/`` inside the package, the library to ``lib/``; both are
git-ignored.  Every call compiles from scratch.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libub.so")

SOURCES = ["ub_api.cpp", "ub_plan.cpp", "gemm_bf16.hip", "gemm_fp8.hip", "quantize_fp8.hip",
           "reduce_partials.hip", "static_scratch.hip"]

ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]
# Device code is compiled without packed-fp32 instructions.
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src, verbose):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [hipcc(), *COMMON]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE]
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__"]
    cmd += ["-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    noise = [ln for ln in res.stderr.splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "warning generated" not in ln]
    if noise and verbose:
        print("\n".join(noise), file=sys.stderr)
    return obj


def build(verbose=False):
    """Compile every source and link ``lib/libub.so``.  Returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs,
           "-L" + os.path.join(ROCM, "lib"), "-lrocprofiler-sdk-roctx", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libub.so failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
