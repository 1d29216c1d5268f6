"""Build libkvq4.so (HIP kernels + C-ABI layer) for gfx950 with hipcc, in-tree.

Usage: python -m quantized_kv_cache_prefill_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvq4.so")
SOURCES = [os.path.join(CSRC, "kvq4_kernels.hip"), os.path.join(CSRC, "kvq4_gemm.hip"),
           os.path.join(CSRC, "kvq4_prefill.hip"),
           os.path.join(CSRC, "kvq4_host.cpp"), os.path.join(CSRC, "kvq4_api.cpp")]
HEADERS = [os.path.join(CSRC, "kvq4_launch.h"), os.path.join(CSRC, "kvq4_device.h"), os.path.join(INCLUDE, "kvq4.h")]

ARCH = "gfx950"

# Device code: gfx950 only; packed-FP32 instructions off; correctly rounded
# fp32 division/sqrt and IEEE denormals kept (the codec's integer decisions
# must match the binary32 definition bit for bit); no fast-math.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkvq4.so)")


def build(verbose: bool = False) -> str:
    """Compile every source and link libkvq4.so next to this file (always rebuilds)."""
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [cc, *HIPCC_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
