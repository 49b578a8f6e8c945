"""Build libfp4.so (the gfx950 HIP library behind include/fp4.h) in-tree.

    python -m block_scaled_bit_fp4_amd.build

Compiles every source with hipcc for gfx950 only.  Flags that matter for the
numerics: -ffp-contract=off (no fused multiply-add contraction, so every
binary32 operation rounds as written) and correctly rounded fp32 division.
Packed-FP32 instructions are disabled for the device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfp4.so")
ARCH = "gfx950"

SOURCES = ["fp4_api.cpp", "fp4_quantize_nvfp4.hip", "fp4_quantize_mxfp4.hip",
           "fp4_quantize_ufp4.hip", "fp4_quantize_mxfp4_oas.hip", "fp4_quantize_e2m1_cap2.hip",
           "fp4_quantize_mxfp4_mbs.hip", "fp4_quantize_mxfp4_oas16.hip", "fp4_quantize_hif4.hip",
           "fp4_dequant.hip", "fp4_gemm.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-I", INCLUDE, "-I", CSRC,
]
DEVICE = [
    "-x", "hip", "--offload-arch=" + ARCH, "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [cc] + COMMON + DEVICE + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    link = [cc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-fno-gpu-rdc"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
