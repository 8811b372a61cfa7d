"""Build libsda.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m sparse_paged_decode_02_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsda.so")
SOURCES = [os.path.join(CSRC, "sda_api.cpp"), os.path.join(CSRC, "sda_kernels.hip"),
           os.path.join(CSRC, "sda_select.hip"), os.path.join(CSRC, "sda_logits.hip"),
           os.path.join(CSRC, "sda_static.hip")]
ARCH = os.environ.get("SDA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # Packed fp32 VALU ops are disabled for all device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The gate's fp32 division must be correctly rounded.
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # MFMA accumulators stay in arch VGPRs: the online-softmax state is loop
    # carried and rescaled by VALU, so AGPR accumulators cost a copy per chunk.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I" + INCLUDE,
    "-I" + CSRC,
]


def build(verbose: bool = True) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd, cwd=PKG)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
