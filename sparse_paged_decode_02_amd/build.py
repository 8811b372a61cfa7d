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
# The gather-ceiling probe (include/sda_probe.h): a measurement library that
# bench.py --gather-ceiling loads; the decode path never does.
PROBE_LIB = os.path.join(PKG, "libsda_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "sda_probe.hip")]
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


def _hipcc(sources, out, verbose):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + ["-o", tmp] + sources
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd, cwd=PKG)
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    """Build libsda.so and the probe library beside it; returns libsda.so."""
    _hipcc(SOURCES, LIB, verbose)
    _hipcc(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
