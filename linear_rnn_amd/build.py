"""Compile the HIP library (gfx950) in-tree: linear_rnn_amd/librwkv7_wkv.so.

    python -m linear_rnn_amd.build

hipcc cross-compiles for gfx950 without a GPU present. Packed-fp32 instruction
selection is disabled (-packed-fp32-ops) and floating-point contraction is off,
so the kernels' explicit fmaf calls fix the arithmetic order.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librwkv7_wkv.so")
ARCH = os.environ.get("RWKV7_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def flags() -> list:
    return ["-O3", "-std=c++17", "--offload-arch=" + ARCH, "-fPIC", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results in ordinary VGPRs: no copies out of the accumulation registers
            # (only the chunk-prep kernel's code changes; the others already use this form)
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-lambda-capture"]


def build(verbose: bool = False) -> str:
    """Compile every source under csrc/ into one shared library (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + flags() + ["-shared", "-o", tmp] + sources() + ["-lrocblas"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
