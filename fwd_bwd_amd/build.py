"""Build libna.so (the HIP kernels and the C ABI of include/na.h) for gfx950, in-tree."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libna.so")
SOURCES = [os.path.join(CSRC, "na_api.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # hardware float atomics for the KV-parallel dq accumulator
    "-munsafe-fp-atomics",
    # MFMA results in ordinary VGPRs: the accumulators are also touched by VALU
    # code (softmax rescale), and AGPR residency costs a copy per use
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", LIB + ".tmp", *SOURCES]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
