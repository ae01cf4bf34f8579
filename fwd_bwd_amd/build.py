"""Build libna.so (the HIP kernels and the C ABI of include/na.h) for gfx950, in-tree."""
from __future__ import annotations

import hashlib
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libna.so")
SOURCES = [os.path.join(CSRC, "na_api.hip"), os.path.join(CSRC, "na_m16.hip"),
           os.path.join(CSRC, "na_unfused.hip"), os.path.join(CSRC, "na_mask.hip")]
# per-source flags: the 16-bit MFMA kernels run without IEEE-mode NaN handling
# (their maxima then need no operand canonicalisation; they form no NaNs)
SOURCE_FLAGS = {"na_m16.hip": ["-fno-honor-nans", "-Xarch_device", "-mno-amdgpu-ieee"]}
OBJDIR = os.path.join(PKG, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # hardware float atomics for the KV-parallel dq accumulator
    "-munsafe-fp-atomics",
    # MFMA results in ordinary VGPRs: the accumulators are also touched by VALU
    # code (softmax rescale), and AGPR residency costs a copy per use
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
]


def source_files():
    """Every file libna.so is built from: the kernel and ABI sources and the
    public header, sorted by name."""
    files = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp"))]
    files.append(os.path.join(ROOT, "include", "na.h"))
    return sorted(files, key=os.path.basename)


def source_sha256() -> str:
    """sha256 over (name, contents) of source_files(); the build embeds it in
    the library (na_source_sha256), so a loaded library can be matched with
    the tree it came from."""
    h = hashlib.sha256()
    for path in source_files():
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link libna.so."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJDIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
           f'-DNA_SOURCE_SHA256="{source_sha256()}"']
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(os.path.basename(src))[0] + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), "-c", *inc,
               "-o", obj, src]
        if verbose:
            print(" ".join(cmd))
        objs.append(obj)
        procs.append((cmd, subprocess.Popen(cmd)))
    for cmd, pr in procs:
        if pr.wait() != 0:
            raise subprocess.CalledProcessError(pr.returncode, cmd)
    link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(link))
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
