"""Builds libsdm.so (HIP kernels + host runtime) for gfx950 with hipcc, in-tree.

Usage:  python -m self_speculative_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsdm.so")
SOURCES = ["sdm_kernels.hip", "sdm_runtime.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libsdm.so")


def build(verbose: bool = False) -> str:
    """Compile every source into self_speculative_amd/libsdm.so (always rebuilds)."""
    out_tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed fp32 VALU ops are kept out of every kernel
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # no implicit multiply-add fusion: each template instantiation of an
           # epilogue (one per activation-tile count) then rounds identically,
           # so a row's result does not depend on the batch it is computed in
           "-ffp-contract=off",
           # MFMA accumulators in VGPRs: the attention's softmax rescale and
           # the GEMM epilogues then work on them without AGPR copies (same
           # instructions and results, fewer moves)
           "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-I", os.path.join(ROOT, "include"),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr[-8000:]}")
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
