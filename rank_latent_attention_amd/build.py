"""Build the gfx950 HIP library (libflare.so) in-tree with hipcc.

Usage: python -m rank_latent_attention_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "flare.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libflare.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def command(out: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # NaN inputs are undefined behaviour of the library: no NaN canonicalisation around max
            "-fno-honor-nans",
            # hipcc must not emit packed-fp32 VALU instructions on this target
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # keep MFMA accumulators in VGPRs (no AGPR copies around the softmax)
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", INCLUDE, SRC, "-o", out]


def build(verbose: bool = False) -> str:
    """Compile csrc/flare.hip into rank_latent_attention_amd/libflare.so (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
