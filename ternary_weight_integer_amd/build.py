"""Build the gfx950 HIP library (libi2s.so) in-tree with hipcc.

Flags: no fast-math, no denormal flushing and no FP contraction, so ``x / s``
stays a correctly rounded IEEE division and every float operation in the
kernels is a single round-to-nearest operation (the epilogue multiply and a
bias add are never fused into an FMA); packed-FP32 instruction selection is
disabled.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "i2s.hip")
HEADER = os.path.join(ROOT, "include", "i2s.h")
LIB = os.path.join(PKG, "libi2s.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the I2_S library needs ROCm's hipcc to build")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-Wall",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-ffp-contract=off",
        "-I", os.path.join(ROOT, "include"),
    ]


def build(verbose: bool = False) -> str:
    """Compile csrc/i2s.hip into libi2s.so next to this file; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *flags(), SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line.
    noise = "-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
