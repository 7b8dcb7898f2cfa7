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
SRCS = [os.path.join(PKG, "csrc", n) for n in ("i2s.hip", "i8s.hip", "noalloc.hip")]
HEADERS = [os.path.join(ROOT, "include", h) for h in ("i2s.h", "i8s.h", "w8a8.h")]
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
        "-Wall",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-ffp-contract=off",
        # Kernel arguments preloaded into SGPRs at wave launch (where the
        # firmware supports it; otherwise the compiler's compatibility
        # prologue loads them), so that the first vector loads need not wait
        # for a scalar load round trip.
        "-mllvm", "-amdgpu-kernarg-preload-count=16",
        "-I", os.path.join(ROOT, "include"),
    ]


# hipcc's host pass does not know the packed-fp32 feature and says so; drop that line.
_NOISE = "-packed-fp32-ops' is not a recognized feature"


def _errors(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines() if _NOISE not in l)


def build(verbose: bool = False) -> str:
    """Compile csrc/*.hip (in parallel, one object each) and link libi2s.so
    next to this file; returns its path."""
    objs = [LIB + "." + os.path.splitext(os.path.basename(src))[0] + ".o" for src in SRCS]
    procs = []
    for src, obj in zip(SRCS, objs):
        cmd = [hipcc(), *flags(), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    failed = []
    for src, p in zip(SRCS, procs):
        _, err = p.communicate()
        err = _errors(err)
        if p.returncode != 0:
            failed.append(f"{os.path.basename(src)} ({p.returncode}):\n{err}")
        elif err.strip() and verbose:
            print(err, file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed: " + "\n".join(failed))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    for obj in objs:
        os.remove(obj)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc link failed ({res.returncode}):\n{_errors(res.stderr)}")
    # A kernel whose host-side stub the compiler dropped links as an
    # undefined symbol; refuse such a library here rather than at first use.
    import ctypes
    try:
        ctypes.CDLL(tmp)
    except OSError as e:
        os.remove(tmp)
        raise RuntimeError(f"built library does not load: {e}") from e
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
