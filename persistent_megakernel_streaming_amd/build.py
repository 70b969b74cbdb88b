"""Builds libcpms.so (the HIP depth-loop library) in-tree for gfx950.

Run as ``python -m persistent_megakernel_streaming_amd.build`` or call
``build()``.  hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libcpms.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Device code: gfx950 only; no fast math; no FMA contraction (explicit fmaf
# where wanted) so both executors and every inlined copy of a body round the
# same way; packed fp32 instructions off.
DEVICE_FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-ffp-contract=off",
                "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wno-unused-command-line-argument"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return r


def build(verbose: bool = False) -> str:
    """Compiles every HIP source and links libcpms.so next to the package."""
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    tmpdir = os.path.join(PKG, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    kobj = os.path.join(tmpdir, "cp_kernels.o")
    pobj = os.path.join(tmpdir, "cp_plan.o")
    _run([HIPCC, *DEVICE_FLAGS, *inc, "-c", os.path.join(CSRC, "cp_kernels.hip"), "-o", kobj])
    _run([HIPCC, *HOST_FLAGS, *inc, "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, "cp_plan.cpp"), "-o", pobj])
    tmp = LIB + f".tmp{os.getpid()}"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", kobj, pobj, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
