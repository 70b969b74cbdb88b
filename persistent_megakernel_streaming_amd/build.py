"""Builds libcpms.so (the HIP depth-loop library) in-tree for gfx950.

Run as ``python -m persistent_megakernel_streaming_amd.build`` or call
``build()``.  hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import os
import re
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
DEVICE_SOURCES = ["cp_kernels.hip", "cp_measure.hip", "cp_static.hip"]


# A vector-memory instruction that reads SGPRs a VALU instruction (such as
# v_readlane, which restores spilled buffer resources) has just written needs
# five wait states.  The compiler inserts them before its own instructions but
# not before inline asm, so every asm block that issues a vector-memory
# instruction must begin with "s_nop 4" (or longer) itself.
_ASM_RE = re.compile(r'asm\s+volatile\s*\(((?:\s*"(?:[^"\\]|\\.)*")+)')
_VMEM_RE = re.compile(r'\b(buffer|global|flat|scratch)_(load|store|atomic)')


def check_asm_guards(path: str) -> int:
    """Raises if an inline-asm block of `path` issues a vector-memory
    instruction without starting with s_nop 4 or longer; returns the number
    of such blocks checked."""
    text = open(path).read()
    n = 0
    for m in _ASM_RE.finditer(text):
        body = "".join(re.findall(r'"((?:[^"\\]|\\.)*)"', m.group(1))).replace("\\n", "\n")
        if not _VMEM_RE.search(body):
            continue
        n += 1
        first = body.strip().split("\n")[0].strip()
        g = re.fullmatch(r"s_nop\s+(\d+)", first)
        if not g or int(g.group(1)) < 4:
            line = text.count("\n", 0, m.start()) + 1
            raise RuntimeError(f"{path}:{line}: inline asm with a vector-memory instruction must start with "
                               f"'s_nop 4' (found {first!r})")
    return n


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
    objs = []
    for name in DEVICE_SOURCES:
        check_asm_guards(os.path.join(CSRC, name))
        objs.append(os.path.join(tmpdir, name.replace(".hip", ".o")))
        _run([HIPCC, *DEVICE_FLAGS, *inc, "-c", os.path.join(CSRC, name), "-o", objs[-1]])
    objs.append(os.path.join(tmpdir, "cp_plan.o"))
    _run([HIPCC, *HOST_FLAGS, *inc, "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, "cp_plan.cpp"), "-o", objs[-1]])
    tmp = LIB + f".tmp{os.getpid()}"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
