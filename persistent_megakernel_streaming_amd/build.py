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
#
# A load written in inline asm writes its output registers some time after it
# issues, while the compiler takes the asm's outputs as written at once: an
# output that shares registers with an input (an address) could be
# overwritten while a later instruction of the block still reads it.  Every
# output of an asm block that loads must therefore be early-clobber ("=&") or
# read-write ("+").
_ASM_RE = re.compile(r'asm\s+volatile\s*\(((?:\s*"(?:[^"\\]|\\.)*")+)\s*(:[^;]*)?\);')
_VMEM_RE = re.compile(r'\b(buffer|global|flat|scratch)_(load|store|atomic)')
_LOAD_RE = re.compile(r'\b((buffer|global|flat|scratch|s)_load|ds_read)')


def check_asm_guards(path: str) -> int:
    """Raises if an inline-asm block of `path` issues a vector- or scalar-memory
    instruction without starting with s_nop 4 or longer, or loads (LDS reads
    included) into an output that is neither early-clobber nor read-write;
    returns the number of blocks with a memory instruction."""
    text = open(path).read()
    n = 0
    for m in _ASM_RE.finditer(text):
        body = "".join(re.findall(r'"((?:[^"\\]|\\.)*)"', m.group(1))).replace("\\n", "\n")
        if not (_VMEM_RE.search(body) or _LOAD_RE.search(body)):
            continue
        n += 1
        line = text.count("\n", 0, m.start()) + 1
        first = body.strip().split("\n")[0].strip()
        g = re.fullmatch(r"s_nop\s+(\d+)", first)
        if (_VMEM_RE.search(body) or re.search(r"\bs_load", body)) and (not g or int(g.group(1)) < 4):
            raise RuntimeError(f"{path}:{line}: inline asm with a memory instruction must start with "
                               f"'s_nop 4' (found {first!r})")
        if _LOAD_RE.search(body):
            outs = (m.group(2) or ":").split(":")[1]
            for c in re.findall(r'"([^"]*)"\s*\(', outs):
                if not (c.startswith("=&") or c.startswith("+")):
                    raise RuntimeError(f"{path}:{line}: inline asm that loads needs early-clobber ('=&') or "
                                       f"read-write ('+') outputs (found {c!r})")
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
