"""Build step: compile the HIP library ``libregen_attn.so`` for gfx950.

Run as ``python -m diffusion_transformer_attention_dit_amd.build``; the
library lands in the package directory (in-tree, so it travels with the
source tree).
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libregen_attn.so")
SOURCES = [os.path.join(CSRC, "regen_attn.hip")]
DEPENDS = SOURCES + [os.path.join(CSRC, h) for h in ("common.hpp", "attention.hpp", "cross.hpp", "gemm.hpp",
                                                     "layout.hpp", "probe.hpp")] + \
    [os.path.join(INCLUDE, "regen_attn.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # Keep packed-FP32 instructions out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The ILP-first iterative scheduler: the attention kernel's loop runs
    # about 2% faster with it (same instructions, same results).
    "-mllvm", "-amdgpu-sched-strategy=iterative-ilp",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra) + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPENDS)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
