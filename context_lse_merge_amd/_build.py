"""Build libdcp.so (the HIP library behind include/dcp.h) in-tree for gfx950.

``python context_lse_merge_amd/_build.py`` or ``build()`` compiles every source
under ``csrc/`` with hipcc.  Packed-FP32 instructions are switched off for all
device code (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdcp.so")
ARCH = "gfx950"

SOURCES = ["dcp_host.cpp", "merge.hip", "mla_decode.hip", "mla_varlen.hip", "noalloc.hip"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
    "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Every rounding is the one the source writes: no implicit contraction of
    # a multiply and an add into an FMA, so that kernels sharing an
    # arithmetic give the same bits however they are inlined or unrolled.
    "-ffp-contract=off",
    # Kernel-argument preloading: the leading scalar arguments of a kernel
    # (up to 16 dwords) arrive in SGPRs when the wavefront starts.  The merge
    # kernels lead with what their first loads need; kernels whose first
    # argument is a struct are unaffected.
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I" + INCLUDE, "-I" + CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the DCP library needs ROCm's hipcc to build")


def build(verbose: bool = False) -> str:
    """Compile every source and link libdcp.so; returns its path."""
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc] + lang + HIPCC_FLAGS + ["-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
