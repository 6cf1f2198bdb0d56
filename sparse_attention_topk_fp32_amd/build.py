"""Build ``libtopk_select.so`` (HIP, gfx950) in-tree with hipcc.

    python -m sparse_attention_topk_fp32_amd.build

The library is a plain C-ABI shared object (``include/topk_select.h``); the
Python binding loads it with ctypes.  Packed-FP32 instructions are disabled
for all device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "topk_select.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtopk_select.so")
ARCH = os.environ.get("TOPK_SELECT_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def command(out: str = LIB, extra=()):
    return [
        hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", INCLUDE, SRC, "-o", out, *extra,
    ]


def build(verbose: bool = False) -> str:
    """Compile the library (always; callers decide when to rebuild)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
