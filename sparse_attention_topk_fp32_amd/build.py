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
# test build: the same source with TKS_TEST_HOOKS (the wait bound settable
# from the host, for exercising the give-up path); never loaded by the
# product binding
HOOKS_LIB = os.path.join(PKG, "libtopk_select_hooks.so")
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
        # leading scalar kernel arguments preloaded into SGPRs at wave launch
        "-mllvm", "-amdgpu-kernarg-preload-count=9",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", INCLUDE, SRC, "-o", out, *extra,
    ]


def build(verbose: bool = False, hooks: bool = True) -> str:
    """Compile the library, and the test-hook build beside it (always;
    callers decide when to rebuild).  The two compilations run in parallel."""
    jobs = [(LIB, ())]
    if hooks:
        jobs.append((HOOKS_LIB, ("-DTKS_TEST_HOOKS",)))
    procs = []
    for out, extra in jobs:
        tmp = out + ".tmp%d" % os.getpid()
        cmd = command(tmp, extra)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((out, tmp, cmd, subprocess.Popen(cmd)))
    failed = [cmd for _, _, cmd, p in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    for out, tmp, _, _ in procs:
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv, hooks="--no-hooks" not in sys.argv))
