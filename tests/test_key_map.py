"""The GPU path's key map, checked exhaustively on the host: the same
header the kernels include (csrc/key_map.h) is compiled into a small C++
program that walks every non-NaN float in value order and checks that the
keys are strictly increasing except at -0 -> +0, where they tie, and that
key 0 ("no element") comes from no non-NaN pattern
(tests/key_map_exhaustive.cpp)."""

from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "sparse_attention_topk_fp32_amd", "csrc")


def test_key_map_over_all_bit_patterns():
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not available")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "key_map_exhaustive")
        subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", "-Wno-unknown-pragmas", "-I", CSRC,
                        os.path.join(HERE, "key_map_exhaustive.cpp"), "-o", exe], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
    assert int(r.stdout.split()[1]) == 2 ** 32 - 2 ** 24 + 2
