"""The allocation-free entry point (topk_select_no_alloc) against topk_select.

Both run the same launch shapes, so the outputs are compared byte for byte
(stronger than the sorted-set parity the oracle tests use), on two calls in a
row where the second input is smaller, for shapes that split a row over many
workgroups and for the one-workgroup-per-row shape.  Inputs beyond the fixed
scratch are rejected before anything is enqueued.  Each case prints its name
before touching the GPU."""

from __future__ import annotations

import sys

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg: str) -> None:
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_topk_fp32_amd as tks

    tks.version()  # loads the library, raises when it is missing
    return torch, tks


def _on_gpu(torch, x, lengths):
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    ld = None if lengths is None else torch.from_numpy(np.asarray(lengths, np.int32)).cuda()
    return xd, ld


def _both(torch, tks, x, lengths, k):
    """(no_alloc output, topk_select output) as host arrays, one stream."""
    xd, ld = _on_gpu(torch, x, lengths)
    rows, n = x.shape
    a = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    b = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    lp = ld.data_ptr() if ld is not None else 0
    rc = tks.topk_select_no_alloc(xd.data_ptr(), rows, n, lp, k, a.data_ptr(), s)
    assert rc == 0, tks._native.error_string(rc)
    rc = tks.topk_select(xd.data_ptr(), rows, n, lp, k, b.data_ptr(), s)
    assert rc == 0, tks._native.error_string(rc)
    torch.cuda.synchronize()
    assert tks.device_status() == 0
    return a.cpu().numpy(), b.cpu().numpy()


def _check_pair(torch, tks, cases):
    for name, x, lengths, k in cases:
        _say("no_alloc %s rows=%d n=%d k=%d" % (name, x.shape[0], x.shape[1], k))
        a, b = _both(torch, tks, x, lengths, k)
        assert a.tobytes() == b.tobytes(), "%s: no_alloc output differs from topk_select" % name
        # the set is the exact top-k (checked against topk_select's, which the
        # oracle tests pin), and every row holds k distinct valid entries
        for r in range(a.shape[0]):
            v = a[r][a[r] >= 0]
            assert np.unique(v).size == v.size


def _normal(seed, rows, n):
    return np.random.default_rng(seed).standard_normal((rows, n)).astype(np.float32)


def test_split_shapes_then_smaller(lib):
    torch, tks = lib
    c2, c1 = W.generate("c2"), W.generate("c1")
    _check_pair(torch, tks, [
        ("c2 (1 row, n=131072)", c2.x, c2.lengths, c2.k),
        ("c1 (1 row, n=16384, smaller)", c1.x, c1.lengths, c1.k),
    ])


def test_batched_then_smaller(lib):
    torch, tks = lib
    c4 = W.generate("c4")
    rng = np.random.default_rng(5)
    x = _normal(6, 8, 40000)
    lengths = rng.integers(0, 40001, size=8).astype(np.int32)
    _check_pair(torch, tks, [
        ("c4 (64 ragged rows, n=131072)", c4.x, c4.lengths, c4.k),
        ("8 ragged rows, n=40000, k=300 (smaller)", x, lengths, 300),
    ])


def test_long_row_then_tiny(lib):
    torch, tks = lib
    c3 = W.generate("c3")
    _check_pair(torch, tks, [
        ("c3 (1 row, n=1048576)", c3.x, c3.lengths, c3.k),
        ("1 row, n=3, k=1 (smaller)", np.array([[1.0, 3.0, 3.0]], np.float32), None, 1),
    ])


def test_row_per_workgroup_then_smaller(lib):
    torch, tks = lib
    _check_pair(torch, tks, [
        ("600 rows, n=8192, k=512", _normal(7, 600, 8192), None, 512),
        ("300 rows, n=4099, k=100 (smaller)", _normal(8, 300, 4099), None, 100),
    ])


def test_beyond_the_scratch_is_rejected(lib):
    torch, tks = lib
    rows, n, k = 64, 1 << 20, 2048
    _say("no_alloc over the limit rows=%d n=%d (rejected on the host)" % (rows, n))
    x = torch.zeros(rows * n, dtype=torch.float32, device="cuda")
    out = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    rc = tks.topk_select_no_alloc(x.data_ptr(), rows, n, 0, k, out.data_ptr(), s)
    assert rc == tks._native.ERROR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert bool((out == -7).all()), "a rejected call wrote its output"
    # the entry point still works afterwards
    c1 = W.generate("c1")
    _check_pair(torch, tks, [("c1 after a rejected call", c1.x, c1.lengths, c1.k)])
