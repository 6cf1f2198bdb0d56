"""The C-ABI library loads and exports what include/topk_select.h declares;
host-side argument checks answer before any HIP call (CPU only)."""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "topk_select.h")


@pytest.fixture(scope="module")
def lib():
    from sparse_attention_topk_fp32_amd import _native

    if not os.path.exists(_native.LIB_PATH):
        pytest.fail("libtopk_select.so is not built: run __graft_entry__.build() or "
                    "python -m sparse_attention_topk_fp32_amd.build")
    return _native.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(topk_\w*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_binding_exports():
    from sparse_attention_topk_fp32_amd import _native

    assert _declared_functions() == sorted(_native.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_error_strings(lib):
    from sparse_attention_topk_fp32_amd import _native

    assert lib.topk_select_version() == 1
    for code in range(8):
        s = _native.error_string(code)
        assert s and s != "unknown status"
    assert _native.error_string(99) == "unknown status"


def _call(lib, logits, rows, n, lengths, k, out):
    return lib.topk_select(logits, rows, n, lengths, k, out, None)


def test_argument_checks_answer_before_any_hip_call(lib):
    from sparse_attention_topk_fp32_amd import _native

    INV = _native.ERROR_INVALID_VALUE
    a = 0x10000000  # stand-in addresses: never dereferenced, validation is host-only
    o = 0x20000000
    assert _call(lib, a, 0, 16, None, 4, o) == _native.SUCCESS  # rows == 0: no-op
    assert _call(lib, a, -1, 16, None, 4, o) == INV
    assert _call(lib, a, 1, 0, None, 1, o) == INV
    assert _call(lib, a, 1, 16, None, 0, o) == INV
    assert _call(lib, a, 1, 16, None, 17, o) == INV
    assert _call(lib, None, 1, 16, None, 4, o) == INV
    assert _call(lib, a, 1, 16, None, 4, None) == INV
    assert _call(lib, a + 2, 1, 16, None, 4, o) == INV  # logits not 4-byte aligned
    assert _call(lib, a, 1, 16, None, 4, o + 1) == INV
    assert _call(lib, a, 2, 16, None, 4, a + 64) == INV  # out overlaps logits
    assert _call(lib, a, 2, 16, o, 4, o + 4) == INV  # out overlaps lengths
    # rows longer than 2^30 logits are refused (offsets stay far from 32-bit limits)
    assert _call(lib, a, 1, (1 << 30) + 1, None, 4, o) == INV
    assert _call(lib, a, 1, 0x7FFFFFFF, None, 4, o) == INV


def test_sorted_argument_checks_answer_before_any_hip_call(lib):
    from sparse_attention_topk_fp32_amd import _native

    INV = _native.ERROR_INVALID_VALUE
    a, o, v = 0x10000000, 0x20000000, 0x30000000  # stand-in addresses, never dereferenced

    def call(logits, rows, n, lengths, k, out, vals):
        return lib.topk_select_sorted(logits, rows, n, lengths, k, out, vals, None)

    assert call(a, 0, 16, None, 4, o, v) == _native.SUCCESS
    assert call(a, 1, 16, None, 17, o, v) == INV
    assert call(a, 1, 16, None, 4, None, v) == INV
    assert call(a, 1, 16, None, 4, o, v + 2) == INV  # values not 4-byte aligned
    assert call(a, 2, 16, None, 4, o, a + 64) == INV  # values overlap logits
    assert call(a, 2, 16, None, 4, o, o + 4) == INV  # values overlap out
    assert call(a, 2, 16, v, 4, o, v + 4) == INV  # values overlap lengths
    assert call(a, 2, 16, None, 4, a + 8, v) == INV  # out overlaps logits
    assert lib.topk_select_sorted_ex(a, 1, 16, None, 4, o, v, None, None) == INV  # no plan


def test_indexer_argument_checks_answer_before_any_hip_call(lib):
    from sparse_attention_topk_fp32_amd import _native

    INV = _native.ERROR_INVALID_VALUE
    q, kc, w, o, lg = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000

    def logits(q_=q, kc_=kc, w_=w, rows=2, n=64, heads=16, dim=64, kstride=0, lengths=None, out=lg):
        return lib.topk_indexer_logits(q_, kc_, w_, rows, n, heads, dim, kstride, lengths, out, None)

    def select(k=8, out=o, logits_out=None, fn="topk_indexer_select", **kw):
        a = dict(q_=q, kc_=kc, w_=w, rows=2, n=64, heads=16, dim=64, kstride=0, lengths=None)
        a.update(kw)
        return getattr(lib, fn)(a["q_"], a["kc_"], a["w_"], a["rows"], a["n"], a["heads"], a["dim"],
                                a["kstride"], a["lengths"], k, out, logits_out, None)

    assert logits(rows=0) == _native.SUCCESS
    assert logits(heads=0) == INV and logits(heads=65) == INV
    assert logits(dim=48) == INV and logits(dim=256) == INV
    assert logits(kstride=4) == INV  # not a multiple of 8 elements
    assert logits(kstride=64 * 64 - 8) == INV  # rows' keys would overlap
    assert logits(q_=q + 8) == INV and logits(kc_=kc + 4) == INV  # 16-byte alignment
    assert logits(out=None) == INV
    assert logits(out=q + 16) == INV  # logits overlap the queries
    for fn in ("topk_indexer_select", "topk_indexer_select_fused"):
        assert select(k=65, fn=fn) == INV and select(k=0, fn=fn) == INV
        assert select(out=None, fn=fn) == INV
        assert select(out=q, fn=fn) == INV  # indices overlap the queries
        assert select(out=lg, logits_out=lg, fn=fn) == INV  # indices overlap the logits output
        assert select(dim=48, fn=fn) == INV
        assert select(rows=0, fn=fn) == _native.SUCCESS


def test_sparse_attention_argument_checks_answer_before_any_hip_call(lib):
    from sparse_attention_topk_fp32_amd import _native

    INV = _native.ERROR_INVALID_VALUE
    q, kc, vc, ix, o = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000

    def call(q_=q, kc_=kc, vc_=vc, idx=ix, rows=2, n=64, heads=16, dim=64, kvstride=0, k=8, scale=0.125, out=o):
        return lib.topk_sparse_attention(q_, kc_, vc_, idx, rows, n, heads, dim, kvstride, k, scale, out, None)

    assert call(rows=0) == _native.SUCCESS
    assert call(heads=0) == INV and call(heads=65) == INV
    assert call(dim=48) == INV and call(k=0) == INV
    assert call(kvstride=12) == INV and call(kvstride=64 * 64 - 8) == INV
    assert call(scale=float("nan")) == INV and call(scale=float("inf")) == INV
    assert call(vc_=vc + 8) == INV and call(idx=ix + 2) == INV
    assert call(out=None) == INV and call(idx=None) == INV
    assert call(out=q) == INV  # output overlaps the queries


def test_variant_table(lib):
    from sparse_attention_topk_fp32_amd import _native

    nv = lib.topk_select_num_variants()
    assert nv >= 2
    seen_resident = set()
    for v in range(nv):
        p = _native.PlanT()
        assert lib.topk_select_variant_info(v, ctypes.byref(p)) == 0
        assert p.block % 64 == 0 and p.block >= 256
        assert p.items % 4 == 0
        seen_resident.add(p.resident)
    assert seen_resident == {0, 1}
    p = _native.PlanT()
    assert lib.topk_select_variant_info(nv, ctypes.byref(p)) == _native.ERROR_INVALID_VALUE
    assert lib.topk_select_plan(1, 16, 17, ctypes.byref(p)) == _native.ERROR_INVALID_VALUE


def test_select_rejects_non_gpu_tensors():
    import torch

    import sparse_attention_topk_fp32_amd as tks

    with pytest.raises(TypeError):
        tks.select(torch.zeros(4, 8), 2)
    with pytest.raises(TypeError):
        tks.select(np.zeros((4, 8), np.float32), 2)
    with pytest.raises(TypeError):
        tks.select_sorted(torch.zeros(4, 8), 2)


def test_stream_read_argument_checks_answer_before_any_hip_call(lib):
    """Null, misaligned or mis-sized arguments are refused on the host (no
    HIP call is made, so this runs without a GPU)."""
    from sparse_attention_topk_fp32_amd import _native

    lib2 = _native.load()
    assert lib2.topk_stream_read(None, 16, 16, None) == _native.ERROR_INVALID_VALUE
    assert lib2.topk_stream_read(16, 16, None, None) == _native.ERROR_INVALID_VALUE
    assert lib2.topk_stream_read(17, 16, 16, None) == _native.ERROR_INVALID_VALUE
    assert lib2.topk_stream_read(16, 0, 16, None) == _native.ERROR_INVALID_VALUE
    assert lib2.topk_stream_read(16, 24, 16, None) == _native.ERROR_INVALID_VALUE
