"""MI355X-native index-only TopK selector (radix select, HIP for gfx950).

Python binding over the C ABI of ``libtopk_select.so`` (``include/topk_select.h``).
PyTorch is used only to allocate device memory and to name the current HIP
stream; the selection itself runs entirely in the library's kernels.

    import torch, sparse_attention_topk_fp32_amd as tks
    idx = tks.select(logits, k=2048)              # int32 [rows, k], unsorted
    idx = tks.select(logits, k=2048, lengths=L)   # per-row valid lengths
    idx, val = tks.select_sorted(logits, k=2048, return_values=True)  # ordered

Semantics (the TopK article "How to Use FlagOS's New Triton-TLE Language to
Build a TopK Selector Faster Than FlashInfer", sections 01, 02 and 5): per row,
the indices of the k largest valid logits, ties at the threshold value going
to the lowest index, -1 in slots past the valid length, order unspecified.
``select_sorted`` gives the same sets in order (value descending, equal values
by index ascending; section 02's need_sorted option), optionally with values.
"""

from __future__ import annotations

import ctypes
from typing import Optional

from . import _native
from ._native import TopkSelectError  # noqa: F401

__all__ = [
    "select",
    "topk_select",
    "topk_select_ex",
    "topk_select_no_alloc",
    "select_sorted",
    "indexer_logits",
    "indexer_select",
    "sparse_attention",
    "topk_select_sorted",
    "topk_indexer_logits",
    "topk_indexer_select",
    "topk_indexer_select_fused",
    "topk_select_sorted_ex",
    "plan",
    "num_variants",
    "variant_info",
    "device_status",
    "release_workspace",
    "version",
    "stream_read",
    "TopkSelectError",
]


def _check(rc: int, what: str) -> None:
    if rc != _native.SUCCESS:
        raise TopkSelectError(rc, what)


def topk_select(logits_ptr: int, rows: int, n: int, lengths_ptr: Optional[int], k: int, out_ptr: int,
                stream: int = 0) -> int:
    """Raw C-ABI call with device pointers; returns the status code."""
    return _native.load().topk_select(logits_ptr or None, rows, n, lengths_ptr or None, k, out_ptr or None,
                                      stream or None)


def topk_select_ex(logits_ptr: int, rows: int, n: int, lengths_ptr: Optional[int], k: int, out_ptr: int,
                   stream: int, variant: int, wgs_per_row: int) -> int:
    """Raw C-ABI call with an explicit launch shape; returns the status code."""
    p = _native.PlanT(variant, wgs_per_row, 0, 0, 0, 0)
    return _native.load().topk_select_ex(logits_ptr or None, rows, n, lengths_ptr or None, k, out_ptr or None,
                                         stream or None, ctypes.byref(p))


def topk_select_no_alloc(logits_ptr: int, rows: int, n: int, lengths_ptr: Optional[int], k: int, out_ptr: int,
                         stream: int = 0) -> int:
    """Raw C-ABI call of the allocation-free entry point; returns the status code."""
    return _native.load().topk_select_no_alloc(logits_ptr or None, rows, n, lengths_ptr or None, k,
                                               out_ptr or None, stream or None)


def topk_select_sorted(logits_ptr: int, rows: int, n: int, lengths_ptr: Optional[int], k: int, out_ptr: int,
                       val_ptr: Optional[int], stream: int = 0) -> int:
    """Raw C-ABI call of the ordered selection; returns the status code."""
    return _native.load().topk_select_sorted(logits_ptr or None, rows, n, lengths_ptr or None, k, out_ptr or None,
                                             val_ptr or None, stream or None)


def topk_select_sorted_ex(logits_ptr: int, rows: int, n: int, lengths_ptr: Optional[int], k: int, out_ptr: int,
                          val_ptr: Optional[int], stream: int, variant: int, wgs_per_row: int) -> int:
    """Raw C-ABI call of the ordered selection with an explicit launch shape."""
    p = _native.PlanT(variant, wgs_per_row, 0, 0, 0, 0)
    return _native.load().topk_select_sorted_ex(logits_ptr or None, rows, n, lengths_ptr or None, k,
                                                out_ptr or None, val_ptr or None, stream or None, ctypes.byref(p))


def topk_indexer_logits(q_ptr: int, kc_ptr: int, w_ptr: int, rows: int, n: int, heads: int, dim: int,
                        kstride: int, lengths_ptr: Optional[int], logits_ptr: int, stream: int = 0) -> int:
    """Raw C-ABI call of the indexer logits; returns the status code."""
    return _native.load().topk_indexer_logits(q_ptr or None, kc_ptr or None, w_ptr or None, rows, n, heads, dim,
                                              kstride, lengths_ptr or None, logits_ptr or None, stream or None)


def topk_indexer_select(q_ptr: int, kc_ptr: int, w_ptr: int, rows: int, n: int, heads: int, dim: int,
                        kstride: int, lengths_ptr: Optional[int], k: int, out_ptr: int,
                        logits_ptr: Optional[int], stream: int = 0) -> int:
    """Raw C-ABI call of the indexer logits followed by the selection."""
    return _native.load().topk_indexer_select(q_ptr or None, kc_ptr or None, w_ptr or None, rows, n, heads, dim,
                                              kstride, lengths_ptr or None, k, out_ptr or None,
                                              logits_ptr or None, stream or None)


def topk_indexer_select_fused(q_ptr: int, kc_ptr: int, w_ptr: int, rows: int, n: int, heads: int, dim: int,
                              kstride: int, lengths_ptr: Optional[int], k: int, out_ptr: int,
                              logits_ptr: Optional[int], stream: int = 0) -> int:
    """Raw C-ABI call of the indexer with the selection's first pass in the
    logits kernel."""
    return _native.load().topk_indexer_select_fused(q_ptr or None, kc_ptr or None, w_ptr or None, rows, n, heads,
                                                    dim, kstride, lengths_ptr or None, k, out_ptr or None,
                                                    logits_ptr or None, stream or None)


def _stream_handle(stream) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return int(getattr(stream, "cuda_stream", stream) or 0)


def _prepare(logits, k, lengths):
    import torch

    if not isinstance(logits, torch.Tensor) or logits.device.type != "cuda":
        raise TypeError("logits must be a GPU tensor")
    if logits.dtype != torch.float32:
        raise TypeError("logits must be float32")
    squeeze = logits.dim() == 1
    x = logits.unsqueeze(0) if squeeze else logits
    if x.dim() != 2:
        raise ValueError("logits must be [rows, n]")
    rows, n = x.shape
    if not x.is_contiguous():
        raise ValueError("logits must be contiguous (row-major, row stride n)")
    lp = None
    if lengths is not None:
        if lengths.dtype != torch.int32 or lengths.device != x.device or lengths.shape != (rows,):
            raise ValueError("lengths must be an int32 [rows] tensor on the logits' device")
        if not lengths.is_contiguous():
            raise ValueError("lengths must be contiguous")
        lp = lengths.data_ptr()
    return x, squeeze, rows, n, lp


def _check_out(t, dtype, rows, k, x, name):
    if t.dtype != dtype or t.shape != (rows, k) or not t.is_contiguous() or t.device != x.device:
        raise ValueError("%s must be a contiguous %s [rows, k] tensor on the logits' device" % (name, dtype))


def select_sorted(logits, k: int, lengths=None, out=None, out_values=None, return_values: bool = False,
                  stream=None, variant: Optional[int] = None, wgs_per_row: Optional[int] = None):
    """``select`` with each row in order: values descending, equal values by
    index ascending, -1 slots last.  With ``return_values`` (or
    ``out_values`` given) also the selected logits, bit for bit, -inf beside
    each -1; returns (indices, values) then, else the indices."""
    import torch

    x, squeeze, rows, n, lp = _prepare(logits, k, lengths)
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=x.device)
    else:
        _check_out(out, torch.int32, rows, k, x, "out")
    want_vals = return_values or out_values is not None
    if want_vals and out_values is None:
        out_values = torch.empty((rows, k), dtype=torch.float32, device=x.device)
    elif want_vals:
        _check_out(out_values, torch.float32, rows, k, x, "out_values")
    vp = out_values.data_ptr() if want_vals else None
    sh = _stream_handle(stream)
    with torch.cuda.device(x.device):
        if variant is None and wgs_per_row is None:
            rc = topk_select_sorted(x.data_ptr(), rows, n, lp, k, out.data_ptr(), vp, sh)
        else:
            if variant is None or wgs_per_row is None:
                raise ValueError("give both variant and wgs_per_row")
            rc = topk_select_sorted_ex(x.data_ptr(), rows, n, lp, k, out.data_ptr(), vp, sh, variant, wgs_per_row)
    _check(rc, "topk_select_sorted")
    if squeeze:
        out = out[0]
        out_values = out_values[0] if want_vals else None
    return (out, out_values) if want_vals else out


def select(logits, k: int, lengths=None, out=None, stream=None, variant: Optional[int] = None,
           wgs_per_row: Optional[int] = None):
    """Indices of the k largest valid logits of each row.

    logits   float32 tensor on the GPU, [rows, n] (or [n]), contiguous rows.
    k        1 <= k <= n.
    lengths  optional int32 GPU tensor [rows] of valid lengths.
    out      optional preallocated int32 GPU tensor [rows, k].
    stream   torch stream (default: the current stream).
    variant, wgs_per_row: optional explicit launch shape (tests, tuning).
    Returns the int32 [rows, k] tensor (``out`` when given)."""
    import torch

    x, squeeze, rows, n, lp = _prepare(logits, k, lengths)
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=x.device)
    else:
        _check_out(out, torch.int32, rows, k, x, "out")
    sh = _stream_handle(stream)
    with torch.cuda.device(x.device):
        if variant is None and wgs_per_row is None:
            rc = topk_select(x.data_ptr(), rows, n, lp, k, out.data_ptr(), sh)
        else:
            if variant is None or wgs_per_row is None:
                raise ValueError("give both variant and wgs_per_row")
            rc = topk_select_ex(x.data_ptr(), rows, n, lp, k, out.data_ptr(), sh, variant, wgs_per_row)
    _check(rc, "topk_select")
    return out[0] if squeeze else out


def _qk_args(q, kc):
    """Shapes of bfloat16 queries [rows, heads, dim] and keys [n, dim]
    (shared by every row) or [rows, n, dim]: (rows, heads, dim, n, kstride)."""
    import torch

    for t, name in ((q, "q"), (kc, "kc")):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.bfloat16:
            raise TypeError("%s must be a bfloat16 GPU tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if q.dim() != 3:
        raise ValueError("q must be [rows, heads, dim]")
    rows, heads, dim = q.shape
    if kc.device != q.device:
        raise ValueError("kc must be on q's device")
    if kc.dim() == 2:
        n, kstride = kc.shape[0], 0
    elif kc.dim() == 3 and kc.shape[0] == rows:
        n, kstride = kc.shape[1], kc.shape[1] * kc.shape[2]
    else:
        raise ValueError("kc must be [n, dim] (shared by every row) or [rows, n, dim]")
    if kc.shape[-1] != dim:
        raise ValueError("kc's last dimension must be q's dim")
    return rows, heads, dim, n, kstride


def _indexer_args(q, kc, w, lengths):
    import torch

    rows, heads, dim, n, kstride = _qk_args(q, kc)
    if not isinstance(w, torch.Tensor) or w.dtype != torch.float32 or w.device != q.device or not w.is_contiguous():
        raise TypeError("w must be a contiguous float32 tensor on q's device")
    if w.shape != (rows, heads):
        raise ValueError("w must be [rows, heads]")
    lp = None
    if lengths is not None:
        if lengths.dtype != torch.int32 or lengths.device != q.device or lengths.shape != (rows,) \
                or not lengths.is_contiguous():
            raise ValueError("lengths must be a contiguous int32 [rows] tensor on q's device")
        lp = lengths.data_ptr()
    return rows, heads, dim, n, kstride, lp


def indexer_logits(q, kc, w, lengths=None, out=None, stream=None):
    """Indexer logits on the matrix cores: out[r, t] = sum_h w[r, h] *
    max(0, q[r, h] . kc[t]) (kc [n, dim] shared by every row, or [rows, n,
    dim]), -inf past the valid length.  q, kc bfloat16; w float32."""
    import torch

    rows, heads, dim, n, kstride, lp = _indexer_args(q, kc, w, lengths)
    if out is None:
        out = torch.empty((rows, n), dtype=torch.float32, device=q.device)
    else:
        _check_out(out, torch.float32, rows, n, q, "out")
    with torch.cuda.device(q.device):
        rc = topk_indexer_logits(q.data_ptr(), kc.data_ptr(), w.data_ptr(), rows, n, heads, dim, kstride, lp,
                                 out.data_ptr(), _stream_handle(stream))
    _check(rc, "topk_indexer_logits")
    return out


def indexer_select(q, kc, w, k: int, lengths=None, out=None, out_logits=None, return_logits: bool = False,
                   stream=None, fused: bool = False):
    """The indexer logits, then the selection of the k largest per row
    (unordered, as ``select``).  Returns the indices, or (indices, logits)
    with ``return_logits`` (or ``out_logits`` given).  ``fused`` calls
    topk_indexer_select_fused (the selection's first pass in the logits
    kernel) instead of topk_indexer_select."""
    import torch

    rows, heads, dim, n, kstride, lp = _indexer_args(q, kc, w, lengths)
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=q.device)
    else:
        _check_out(out, torch.int32, rows, k, q, "out")
    want = return_logits or out_logits is not None
    if want and out_logits is None:
        out_logits = torch.empty((rows, n), dtype=torch.float32, device=q.device)
    elif want:
        _check_out(out_logits, torch.float32, rows, n, q, "out_logits")
    fn = topk_indexer_select_fused if fused else topk_indexer_select
    with torch.cuda.device(q.device):
        rc = fn(q.data_ptr(), kc.data_ptr(), w.data_ptr(), rows, n, heads, dim, kstride, lp, k, out.data_ptr(),
                out_logits.data_ptr() if want else None, _stream_handle(stream))
    _check(rc, "topk_indexer_select_fused" if fused else "topk_indexer_select")
    return (out, out_logits) if want else out


def topk_sparse_attention(q_ptr: int, kc_ptr: int, vc_ptr: int, idx_ptr: int, rows: int, n: int, heads: int,
                          dim: int, kvstride: int, k: int, scale: float, out_ptr: int, stream: int = 0) -> int:
    """Raw C-ABI call of the attention over the selected positions."""
    return _native.load().topk_sparse_attention(q_ptr or None, kc_ptr or None, vc_ptr or None, idx_ptr or None,
                                                rows, n, heads, dim, kvstride, k, float(scale), out_ptr or None,
                                                stream or None)


def sparse_attention(q, kc, vc, idx, scale: Optional[float] = None, out=None, stream=None):
    """Attention of the query heads over the selected positions only:
    out[r, h] = sum_j softmax_j(scale q[r, h] . kc[idx[r, j]]) vc[idx[r, j]]
    (slots holding -1 are skipped).  q [rows, heads, dim] bfloat16; kc, vc
    bfloat16 [n, dim] (shared by every row) or [rows, n, dim]; idx int32
    [rows, k] (e.g. from ``select``); scale defaults to 1/sqrt(dim).
    Returns float32 [rows, heads, dim]."""
    import math

    import torch

    rows, heads, dim, n, kvstride = _qk_args(q, kc)
    if not isinstance(vc, torch.Tensor) or vc.dtype != torch.bfloat16 or vc.shape != kc.shape \
            or vc.device != q.device or not vc.is_contiguous():
        raise ValueError("vc must be a contiguous bfloat16 tensor shaped like kc on q's device")
    if not isinstance(idx, torch.Tensor) or idx.dtype != torch.int32 or idx.dim() != 2 or idx.shape[0] != rows \
            or idx.device != q.device or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 [rows, k] tensor on q's device")
    k = idx.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(dim)
    if out is None:
        out = torch.empty((rows, heads, dim), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or out.shape != (rows, heads, dim) or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous float32 [rows, heads, dim] tensor on q's device")
    with torch.cuda.device(q.device):
        rc = topk_sparse_attention(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), idx.data_ptr(), rows, n, heads, dim,
                                   kvstride, k, scale, out.data_ptr(), _stream_handle(stream))
    _check(rc, "topk_sparse_attention")
    return out


def plan(rows: int, n: int, k: int) -> dict:
    """The launch shape the library picks for (rows, n, k) on the current device."""
    p = _native.PlanT()
    _check(_native.load().topk_select_plan(rows, n, k, ctypes.byref(p)), "topk_select_plan")
    return {f: getattr(p, f) for f, _ in _native.PlanT._fields_}


def num_variants() -> int:
    return int(_native.load().topk_select_num_variants())


def variant_info(v: int) -> dict:
    p = _native.PlanT()
    _check(_native.load().topk_select_variant_info(v, ctypes.byref(p)), "topk_select_variant_info")
    return {f: getattr(p, f) for f, _ in _native.PlanT._fields_}


def device_status(stream=None) -> int:
    """Synchronise the stream and return (and clear) the device-side error flags."""
    flags = ctypes.c_int32(0)
    rc = _native.load().topk_select_device_status(_stream_handle(stream) or None, ctypes.byref(flags))
    if rc not in (_native.SUCCESS, _native.ERROR_DEVICE_FLAG):
        raise TopkSelectError(rc, "topk_select_device_status")
    return int(flags.value)


def release_workspace() -> None:
    _check(_native.load().topk_select_release_workspace(), "topk_select_release_workspace")


def version() -> int:
    return int(_native.load().topk_select_version())


def stream_read(buf, sink, stream=None) -> None:
    """One streaming read of the device tensor `buf` (16-byte aligned, a
    multiple of 16 bytes) on `stream`; `sink` is a device int32/uint32
    tensor of at least one element.  For measuring achievable read bandwidth."""
    nbytes = buf.numel() * buf.element_size()
    _check(_native.load().topk_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), _stream_handle(stream)),
           "topk_stream_read")
