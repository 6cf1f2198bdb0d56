"""CPU oracle for the index-only TopK selector.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``sparse_attention_topk_fp32_amd``) never imports it, and this package never
imports the product library: the two share no code.

Contents
--------
* ``topk`` / ``kth_largest`` - the plain definition (``topk_oracle.c``): sort
  the valid positions of each row by (value descending, index ascending) with
  IEEE float comparisons and keep the first k.  Compiled with gcc, no
  fast-math.
* ``topk_sorted`` - the same selection in that order, with the selected
  values (the ordered output of the article's radix_topk, section 02).
* ``indexer_logits`` - the logits the selector is fed (DSA step 1 of the
  article's section 01), in double precision from bf16 inputs, with the
  magnitude of the summed terms (the scale of float32 rounding errors).
* ``sparse_attention`` - attention of the query heads over the selected
  positions only (DSA step 3), in double precision, with the error scales.
* ``pages_radix`` - the article's radix-select method restated in Python
  (mapping, digit histograms, threshold bucket, collection), a second route
  used to pin the first.

Parity pins (tests/test_oracle_pins.py): brute force over all k-subsets of tiny
rows, the article's method (``pages_radix``), numpy's stable argsort, closed
forms, the worked value the article prints (839 -> 100), and the selection
invariants; for the indexer logits, closed forms (one-hot queries, queries
opposite to every key), numpy matrix products in float64, linearity in the
weights and independence of the head order; for the attention over the
selected positions, closed forms (one position gives its value row, equal
scores the mean of the value rows, none gives zeros), numpy matrix products
and softmax in float64, independence of the slot order, linearity in the
values and invariance to a score shift.  No oracle function is left
unpinned.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "topk_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

ORACLE_OK, ORACLE_ERR_ARG, ORACLE_ERR_NAN, ORACLE_ERR_NOMEM = 0, 1, 2, 3


def build(force: bool = False) -> str:
    """Compile ``topk_oracle.c`` into ``liboracle.so`` with gcc (-O2, no
    fast-math, so subnormals compare as themselves)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-Wall", "-Werror",
             _SRC, "-o", tmp],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I = ctypes.c_int32
            lib.oracle_topk.argtypes = [P, I, I, P, I, P]
            lib.oracle_topk.restype = ctypes.c_int
            lib.oracle_topk_sorted.argtypes = [P, I, I, P, I, P, P]
            lib.oracle_topk_sorted.restype = ctypes.c_int
            lib.oracle_indexer_logits.argtypes = [P, P, P, I, I, I, I, ctypes.c_int64, P, P]
            lib.oracle_indexer_logits.restype = ctypes.c_int
            lib.oracle_sparse_attention.argtypes = [P, P, P, P, I, I, I, I, ctypes.c_int64, I, ctypes.c_double,
                                                    P, P, P]
            lib.oracle_sparse_attention.restype = ctypes.c_int
            lib.oracle_kth_largest.argtypes = [P, I, I, I, P]
            lib.oracle_kth_largest.restype = ctypes.c_int
            _lib = lib
    return _lib


def topk(x: np.ndarray, k: int, lengths: Optional[np.ndarray] = None) -> np.ndarray:
    """Oracle selection: int32 [rows, k], each row in (value desc, index asc)
    order, padded with -1 when the valid length is below k."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    rows, n = x.shape
    out = np.empty((rows, k), dtype=np.int32)
    lp = None
    if lengths is not None:
        lengths = np.ascontiguousarray(lengths, dtype=np.int32)
        assert lengths.shape == (rows,)
        lp = lengths.ctypes.data
    rc = lib.oracle_topk(x.ctypes.data, rows, n, lp, int(k), out.ctypes.data)
    if rc == ORACLE_ERR_NAN:
        raise ValueError("NaN among the valid logits (outside the selector's contract)")
    if rc != ORACLE_OK:
        raise ValueError("oracle_topk failed with code %d" % rc)
    return out


def topk_sorted(x: np.ndarray, k: int, lengths: Optional[np.ndarray] = None):
    """Ordered oracle selection: (int32 [rows, k] indices in (value desc,
    index asc) order, float32 [rows, k] values at those indices, -inf beside
    each -1)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    rows, n = x.shape
    out = np.empty((rows, k), dtype=np.int32)
    val = np.empty((rows, k), dtype=np.float32)
    lp = None
    if lengths is not None:
        lengths = np.ascontiguousarray(lengths, dtype=np.int32)
        assert lengths.shape == (rows,)
        lp = lengths.ctypes.data
    rc = lib.oracle_topk_sorted(x.ctypes.data, rows, n, lp, int(k), out.ctypes.data, val.ctypes.data)
    if rc == ORACLE_ERR_NAN:
        raise ValueError("NaN among the valid logits (outside the selector's contract)")
    if rc != ORACLE_OK:
        raise ValueError("oracle_topk_sorted failed with code %d" % rc)
    return out, val


def indexer_logits(q: np.ndarray, kc: np.ndarray, w: np.ndarray):
    """Indexer logits: q [rows, H, d], kc [n, d] (shared by every row) or
    [rows, n, d], w [rows, H]; float32 arrays holding bf16 values.  Returns
    (logits, absterm), both float64 [rows, n]: logits[r, t] = sum_h w[r, h] *
    max(0, q[r, h] . kc[t]); absterm[r, t] = sum_h |w[r, h]| * sum_i
    |q[r, h, i] * kc[t, i]|."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    kc = np.ascontiguousarray(kc, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, H, d = q.shape
    assert w.shape == (rows, H)
    if kc.ndim == 2:
        n = kc.shape[0]
        kstride = 0
    else:
        assert kc.shape[0] == rows
        n = kc.shape[1]
        kstride = n * d
    assert kc.shape[-1] == d
    logits = np.empty((rows, n), dtype=np.float64)
    absterm = np.empty((rows, n), dtype=np.float64)
    rc = lib.oracle_indexer_logits(q.ctypes.data, kc.ctypes.data, w.ctypes.data, rows, n, H, d, kstride,
                                   logits.ctypes.data, absterm.ctypes.data)
    if rc != ORACLE_OK:
        raise ValueError("oracle_indexer_logits failed with code %d" % rc)
    return logits, absterm


def sparse_attention(q: np.ndarray, kc: np.ndarray, vc: np.ndarray, idx: np.ndarray, scale: float):
    """Attention over the selected positions: q [rows, H, d]; kc, vc [n, d]
    (shared by every row) or [rows, n, d]; idx int32 [rows, k] (-1: no
    position).  Returns (out, mag, smax): out [rows, H, d] float64 =
    sum_j softmax_j(scale q . K[idx_j]) V[idx_j]; mag [rows, H, d] = sum_j
    p_j |V[idx_j]|; smax [rows, H] = max_j scale * sum_i |q_i K[idx_j]_i|."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    kc = np.ascontiguousarray(kc, dtype=np.float32)
    vc = np.ascontiguousarray(vc, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    rows, H, d = q.shape
    k = idx.shape[1]
    assert idx.shape == (rows, k) and kc.shape == vc.shape
    if kc.ndim == 2:
        n, kvstride = kc.shape[0], 0
    else:
        assert kc.shape[0] == rows
        n, kvstride = kc.shape[1], kc.shape[1] * d
    out = np.empty((rows, H, d), np.float64)
    mag = np.empty((rows, H, d), np.float64)
    smax = np.empty((rows, H), np.float64)
    rc = lib.oracle_sparse_attention(q.ctypes.data, kc.ctypes.data, vc.ctypes.data, idx.ctypes.data, rows, n, H, d,
                                     kvstride, k, float(scale), out.ctypes.data, mag.ctypes.data, smax.ctypes.data)
    if rc != ORACLE_OK:
        raise ValueError("oracle_sparse_attention failed with code %d" % rc)
    return out, mag, smax


def kth_largest(row: np.ndarray, k: int, length: Optional[int] = None) -> float:
    """The k-th largest valid value of one row, with multiplicity."""
    lib = _load()
    row = np.ascontiguousarray(row, dtype=np.float32).ravel()
    L = row.shape[0] if length is None else int(length)
    v = ctypes.c_float()
    rc = lib.oracle_kth_largest(row.ctypes.data, row.shape[0], L, int(k), ctypes.addressof(v))
    if rc != ORACLE_OK:
        raise ValueError("oracle_kth_largest failed with code %d" % rc)
    return float(np.float32(v.value))
