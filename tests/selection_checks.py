"""Checks on a selected index row that hold whatever produced it.

The selector's contract (TopK article, sections 01 and 02): per row, the
indices of the k largest valid values, each index once, ties at the
threshold value going to the lowest indices, -1 in slots that hold no index
(section 5's output flush).
"""

from __future__ import annotations

import numpy as np


def valid_length(n: int, lengths, r: int) -> int:
    if lengths is None:
        return n
    return int(min(max(int(lengths[r]), 0), n))


def check_row_invariants(x_row: np.ndarray, L: int, k: int, sel: np.ndarray) -> None:
    """Raise AssertionError unless ``sel`` is the unique correct selection for
    the valid prefix ``x_row[:L]``: k entries, min(k, L) distinct indices in
    [0, L), -1 in the rest, every selected value >= every unselected valid
    value, and among values equal to the smallest selected value the selected
    indices all lie below the unselected ones."""
    sel = np.asarray(sel)
    assert sel.shape == (k,), sel.shape
    take = min(k, L)
    valid = sel[sel >= 0]
    assert int((sel == -1).sum()) == k - take, "wrong number of -1 slots"
    assert valid.size == take, "wrong number of indices"
    assert np.all(valid < L), "index past the valid length"
    assert np.unique(valid).size == take, "duplicate index"
    if take == 0 or take == L:
        return
    xv = x_row[:L].astype(np.float64)
    chosen = np.zeros(L, dtype=bool)
    chosen[valid] = True
    lo = xv[chosen].min()
    hi = xv[~chosen].max()
    assert lo >= hi, "an unselected value exceeds a selected one"
    if lo == hi:
        tied = np.nonzero(xv == lo)[0]
        tsel = tied[chosen[tied]]
        tun = tied[~chosen[tied]]
        assert tsel.max() < tun.min(), "ties at the threshold not taken lowest index first"


def check_row_order(x_row: np.ndarray, L: int, k: int, sel: np.ndarray, vals=None) -> None:
    """Raise AssertionError unless ``sel`` is the correct selection (as in
    check_row_invariants) laid out in order: values descending, equal values
    by index ascending, the -1 slots last; and, when ``vals`` is given, each
    value is the logit at its index bit for bit, -inf beside each -1."""
    sel = np.asarray(sel)
    check_row_invariants(x_row, L, k, sel)
    take = min(k, L)
    assert np.all(sel[:take] >= 0) and np.all(sel[take:] == -1), "-1 slots not at the end"
    s = sel[:take].astype(np.int64)
    xv = x_row.astype(np.float64)[s]
    if take > 1:
        a, b = xv[:-1], xv[1:]
        ok = (a > b) | ((a == b) & (s[:-1] < s[1:]))
        assert np.all(ok), "out of order at position %d" % int(np.argmin(ok))
    if vals is not None:
        vals = np.asarray(vals, dtype=np.float32)
        assert vals.shape == (k,)
        want = x_row[s].astype(np.float32)
        assert np.array_equal(vals[:take].view(np.uint32), want.view(np.uint32)), "values differ from the logits"
        assert np.all(vals[take:] == -np.inf), "padding values are not -inf"


def same_sets(a: np.ndarray, b: np.ndarray) -> bool:
    """Row-wise equality of two [rows, k] index arrays as sorted multisets."""
    return np.array_equal(np.sort(a, axis=-1), np.sort(b, axis=-1))


def check_rows_vectorized(x: np.ndarray, lengths, k: int, sel: np.ndarray, block: int = 256) -> None:
    """check_row_invariants for many rows at once (numpy, row blocks)."""
    rows, n = x.shape
    col = np.arange(n)
    for r0 in range(0, rows, block):
        r1 = min(rows, r0 + block)
        xb = x[r0:r1]
        sb = np.asarray(sel[r0:r1])
        R = r1 - r0
        L = np.full(R, n) if lengths is None else np.clip(np.asarray(lengths[r0:r1]).astype(np.int64), 0, n)
        take = np.minimum(k, L)
        assert np.array_equal((sb == -1).sum(1), k - take), "wrong number of -1 slots"
        valid_sel = sb >= 0
        assert np.array_equal(valid_sel.sum(1), take), "wrong number of indices"
        assert np.all(np.where(valid_sel, sb, 0) < L[:, None]), "index past the valid length"
        ss = np.sort(np.where(valid_sel, sb, -1), axis=1)
        dup = (np.diff(ss, axis=1) == 0) & (ss[:, 1:] >= 0)
        assert not dup.any(), "duplicate index"
        chosen = np.zeros((R, n), dtype=bool)
        rr = np.repeat(np.arange(R), k)
        flat = sb.reshape(-1)
        m = flat >= 0
        chosen[rr[m], flat[m]] = True
        valid = col[None, :] < L[:, None]
        xf = xb.astype(np.float64)
        lo = np.where(chosen, xf, np.inf).min(1)
        hi = np.where(valid & ~chosen, xf, -np.inf).max(1)
        assert np.all(lo >= hi), "an unselected value exceeds a selected one"
        tie = valid & (xf == lo[:, None])
        max_sel_tie = np.where(tie & chosen, col[None, :], -1).max(1)
        min_uns_tie = np.where(tie & ~chosen, col[None, :], n).min(1)
        assert np.all(max_sel_tie < min_uns_tie), "ties at the threshold not taken lowest index first"
