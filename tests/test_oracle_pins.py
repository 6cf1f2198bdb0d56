"""Pins of the CPU oracle to things other than itself (CPU only).

The oracle (``oracle/topk_oracle.c``) is the plain definition of the TopK
article's selector: sort valid positions by (value desc, index asc), keep k.
Each test below checks it against an independent source:

* brute force over every k-subset of tiny rows, kept by the defining property;
* the article's radix-select method restated step by step (``oracle.pages_radix``);
* numpy's stable sort (a library routine for the same order);
* closed forms of rows whose answer is known;
* hand-worked cases and the one value the article prints (``tests/golden``);
* the invariants every correct selection satisfies.
"""

from __future__ import annotations

import itertools
import math
import os

import numpy as np
import pytest

import oracle
from oracle import pages_radix
from tests.selection_checks import check_row_invariants, check_row_order, same_sets

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SUB = np.float32(1e-45)  # smallest positive subnormal float32
ALPHABET = np.array([-np.inf, -1.0, -0.0, 0.0, SUB, -SUB, 1.0, np.inf], dtype=np.float32)


def _parse_floats(s):
    return np.array([float(t) for t in s.split()], dtype=np.float32)


def _golden_cases():
    cases = []
    with open(os.path.join(GOLDEN, "hand_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals, k, length, expect = [p.strip() for p in line.split("|")]
            L = None if length == "all" else int(length)
            cases.append((_parse_floats(vals), int(k), L, [int(t) for t in expect.split()]))
    return cases


# ---------------------------------------------------------------- golden

@pytest.mark.parametrize("vals,k,L,expect", _golden_cases())
def test_hand_cases(vals, k, L, expect):
    lengths = None if L is None else np.array([L], dtype=np.int32)
    got = oracle.topk(vals[None, :], k, lengths)[0]
    assert sorted(got.tolist()) == expect
    # the article's method reaches the same set
    assert sorted(pages_radix.radix_topk_row(vals.tolist(), k, L)) == expect


def test_place_value_printed_by_article():
    with open(os.path.join(GOLDEN, "pages_place_value.txt")) as f:
        rows = [l.split("|") for l in f if l.strip() and not l.startswith("#")]
    assert rows, "empty fixture"
    for a, b in rows:
        assert pages_radix.highest_power_of_10(int(a)) == int(b)


# ---------------------------------------------------------------- brute force

def _brute_force_sets(x, L, k):
    """Every k-subset S of [0, L) such that each chosen element beats each
    unchosen one (larger value, or equal value and smaller index)."""
    found = []
    for S in itertools.combinations(range(L), k):
        s = set(S)
        ok = True
        for i in S:
            for j in range(L):
                if j in s:
                    continue
                if not (x[i] > x[j] or (x[i] == x[j] and i < j)):
                    ok = False
                    break
            if not ok:
                break
        if ok:
            found.append(list(S))
    return found


def test_brute_force_tiny_rows():
    rng = np.random.default_rng(20261202)
    checked = 0
    for n in range(1, 9):
        for _ in range(40):
            x = rng.choice(ALPHABET, size=n)
            L = int(rng.integers(0, n + 1)) if rng.random() < 0.3 else n
            for k in range(1, n + 1):
                got = oracle.topk(x[None, :], k, np.array([L], np.int32))[0]
                if L < k:
                    assert sorted(got.tolist()) == [-1] * (k - L) + list(range(L))
                    continue
                sets = _brute_force_sets(x.astype(np.float64), L, k)
                assert len(sets) == 1, (x, L, k, sets)  # the selection is unique
                assert sorted(got.tolist()) == sets[0], (x, L, k)
                checked += 1
    assert checked > 500


# ---------------------------------------------------------------- the article's method

def test_article_method_matches_oracle_random_ties():
    rng = np.random.default_rng(7)
    for trial in range(300):
        n = int(rng.integers(1, 400))
        kind = trial % 3
        if kind == 0:
            x = rng.choice(ALPHABET, size=n)
        elif kind == 1:
            x = rng.integers(-3, 4, size=n).astype(np.float32)  # heavy ties
        else:
            x = rng.standard_normal(n).astype(np.float32)
        k = int(rng.integers(1, n + 1))
        got = oracle.topk(x[None, :], k)[0]
        ref, tkey = pages_radix.radix_topk_indices(x.tolist(), k)
        assert sorted(got.tolist()) == sorted(ref)
        # both routes agree on the threshold T (the k-th largest value)
        assert pages_radix.float_to_ordered_u32(oracle.kth_largest(x, k)) == tkey


def test_article_method_on_workload_prefix():
    import workloads as W

    for name in ("c1", "c2", "c3"):
        w = W.generate(name)
        x = w.x[0, :3000]
        got = oracle.topk(x[None, :], 300)[0]
        ref = pages_radix.radix_topk_row(x.tolist(), 300)
        assert sorted(got.tolist()) == sorted(ref), name


# ---------------------------------------------------------------- numpy stable sort

def _numpy_select(x, L, k):
    xv = x[:L]
    order = np.lexsort((np.arange(L), -xv.astype(np.float64)))
    sel = order[:k].astype(np.int32)
    return np.concatenate([sel, -np.ones(k - len(sel), np.int32)])


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_numpy_stable_sort_on_workloads(name):
    import workloads as W

    w = W.generate(name)
    got = oracle.topk(w.x, w.k, w.lengths)
    for r in range(w.x.shape[0]):
        L = w.x.shape[1] if w.lengths is None else int(w.lengths[r])
        assert sorted(got[r].tolist()) == sorted(_numpy_select(w.x[r], L, w.k).tolist())


def test_numpy_stable_sort_on_sampled_causal_rows():
    import workloads as W

    w = W.generate("c5", rows=[0, 1, 2047, 4095])
    got = oracle.topk(w.x, w.k, w.lengths)
    for r in range(4):
        L = int(w.lengths[r])
        assert sorted(got[r].tolist()) == sorted(_numpy_select(w.x[r], L, w.k).tolist())
        check_row_invariants(w.x[r], L, w.k, got[r])


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("L,k", [(1, 1), (5, 3), (100, 100), (4096, 2048), (10000, 2048), (3, 2048)])
def test_closed_forms(L, k):
    n = max(L, k)
    idx = np.arange(n)
    want_low = list(range(min(k, L))) + [-1] * max(0, k - L)
    lengths = np.array([L], np.int32)
    # constant row: lowest indices
    x = np.full(n, 0.25, np.float32)
    assert sorted(oracle.topk(x[None], k, lengths)[0].tolist()) == sorted(want_low)
    # descending ramp: the first k
    x = (-idx).astype(np.float32)
    assert sorted(oracle.topk(x[None], k, lengths)[0].tolist()) == sorted(want_low)
    # all -inf: lowest indices
    x = np.full(n, -np.inf, np.float32)
    assert sorted(oracle.topk(x[None], k, lengths)[0].tolist()) == sorted(want_low)
    # ascending ramp: the last k valid positions
    x = idx.astype(np.float32)
    got = sorted(oracle.topk(x[None], k, lengths)[0].tolist())
    if L >= k:
        assert got == list(range(L - k, L))
    else:
        assert got == sorted(want_low)


def test_k_equal_one_is_first_argmax():
    rng = np.random.default_rng(3)
    for _ in range(200):
        n = int(rng.integers(1, 300))
        x = rng.integers(-5, 5, size=n).astype(np.float32)
        assert oracle.topk(x[None], 1)[0, 0] == int(np.argmax(x))


def test_k_equal_length_is_everything():
    x = np.random.default_rng(4).standard_normal(777).astype(np.float32)
    assert sorted(oracle.topk(x[None], 777)[0].tolist()) == list(range(777))


def test_zero_length_rows_are_all_padding():
    x = np.ones((3, 10), np.float32)
    got = oracle.topk(x, 4, np.array([0, -5, 2], np.int32))
    assert got[0].tolist() == [-1] * 4 and got[1].tolist() == [-1] * 4
    assert sorted(got[2].tolist()) == [-1, -1, 0, 1]


def test_lengths_beyond_n_are_clamped():
    x = np.arange(8, dtype=np.float32)[None]
    assert sorted(oracle.topk(x, 2, np.array([100], np.int32))[0].tolist()) == [6, 7]


# ---------------------------------------------------------------- invariants

def test_invariants_hold_on_oracle_outputs():
    rng = np.random.default_rng(11)
    for _ in range(200):
        n = int(rng.integers(1, 600))
        x = rng.choice(ALPHABET, size=n) if rng.random() < 0.5 else rng.standard_normal(n).astype(np.float32)
        k = int(rng.integers(1, n + 1))
        L = int(rng.integers(0, n + 1))
        got = oracle.topk(x[None], k, np.array([L], np.int32))[0]
        check_row_invariants(x, L, k, got)


def test_invariant_checker_rejects_planted_mistakes():
    """A wrong selection (highest-index ties, a dropped element, a value swap)
    must be caught by the checker the GPU tests rely on."""
    x = np.array([3, 5, 5, 5, 1, 7], np.float32)
    good = oracle.topk(x[None], 3)[0]
    check_row_invariants(x, 6, 3, good)
    for bad in ([5, 3, 2], [5, 1, 1], [5, 1, 0], [5, 1, -1], [5, 4, 1]):
        with pytest.raises(AssertionError):
            check_row_invariants(x, 6, 3, np.array(bad, np.int32))


# ---------------------------------------------------------------- key map of the article's method

def test_mapping_step_orders_like_floats():
    rng = np.random.default_rng(5)
    specials = np.array(
        [-np.inf, -np.finfo(np.float32).max, -1.0, -np.finfo(np.float32).tiny, -SUB, -0.0, 0.0, SUB,
         np.finfo(np.float32).tiny, 1.0, np.finfo(np.float32).max, np.inf], dtype=np.float32)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[~np.isnan(vals)]
    allv = np.concatenate([specials, vals, rng.standard_normal(2000).astype(np.float32)])
    keys = np.array([pages_radix.float_to_ordered_u32(float(v)) for v in allv], dtype=np.uint64)
    order = np.argsort(allv.astype(np.float64), kind="stable")
    sv, sk = allv[order].astype(np.float64), keys[order]
    for a in range(len(sv) - 1):
        if sv[a] < sv[a + 1]:
            assert sk[a] < sk[a + 1]
        else:
            assert sk[a] == sk[a + 1]
    assert pages_radix.float_to_ordered_u32(-0.0) == pages_radix.float_to_ordered_u32(0.0)
    # every non-NaN key fits in 32 bits and is non-negative
    assert all(0 <= int(kk) < 2**32 for kk in keys)


def test_oracle_rejects_nan_and_bad_arguments():
    x = np.array([[1.0, math.nan, 2.0]], np.float32)
    with pytest.raises(ValueError):
        oracle.topk(x, 1)
    # a NaN past the valid length is never read
    assert oracle.topk(x, 1, np.array([1], np.int32))[0].tolist() == [0]
    with pytest.raises(ValueError):
        oracle.topk(np.ones((1, 3), np.float32), 4)
    with pytest.raises(ValueError):
        oracle.topk(np.ones((1, 3), np.float32), 0)


def test_same_sets_helper():
    assert same_sets(np.array([[1, 2, 3]]), np.array([[3, 1, 2]]))
    assert not same_sets(np.array([[1, 2, 3]]), np.array([[3, 1, 4]]))


# ---------------------------------------------------------------- ordered output (need_sorted)

def _ordered_ok(x, seq):
    """Defining property of the ordered output: values never increase, equal
    values have increasing indices."""
    return all(x[a] > x[b] or (x[a] == x[b] and a < b) for a, b in zip(seq, seq[1:]))


def test_sorted_brute_force_tiny_rows():
    """Every ordered k-sequence of distinct valid positions that is a correct
    selection and satisfies the order property: exactly one exists, and it is
    the oracle's ordered output."""
    rng = np.random.default_rng(99)
    checked = 0
    for n in range(1, 7):
        for _ in range(25):
            x = rng.choice(ALPHABET, size=n)
            L = int(rng.integers(0, n + 1)) if rng.random() < 0.3 else n
            xv = x.astype(np.float64)
            for k in range(1, n + 1):
                idx, vals = oracle.topk_sorted(x[None, :], k, np.array([L], np.int32))
                take = min(k, L)
                found = []
                for seq in itertools.permutations(range(L), take):
                    row = np.array(list(seq) + [-1] * (k - take), np.int32)
                    try:
                        check_row_invariants(x, L, k, row)
                    except AssertionError:
                        continue
                    if _ordered_ok(xv, seq):
                        found.append(list(seq))
                assert len(found) == 1, (x, L, k, found)
                assert idx[0, :take].tolist() == found[0] and np.all(idx[0, take:] == -1)
                check_row_order(x, L, k, idx[0], vals[0])
                checked += 1
    assert checked > 200


def test_sorted_matches_article_method_with_need_sorted():
    rng = np.random.default_rng(17)
    for trial in range(200):
        n = int(rng.integers(1, 300))
        kind = trial % 3
        if kind == 0:
            x = rng.choice(ALPHABET, size=n)
        elif kind == 1:
            x = rng.integers(-3, 4, size=n).astype(np.float32)
        else:
            x = rng.standard_normal(n).astype(np.float32)
        k = int(rng.integers(1, n + 1))
        idx, _ = oracle.topk_sorted(x[None, :], k)
        assert idx[0].tolist() == pages_radix.radix_topk_sorted(x.tolist(), k)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_sorted_matches_numpy_lexsort_on_workloads(name):
    import workloads as W

    w = W.generate(name)
    rows = range(w.x.shape[0]) if w.x.shape[0] <= 8 else range(0, w.x.shape[0], 9)
    for r in rows:
        L = w.x.shape[1] if w.lengths is None else int(w.lengths[r])
        lr = None if w.lengths is None else w.lengths[r:r + 1]
        idx, vals = oracle.topk_sorted(w.x[r:r + 1], w.k, lr)
        assert np.array_equal(idx[0], _numpy_select(w.x[r], L, w.k))
        check_row_order(w.x[r], L, w.k, idx[0], vals[0])


@pytest.mark.parametrize("L,k", [(1, 1), (5, 3), (100, 100), (4096, 2048), (3, 2048)])
def test_sorted_closed_forms(L, k):
    n = max(L, k)
    idx = np.arange(n)
    lengths = np.array([L], np.int32)
    take = min(k, L)
    low = list(range(take)) + [-1] * (k - take)
    for x in (np.full(n, 0.25, np.float32), (-idx).astype(np.float32), np.full(n, -np.inf, np.float32)):
        got, vals = oracle.topk_sorted(x[None], k, lengths)
        assert got[0].tolist() == low
        assert np.array_equal(vals[0, :take], x[:take]) and np.all(vals[0, take:] == -np.inf)
    # ascending ramp: the last positions, largest first
    got, vals = oracle.topk_sorted(idx.astype(np.float32)[None], k, lengths)
    assert got[0].tolist() == list(range(L - 1, L - 1 - take, -1)) + [-1] * (k - take)


def test_sorted_values_keep_the_sign_of_zero():
    x = np.array([-0.0, 0.0, -1.0, -0.0], np.float32)
    idx, vals = oracle.topk_sorted(x[None], 3)
    assert idx[0].tolist() == [0, 1, 3]
    assert vals[0].view(np.uint32).tolist() == [0x80000000, 0, 0x80000000]


def test_order_checker_rejects_planted_mistakes():
    x = np.array([3, 5, 5, 5, 1, 7, -0.0], np.float32)
    idx, vals = oracle.topk_sorted(x[None], 4)
    check_row_order(x, 7, 4, idx[0], vals[0])
    bad = idx[0].copy()
    bad[[1, 2]] = bad[[2, 1]]  # equal values, indices descending
    with pytest.raises(AssertionError):
        check_row_order(x, 7, 4, bad)
    bad = idx[0].copy()
    bad[[0, 1]] = bad[[1, 0]]  # smaller value first
    with pytest.raises(AssertionError):
        check_row_order(x, 7, 4, bad)
    badv = vals[0].copy()
    badv[0] = 6.0
    with pytest.raises(AssertionError):
        check_row_order(x, 7, 4, idx[0], badv)
    # -0.0 reported as +0.0 is caught
    i2, v2 = oracle.topk_sorted(x[None], 7)
    v2 = v2[0].copy()
    v2[-1] = 0.0
    with pytest.raises(AssertionError):
        check_row_order(x, 7, 7, i2[0], v2)
    # padding not at the end is caught
    i3, _ = oracle.topk_sorted(x[None], 7, np.array([5], np.int32))
    row = i3[0].copy()
    row[[0, 5]] = row[[5, 0]]
    with pytest.raises(AssertionError):
        check_row_order(x, 5, 7, row)


# ---------------------------------------------------------------- indexer logits (DSA step 1)

def test_indexer_logits_closed_forms():
    # one-hot queries pick one key coordinate per head: logits = sum_h w_h * max(0, K[t, j_h])
    d, H, n = 8, 3, 5
    q = np.zeros((1, H, d), np.float32)
    picks = [1, 4, 7]
    for h, j in enumerate(picks):
        q[0, h, j] = 1.0
    K = np.arange(n * d, dtype=np.float32).reshape(n, d) - 20.0
    w = np.array([[0.5, 2.0, 0.25]], np.float32)
    lg, ab = oracle.indexer_logits(q, K, w)
    for t in range(n):
        want = sum(w[0, h] * max(0.0, K[t, j]) for h, j in enumerate(picks))
        assert lg[0, t] == want
        assert ab[0, t] == sum(w[0, h] * abs(K[t, j]) for h, j in enumerate(picks))
    # a query opposite to every key: every head is cut to zero by the ReLU
    K2 = np.abs(np.random.default_rng(1).standard_normal((6, d))).astype(np.float32) + 0.5
    q2 = -np.ones((1, 2, d), np.float32)
    lg2, _ = oracle.indexer_logits(q2, K2, np.ones((1, 2), np.float32))
    assert np.all(lg2 == 0.0)
    # one head, one dimension: w * max(0, q * k)
    lg3, _ = oracle.indexer_logits(np.array([[[3.0]]], np.float32), np.array([[2.0], [-1.0]], np.float32),
                                   np.array([[0.5]], np.float32))
    assert lg3.tolist() == [[3.0, 0.0]]


@pytest.mark.parametrize("shared", [True, False])
def test_indexer_logits_match_matrix_route(shared):
    """A second route: numpy matrix products in float64."""
    import workloads as W

    wl = W.draw(rows=3, n=300, heads=7, dim=32, k=16, seed=9, shared_keys=shared)
    lg, ab = oracle.indexer_logits(wl.q, wl.kc, wl.w)
    for r in range(3):
        K = (wl.kc if shared else wl.kc[r]).astype(np.float64)
        S = wl.q[r].astype(np.float64) @ K.T  # [H, n]
        want = wl.w[r].astype(np.float64) @ np.maximum(S, 0.0)
        mag = np.abs(wl.w[r].astype(np.float64)) @ (np.abs(wl.q[r].astype(np.float64)) @ np.abs(K.T))
        assert np.allclose(lg[r], want, rtol=1e-12, atol=1e-12)
        assert np.allclose(ab[r], mag, rtol=1e-12, atol=1e-12)


def test_indexer_logits_linear_in_weights_and_blind_to_head_order():
    import workloads as W

    wl = W.draw(rows=2, n=64, heads=5, dim=16, k=8, seed=3)
    lg, _ = oracle.indexer_logits(wl.q, wl.kc, wl.w)
    lg2, _ = oracle.indexer_logits(wl.q, wl.kc, (wl.w * 2).astype(np.float32))
    assert np.array_equal(lg2, 2 * lg)
    perm = np.array([3, 0, 4, 1, 2])
    lg3, _ = oracle.indexer_logits(np.ascontiguousarray(wl.q[:, perm]), wl.kc, np.ascontiguousarray(wl.w[:, perm]))
    assert np.allclose(lg3, lg, rtol=1e-13, atol=0)


# ---------------------------------------------------------------- attention over the selected positions (DSA step 3)

def test_sparse_attention_closed_forms():
    rng = np.random.default_rng(4)
    K = rng.standard_normal((10, 8)).astype(np.float32)
    V = rng.standard_normal((10, 8)).astype(np.float32)
    q = rng.standard_normal((1, 3, 8)).astype(np.float32)
    # one selected position: its value row, whatever the scores
    out, _, _ = oracle.sparse_attention(q, K, V, np.array([[-1, 6, -1]], np.int32), 0.7)
    assert np.array_equal(out[0], np.repeat(V[6][None].astype(np.float64), 3, axis=0))
    # equal scores (zero query): the mean of the selected value rows
    sel = [1, 4, 9, 0]
    out, _, _ = oracle.sparse_attention(np.zeros((1, 2, 8), np.float32), K, V, np.array([sel], np.int32), 1.0)
    assert np.allclose(out[0], V[sel].astype(np.float64).mean(axis=0)[None], rtol=1e-14, atol=1e-15)
    # no selected position: zeros
    out, _, _ = oracle.sparse_attention(q, K, V, np.full((1, 4), -1, np.int32), 1.0)
    assert np.all(out == 0.0)


def test_sparse_attention_matches_numpy_route_and_ignores_slot_order():
    import workloads as W

    wl = W.draw_attention(rows=3, n=200, heads=5, dim=16, k=40, seed=8, lengths="uniform")
    scale = 0.25
    out, mag, smax = oracle.sparse_attention(wl.q, wl.kc, wl.vc, wl.idx, scale)
    for r in range(3):
        sel = wl.idx[r][wl.idx[r] >= 0]
        K = wl.kc[r][sel].astype(np.float64)
        V = wl.vc[r][sel].astype(np.float64)
        S = scale * (wl.q[r].astype(np.float64) @ K.T)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        assert np.allclose(out[r], P @ V, rtol=1e-12, atol=1e-12)
        assert np.allclose(mag[r], P @ np.abs(V), rtol=1e-12, atol=1e-12)
        assert np.allclose(smax[r], (scale * (np.abs(wl.q[r].astype(np.float64)) @ np.abs(K.T))).max(axis=1))
    perm = np.random.default_rng(1).permutation(wl.idx.shape[1])
    out2, _, _ = oracle.sparse_attention(wl.q, wl.kc, wl.vc, np.ascontiguousarray(wl.idx[:, perm]), scale)
    assert np.allclose(out2, out, rtol=1e-13, atol=1e-14)


def test_sparse_attention_is_linear_in_values_and_shift_invariant_in_scores():
    import workloads as W

    wl = W.draw_attention(rows=2, n=64, heads=3, dim=8, k=10, seed=5, shared_kv=True)
    out, _, _ = oracle.sparse_attention(wl.q, wl.kc, wl.vc, wl.idx, 0.5)
    out2, _, _ = oracle.sparse_attention(wl.q, wl.kc, (2 * wl.vc).astype(np.float32), wl.idx, 0.5)
    assert np.allclose(out2, 2 * out, rtol=1e-14, atol=1e-15)
    # a key component every selected key shares adds the same score to all:
    # append a constant column to the keys and a matching query column
    kc2 = np.concatenate([wl.kc, np.ones((wl.kc.shape[0], 1), np.float32)], axis=1)
    vc2 = np.concatenate([wl.vc, np.zeros((wl.vc.shape[0], 1), np.float32)], axis=1)
    q2 = np.concatenate([wl.q, np.full(wl.q.shape[:2] + (1,), 3.0, np.float32)], axis=2)
    out3, _, _ = oracle.sparse_attention(q2, kc2, vc2, wl.idx, 0.5)
    assert np.allclose(out3[:, :, :-1], out, rtol=1e-12, atol=1e-13)
