"""GPU parity of the indexer that feeds the selector (DSA step 1 of the TopK
article's section 01): the matrix-core logits against the oracle's double
precision logits within the float32 rounding bound, and the selection on
those logits against the oracle's selection on the same (GPU) logits,
bit-exact as sets (the decision is taken in the kernel's precision on both
sides).  Each case prints its name before touching the GPU."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from tests.test_gpu_parity import _say

pytestmark = pytest.mark.gpu

U = 2.0 ** -24  # float32 unit roundoff


@pytest.fixture(scope="module")
def torch_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_topk_fp32_amd as tks

    tks.version()
    return torch


def _dev(torch, wl):
    q = torch.from_numpy(wl.q).cuda().to(torch.bfloat16)
    kc = torch.from_numpy(wl.kc).cuda().to(torch.bfloat16)
    w = torch.from_numpy(wl.w).cuda()
    L = None if wl.lengths is None else torch.from_numpy(wl.lengths).cuda()
    return q, kc, w, L


def assert_logits_close(wl, got, rows=None):
    """|got - exact| <= (dim + heads + 2) * u * sum_h |w| sum_i |q k|; -inf
    past each valid length."""
    rows = np.arange(wl.q.shape[0]) if rows is None else np.asarray(rows)
    q, w = wl.q[rows], wl.w[rows]
    kc = wl.kc if wl.kc.ndim == 2 else wl.kc[rows]
    want, mag = oracle.indexer_logits(q, kc, w)
    H, d = wl.q.shape[1], wl.q.shape[2]
    n = want.shape[1]
    for i, r in enumerate(rows):
        L = n if wl.lengths is None else int(min(max(int(wl.lengths[r]), 0), n))
        g = got[i].astype(np.float64)
        assert np.all(np.isneginf(g[L:])), "positions past the valid length must be -inf"
        err = np.abs(g[:L] - want[i, :L])
        bound = (d + H + 2) * U * mag[i, :L] + 1e-30
        bad = np.nonzero(err > bound)[0]
        assert bad.size == 0, "row %d: %d logits outside the rounding bound (first t=%d: got %r want %r bound %r)" % (
            r, bad.size, bad[0], g[bad[0]], want[i, bad[0]], bound[bad[0]])


def _cases():
    out = []
    for rows, n, heads, dim, shared, lengths in [
        (1, 1, 1, 32, False, None),
        (1, 63, 16, 32, False, None),
        (2, 300, 5, 64, True, None),
        (3, 1000, 17, 128, False, "uniform"),
        (2, 4100, 40, 64, False, None),
        (1, 5000, 64, 128, False, None),
        (4, 2049, 64, 32, True, "uniform"),
        (2, 777, 33, 128, True, None),
    ]:
        out.append(pytest.param(rows, n, heads, dim, shared, lengths,
                                id="r%d_n%d_h%d_d%d_%s_%s" % (rows, n, heads, dim, "shared" if shared else "own",
                                                              lengths or "full")))
    return out


@pytest.mark.parametrize("rows,n,heads,dim,shared,lengths", _cases())
def test_indexer_logits_and_selection(torch_gpu, rows, n, heads, dim, shared, lengths):
    import sparse_attention_topk_fp32_amd as tks

    wl = W.draw(rows, n, heads, dim, k=min(n, 100), seed=n + heads, shared_keys=shared, lengths=lengths)
    _say("indexer rows=%d n=%d heads=%d dim=%d shared=%s lengths=%s" % (rows, n, heads, dim, shared, lengths))
    q, kc, w, L = _dev(torch_gpu, wl)
    lg = tks.indexer_logits(q, kc, w, lengths=L).cpu().numpy()
    assert_logits_close(wl, lg)
    k = wl.k
    idx, lg2 = tks.indexer_select(q, kc, w, k, lengths=L, return_logits=True)
    assert tks.device_status() == 0
    lg2 = lg2.cpu().numpy()
    assert np.array_equal(lg2.view(np.uint32), lg.view(np.uint32)), "the two entry points computed different logits"
    want = oracle.topk(lg2, k, wl.lengths)
    assert np.array_equal(np.sort(idx.cpu().numpy(), 1), np.sort(want, 1))


def test_indexer_batch1_decode_workload(torch_gpu):
    import sparse_attention_topk_fp32_amd as tks

    wl = W.generate_indexer("idx_b1_n128k_h64_d128")
    _say("indexer workload %s" % wl.config.name)
    q, kc, w, L = _dev(torch_gpu, wl)
    idx, lg = tks.indexer_select(q, kc, w, wl.k, lengths=L, return_logits=True)
    assert tks.device_status() == 0
    lg = lg.cpu().numpy()
    assert_logits_close(wl, lg)
    want = oracle.topk(lg, wl.k, wl.lengths)
    assert np.array_equal(np.sort(idx.cpu().numpy(), 1), np.sort(want, 1))
    # the scratch path (no logits output) selects the same set
    idx2 = tks.indexer_select(q, kc, w, wl.k, lengths=L)
    assert np.array_equal(np.sort(idx2.cpu().numpy(), 1), np.sort(want, 1))


def test_indexer_batched_ragged_workload(torch_gpu):
    import sparse_attention_topk_fp32_amd as tks

    wl = W.generate_indexer("idx_b64_n16k_h64_d128_ragged")
    _say("indexer workload %s" % wl.config.name)
    q, kc, w, L = _dev(torch_gpu, wl)
    idx, lg = tks.indexer_select(q, kc, w, wl.k, lengths=L, return_logits=True)
    assert tks.device_status() == 0
    lg = lg.cpu().numpy()
    sample = [0, 1, 17, 40, 63]
    assert_logits_close(wl, lg[sample], rows=sample)
    want = oracle.topk(lg, wl.k, wl.lengths)
    assert np.array_equal(np.sort(idx.cpu().numpy(), 1), np.sort(want, 1))
