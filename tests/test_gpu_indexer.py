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
    idx3, lg3 = tks.indexer_select(q, kc, w, k, lengths=L, return_logits=True, fused=True)
    assert tks.device_status() == 0
    assert np.array_equal(lg3.cpu().numpy().view(np.uint32), lg.view(np.uint32)), "the fused form's logits differ"
    assert np.array_equal(np.sort(idx3.cpu().numpy(), 1), np.sort(want, 1))


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


def _sample_groups(n):
    """The groups of 64 tokens that topk_indexer_select_fused samples for
    its bound: every F-th group (F the smallest power of two from 2 that
    keeps 64 or fewer), group j F + F - 1 for j < ng // F."""
    ng = (n + 63) // 64
    F = 2
    while ng // F > 64:
        F *= 2
    return [j * F + F - 1 for j in range(ng // F)]


def _select_and_check(torch_gpu, wl, label, fused=False):
    import sparse_attention_topk_fp32_amd as tks

    _say(label + (" (fused)" if fused else ""))
    q, kc, w, L = _dev(torch_gpu, wl)
    idx, lg = tks.indexer_select(q, kc, w, wl.k, lengths=L, return_logits=True, fused=fused)
    assert tks.device_status() == 0
    lg = lg.cpu().numpy()
    want = oracle.topk(lg, wl.k, wl.lengths)
    assert np.array_equal(np.sort(idx.cpu().numpy(), 1), np.sort(want, 1))
    return idx.cpu().numpy(), lg


@pytest.mark.parametrize("fused", [False, True], ids=["two_launch", "fused"])
@pytest.mark.parametrize("rows,n,heads,dim,k,lengths", [
    (5, 12345, 20, 64, 1000, "uniform"),  # ragged rows, n not a multiple of 64
    (1, 16384, 64, 128, 5000, None),      # large k
    (1, 16384, 64, 128, 7000, None),
    (2, 65, 8, 32, 64, None),              # one token past a group of 64
    (3, 200000, 16, 32, 2048, None),      # n not a multiple of 64
    (8, 65536, 64, 128, 4096, "uniform"),
])
def test_indexer_selection_shapes(torch_gpu, rows, n, heads, dim, k, lengths, fused):
    wl = W.draw(rows, n, heads, dim, k=k, seed=rows * 7 + n % 1000 + k, lengths=lengths)
    if lengths == "uniform":
        # some rows short of k (every valid token selected), one empty
        wl.lengths[0] = min(k, n)
        if rows > 2:
            wl.lengths[1] = 0
    _select_and_check(torch_gpu, wl, "indexer shape rows=%d n=%d heads=%d dim=%d k=%d %s" % (
        rows, n, heads, dim, k, lengths or "full"), fused)


@pytest.mark.parametrize("fused", [False, True], ids=["two_launch", "fused"])
@pytest.mark.parametrize("scale,label", [(8.0, "periodic groups above the row"),
                                         (0.125, "periodic groups below the row")])
def test_indexer_selection_periodic_rows(torch_gpu, scale, label, fused):
    """Rows with a period: the keys of every F-th group of 64 tokens scaled
    (exactly, by a power of two) so that their logits lie far above or far
    below the rest.  The groups are the fused form's sample, so its bound
    lies far above the row's k-th largest (fewer than k candidates) or far
    below it (more than its buffer): it selects by passes over the logits.
    Exact against the oracle on the emitted logits either way."""
    n, k = 65536, 2048
    wl = W.draw(1, n, 16, 64, k=k, seed=5 + int(scale * 8))
    for g in _sample_groups(n):
        wl.kc[0, 64 * g:64 * g + 64] *= np.float32(scale)
    _select_and_check(torch_gpu, wl, "indexer %s n=%d k=%d" % (label, n, k), fused)


def test_indexer_selection_is_repeatable(torch_gpu):
    """Both indexer selections write the same bytes on every call (positions
    follow from block scans and exact ranks, not from timing)."""
    import sparse_attention_topk_fp32_amd as tks

    for name in ("idx_b1_n128k_h64_d128", "idx_b64_n16k_h64_d128_ragged"):
        wl = W.generate_indexer(name)
        _say("indexer repeatability %s" % name)
        q, kc, w, L = _dev(torch_gpu, wl)
        for fused in (False, True):
            first = tks.indexer_select(q, kc, w, wl.k, lengths=L, fused=fused).cpu().numpy()
            for _ in range(3):
                again = tks.indexer_select(q, kc, w, wl.k, lengths=L, fused=fused).cpu().numpy()
                assert np.array_equal(first, again), fused
            assert tks.device_status() == 0



@pytest.mark.parametrize("fused", [False, True], ids=["two_launch", "fused"])
def test_indexer_selection_drifting_rows(torch_gpu, fused):
    """Rows whose logits grow along the row (keys of the third quarter
    scaled by 2, of the last by 4, exactly): the k largest all sit in the
    last quarter, away from most of the rows' sampled groups.  Exact
    against the oracle on the emitted logits."""
    rows, n, k = 32, 16384, 2048
    wl = W.draw(rows, n, 16, 64, k=k, seed=91)
    wl.kc[:, n // 2:3 * n // 4] *= np.float32(2.0)
    wl.kc[:, 3 * n // 4:] *= np.float32(4.0)
    _select_and_check(torch_gpu, wl, "indexer drifting rows=%d n=%d k=%d" % (rows, n, k), fused)


def test_indexer_fused_graph_replay_and_streams(torch_gpu):
    """The fused form's per-row state (epochs, tags) lives in device memory:
    captured in a graph, every replay (with eager calls between) writes the
    eager call's bytes; calls on two streams at once (each with its own
    workspace) both match it."""
    import sparse_attention_topk_fp32_amd as tks

    torch = torch_gpu
    wl = W.generate_indexer("idx_b64_n16k_h64_d128_ragged")
    _say("indexer fused: graph replay x3 and two streams")
    q, kc, w, L = _dev(torch, wl)
    rows = wl.q.shape[0]
    s = torch.cuda.Stream()
    out = torch.full((rows, wl.k), -7, dtype=torch.int32, device="cuda")
    with torch.cuda.stream(s):
        eager = tks.indexer_select(q, kc, w, wl.k, lengths=L, fused=True).clone()
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            tks.indexer_select(q, kc, w, wl.k, lengths=L, out=out, fused=True)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        _ = tks.indexer_select(q, kc, w, wl.k, lengths=L, fused=True)  # eager work between replays
        torch.cuda.synchronize()
    assert tks.device_status(s) == 0
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    o1 = torch.empty_like(out)
    o2 = torch.empty_like(out)
    torch.cuda.synchronize()
    for _ in range(4):
        with torch.cuda.stream(s1):
            tks.indexer_select(q, kc, w, wl.k, lengths=L, out=o1, fused=True)
        with torch.cuda.stream(s2):
            tks.indexer_select(q, kc, w, wl.k, lengths=L, out=o2, fused=True)
        torch.cuda.synchronize()
        assert torch.equal(o1, eager) and torch.equal(o2, eager)
    assert tks.device_status(s1) == 0 and tks.device_status(s2) == 0
    lg = tks.indexer_logits(q, kc, w, lengths=L).cpu().numpy()
    want = oracle.topk(lg, wl.k, wl.lengths)
    assert np.array_equal(np.sort(eager.cpu().numpy(), 1), np.sort(want, 1))
