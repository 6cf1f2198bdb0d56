"""GPU parity of the attention over the selected positions (DSA step 3 of
the TopK article's section 01) against the oracle's double precision result,
within the float32/bf16 rounding bound stated with the C ABI; and the three
steps chained (indexer logits, selection, attention) against the oracle fed
the GPU's own selection.  Each case prints its name before touching the GPU."""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import workloads as W
from tests.test_gpu_parity import _say

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module")
def torch_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_topk_fp32_amd as tks

    tks.version()
    return torch


def _bf16(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16)


def assert_attention_close(q, kc, vc, idx, scale, got):
    want, mag, smax = oracle.sparse_attention(q, kc, vc, idx, scale)
    d = q.shape[2]
    k = idx.shape[1]
    # P is carried as two bf16 terms (hi + lo within 2^-16 p), hence 2^-16
    coef = 2 * (d + 2) * U * smax[:, :, None] + 2.0 ** -16 + (k + 64) * U + 2.0 ** -20
    bound = coef * mag + 1e-30
    err = np.abs(got.astype(np.float64) - want)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, "%d outputs outside the bound (first %s: got %r want %r bound %r)" % (
        len(bad), tuple(bad[0]), got[tuple(bad[0])], want[tuple(bad[0])], bound[tuple(bad[0])])
    # rows without a position give zeros
    empty = ~(idx >= 0).any(axis=1)
    assert np.all(got[empty] == 0.0)


def _cases():
    out = []
    for rows, n, heads, dim, k, shared, lengths in [
        (1, 50, 1, 32, 1, False, None),
        (1, 300, 16, 64, 64, False, None),
        (2, 1000, 5, 128, 100, True, None),
        (3, 5000, 16, 128, 2048, False, "uniform"),
        (2, 3000, 40, 64, 700, False, None),
        (4, 2500, 64, 128, 300, True, "uniform"),
        (2, 100, 17, 32, 130, False, None),
        # several combine batches of 32 chunks (79 chunks: a ragged last one)
        (1, 9000, 8, 64, 5000, False, None),
        # more than 256 (row, head) pairs: batches of 16 chunks (24 chunks)
        (20, 3000, 16, 32, 1500, False, "uniform"),
        # at least 512 WGs of two 64-slot sub-chunks: 128 slots per WG (a
        # ragged last WG; empty slots past each row's length)
        (48, 3000, 16, 64, 1500, False, "uniform"),
        (520, 200, 4, 32, 100, True, None),
        # at least 512 WGs of four sub-chunks: 256 slots per WG (the last
        # WG of a row ragged in its fourth sub-chunk), 16, 40 and 64 heads
        (130, 2000, 16, 128, 1000, False, "uniform"),
        (260, 1500, 40, 64, 500, True, None),
        (520, 800, 64, 32, 300, False, "uniform"),
    ]:
        out.append(pytest.param(rows, n, heads, dim, k, shared, lengths,
                                id="r%d_n%d_h%d_d%d_k%d_%s_%s" % (rows, n, heads, dim, k,
                                                                  "shared" if shared else "own", lengths or "full")))
    return out


@pytest.mark.parametrize("rows,n,heads,dim,k,shared,lengths", _cases())
def test_sparse_attention_parity(torch_gpu, rows, n, heads, dim, k, shared, lengths):
    import sparse_attention_topk_fp32_amd as tks

    wl = W.draw_attention(rows, n, heads, dim, k, seed=rows * 1000 + n + k, shared_kv=shared, lengths=lengths)
    _say("attention rows=%d n=%d heads=%d dim=%d k=%d shared=%s" % (rows, n, heads, dim, k, shared))
    scale = 1.0 / math.sqrt(dim)
    got = tks.sparse_attention(_bf16(torch_gpu, wl.q), _bf16(torch_gpu, wl.kc), _bf16(torch_gpu, wl.vc),
                               torch_gpu.from_numpy(wl.idx).cuda(), scale).cpu().numpy()
    assert tks.device_status() == 0
    assert_attention_close(wl.q, wl.kc, wl.vc, wl.idx, scale, got)


def test_sparse_attention_skips_empty_and_out_of_range_slots(torch_gpu):
    import sparse_attention_topk_fp32_amd as tks

    wl = W.draw_attention(3, 400, 8, 64, 96, seed=77)
    idx = wl.idx.copy()
    idx[0, ::3] = -1
    idx[1, 5] = 400          # past n: holds no position
    idx[1, 6] = -12345
    idx[2, :] = -1           # no position at all: zeros
    _say("attention with empty / out-of-range slots")
    got = tks.sparse_attention(_bf16(torch_gpu, wl.q), _bf16(torch_gpu, wl.kc), _bf16(torch_gpu, wl.vc),
                               torch_gpu.from_numpy(idx).cuda(), 0.125).cpu().numpy()
    clean = np.where((idx >= 0) & (idx < 400), idx, -1).astype(np.int32)
    assert_attention_close(wl.q, wl.kc, wl.vc, clean, 0.125, got)


@pytest.mark.parametrize("name", ["att_b1_n128k_h16_d128_k2048", "att_b64_n16k_h16_d128_k2048_ragged"])
def test_sparse_attention_workloads(torch_gpu, name):
    import sparse_attention_topk_fp32_amd as tks

    wl = W.generate_attention(name)
    _say("attention workload %s" % name)
    scale = 1.0 / math.sqrt(wl.q.shape[2])
    got = tks.sparse_attention(_bf16(torch_gpu, wl.q), _bf16(torch_gpu, wl.kc), _bf16(torch_gpu, wl.vc),
                               torch_gpu.from_numpy(wl.idx).cuda(), scale).cpu().numpy()
    assert tks.device_status() == 0
    rows = np.arange(wl.q.shape[0]) if wl.q.shape[0] <= 8 else np.array([0, 1, 17, 40, 63])
    assert_attention_close(wl.q[rows], wl.kc[rows], wl.vc[rows], wl.idx[rows], scale, got[rows])


def test_decode_pipeline_indexer_selection_attention(torch_gpu):
    """The three DSA steps on the GPU: logits from the indexer, the k largest,
    attention over them; each step checked against the oracle fed the GPU's
    output of the step before."""
    import sparse_attention_topk_fp32_amd as tks

    torch = torch_gpu
    rows, n, k = 4, 20000, 512
    ix = W.draw(rows, n, heads=32, dim=64, k=k, seed=5, lengths="uniform")
    at = W.draw_attention(rows, n, heads=16, dim=128, k=k, seed=6)
    _say("pipeline rows=%d n=%d k=%d" % (rows, n, k))
    L = torch.from_numpy(ix.lengths).cuda()
    idx, logits = tks.indexer_select(_bf16(torch, ix.q), _bf16(torch, ix.kc), torch.from_numpy(ix.w).cuda(), k,
                                     lengths=L, return_logits=True)
    out = tks.sparse_attention(_bf16(torch, at.q), _bf16(torch, at.kc), _bf16(torch, at.vc), idx)
    assert tks.device_status() == 0
    idx_h = idx.cpu().numpy()
    assert np.array_equal(np.sort(idx_h, 1), np.sort(oracle.topk(logits.cpu().numpy(), k, ix.lengths), 1))
    assert_attention_close(at.q, at.kc, at.vc, idx_h, 1.0 / math.sqrt(128), out.cpu().numpy())


def test_graph_replay_of_indexer_and_attention(torch_gpu):
    """Both steps captured in one HIP graph and replayed, with eager work and
    synchronisations between replays: every replay gives the eager result."""
    import sparse_attention_topk_fp32_amd as tks

    torch = torch_gpu
    rows, n, k = 3, 9000, 256
    ix = W.draw(rows, n, heads=16, dim=64, k=k, seed=12, lengths="uniform")
    at = W.draw_attention(rows, n, heads=16, dim=64, k=k, seed=13)
    _say("graph replay x3: indexer selection then attention")
    q, kc, w = _bf16(torch, ix.q), _bf16(torch, ix.kc), torch.from_numpy(ix.w).cuda()
    L = torch.from_numpy(ix.lengths).cuda()
    aq, ak, av = _bf16(torch, at.q), _bf16(torch, at.kc), _bf16(torch, at.vc)
    idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    out = torch.zeros((rows, 16, 64), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        e_idx = tks.indexer_select(q, kc, w, k, lengths=L).clone()
        tks.sparse_attention(aq, ak, av, e_idx)  # allocates the scratch outside the capture
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            tks.indexer_select(q, kc, w, k, lengths=L, out=idx)
            tks.sparse_attention(aq, ak, av, idx, out=out)
    want_sets = torch.sort(e_idx, dim=1).values
    for rep in range(3):
        idx.fill_(-7)
        out.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.sort(idx, dim=1).values, want_sets), rep
        # the slot order may differ from the eager call (so may the rounding
        # of the chunked softmax): check each replay against the oracle
        assert_attention_close(at.q, at.kc, at.vc, idx.cpu().numpy(), 1.0 / math.sqrt(64), out.cpu().numpy())
        _ = tks.indexer_select(q, kc, w, k, lengths=L)
        torch.cuda.synchronize()
    assert tks.device_status(s) == 0
