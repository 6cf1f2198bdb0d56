"""GPU parity of the ordered selection (``topk_select_sorted``): indices in
(value descending, index ascending) order and the selected values, compared
with the oracle's ordered output element by element (bit-exact), on the
workloads, the edge cases and every selection kernel path.  Each case prints
its name before touching the GPU."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from tests.selection_checks import check_row_order
from tests.test_gpu_parity import _edge_cases, _one_wg_per_row_variants, _say, _variant_shapes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_topk_fp32_amd as tks

    tks.version()
    return torch


def run_sorted(torch, x, k, lengths=None, variant=None, wgs=None, values=True):
    import sparse_attention_topk_fp32_amd as tks

    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None]
    xd = torch.from_numpy(x).cuda()
    lg = None if lengths is None else torch.from_numpy(np.asarray(lengths, np.int32)).cuda()
    r = tks.select_sorted(xd, k, lengths=lg, return_values=values, variant=variant, wgs_per_row=wgs)
    flags = tks.device_status()
    assert flags == 0, "device-side error flags raised: %d" % flags
    if values:
        return r[0].cpu().numpy(), r[1].cpu().numpy()
    return r.cpu().numpy(), None


def assert_sorted_parity(x, k, lengths, idx, vals):
    want_idx, want_val = oracle.topk_sorted(x, k, lengths)
    bad = np.nonzero((idx != want_idx).any(axis=1))[0]
    assert bad.size == 0, "rows differ from the oracle: %s (first: got %s... want %s...)" % (
        bad[:8].tolist(), idx[bad[0]][:8].tolist(), want_idx[bad[0]][:8].tolist())
    if vals is not None:
        assert np.array_equal(vals.view(np.uint32), want_val.view(np.uint32)), "values differ from the oracle"


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_sorted_workload_parity(torch_gpu, name):
    w = W.generate(name)
    _say("sorted workload %s rows=%d n=%d" % (name, *w.x.shape))
    idx, vals = run_sorted(torch_gpu, w.x, w.k, w.lengths)
    assert_sorted_parity(w.x, w.k, w.lengths, idx, vals)


def test_sorted_causal_4096_rows(torch_gpu):
    """Every one of the 4,096 rows against the oracle (rows split over host
    threads; the oracle's C loop runs outside the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    w = W.generate("c5")
    _say("sorted workload c5 rows=%d n=%d (all rows on GPU, all rows checked)" % w.x.shape)
    idx, vals = run_sorted(torch_gpu, w.x, w.k, w.lengths)
    bounds = np.linspace(0, w.x.shape[0], 17).astype(int)

    def check(ab):
        a, b = ab
        assert_sorted_parity(w.x[a:b], w.k, w.lengths[a:b], idx[a:b], vals[a:b])

    with ThreadPoolExecutor(max_workers=16) as ex:
        list(ex.map(check, zip(bounds[:-1], bounds[1:])))
    rng = np.random.default_rng(5)
    for r in rng.integers(0, 4096, size=16):
        check_row_order(w.x[r], int(w.lengths[r]), w.k, idx[r], vals[r])


@pytest.mark.parametrize("x,k,lengths", _edge_cases())
def test_sorted_edge_case(torch_gpu, request, x, k, lengths):
    _say("sorted edge %s shape=%s k=%d" % (request.node.callspec.id, x.shape, k))
    x2 = x if x.ndim == 2 else x[None]
    idx, vals = run_sorted(torch_gpu, x2, k, lengths)
    assert_sorted_parity(x2, k, lengths, idx, vals)


@pytest.mark.parametrize("x,k,lengths", _edge_cases())
def test_sorted_edge_case_one_wg_per_row(torch_gpu, request, x, k, lengths):
    x2 = x if x.ndim == 2 else x[None]
    for v in _one_wg_per_row_variants():
        _say("sorted edge %s variant %d" % (request.node.callspec.id, v))
        idx, vals = run_sorted(torch_gpu, x2, k, lengths, variant=v, wgs=1)
        assert_sorted_parity(x2, k, lengths, idx, vals)


def test_sorted_drifting_rows_one_wg_per_row(torch_gpu):
    from tests.test_gpu_parity import _drifting_rows

    x, lengths = _drifting_rows()
    for v in _one_wg_per_row_variants():
        _say("sorted drifting rows variant %d" % v)
        idx, vals = run_sorted(torch_gpu, x, 2048, lengths, variant=v, wgs=1)
        assert_sorted_parity(x, 2048, lengths, idx, vals)


@pytest.mark.parametrize("case", ["ties_bf16_131072", "tie_storm_40000", "ragged_4rows"])
def test_sorted_every_variant_and_split(torch_gpu, case):
    """Every selection kernel path records the keys the sort uses."""
    import sparse_attention_topk_fp32_amd as tks

    rng = np.random.default_rng(len(case) + 100)
    lengths = None
    if case == "ties_bf16_131072":
        x = W.bf16_round(rng.standard_normal((1, 131072)).astype(np.float32))
    elif case == "tie_storm_40000":
        x = np.full((1, 40000), 2.0, np.float32)
        x[0, rng.integers(0, 40000, 500)] = 3.0
    else:
        x = rng.standard_normal((4, 50000)).astype(np.float32)
        lengths = np.array([50000, 4097, 30001, 2000], np.int32)
    rows, n = x.shape
    k = 2048
    ran = 0
    for v, info in _variant_shapes():
        per_wg = info["block"] * info["items"]
        gmin = -(-(n + 6) // per_wg) if info["resident"] else 1
        for G in sorted({gmin, 2 * gmin, 8}):
            if G < gmin:
                continue
            _say("sorted variant %d G=%d case=%s" % (v, G, case))
            try:
                idx, vals = run_sorted(torch_gpu, x, k, lengths, variant=v, wgs=G)
            except tks.TopkSelectError as e:
                assert e.status == 1, e
                continue
            assert_sorted_parity(x, k, lengths, idx, vals)
            ran += 1
    assert ran >= 8


@pytest.mark.parametrize("k", [1, 64, 1000, 1024, 1025, 2048, 4096, 4097, 8192, 8193, 16384, 40000])
def test_sorted_k_sizes(torch_gpu, k):
    """Every sort shape: one on-chip sort of 1K, 2K, 4K or 8K entries, and
    runs of 8K merged in one or more passes."""
    rng = np.random.default_rng(k)
    x = W.bf16_round(rng.standard_normal((3, 50000)).astype(np.float32))
    lengths = np.array([50000, k // 2, 31000], np.int32)
    _say("sorted k=%d rows=3 n=50000" % k)
    idx, vals = run_sorted(torch_gpu, x, k, lengths)
    assert_sorted_parity(x, k, lengths, idx, vals)


@pytest.mark.parametrize("k", [16, 1000, 1025, 2048, 4096])
def test_sorted_k_sizes_many_rows(torch_gpu, k):
    """Many rows: one sorting WG per row (the few-row calls above take the
    ranking kernel for k <= 4096)."""
    rng = np.random.default_rng(k + 7)
    rows = 40 if k > 16 else 200000
    n = 6000 if k > 16 else 40
    x = W.bf16_round(rng.standard_normal((rows, n)).astype(np.float32))
    lengths = rng.integers(0, n + 1, size=rows).astype(np.int32)
    _say("sorted k=%d rows=%d n=%d" % (k, rows, n))
    idx, vals = run_sorted(torch_gpu, x, k, lengths)
    sample = np.arange(0, rows, max(1, rows // 64))
    assert_sorted_parity(x[sample], k, lengths[sample], idx[sample], vals[sample])


def test_sorted_indices_only_and_repeat(torch_gpu):
    w = W.generate("c2")
    _say("sorted indices only, repeated x10")
    idx0, vals = run_sorted(torch_gpu, w.x, w.k)
    for _ in range(10):
        idx, none = run_sorted(torch_gpu, w.x, w.k, values=False)
        assert none is None
        assert np.array_equal(idx, idx0)  # the order is fully determined


def test_sorted_graph_replay_matches_eager(torch_gpu):
    import sparse_attention_topk_fp32_amd as tks

    torch = torch_gpu
    _say("sorted graph replay x3 (batch-1 row and 64 ragged rows)")
    for name in ("c2", "c4"):
        w = W.generate(name)
        x = torch.from_numpy(w.x).cuda()
        L = None if w.lengths is None else torch.from_numpy(w.lengths).cuda()
        s = torch.cuda.Stream()
        out = torch.full((w.x.shape[0], w.k), -7, dtype=torch.int32, device="cuda")
        val = torch.zeros((w.x.shape[0], w.k), dtype=torch.float32, device="cuda")
        with torch.cuda.stream(s):
            e_idx, e_val = tks.select_sorted(x, w.k, lengths=L, return_values=True)
            e_idx, e_val = e_idx.clone(), e_val.clone()
            s.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                tks.select_sorted(x, w.k, lengths=L, out=out, out_values=val)
        for rep in range(3):
            out.fill_(-7)
            val.fill_(0.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, e_idx), (name, rep)
            assert torch.equal(val.view(torch.int32), e_val.view(torch.int32)), (name, rep)
            _ = tks.select_sorted(x, w.k, lengths=L)
            torch.cuda.synchronize()
        assert tks.device_status(s) == 0
        assert_sorted_parity(w.x, w.k, w.lengths, out.cpu().numpy(), val.cpu().numpy())


def test_sorted_values_keep_the_sign_of_zero(torch_gpu):
    x = np.zeros(5000, np.float32)
    x[::2] = -0.0
    x[:10] = 1.0
    _say("sorted signed zeros, k=100")
    idx, vals = run_sorted(torch_gpu, x[None], 100)
    assert_sorted_parity(x[None], 100, None, idx, vals)
    assert (vals[0, 10:].view(np.uint32) == 0x80000000).sum() == 45
