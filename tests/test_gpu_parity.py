"""GPU parity: the HIP selector against the CPU oracle, element by element as
sorted index sets (bit-exact), on every workload and on the edge cases of the
method.  Each case prints its name before touching the GPU."""

from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import workloads as W
from tests.selection_checks import check_row_invariants, check_rows_vectorized

pytestmark = pytest.mark.gpu


def _say(msg: str) -> None:
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_topk_fp32_amd as tks

    tks.version()  # loads the library, raises when it is missing
    return torch


def run_gpu(torch, x: np.ndarray, k: int, lengths=None, offset: int = 0, variant=None, wgs=None, stream=None):
    """Copy x (rows, n) to the GPU starting `offset` floats into a buffer (to
    test unaligned rows), select, and return the host result."""
    import sparse_attention_topk_fp32_amd as tks

    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None]
    rows, n = x.shape
    buf = torch.empty(rows * n + offset + 4, dtype=torch.float32, device="cuda")
    view = buf[offset: offset + rows * n].view(rows, n)
    view.copy_(torch.from_numpy(x))
    lg = None if lengths is None else torch.from_numpy(np.asarray(lengths, np.int32)).cuda()
    out = tks.select(view, k, lengths=lg, variant=variant, wgs_per_row=wgs, stream=stream)
    flags = tks.device_status(stream)
    assert flags == 0, "device-side error flags raised: %d" % flags
    return out.cpu().numpy()


def assert_parity(x, k, lengths, got):
    want = oracle.topk(x, k, lengths)
    gs = np.sort(got, axis=1)
    ws = np.sort(want, axis=1)
    bad = np.nonzero((gs != ws).any(axis=1))[0]
    assert bad.size == 0, "rows differ from the oracle: %s (first: got %s... want %s...)" % (
        bad[:8].tolist(), gs[bad[0]][:8].tolist(), ws[bad[0]][:8].tolist())


# ----------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_workload_full_parity(torch_gpu, name):
    w = W.generate(name)
    _say("workload %s %s rows=%d n=%d" % (name, w.config.name, *w.x.shape))
    got = run_gpu(torch_gpu, w.x, w.k, w.lengths)
    assert_parity(w.x, w.k, w.lengths, got)
    check_rows_vectorized(w.x, w.lengths, w.k, got)


def test_workload_causal_4096_rows(torch_gpu):
    w = W.generate("c5")
    _say("workload c5 %s rows=%d n=%d (all rows on GPU)" % (w.config.name, *w.x.shape))
    got = run_gpu(torch_gpu, w.x, w.k, w.lengths)
    rng = np.random.default_rng(99)
    sample = np.unique(np.concatenate([[0, 1, 2047, 4094, 4095], rng.integers(0, 4096, size=27)]))
    assert_parity(w.x[sample], w.k, w.lengths[sample], got[sample])
    check_rows_vectorized(w.x, w.lengths, w.k, got)


@pytest.mark.parametrize("name", ["c4", "c5"])
def test_lengths_null_matches_minus_inf_tail(torch_gpu, name):
    """Past the valid length the workloads hold -inf; with every valid length
    >= 4096 > k those positions are never selected, so omitting `lengths`
    must give the same sets."""
    w = W.generate(name, rows=np.arange(0, W.config(name).rows, max(1, W.config(name).rows // 64)))
    _say("lengths NULL vs given, %s rows=%d" % (name, w.x.shape[0]))
    a = run_gpu(torch_gpu, w.x, w.k, w.lengths)
    b = run_gpu(torch_gpu, w.x, w.k, None)
    assert np.array_equal(np.sort(a, 1), np.sort(b, 1))


# ----------------------------------------------------------------- edge cases

def _edge_cases():
    rng = np.random.default_rng(2026)
    cases = []

    def add(name, x, k, lengths=None):
        cases.append(pytest.param(np.asarray(x, np.float32), k, lengths, id=name))

    for n in (1, 2, 3, 5, 7, 64):
        x = rng.standard_normal(n)
        for k in sorted({1, max(1, n // 2), n}):
            add("tiny_n%d_k%d" % (n, k), x, k)
    add("n1001_not_mult4", rng.standard_normal(1001), 100)
    add("n4099_k2048", rng.standard_normal(4099), 2048)
    add("k_equals_n", rng.standard_normal(5000), 5000)
    add("k_n_minus_1", rng.standard_normal(5000), 4999)
    add("k_5000_over_capacity", rng.standard_normal(16384), 5000)
    add("k_12000_over_capacity", rng.standard_normal(16384), 12000)
    x = rng.standard_normal((6, 3000))
    add("lengths_mixed", x, 2048, np.array([0, 1, 2047, 2048, 2049, 3000], np.int32))
    add("lengths_out_of_range", x[:3], 16, np.array([-7, 5000, 17], np.int32))
    add("all_equal_20000", np.full(20000, 0.5), 2048)
    add("all_equal_65536", np.full(65536, -3.0), 2048)
    add("all_minus_inf", np.full(10000, -np.inf), 2048)
    add("all_plus_inf", np.full(10000, np.inf), 100)
    v = rng.standard_normal(30000)
    v[rng.random(30000) < 0.3] = -np.inf
    v[rng.random(30000) < 0.01] = np.inf
    add("mixed_infinities", v, 2048)
    z = np.where(rng.random(20000) < 0.5, -0.0, 0.0)
    z[:100] = 1.0
    add("signed_zeros_at_threshold", z, 2048)
    d = np.array([1e-45, -1e-45, 3e-45, 0.0, -0.0], np.float32)[rng.integers(0, 5, 20000)]
    add("subnormals_at_threshold", d, 3000)
    add("ascending_ramp", np.arange(70000), 2048)
    add("descending_ramp", -np.arange(70000), 2048)
    # rows whose first chunks misrepresent the rest (a sampled estimate of
    # the threshold is far off): the exact fallback must take over
    add("descending_values_k30000", np.arange(70000, 0, -1), 30000)
    hi_head = rng.standard_normal(40000)
    hi_head[:6000] += 50.0
    add("large_values_first", hi_head, 2048)
    lo_head = rng.standard_normal(40000)
    lo_head[:6000] -= 50.0
    add("small_values_first", lo_head, 2048)
    # long rows (the ones that take the sampled window round)
    long_hi = rng.standard_normal(600000)
    long_hi[:1000] += 50.0  # fewer than k large values, all in the sample
    add("long_row_large_values_first", long_hi, 2048)
    add("long_row_descending_k300000", np.arange(600000, 0, -1), 300000)
    add("long_row_normal", rng.standard_normal(600000), 2048)
    # 256 distinct values, each 256 times: keys agree on their top 24 bits
    base = np.float32(1.0).view(np.uint32)
    add("top24_bits_shared", (base + (np.arange(65536) % 256).astype(np.uint32)).view(np.float32), 2048)
    add("bf16_quantized", W.bf16_round(rng.standard_normal(131072).astype(np.float32)), 2048)
    add("small_alphabet", rng.integers(-3, 4, 50000), 2048)
    add("multirow_small_alphabet", rng.integers(-2, 3, (8, 9000)), 1000)
    return cases


@pytest.mark.parametrize("x,k,lengths", _edge_cases())
def test_edge_case(torch_gpu, request, x, k, lengths):
    _say("edge %s shape=%s k=%d" % (request.node.callspec.id, x.shape, k))
    x2 = x if x.ndim == 2 else x[None]
    got = run_gpu(torch_gpu, x2, k, lengths)
    assert_parity(x2, k, lengths, got)
    for r in range(x2.shape[0]):
        L = x2.shape[1] if lengths is None else int(min(max(int(lengths[r]), 0), x2.shape[1]))
        check_row_invariants(x2[r], L, k, got[r])


def _one_wg_per_row_variants():
    import sparse_attention_topk_fp32_amd as tks

    return [v for v in range(tks.num_variants()) if tks.variant_info(v)["first_bits"] == 12]


@pytest.mark.parametrize("x,k,lengths", _edge_cases())
def test_edge_case_one_wg_per_row(torch_gpu, request, x, k, lengths):
    """The same edge cases through the one-WG-per-row kernels (12-bit first
    digit, streamed tiles)."""
    x2 = x if x.ndim == 2 else x[None]
    for v in _one_wg_per_row_variants():
        _say("edge %s variant %d" % (request.node.callspec.id, v))
        got = run_gpu(torch_gpu, x2, k, lengths, variant=v, wgs=1)
        assert_parity(x2, k, lengths, got)


@pytest.mark.parametrize("case", ["normal", "tie_storm"])
def test_rows_past_2_pow_24(torch_gpu, case):
    """A row longer than 2^24 (indices need all 32 index bits; the default
    shape streams it over many WGs): normal values, and a tie storm whose
    threshold is settled on the index digits."""
    rng = np.random.default_rng(24)
    n = (1 << 24) + 5
    if case == "normal":
        x = rng.standard_normal(n, dtype=np.float32)
    else:
        x = np.full(n, 1.5, np.float32)
        x[rng.integers(0, n, 700)] = 2.5
    _say("row past 2^24: n=%d case=%s" % (n, case))
    got = run_gpu(torch_gpu, x[None], 2048)
    assert_parity(x[None], 2048, None, got)
    for v in _one_wg_per_row_variants():
        _say("row past 2^24: case=%s variant %d (one WG)" % (case, v))
        got = run_gpu(torch_gpu, x[None], 2048, variant=v, wgs=1)
        assert_parity(x[None], 2048, None, got)


def _drifting_rows():
    """Rows whose first tile misjudges the bound of the one-WG-per-row
    kernels: a run of large values after a normal first tile (a tile that
    overflows the candidate buffer), a rising trend, a dense value band at
    the threshold (many elements in one 12-bit bin), a control row, and a
    falling trend (the first tile's bound is too high for the rest of the
    row: fewer than k elements end up buffered)."""
    rng = np.random.default_rng(2048)
    n = 65536
    x = rng.standard_normal((6, n)).astype(np.float32)
    x[0, 8192:4 * 8192] += 10.0
    x[1] += np.arange(n, dtype=np.float32) / 4000.0
    x[2, :] = 1.0 + rng.integers(0, 64, n).astype(np.float32) / 4096.0  # 64 values inside one 12-bit bin
    x[3, 8192:9000] += 10.0  # fewer than k large ones: the bound overshoots
    x[5] -= np.arange(n, dtype=np.float32) / 4000.0
    lengths = np.array([n, n, n, n, 50000, n], np.int32)
    return x, lengths


def test_drifting_rows_one_wg_per_row(torch_gpu):
    x, lengths = _drifting_rows()
    for v in _one_wg_per_row_variants():
        _say("drifting rows variant %d" % v)
        got = run_gpu(torch_gpu, x, 2048, lengths, variant=v, wgs=1)
        assert_parity(x, 2048, lengths, got)


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_unaligned_rows_one_wg_per_row(torch_gpu, offset):
    rng = np.random.default_rng(10 + offset)
    for rows, n in ((2, 70001), (3, 10001), (5, 4097)):
        x = rng.standard_normal((rows, n)).astype(np.float32)
        for v in _one_wg_per_row_variants():
            _say("unaligned offset=%d rows=%d n=%d variant %d" % (offset, rows, n, v))
            got = run_gpu(torch_gpu, x, 1024, offset=offset, variant=v, wgs=1)
            assert_parity(x, 1024, None, got)


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_unaligned_rows(torch_gpu, offset):
    rng = np.random.default_rng(offset)
    for rows, n in ((1, 131072), (3, 10001), (5, 4097)):
        x = rng.standard_normal((rows, n)).astype(np.float32)
        _say("unaligned offset=%d rows=%d n=%d" % (offset, rows, n))
        got = run_gpu(torch_gpu, x, 1024, offset=offset)
        assert_parity(x, 1024, None, got)


# ----------------------------------------------------------------- every kernel path

def _variant_shapes():
    import sparse_attention_topk_fp32_amd as tks

    out = []
    for v in range(tks.num_variants()):
        info = tks.variant_info(v)
        out.append((v, info))
    return out


@pytest.mark.parametrize("case", ["normal_131072", "ties_bf16_131072", "tie_storm_40000", "ragged_4rows"])
def test_every_variant_and_split(torch_gpu, case):
    import sparse_attention_topk_fp32_amd as tks

    rng = np.random.default_rng(len(case))
    lengths = None
    if case == "normal_131072":
        x = rng.standard_normal((1, 131072)).astype(np.float32)
    elif case == "ties_bf16_131072":
        x = W.bf16_round(rng.standard_normal((1, 131072)).astype(np.float32))
    elif case == "tie_storm_40000":
        x = np.full((1, 40000), 2.0, np.float32)
        x[0, rng.integers(0, 40000, 500)] = 3.0
    else:
        x = rng.standard_normal((4, 50000)).astype(np.float32)
        lengths = np.array([50000, 4097, 30001, 2000], np.int32)
    rows, n = x.shape
    k = 2048
    want = np.sort(oracle.topk(x, k, lengths), 1)
    ran = 0
    for v, info in _variant_shapes():
        per_wg = info["block"] * info["items"]
        gmin = -(-(n + 6) // per_wg) if info["resident"] else 1
        for G in sorted({gmin, gmin + 1, 2 * gmin, 8, 32}):
            if G < gmin:
                continue
            _say("variant %d %s G=%d case=%s" % (v, info, G, case))
            try:
                got = run_gpu(torch_gpu, x, k, lengths, variant=v, wgs=G)
            except tks.TopkSelectError as e:
                assert e.status == 1, e  # shape rejected (cannot cover the row / not co-resident)
                continue
            assert np.array_equal(np.sort(got, 1), want), (v, G, case)
            ran += 1
    assert ran >= 8


@pytest.mark.parametrize("shape", [None, (7, 32), (8, 64)])
def test_window_round_length_boundary(torch_gpu, shape):
    """Rows around the length from which the sampled 12-bit window round is
    taken (524,288), in a call long enough to compile it in: rows at, above
    and one below the boundary, with ties (bf16-rounded values)."""
    rng = np.random.default_rng(524288)
    n = 600000
    x = W.bf16_round(rng.standard_normal((3, n)).astype(np.float32))
    lengths = np.array([n, 524288, 524287], np.int32)
    variant, wgs = shape if shape is not None else (None, None)
    _say("window boundary rows=3 n=%d lengths=%s shape=%s" % (n, lengths.tolist(), shape))
    got = run_gpu(torch_gpu, x, 2048, lengths, variant=variant, wgs=wgs)
    assert_parity(x, 2048, lengths, got)
    _say("window boundary 1 x 524288, no lengths")
    got = run_gpu(torch_gpu, x[:1, :524288], 2048, None, variant=variant, wgs=wgs)
    assert_parity(x[:1, :524288], 2048, None, got)


# ----------------------------------------------------------------- calling conventions

@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_repeat_calls_are_deterministic(torch_gpu, name):
    """The output order is unspecified but fixed by the input and the launch
    shape: repeated calls write identical bytes."""
    import sparse_attention_topk_fp32_amd as tks

    w = W.generate(name)
    _say("repeat x20 on %s, byte equality" % w.config.name)
    x = torch_gpu.from_numpy(w.x).cuda()
    L = None if w.lengths is None else torch_gpu.from_numpy(w.lengths).cuda()
    first = tks.select(x, w.k, lengths=L)
    for _ in range(20):
        again = tks.select(x, w.k, lengths=L)
        assert torch_gpu.equal(again, first)
    assert tks.device_status() == 0
    assert_parity(w.x, w.k, w.lengths, first.cpu().numpy())


def test_repeat_calls_are_deterministic_many_rows(torch_gpu):
    """The one-WG-per-row kernel (many rows), repeated: identical bytes."""
    import sparse_attention_topk_fp32_amd as tks

    w = W.generate("c5", rows=np.arange(0, 4096, 8))
    _say("repeat x5 on 512 causal rows, byte equality")
    x = torch_gpu.from_numpy(w.x).cuda()
    L = torch_gpu.from_numpy(w.lengths).cuda()
    first = tks.select(x, w.k, lengths=L)
    for _ in range(5):
        assert torch_gpu.equal(tks.select(x, w.k, lengths=L), first)
    assert tks.device_status() == 0


def test_single_workgroup_rows_repeat(torch_gpu):
    """One streaming workgroup per row (the path for rows too long to keep on
    chip), repeated: identical bytes every time."""
    import sparse_attention_topk_fp32_amd as tks

    w = W.generate("c5", rows=np.arange(64))
    _say("identical bytes x5, one streaming WG per row")
    x = torch_gpu.from_numpy(w.x).cuda()
    L = torch_gpu.from_numpy(w.lengths).cuda()
    v = next(v for v in range(tks.num_variants())
             if not tks.variant_info(v)["resident"])  # one streaming WG covers any row
    first = tks.select(x, w.k, lengths=L, variant=v, wgs_per_row=1)
    for _ in range(5):
        again = tks.select(x, w.k, lengths=L, variant=v, wgs_per_row=1)
        assert torch_gpu.equal(again, first)
    assert_parity(w.x, w.k, w.lengths, first.cpu().numpy())


def test_non_default_stream_and_preallocated_out(torch_gpu):
    import sparse_attention_topk_fp32_amd as tks

    torch = torch_gpu
    w = W.generate("c4", rows=np.arange(16))
    _say("side stream, preallocated out")
    s = torch.cuda.Stream()
    x = torch.from_numpy(w.x).cuda()
    L = torch.from_numpy(w.lengths).cuda()
    out = torch.full((16, w.k), 7, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        r = tks.select(x, w.k, lengths=L, out=out)
    assert r.data_ptr() == out.data_ptr()
    s.synchronize()
    assert tks.device_status(s) == 0
    assert_parity(w.x, w.k, w.lengths, out.cpu().numpy())


def test_zero_rows_and_one_dim_input(torch_gpu):
    import sparse_attention_topk_fp32_amd as tks

    torch = torch_gpu
    _say("rows=0 and 1-D input")
    out = tks.select(torch.empty((0, 100), device="cuda"), 10)
    assert out.shape == (0, 10)
    x = np.random.default_rng(1).standard_normal(3000).astype(np.float32)
    got = tks.select(torch.from_numpy(x).cuda(), 50).cpu().numpy()
    assert sorted(got.tolist()) == sorted(oracle.topk(x, 50)[0].tolist())


def test_invalid_arguments_enqueue_nothing(torch_gpu):
    import sparse_attention_topk_fp32_amd as tks

    torch = torch_gpu
    _say("invalid arguments")
    x = torch.randn(2, 100, device="cuda")
    out = torch.full((2, 101), 5, dtype=torch.int32, device="cuda")
    with pytest.raises(tks.TopkSelectError):
        tks.select(x, 101, out=out)
    with pytest.raises(tks.TopkSelectError):
        tks.select(x, 0)
    torch.cuda.synchronize()
    assert int((out != 5).sum()) == 0


def test_graph_replay_matches_eager(torch_gpu):
    """The benchmark replays captured launches: every replay, with eager work
    and synchronisations in between, must give the eager result."""
    import sparse_attention_topk_fp32_amd as tks

    torch = torch_gpu
    _say("graph replay x4 (batch-1 row and 64 ragged rows)")
    for name in ("c2", "c4"):
        w = W.generate(name)
        x = torch.from_numpy(w.x).cuda()
        L = None if w.lengths is None else torch.from_numpy(w.lengths).cuda()
        s = torch.cuda.Stream()
        out = torch.full((w.x.shape[0], w.k), -7, dtype=torch.int32, device="cuda")
        with torch.cuda.stream(s):
            eager = tks.select(x, w.k, lengths=L).clone()
            s.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                tks.select(x, w.k, lengths=L, out=out)
        for rep in range(4):
            out.fill_(-7)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), (name, rep)
            _ = tks.select(x, w.k, lengths=L)  # eager work between replays
            torch.cuda.synchronize()
        assert tks.device_status(s) == 0
        assert_parity(w.x, w.k, w.lengths, out.cpu().numpy())


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_graph_survives_workspace_growth(torch_gpu):
    """A graph keeps the buffers it was captured with: a first call inside a
    capture (no workspace yet) is refused with the capture error and
    enqueues nothing; after an eager warm-up, a captured call keeps giving
    the eager result even after a larger eager call on the same stream has
    grown the workspace (the old buffers are retired, not freed)."""
    import sparse_attention_topk_fp32_amd as tks

    torch = torch_gpu
    _say("graph capture: refused first call, growth between replays")
    tks.release_workspace()
    w1, w4 = W.generate("c2"), W.generate("c4")
    x1 = torch.from_numpy(w1.x).cuda()
    x4 = torch.from_numpy(w4.x).cuda()
    L4 = torch.from_numpy(w4.lengths).cuda()
    out1 = torch.full((1, w1.k), -7, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g0 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with pytest.raises(tks.TopkSelectError):
            with torch.cuda.graph(g0, stream=s):
                tks.select(x1, w1.k, out=out1)
    torch.cuda.synchronize()
    assert int((out1 != -7).sum()) == 0
    with torch.cuda.stream(s):
        eager = tks.select(x1, w1.k).clone()
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            tks.select(x1, w1.k, out=out1)
        big = tks.select(x4, w4.k, lengths=L4)  # 64 rows: the row table and the stage grow
    torch.cuda.synchronize()
    assert_parity(w4.x, w4.k, w4.lengths, big.cpu().numpy())
    for rep in range(3):
        out1.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out1, eager), rep
    assert tks.device_status(s) == 0
    assert_parity(w1.x, w1.k, None, out1.cpu().numpy())


def test_workspace_reuse_across_row_counts(torch_gpu):
    """Calls with different row counts reuse one workspace: per-row scratch
    must never be overlapped by another call's staging area (a one-row split
    call followed by a many-row split call once left row 1 dirty)."""
    import sparse_attention_topk_fp32_amd as tks

    _say("workspace reuse: 1 row, 8 rows, 1 row (big k), 8 rows")
    tks.release_workspace()
    rng = np.random.default_rng(77)
    one = rng.standard_normal((1, 131072)).astype(np.float32)
    eight = rng.integers(-2, 3, (8, 9000)).astype(np.float32)
    for x, k in ((one, 2048), (eight, 1000), (one, 9000), (eight, 1000), (eight[:3], 16)):
        got = run_gpu(torch_gpu, x, k)
        assert_parity(x, k, None, got)


def test_stream_read_runs(torch_gpu):
    """The bandwidth yardstick: a plain streaming read launches and leaves
    the sink alone on ordinary data."""
    import sparse_attention_topk_fp32_amd as tks

    _say("stream_read 64 MiB")
    buf = torch_gpu.ones(16 << 20, dtype=torch_gpu.float32, device="cuda")
    sink = torch_gpu.full((1,), 7, dtype=torch_gpu.int32, device="cuda")
    tks.stream_read(buf, sink)
    torch_gpu.cuda.synchronize()
    assert int(sink.item()) == 7
