"""The bounded wait's give-up path, forced from the host in a test build
(libtopk_select_hooks.so: the same source with TKS_TEST_HOOKS, whose wait
bound the host can set).  With the bound at 0 every finishing workgroup gives
up before its first poll: it raises flag 1 and finishes its row by passes over
the logits, so the output is still exact and every kernel ends normally.
topk_select_device_status then reports flag 1 and clears the workspace (late
counts and candidates of the other workgroups), and the next call with the
normal bound is exact.  Each case prints its name before touching the GPU."""

from __future__ import annotations

import ctypes
import os
import sys

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

HOOKS = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "sparse_attention_topk_fp32_amd",
                     "libtopk_select_hooks.so")
DEFAULT_LIMIT = 200000000  # 2 s of the 100 MHz constant clock


def _say(msg: str) -> None:
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def hooks():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(HOOKS):
        pytest.fail("the test build is missing: run python -m sparse_attention_topk_fp32_amd.build")
    lib = ctypes.CDLL(HOOKS)
    P, I = ctypes.c_void_p, ctypes.c_int32
    lib.topk_select.argtypes = [P, I, I, P, I, P, P]
    lib.topk_select.restype = ctypes.c_int
    lib.topk_select_device_status.argtypes = [P, ctypes.POINTER(ctypes.c_int32)]
    lib.topk_select_device_status.restype = ctypes.c_int
    lib.topk_select_test_set_spin_limit.argtypes = [ctypes.c_uint64]
    lib.topk_select_test_set_spin_limit.restype = ctypes.c_int
    yield torch, lib
    lib.topk_select_test_set_spin_limit(DEFAULT_LIMIT)


def _run(torch, lib, w, stream):
    rows, n = w.x.shape
    x = torch.from_numpy(w.x).cuda()
    lg = None if w.lengths is None else torch.from_numpy(w.lengths).cuda()
    out = torch.full((rows, w.k), -7, dtype=torch.int32, device="cuda")
    rc = lib.topk_select(x.data_ptr(), rows, n, None if lg is None else lg.data_ptr(), w.k, out.data_ptr(),
                         stream.cuda_stream)
    assert rc == 0
    flags = ctypes.c_int32(-1)
    st = lib.topk_select_device_status(stream.cuda_stream, ctypes.byref(flags))
    return out.cpu().numpy(), st, flags.value


def _exact(w, got):
    want = oracle.topk(w.x, w.k, w.lengths)
    assert np.array_equal(np.sort(got, 1), np.sort(want, 1)), "output differs from the oracle"


@pytest.mark.parametrize("name", ["c2", "c4"])
def test_waits_that_give_up_still_select_exactly(hooks, name):
    torch, lib = hooks
    w = W.generate(name)
    stream = torch.cuda.Stream()
    _say("give-up %s rows=%d n=%d: wait bound 0" % (name, *w.x.shape))
    assert lib.topk_select_test_set_spin_limit(0) == 0
    got, st, flags = _run(torch, lib, w, stream)
    assert st == 5 and flags == 1, (st, flags)  # DEVICE_FLAG, timeout flag only
    _exact(w, got)
    _say("give-up %s: normal bound again after device_status cleared the workspace" % name)
    assert lib.topk_select_test_set_spin_limit(DEFAULT_LIMIT) == 0
    for _ in range(3):
        got, st, flags = _run(torch, lib, w, stream)
        assert st == 0 and flags == 0, (st, flags)
        _exact(w, got)


def test_indexer_candidates_give_up_still_select_exactly(hooks):
    """topk_indexer_select_fused with the wait bound at 0: its
    tile workgroups give up waiting for the row's bound and mark their
    counts, every kernel still ends, flag 1 is raised, and the finishing
    workgroup selects the row by passes over the logits, exactly.  After
    device_status, calls with the normal bound are exact."""
    torch, lib = hooks
    P, I = ctypes.c_void_p, ctypes.c_int32
    lib.topk_indexer_select_fused.argtypes = [P, P, P, I, I, I, I, ctypes.c_int64, P, I, P, P, P]
    lib.topk_indexer_select_fused.restype = ctypes.c_int
    wl = W.generate_indexer("idx_b1_n128k_h64_d128")
    rows, H, d = wl.q.shape
    n = wl.kc.shape[-2]
    q = torch.from_numpy(wl.q).cuda().to(torch.bfloat16)
    kc = torch.from_numpy(wl.kc).cuda().to(torch.bfloat16)
    w = torch.from_numpy(wl.w).cuda()
    stream = torch.cuda.Stream()

    def call():
        out = torch.full((rows, wl.k), -7, dtype=torch.int32, device="cuda")
        lg = torch.empty((rows, n), dtype=torch.float32, device="cuda")
        rc = lib.topk_indexer_select_fused(q.data_ptr(), kc.data_ptr(), w.data_ptr(), rows, n, H, d, n * d, None, wl.k,
                                     out.data_ptr(), lg.data_ptr(), stream.cuda_stream)
        assert rc == 0
        flags = ctypes.c_int32(-1)
        st = lib.topk_select_device_status(stream.cuda_stream, ctypes.byref(flags))
        return out.cpu().numpy(), lg.cpu().numpy(), st, flags.value

    _say("give-up indexer %s: normal bound" % wl.config.name)
    _, lg_ref, st, flags = call()
    assert st == 0 and flags == 0, (st, flags)
    _say("give-up indexer: wait bound 0")
    assert lib.topk_select_test_set_spin_limit(0) == 0
    got, lg, st, flags = call()
    assert st == 5 and flags == 1, (st, flags)
    assert np.array_equal(lg.view(np.uint32), lg_ref.view(np.uint32)), "logits differ after the give-up"
    want = oracle.topk(lg_ref, wl.k, None)
    assert np.array_equal(np.sort(got, 1), np.sort(want, 1)), "output differs from the oracle"
    _say("give-up indexer: normal bound again after device_status cleared the workspace")
    assert lib.topk_select_test_set_spin_limit(DEFAULT_LIMIT) == 0
    for _ in range(3):
        got, lg, st, flags = call()
        assert st == 0 and flags == 0, (st, flags)
        assert np.array_equal(np.sort(got, 1), np.sort(want, 1)), "output differs from the oracle"
