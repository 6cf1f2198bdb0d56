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

