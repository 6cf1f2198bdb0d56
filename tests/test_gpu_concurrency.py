"""Several host threads, each enqueuing selections on a stream of its own at
the same time: calls are serialised on the host only while they enqueue, each
(device, stream) has its own workspace, and a row's workgroups wait only for
workgroups of their own launch, so the launches may overlap on the device in
any way.  Every result must be the oracle's set, byte-identical across the
repeats of a thread, with no device-side flag.  Each case prints its name
before touching the GPU."""

from __future__ import annotations

import sys
import threading

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg: str) -> None:
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def test_threads_on_their_own_streams():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_topk_fp32_amd as tks

    rng = np.random.default_rng(2024)
    cases = []
    # split rows (many WGs per row, waits between them), a ragged batch and a
    # one-WG-per-row batch
    for t in range(2):
        x = rng.standard_normal((1, 131072)).astype(np.float32)
        cases.append(("1x131072 seed %d" % t, x, None, 2048))
    c4 = W.generate("c4")
    cases.append(("c4 64x131072 ragged", c4.x, c4.lengths, c4.k))
    x = rng.standard_normal((512, 8192)).astype(np.float32)
    cases.append(("512x8192", x, None, 256))
    dev = []
    for name, x, lengths, k in cases:
        xd = torch.from_numpy(x).cuda()
        ld = None if lengths is None else torch.from_numpy(lengths).cuda()
        dev.append((xd, ld, k))
    iters = 8
    results = [[None] * iters for _ in cases]
    errors = []
    streams = [torch.cuda.Stream() for _ in cases]
    outs = [[torch.empty((x.shape[0], k), dtype=torch.int32, device="cuda") for _ in range(iters)]
            for (_, x, _, k) in cases]
    torch.cuda.synchronize()
    start = threading.Barrier(len(cases))

    def worker(i):
        try:
            xd, ld, k = dev[i]
            s = streams[i]
            start.wait()
            for it in range(iters):
                tks.select(xd, k, lengths=ld, out=outs[i][it], stream=s)
            s.synchronize()
            for it in range(iters):
                results[i][it] = outs[i][it].cpu().numpy()
        except Exception as e:  # reported below
            errors.append((i, repr(e)))

    _say("concurrency: %d threads x %d calls, one stream each" % (len(cases), iters))
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for i, (name, x, lengths, k) in enumerate(cases):
        assert tks.device_status(streams[i]) == 0, name
        want = np.sort(oracle.topk(x, k, lengths), 1)
        for it in range(iters):
            assert results[i][it] is not None, name
            assert results[i][it].tobytes() == results[i][0].tobytes(), "%s: repeat %d differs" % (name, it)
        assert np.array_equal(np.sort(results[i][0], 1), want), "%s differs from the oracle" % name
