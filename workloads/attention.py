"""Seeded synthetic inputs of the attention that consumes the selection.

The TopK article (section 01) names the third DSA step: attention computed
only on the keys and values of the k selected positions.  These workloads
feed it: per query row, H attention heads of dimension d (queries), one key
and one value of dimension d per historical token (shared by the heads),
and the k selected positions.  The positions are drawn here (k distinct
valid positions per row in random order, -1 in the slots past a short row's
valid length), not computed by a selection: nothing in this module scores,
selects or attends.

* q[r, h, :], K[t, :], V[t, :] ~ N(0, 1) per element, rounded to bf16;
* valid lengths U{1024..n} (rows shorter than k get -1 slots) or none.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .synth import bf16_round

_LENGTH_STREAM = (1 << 32) + 1


@dataclass(frozen=True)
class AttentionConfig:
    name: str
    rows: int
    n: int
    heads: int
    dim: int
    k: int
    seed: int
    lengths: Optional[str]
    note: str


ATTENTION_CONFIGS = {
    c.name: c
    for c in [
        AttentionConfig("att_b1_n128k_h16_d128_k2048", 1, 131072, 16, 128, 2048, 31, None,
                        "batch-1 decode: 1 query of 16 heads x 128 over 2,048 of 131,072 keys/values"),
        AttentionConfig("att_b64_n16k_h16_d128_k2048_ragged", 64, 16384, 16, 128, 2048, 32, "uniform",
                        "64 queries, each with its own 16,384 keys/values, valid length U{1024..16384}"),
    ]
}


@dataclass
class AttentionWorkload:
    config: Optional[AttentionConfig]
    q: np.ndarray  # float32 [rows, H, d], bf16 values
    kc: np.ndarray  # float32 [rows, n, d] or [n, d], bf16 values
    vc: np.ndarray  # same shape as kc
    idx: np.ndarray  # int32 [rows, k]
    lengths: Optional[np.ndarray]


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def draw_attention(rows: int, n: int, heads: int, dim: int, k: int, seed: int, shared_kv: bool = False,
                   lengths: Optional[str] = None, config: Optional[AttentionConfig] = None) -> AttentionWorkload:
    L = np.full(rows, n, np.int64)
    if lengths == "uniform":
        L = _rng(seed, _LENGTH_STREAM).integers(min(1024, n), n, size=rows, endpoint=True)
    q = np.empty((rows, heads, dim), np.float32)
    shape = (n, dim) if shared_kv else (rows, n, dim)
    kc = np.empty(shape, np.float32)
    vc = np.empty(shape, np.float32)
    idx = np.full((rows, k), -1, np.int32)
    for r in range(rows):
        g = _rng(seed, r)
        q[r] = bf16_round(g.standard_normal((heads, dim), dtype=np.float32))
        if not shared_kv:
            kc[r] = bf16_round(g.standard_normal((n, dim), dtype=np.float32))
            vc[r] = bf16_round(g.standard_normal((n, dim), dtype=np.float32))
        take = int(min(k, L[r]))
        idx[r, :take] = g.choice(int(L[r]), size=take, replace=False)
    if shared_kv:
        g = _rng(seed, 1 << 31)
        kc[:] = bf16_round(g.standard_normal((n, dim), dtype=np.float32))
        vc[:] = bf16_round(g.standard_normal((n, dim), dtype=np.float32))
    return AttentionWorkload(config, q, kc, vc, idx, None if lengths is None else L.astype(np.int32))


def generate_attention(name: str) -> AttentionWorkload:
    c = ATTENTION_CONFIGS[name]
    return draw_attention(c.rows, c.n, c.heads, c.dim, c.k, c.seed, False, c.lengths, c)
