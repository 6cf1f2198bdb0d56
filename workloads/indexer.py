"""Seeded synthetic inputs of the indexer that produces the selector's logits.

The TopK article (section 01) lists the three steps of DSA-style decoding:
logits of the current query against every historical token, the TopK
selection, attention over the selected tokens.  These workloads feed the
first step: per query row, H indexer heads of dimension d (queries), one key
of dimension d per historical token, and one weight per head.  All values are
drawn here; nothing in this module computes logits or selects.

* queries q[r, h, :] ~ N(0, 1/d) per element, rounded to bf16;
* keys K[t, :] ~ N(0, 1) per element, rounded to bf16 (one key array per row,
  or one shared by every row);
* head weights w[r, h] ~ U(0, 1), float32;
* valid lengths as for the batched selector workload (uniform) or none.

With these scales each head's dot product is close to N(0, 1), so the logits
have the shape of the causal selector workload's values: a U(0,1)-weighted
sum of ReLU(N(0,1)) terms.  Row r draws from PCG64(SeedSequence([seed, r])),
the lengths from their own stream.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .synth import bf16_round

_LENGTH_STREAM = (1 << 32) + 1


@dataclass(frozen=True)
class IndexerConfig:
    name: str
    rows: int
    n: int
    heads: int
    dim: int
    k: int
    seed: int
    shared_keys: bool
    lengths: Optional[str]  # None | "uniform"
    note: str


INDEXER_CONFIGS = {
    c.name: c
    for c in [
        IndexerConfig("idx_b1_n128k_h64_d128", 1, 131072, 64, 128, 2048, 21, False, None,
                      "batch-1 decode: 1 query, 64 heads x 128, 131,072 keys of 128 (bf16)"),
        IndexerConfig("idx_b64_n16k_h64_d128_ragged", 64, 16384, 64, 128, 2048, 22, False, "uniform",
                      "batched decode: 64 queries, each with its own 16,384 keys, valid length U{2048..16384}"),
    ]
}


@dataclass
class IndexerWorkload:
    config: Optional[IndexerConfig]
    q: np.ndarray  # float32 [rows, H, d], bf16 values
    kc: np.ndarray  # float32 [n, d] (shared) or [rows, n, d], bf16 values
    w: np.ndarray  # float32 [rows, H]
    lengths: Optional[np.ndarray]  # int32 [rows] or None
    k: int


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def draw(rows: int, n: int, heads: int, dim: int, k: int, seed: int, shared_keys: bool = False,
         lengths: Optional[str] = None, config: Optional[IndexerConfig] = None) -> IndexerWorkload:
    """Draw an indexer workload of the given shape."""
    q = np.empty((rows, heads, dim), np.float32)
    w = np.empty((rows, heads), np.float32)
    kc = np.empty((n, dim) if shared_keys else (rows, n, dim), np.float32)
    scale = np.float32(1.0 / np.sqrt(dim))
    for r in range(rows):
        g = _rng(seed, r)
        q[r] = bf16_round(g.standard_normal((heads, dim), dtype=np.float32) * scale)
        w[r] = g.random(heads, dtype=np.float32)
        if not shared_keys:
            kc[r] = bf16_round(g.standard_normal((n, dim), dtype=np.float32))
    if shared_keys:
        kc[:] = bf16_round(_rng(seed, 1 << 31).standard_normal((n, dim), dtype=np.float32))
    L = None
    if lengths == "uniform":
        L = _rng(seed, _LENGTH_STREAM).integers(min(2048, max(1, n // 4)), n, size=rows, endpoint=True).astype(np.int32)
    return IndexerWorkload(config, q, kc, w, L, k)


def generate_indexer(name: str) -> IndexerWorkload:
    c = INDEXER_CONFIGS[name]
    return draw(c.rows, c.n, c.heads, c.dim, c.k, c.seed, c.shared_keys, c.lengths, c)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The bf16 bit patterns (uint16) of float32 values that are bf16 values."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)
