"""Seeded synthetic indexer-logit workloads.

The TopK selector article ("How to Use FlagOS's New Triton-TLE Language to
Build a TopK Selector Faster Than FlashInfer") measures the selector on DSA
indexer logits: one query row at sequence lengths 131072 and 262144 (up to
512K) for batch 1, and 64 rows for the batched case (its results 2 and 3).  No
dataset is involved; the five workloads below stand in for those logits with
the shapes, value distributions and valid-length structure stated next to
each.  Every value is a pure function of (workload seed, row): row ``r`` draws
from its own ``numpy`` PCG64 stream seeded with ``SeedSequence([seed, r])``, so
any single row can be regenerated alone (the oracle's sampled checks rely on
that) and rows can be generated in parallel.

Nothing in this module selects, ranks or compares logits.
"""

from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

K_DEFAULT = 2048
_LENGTH_STREAM = (1 << 32) + 1  # SeedSequence entropy word for per-row lengths


@dataclass(frozen=True)
class Config:
    name: str
    rows: int
    n: int
    k: int
    seed: int
    values: str  # "normal" | "normal_bf16" | "outlier_bf16" | "relu_mix8"
    lengths: Optional[str]  # None (all valid) | "uniform" | "causal"
    note: str


CONFIGS = {
    c.name: c
    for c in [
        Config("b1_n16k_normal", 1, 16384, K_DEFAULT, 1, "normal", None,
               "1 row x 16,384, fp32 N(0,1)"),
        Config("b1_n128k_bf16", 1, 131072, K_DEFAULT, 2, "normal_bf16", None,
               "1 row x 131,072, N(0,1) rounded to bf16 (RNE) then widened: "
               "many exact ties; the batch-1 decode latency case"),
        Config("b1_n1m_outlier_bf16", 1, 1 << 20, K_DEFAULT, 3, "outlier_bf16", None,
               "1 row x 1,048,576, 99% N(0,1) + 1% N(6,1) outliers, bf16-rounded"),
        Config("b64_n128k_ragged", 64, 131072, K_DEFAULT, 4, "normal", "uniform",
               "64 rows x 131,072, fp32 N(0,1), valid length U{4096..131072}, "
               "-inf past it"),
        Config("b4096_n64k_causal_relu8", 4096, 65536, K_DEFAULT, 5, "relu_mix8", "causal",
               "4,096 rows x 65,536, valid length 61,440 + r (causal), values "
               "sum_j w[r][j]*ReLU(z_j) over 8 draws, w ~ U(0,1) per row, -inf past it"),
    ]
}

# Short aliases used by the tests and the bench command line.
ALIASES = {
    "c1": "b1_n16k_normal",
    "c2": "b1_n128k_bf16",
    "c3": "b1_n1m_outlier_bf16",
    "c4": "b64_n128k_ragged",
    "c5": "b4096_n64k_causal_relu8",
}


def config(name: str) -> Config:
    return CONFIGS[ALIASES.get(name, name)]


@dataclass
class Workload:
    config: Config
    x: np.ndarray  # float32 [rows, n], C-contiguous
    lengths: Optional[np.ndarray]  # int32 [rows] or None
    row_ids: np.ndarray  # int64 [rows]: which rows of the full workload these are

    @property
    def k(self) -> int:
        return self.config.k


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned
    widened back to float32.  Inputs must be finite (all generated values are)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def lengths_for(cfg: Config) -> Optional[np.ndarray]:
    """Per-row valid lengths of the full workload (int32), or None when every
    position of every row is valid."""
    if cfg.lengths is None:
        return None
    if cfg.lengths == "uniform":
        g = _rng(cfg.seed, _LENGTH_STREAM)
        return g.integers(4096, 131072, size=cfg.rows, endpoint=True).astype(np.int32)
    if cfg.lengths == "causal":
        return (61440 + np.arange(cfg.rows, dtype=np.int64)).astype(np.int32)
    raise ValueError(cfg.lengths)


def gen_row(cfg: Config, r: int, length: Optional[int] = None, out: Optional[np.ndarray] = None):
    """Row ``r`` of the workload as float32 [n]; positions >= length are -inf."""
    n = cfg.n
    L = n if length is None else int(length)
    row = np.empty(n, dtype=np.float32) if out is None else out
    g = _rng(cfg.seed, r)
    if cfg.values == "normal":
        v = g.standard_normal(L, dtype=np.float32)
    elif cfg.values == "normal_bf16":
        v = bf16_round(g.standard_normal(L, dtype=np.float32))
    elif cfg.values == "outlier_bf16":
        z = g.standard_normal(L, dtype=np.float32)
        is_outlier = g.random(L) < 0.01
        v = bf16_round(np.where(is_outlier, z + np.float32(6.0), z).astype(np.float32))
    elif cfg.values == "relu_mix8":
        w = g.random(8, dtype=np.float32)
        z = g.standard_normal((8, L), dtype=np.float32)
        v = np.zeros(L, dtype=np.float32)
        for j in range(8):  # fp32 multiply then fp32 add, j = 0..7, no fused multiply-add
            v = v + w[j] * np.maximum(z[j], np.float32(0.0))
    else:
        raise ValueError(cfg.values)
    row[:L] = v
    row[L:] = -np.inf
    return row


def generate(name: str, rows=None, threads: Optional[int] = None) -> Workload:
    """Generate the workload (all rows, or the listed row ids)."""
    cfg = config(name)
    row_ids = np.arange(cfg.rows, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    all_lengths = lengths_for(cfg)
    lengths = None if all_lengths is None else np.ascontiguousarray(all_lengths[row_ids])
    x = np.empty((len(row_ids), cfg.n), dtype=np.float32)

    def work(lo_hi):
        lo, hi = lo_hi
        for i in range(lo, hi):
            L = None if lengths is None else int(lengths[i])
            gen_row(cfg, int(row_ids[i]), L, out=x[i])

    nrow = len(row_ids)
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    threads = max(1, min(threads, nrow))
    step = (nrow + threads - 1) // threads
    parts = [(i, min(nrow, i + step)) for i in range(0, nrow, step)]
    if len(parts) == 1:
        work(parts[0])
    else:
        with ThreadPoolExecutor(len(parts)) as ex:
            list(ex.map(work, parts))
    return Workload(cfg, x, lengths, row_ids)


def sha256_of(w: Workload) -> str:
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(w.x).tobytes())
    if w.lengths is not None:
        h.update(np.ascontiguousarray(w.lengths).tobytes())
    return h.hexdigest()
