"""Seeded synthetic score rows shaped like the indexer's selection workload.

This module only draws random numbers.  It holds none of the selection
arithmetic, imports neither the GPU binding nor the oracle, and is the one
piece of code both sides' callers share.

The rows stand in for indexer scores over a 16K-1M token context ("The Secret
GPU Kernel Behind DeepSeek V4.1 Flash", transcript 1:48-3:05: each indexer
query scores every cached position and 512 are kept; the built-in selection
is measured from 16,000 to a million scores).  No public dataset or trained
weights are involved.  Every array is drawn in float64 with numpy's PCG64 and
rounded once to float32.

Named workloads (rows x n, k):
  small     4 x 16,384,   k=512   N(0,1)
  outlier   64 x 131,072, k=512   N(0,1), 1% of positions per row from N(4,1)
  one_row   1 x 1,048,576, k=512  N(0,1)  (one row: must be split over CUs)
  adverse   128 x 1,048,576, k=512  even rows strictly ascending by position,
                                    odd rows quantized to 256 levels
  ragged    256 x 262,144, k=2048 lengths uniform in [1, 262,144], scores
                                    N(0,1) + 0.5*log1p(position), -inf padding

Vocabulary-sized workload (``vocab``): 128 rows of 129,000 N(0,1) scores
(the page's test file sweeps a vocabulary of 129,000, transcript 8:00) with
k = 4,096, above the page's own kernel's limit of about 4,000 (5:45).

Pooled workload (``pooled``): the rows an indexer above the pooling layer
sees (transcript 7:22-7:46: blocks of 8 positions, 2,000 blocks kept, the
newest pinned, about 16,000 candidates of a long context).  128 query rows
over a 1,048,576-position context; each row's pool has 2,000 slots of 8
positions: the 16 newest blocks first (newest first), then 1,984 distinct
older blocks drawn uniformly, and N(0,1) scores for the 16,000 pooled
positions; top-512.  The blocks are drawn at random rather than chosen by a
pooling pass, so this module stays free of the method's arithmetic.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class Workload:
    name: str
    scores: np.ndarray            # float32 [rows][n], C-contiguous
    lengths: np.ndarray | None    # int32 [rows] or None (all rows full)
    k: int
    seed: int
    description: str

    @property
    def rows(self) -> int:
        return self.scores.shape[0]

    @property
    def n(self) -> int:
        return self.scores.shape[1]

    def valid_elements(self) -> int:
        """Number of scores the selection must read: sum of row lengths."""
        if self.lengths is None:
            return self.rows * self.n
        return int(np.clip(self.lengths.astype(np.int64), 0, self.n).sum())


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_rows(rows: int, n: int, seed: int) -> np.ndarray:
    return _rng(seed).standard_normal((rows, n)).astype(np.float32)


def strictly_ascending(v: np.ndarray) -> np.ndarray:
    """Sorted float32 row made strictly increasing by nudging repeats up one ulp."""
    v = np.sort(v.astype(np.float32))
    while True:
        bad = np.nonzero(v[1:] <= v[:-1])[0]
        if bad.size == 0:
            return v
        v[bad + 1] = np.nextafter(v[bad], np.float32(np.inf))


def quantized_levels(x: np.ndarray) -> np.ndarray:
    """256 levels q/32 with q = clip(floor(32 x), -128, 127) (no -0.0 possible)."""
    q = np.clip(np.floor(32.0 * x), -128, 127).astype(np.int64)
    return (q.astype(np.float64) / 32.0).astype(np.float32)


def small(seed: int = 101) -> Workload:
    return Workload("small", normal_rows(4, 16384, seed), None, 512, seed,
                    "4 rows x 16,384 fp32 N(0,1), k=512")


def outlier(seed: int = 102, rows: int = 64, n: int = 131072) -> Workload:
    g = _rng(seed)
    x = g.standard_normal((rows, n))
    m = int(round(0.01 * n))
    for r in range(rows):
        pos = g.choice(n, size=m, replace=False)
        x[r, pos] = g.normal(4.0, 1.0, size=m)
    return Workload("outlier", x.astype(np.float32), None, 512, seed,
                    f"{rows} rows x {n:,} fp32 N(0,1) with {m} positions/row from N(4,1), k=512")


def one_row(seed: int = 103, n: int = 1 << 20) -> Workload:
    return Workload("one_row", normal_rows(1, n, seed), None, 512, seed,
                    f"1 row x {n:,} fp32 N(0,1), k=512")


def adverse(seed: int = 104, rows: int = 128, n: int = 1 << 20) -> Workload:
    g = _rng(seed)
    out = np.empty((rows, n), dtype=np.float32)
    for r in range(rows):
        x = g.standard_normal(n)
        if r % 2 == 0:
            out[r] = strictly_ascending(x.astype(np.float32))
        else:
            out[r] = quantized_levels(x)
    return Workload("adverse", out, None, 512, seed,
                    f"{rows} rows x {n:,} fp32, k=512; even rows strictly ascending, "
                    "odd rows quantized to 256 levels")


def ragged(seed: int = 105, rows: int = 256, n: int = 262144, k: int = 2048) -> Workload:
    g = _rng(seed)
    lengths = g.integers(1, n, size=rows, endpoint=True).astype(np.int32)
    out = np.full((rows, n), -np.inf, dtype=np.float32)
    pos = np.arange(n, dtype=np.float64)
    trend = 0.5 * np.log1p(pos)
    for r in range(rows):
        L = int(lengths[r])
        out[r, :L] = (g.standard_normal(L) + trend[:L]).astype(np.float32)
    return Workload("ragged", out, lengths, k, seed,
                    f"{rows} ragged rows, lengths uniform in [1, {n:,}], padded to {n:,} "
                    f"with -inf, scores N(0,1)+0.5*log1p(position), k={k}")


@dataclass
class PooledWorkload:
    name: str
    pool_scores: np.ndarray       # float32 [rows][keep * group]
    pool_idx: np.ndarray          # int32 [rows][keep], -1 = empty slot
    lengths: np.ndarray | None    # int32 [rows] context lengths or None (all n)
    n: int                        # context length
    group: int
    k: int
    seed: int
    description: str

    @property
    def rows(self) -> int:
        return self.pool_idx.shape[0]

    @property
    def keep(self) -> int:
        return self.pool_idx.shape[1]


def random_pool(g: np.random.Generator, L: int, group: int, keep: int, pinned: int) -> np.ndarray:
    """Pool slots for one row of length L: the newest min(pinned, nb) blocks,
    newest first, then distinct older blocks drawn uniformly, then -1
    (at most `keep` slots in all)."""
    nb = -(-L // group)
    P = min(pinned, nb, keep)
    out = np.full(keep, -1, dtype=np.int32)
    out[:P] = np.arange(nb - 1, nb - 1 - P, -1)
    m = min(keep - P, nb - P)
    if m > 0:
        out[P:P + m] = g.choice(nb - P, size=m, replace=False)
    return out


def pooled(seed: int = 106, rows: int = 128, n: int = 1 << 20, group: int = 8,
           keep: int = 2000, pinned: int = 16, k: int = 512) -> PooledWorkload:
    g = _rng(seed)
    idx = np.stack([random_pool(g, n, group, keep, pinned) for _ in range(rows)])
    sc = g.standard_normal((rows, keep * group)).astype(np.float32)
    return PooledWorkload("pooled", sc, idx, None, n, group, k, seed,
                          f"{rows} rows over a {n:,}-position context; pools of {keep:,} blocks "
                          f"of {group} ({pinned} newest pinned, the rest drawn uniformly), "
                          f"N(0,1) scores for the {keep * group:,} pooled positions, k={k}")


def vocab(seed: int = 107, rows: int = 128, n: int = 129_000, k: int = 4096) -> Workload:
    return Workload("vocab", normal_rows(rows, n, seed), None, k, seed,
                    f"{rows} rows x {n:,} fp32 N(0,1), k={k:,}")


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), as float32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32)


@dataclass
class DecodeWorkload:
    name: str
    q: np.ndarray       # float32 [rows][heads][dqk], values exact in bfloat16
    kv: np.ndarray      # float32 [n][dqk], values exact in bfloat16
    idx: np.ndarray     # int32 [rows][k]
    dv: int
    scale: float
    seed: int
    description: str


def decode(seed: int = 108, rows: int = 128, heads: int = 16, n: int = 1 << 20, k: int = 512,
           dqk: int = 576, dv: int = 512) -> DecodeWorkload:
    """Sparse-attention decode inputs: N(0,1) queries and cache entries rounded
    to bfloat16, k distinct positions per row drawn uniformly (standing in for
    the indexer's picks), softmax scale 1/sqrt(dqk)."""
    g = _rng(seed)
    q = bf16_round(g.standard_normal((rows, heads, dqk)).astype(np.float32))
    kv = bf16_round(g.standard_normal((n, dqk)).astype(np.float32))
    idx = np.stack([g.choice(n, size=k, replace=False) for _ in range(rows)]).astype(np.int32)
    return DecodeWorkload("decode", q, kv, idx, dv, float(1.0 / np.sqrt(dqk)), seed,
                          f"{rows} rows x {heads} heads, dqk={dqk}, dv={dv}, latent cache of "
                          f"{n:,} entries (bf16), k={k} selected positions per row")


def decode_positions(rows: int, n: int, k: int, seed: int) -> np.ndarray:
    """Another draw of the decode workload's selections: k distinct
    positions per row, uniform over [0, n), int32 [rows][k]."""
    g = _rng(seed)
    return np.stack([g.choice(n, size=k, replace=False) for _ in range(rows)]).astype(np.int32)


WORKLOADS = {
    "vocab": vocab,
    "small": small,
    "outlier": outlier,
    "one_row": one_row,
    "adverse": adverse,
    "ragged": ragged,
}


def make(name: str, **kw) -> Workload:
    return WORKLOADS[name](**kw)
