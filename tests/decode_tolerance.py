"""Per-element error bound for the sparse-attention decode (test side).

The kernel multiplies bf16 inputs exactly and sums in fp32, so its scores
are off by far less than 1e-4; each softmax weight is rounded to bf16 before
the value product (relative error at most 2^-9) and the running sum adds the
rounded weights.  The output is then the convex combination with weights
p~_j = p_j (1 + e_j) / (1 + sum_i p_i e_i), |e_j| <= 2^-9, so element c of a
head's output differs from the exact one by at most about
2^-8 * sum_j p_j |v_jc|.  The bound used is twice that, plus 1e-6 for fp32
accumulation:

    bound[r][h][c] = 2^-7 * sum_j p_j |v_jc| + 1e-6

with p the exact softmax of the row's selected positions (the same readings
as the oracle: out-of-range indices select nothing, a repeated index counts
twice).  It is computed here in float64, beside the oracle's output, and
shares no code with the oracle.
"""

from __future__ import annotations

import numpy as np


def decode_error_bound(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, scale: float,
                       dv: int) -> np.ndarray:
    """float64 [rows][heads][dv] bound for q [rows][heads][dqk], kv [n][dqk], idx [rows][k]."""
    rows, heads, _ = q.shape
    n = kv.shape[0]
    bound = np.full((rows, heads, dv), 1e-6, dtype=np.float64)
    for r in range(rows):
        j = idx[r][(idx[r] >= 0) & (idx[r] < n)].astype(np.int64)
        if j.size == 0:
            continue
        keys = kv[j].astype(np.float64)                       # [m][dqk]
        logits = scale * (q[r].astype(np.float64) @ keys.T)    # [heads][m]
        logits -= logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        p /= p.sum(axis=1, keepdims=True)
        bound[r] += 2.0 ** -7 * (p @ np.abs(keys[:, :dv]))
    return bound


def within(got: np.ndarray, want: np.ndarray, bound: np.ndarray) -> tuple[bool, float]:
    """(all elements within the bound, largest |error| / bound)."""
    ratio = np.abs(got.astype(np.float64) - want) / bound
    return bool(np.all(ratio <= 1.0)), float(ratio.max())
