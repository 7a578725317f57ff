"""CPU oracle for the sparse-attention decode over selected indices.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may call it; the GPU library shares no
code with it.

What it computes (the plain definition, in float64): the layers that
consume the indexer's picks attend only to the selected positions
("The Secret GPU Kernel Behind DeepSeek V4.1 Flash", transcript 1:48-2:13:
the indexer chooses which positions the expensive attention reads; the
sparse-MLA decode kernel of "The Full-Stack Optimization of DeepSeek-V4-Flash
on Blackwell GPUs", chunk 68.0 summary, which splits the top-k dimension and
merges the parts by their log-sum-exp).  Readings where the pages are
silent:
  * One latent cache ``kv[n][dqk]`` is shared by every head (the MLA
    layout); a head's values are the first ``dv`` channels of the same
    entries.
  * Row r's query for head h is ``q[r][h][:]``; its scores are
    ``scale * q[r][h] . kv[j]`` for the selected positions j = idx[r][t]
    with 0 <= j < n (negative or out-of-range entries are skipped, so the
    top-k filler -1 selects nothing); a position listed twice counts twice.
  * ``out[r][h] = sum_j softmax(scores)_j * kv[j][:dv]``; a row with no
    selected position gives zeros.
Inputs are float arrays whose values are exactly representable in bfloat16
(the GPU takes their bit patterns); every step here is float64.
"""

from __future__ import annotations

import numpy as np


def sparse_decode(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, scale: float, dv: int) -> np.ndarray:
    """q [rows][heads][dqk], kv [n][dqk], idx [rows][k] -> out float64 [rows][heads][dv]."""
    rows, heads, dqk = q.shape
    n = kv.shape[0]
    out = np.zeros((rows, heads, dv), dtype=np.float64)
    for r in range(rows):
        sel = [int(j) for j in idx[r] if 0 <= int(j) < n]
        if not sel:
            continue
        K = kv[sel].astype(np.float64)                    # [m][dqk]
        for h in range(heads):
            s = scale * (K @ q[r, h].astype(np.float64))  # [m]
            w = np.exp(s - s.max())
            p = w / w.sum()
            out[r, h] = p @ K[:, :dv]
    return out
