"""The decode's per-element tolerance catches a mis-weighted split (CPU)."""

from __future__ import annotations

import numpy as np

from decode_tolerance import decode_error_bound, within
from oracle.decode import sparse_decode
from sparse_attention_indexer_row_amd import workloads


def _case(seed=3, rows=3, heads=16, dqk=576, dv=512, n=20000, k=512):
    g = np.random.Generator(np.random.PCG64(seed))
    q = workloads.bf16_round(g.standard_normal((rows, heads, dqk)).astype(np.float32))
    kv = workloads.bf16_round(g.standard_normal((n, dqk)).astype(np.float32))
    idx = np.stack([g.choice(n, size=k, replace=False) for _ in range(rows)]).astype(np.int32)
    return q, kv, idx, 1.0 / np.sqrt(dqk), dv


def _split_weighted(q, kv, idx, scale, dv, splits=4, bad=1, factor=1.2):
    """The split-K result with split `bad`'s weight scaled by `factor` in the
    log-sum-exp combine (each split's exact partial output, max and sum)."""
    rows, heads, _ = q.shape
    out = np.zeros((rows, heads, dv))
    for r in range(rows):
        parts = np.array_split(idx[r], splits)
        for h in range(heads):
            o, m, l = [], [], []
            for part in parts:
                keys = kv[part].astype(np.float64)
                s = scale * (keys @ q[r, h].astype(np.float64))
                w = np.exp(s - s.max())
                o.append(w @ keys[:, :dv] / w.sum())
                m.append(s.max())
                l.append(w.sum())
            M = max(m)
            cw = np.array([np.exp(mi - M) * li for mi, li in zip(m, l)])
            cw[bad] *= factor
            out[r, h] = sum(c * oi for c, oi in zip(cw, o)) / cw.sum()
    return out


def test_exact_split_combine_is_within_the_bound():
    q, kv, idx, scale, dv = _case()
    want = sparse_decode(q, kv, idx, scale, dv)
    b = decode_error_bound(q, kv, idx, scale, dv)
    ok, worst = within(_split_weighted(q, kv, idx, scale, dv, factor=1.0), want, b)
    assert ok and worst < 1e-3


def test_split_weighted_20_percent_high_fails_the_bound():
    q, kv, idx, scale, dv = _case()
    want = sparse_decode(q, kv, idx, scale, dv)
    b = decode_error_bound(q, kv, idx, scale, dv)
    ok, worst = within(_split_weighted(q, kv, idx, scale, dv, factor=1.2), want, b)
    assert not ok and worst > 1.5


def test_bf16_rounded_weights_stay_within_the_bound():
    # The arithmetic the bound is derived from: softmax weights rounded to
    # bf16 (round to nearest even) and renormalised by their rounded sum.
    q, kv, idx, scale, dv = _case(seed=4, rows=2)
    want = sparse_decode(q, kv, idx, scale, dv)
    b = decode_error_bound(q, kv, idx, scale, dv)
    got = np.zeros_like(want)
    for r in range(q.shape[0]):
        keys = kv[idx[r]].astype(np.float64)
        for h in range(q.shape[1]):
            s = scale * (keys @ q[r, h].astype(np.float64))
            w = workloads.bf16_round(np.exp(s - s.max()).astype(np.float32)).astype(np.float64)
            got[r, h] = w @ keys[:, :dv] / w.sum()
    ok, worst = within(got, want, b)
    assert ok, worst
