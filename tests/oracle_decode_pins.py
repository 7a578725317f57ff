"""Checks that pin the decode oracle to facts that do not come from it.

Each check takes ``decode(q, kv, idx, scale, dv) -> out`` and raises
``AssertionError`` on a mismatch.  Sources of truth:
  * one selected position: the output is that position's value row;
  * a zero query: every score is equal, so the output is the plain mean of
    the selected value rows (duplicates counted twice);
  * two positions with scores a and b: weights 1/(1+e^(b-a)) and its
    complement, written from the two-point softmax closed form;
  * the order of the selected positions, and the filler -1, change nothing;
  * a hand-derived case in ``golden/decode_cases.json``.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "decode_cases.json")


def _close(a, b, what, tol=1e-12):
    assert np.allclose(a, b, rtol=tol, atol=tol), f"{what}: {a} != {b}"


def pin_single_position(decode):
    g = np.random.default_rng(61)
    q = g.standard_normal((2, 3, 8))
    kv = g.standard_normal((10, 8))
    idx = np.array([[4, -1, -1], [-1, 7, 12]])   # 12 is out of range: skipped
    out = decode(q, kv, idx, 0.5, 5)
    for h in range(3):
        _close(out[0, h], kv[4, :5], "single position row 0")
        _close(out[1, h], kv[7, :5], "single position row 1")


def pin_zero_query_is_mean(decode):
    g = np.random.default_rng(62)
    kv = g.standard_normal((20, 6))
    q = np.zeros((1, 2, 6))
    idx = np.array([[3, 9, 9, 14]])
    out = decode(q, kv, idx, 1.0, 6)
    want = (kv[3] + 2 * kv[9] + kv[14]) / 4.0
    _close(out[0, 0], want, "zero query mean")
    _close(out[0, 1], want, "zero query mean, head 1")


def pin_two_point_softmax(decode):
    kv = np.zeros((5, 3))
    kv[1] = [1.0, 0.0, 2.0]
    kv[3] = [0.0, 1.0, -1.0]
    q = np.array([[[0.5, 1.5, 0.0]]])
    scale = 0.8
    a = scale * (0.5 * 1.0)          # score of position 1
    b = scale * (1.5 * 1.0)          # score of position 3
    w1 = 1.0 / (1.0 + math.exp(b - a))
    want = w1 * kv[1] + (1.0 - w1) * kv[3]
    out = decode(q, kv, np.array([[3, 1]]), scale, 3)
    _close(out[0, 0], want, "two-point softmax")


def pin_order_and_filler_irrelevant(decode):
    g = np.random.default_rng(63)
    q = g.standard_normal((3, 4, 16))
    kv = g.standard_normal((50, 16))
    idx = np.stack([g.choice(50, size=12, replace=False) for _ in range(3)])
    out = decode(q, kv, idx, 0.25, 8)
    shuffled = np.stack([np.concatenate([g.permutation(r), [-1, -1]]) for r in idx])
    _close(decode(q, kv, shuffled, 0.25, 8), out, "order and filler", tol=1e-12)


def pin_golden(decode):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        out = decode(np.array(c["q"], dtype=np.float64), np.array(c["kv"], dtype=np.float64),
                     np.array(c["idx"]), c["scale"], c["dv"])
        _close(out, np.array(c["out"], dtype=np.float64), c["name"], tol=1e-9)


DECODE_PINS = [pin_single_position, pin_zero_query_is_mean, pin_two_point_softmax,
               pin_order_and_filler_irrelevant, pin_golden]
