"""Checks that pin the CPU oracle to facts that do not come from the oracle.

Each check takes ``topk(scores, k, lengths) -> (values, indices)`` and raises
``AssertionError`` on a mismatch.  They are used twice: against the real
oracle, and against deliberately broken copies of it (a planted mistake must
trip at least one check).

Sources of truth used here, none of them the oracle's own comparator:
  * hand-derived cases in ``golden/oracle_cases.json``;
  * numpy's ``argmax`` (first maximum) for k = 1 and numpy's stable
    ``argsort`` of the negated row for k = L, on rows without zeros (numpy
    treats -0.0 == +0.0, so zeros are covered by the other routes);
  * exhaustive enumeration of every row of length 4 over the alphabet
    {-inf, -1, -0.0, +0.0, 1, +inf}, ranked through the IEEE-754 totalOrder
    integer mapping of the float32 bit patterns (a route the oracle does not
    use: it compares floats and breaks the zero pair by sign).
"""

from __future__ import annotations

import itertools
import json
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_cases.json")


def parse_value(s: str) -> np.float32:
    if s.startswith("bits:"):
        return np.frombuffer(struct.pack("<I", int(s[5:], 16)), dtype=np.float32)[0]
    return np.float32(float(s))


def bits_of(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def total_order_key(a: np.ndarray) -> np.ndarray:
    """IEEE-754 totalOrder as unsigned integers (valid for every non-NaN float)."""
    b = bits_of(a).astype(np.uint64)
    neg = (b >> np.uint64(31)) == 1
    return np.where(neg, np.uint64(0xFFFFFFFF) - b, b | np.uint64(0x80000000))


def expected_by_key(row: np.ndarray, L: int, k: int):
    """Top-k of row[:L] via the integer totalOrder key, ties by lower index."""
    L = max(0, min(L, row.size))
    key = total_order_key(row[:L]).astype(np.int64)
    order = np.lexsort((np.arange(L), -key))
    m = min(k, L)
    vals = np.full(k, -np.inf, dtype=np.float32)
    idx = np.full(k, -1, dtype=np.int32)
    vals[:m] = row[order[:m]]
    idx[:m] = order[:m]
    return vals, idx


def check_golden(topk):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        rows = np.array([[parse_value(v) for v in r] for r in c["rows"]], dtype=np.float32)
        lengths = None if c["lengths"] is None else np.array(c["lengths"], dtype=np.int32)
        vals, idx = topk(rows, c["k"], lengths)
        ev = np.array([[parse_value(v) for v in r] for r in c["expect_values"]], dtype=np.float32)
        ei = np.array(c["expect_indices"], dtype=np.int32)
        assert np.array_equal(idx, ei), f"{c['name']}: indices {idx.tolist()} != {ei.tolist()}"
        assert np.array_equal(bits_of(vals), bits_of(ev)), (
            f"{c['name']}: value bits {bits_of(vals).tolist()} != {bits_of(ev).tolist()}")


def check_argmax(topk, seed: int = 7):
    g = np.random.default_rng(seed)
    # heavy ties (few levels, no zero level) so "first maximum" matters
    rows = (g.integers(1, 9, size=(64, 300)) * np.float32(0.5)).astype(np.float32)
    rows[::3] = g.standard_normal((rows[::3].shape)).astype(np.float32) + np.float32(10.0)
    vals, idx = topk(rows, 1, None)
    exp = np.argmax(rows, axis=1)
    assert np.array_equal(idx[:, 0], exp), "k=1 does not pick the first maximum"
    assert np.array_equal(bits_of(vals[:, 0]), bits_of(rows[np.arange(64), exp]))


def check_full_sort(topk, seed: int = 8):
    g = np.random.default_rng(seed)
    n = 257
    rows = g.standard_normal((16, n)).astype(np.float32)
    rows[1::2] = np.round(rows[1::2] * 2) / 2 + np.float32(0.25)   # ties, never zero
    rows[rows == 0] = np.float32(0.125)
    rows[3, 5] = np.inf
    rows[3, 6] = -np.inf
    vals, idx = topk(rows, n, None)
    for r in range(rows.shape[0]):
        exp = np.argsort(-rows[r], kind="stable")
        assert np.array_equal(idx[r], exp), f"row {r}: k=L differs from stable descending sort"
        assert np.array_equal(bits_of(vals[r]), bits_of(rows[r][exp]))


ALPHABET = np.array([-np.inf, -1.0, -0.0, 0.0, 1.0, np.inf], dtype=np.float32)


def check_exhaustive_alphabet(topk, n: int = 4):
    rows = np.array(list(itertools.product(range(ALPHABET.size), repeat=n)))
    rows = ALPHABET[rows].astype(np.float32)
    R = rows.shape[0]
    lens = (np.arange(R) % (n + 2)).astype(np.int32) - 1      # -1 .. n
    for k in range(1, n + 2):
        for lengths in (None, lens):
            vals, idx = topk(rows, k, lengths)
            for r in range(R):
                L = n if lengths is None else int(lengths[r])
                ev, ei = expected_by_key(rows[r], L, k)
                assert np.array_equal(idx[r], ei), (
                    f"row {rows[r].tolist()} L={L} k={k}: {idx[r].tolist()} != {ei.tolist()}")
                assert np.array_equal(bits_of(vals[r]), bits_of(ev))


ALL_PINS = (check_golden, check_argmax, check_full_sort, check_exhaustive_alphabet)
