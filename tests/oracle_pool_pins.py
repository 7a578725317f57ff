"""Checks that pin the oracle's block-max pooled pre-selection to facts that
do not come from the oracle.

Each check takes ``pool(scores, group, keep, pinned, lengths) -> (values,
indices)`` and raises ``AssertionError`` on a mismatch.  Sources of truth:
  * hand-derived cases in ``golden/pool_cases.json``;
  * a route through the IEEE-754 totalOrder integer key: block scores as the
    integer maximum over a padded reshape, the older blocks ranked by
    ``lexsort`` on (-key, block) -- neither step is the oracle's comparator;
  * group = 1 with nothing pinned is an exact top-k, checked against numpy's
    stable argsort on rows without zeros.
"""

from __future__ import annotations

import json
import os

import numpy as np

from oracle_pins import bits_of, parse_value, total_order_key

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pool_cases.json")


def key_to_float(key: np.ndarray) -> np.ndarray:
    key = key.astype(np.uint64)
    neg = key < np.uint64(0x80000000)
    bits = np.where(neg, np.uint64(0xFFFFFFFF) - key, key - np.uint64(0x80000000))
    return bits.astype(np.uint32).view(np.float32)


def expected_pool(row: np.ndarray, L: int, group: int, keep: int, pinned: int):
    L = max(0, min(L, row.size))
    nb = -(-L // group)
    vals = np.full(keep, -np.inf, dtype=np.float32)
    idx = np.full(keep, -1, dtype=np.int32)
    if nb == 0:
        return vals, idx
    key = np.zeros(nb * group, dtype=np.int64)   # padding key 0 lies below every float
    key[:L] = total_order_key(row[:L]).astype(np.int64)
    bkey = key.reshape(nb, group).max(axis=1)
    P = min(pinned, nb)
    s = 0
    for b in range(nb - 1, nb - 1 - P, -1):
        vals[s], idx[s] = key_to_float(np.array([bkey[b]]))[0], b
        s += 1
    older = nb - P
    order = np.lexsort((np.arange(older), -bkey[:older]))
    take = min(keep - P, older)
    for b in order[:take]:
        vals[s], idx[s] = key_to_float(np.array([bkey[b]]))[0], b
        s += 1
    return vals, idx


def _same(gv, gi, ev, ei, what):
    assert np.array_equal(gi, ei), f"{what}: indices {gi} != {ei}"
    assert np.array_equal(bits_of(gv), bits_of(ev)), f"{what}: values {gv} != {ev}"


def pin_golden(pool):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        row = np.array([parse_value(str(v)) for v in c["row"]], dtype=np.float32)[None, :]
        lengths = np.array([c["length"]], dtype=np.int32) if "length" in c else None
        v, i = pool(row, c["group"], c["keep"], c["pinned"], lengths)
        ev = np.array([parse_value(str(x)) for x in c["values"]], dtype=np.float32)
        _same(v[0], i[0], ev, np.array(c["indices"], dtype=np.int32), c["name"])


def pin_integer_key_route(pool):
    g = np.random.default_rng(41)
    for trial in range(40):
        n = int(g.integers(1, 300))
        group = int(g.integers(1, 10))
        keep = int(g.integers(1, 40))
        pinned = int(g.integers(0, keep + 1))
        rows = 3
        if trial % 2:
            x = np.float32(g.integers(-3, 4, size=(rows, n))) / np.float32(2.0)   # many ties
            x[g.random((rows, n)) < 0.1] = np.float32(-0.0)
        else:
            x = g.standard_normal((rows, n)).astype(np.float32)
        lengths = g.integers(-2, n + 3, size=rows).astype(np.int32)
        v, i = pool(x, group, keep, pinned, lengths)
        for r in range(rows):
            ev, ei = expected_pool(x[r], int(lengths[r]), group, keep, pinned)
            _same(v[r], i[r], ev, ei, f"trial {trial} row {r}")


def pin_group_one_is_topk(pool):
    g = np.random.default_rng(42)
    x = g.standard_normal((4, 500)).astype(np.float32)
    x[x == 0] = np.float32(0.5)
    for k in (1, 7, 500):
        v, i = pool(x, 1, k, 0, None)
        for r in range(4):
            order = np.argsort(-x[r], kind="stable")[:k]
            _same(v[r], i[r], x[r][order], order.astype(np.int32), f"group 1 k={k}")


def pin_pinned_are_newest(pool):
    g = np.random.default_rng(43)
    x = g.standard_normal((2, 97)).astype(np.float32)
    v, i = pool(x, 8, 20, 5, None)   # 13 blocks, the last one partial
    nb = 13
    assert list(i[0, :5]) == [nb - 1 - j for j in range(5)], i[0, :5]
    assert np.all(i[:, 5:13] >= 0) and np.all(i[:, 13:] == -1)
    assert len(set(i[0, :13].tolist())) == 13


POOL_PINS = [pin_golden, pin_integer_key_route, pin_group_one_is_topk, pin_pinned_are_newest]
