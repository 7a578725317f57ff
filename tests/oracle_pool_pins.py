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


# ---- selection inside a block pool ----------------------------------------
#
# Each check takes ``pooled(pool_scores, pool_idx, group, k, n, lengths) ->
# (values, positions)``.  Sources of truth:
#   * hand-derived cases in ``golden/pooled_cases.json``;
#   * a pool of every block, in a shuffled slot order, over a zero-free row is
#     the row's plain top-k: numpy's stable argsort of the row;
#   * moving pool slots (with their scores) changes nothing;
#   * brute force through the totalOrder integer key: candidate positions
#     listed by a broadcast, ranked by ``lexsort`` on (-key, position).

POOLED_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                             "pooled_cases.json")


def pin_pooled_golden(pooled):
    with open(POOLED_GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        ps = np.array([parse_value(str(v)) for v in c["pool_scores"]], dtype=np.float32)[None, :]
        pi = np.array(c["pool_idx"], dtype=np.int32)[None, :]
        lengths = np.array([c["length"]], dtype=np.int32) if "length" in c else None
        v, i = pooled(ps, pi, c["group"], c["k"], c["n"], lengths)
        ev = np.array([parse_value(str(x)) for x in c["values"]], dtype=np.float32)
        _same(v[0], i[0], ev, np.array(c["indices"], dtype=np.int32), c["name"])


def _gather(x, pool_idx, group):
    """pool_scores for a full-row score array x[rows][n] (positions past n read 0)."""
    rows, keep = pool_idx.shape
    n = x.shape[1]
    pos = pool_idx[:, :, None].astype(np.int64) * group + np.arange(group)[None, None, :]
    ok = (pool_idx[:, :, None] >= 0) & (pos < n)
    out = np.zeros((rows, keep, group), dtype=np.float32)
    r = np.broadcast_to(np.arange(rows)[:, None, None], pos.shape)
    out[ok] = x[r[ok], pos[ok]]
    return out.reshape(rows, keep * group)


def pin_pooled_full_pool_is_topk(pooled):
    g = np.random.default_rng(51)
    for group, n in [(1, 300), (4, 301), (8, 1000)]:
        x = g.standard_normal((3, n)).astype(np.float32)
        x[x == 0] = np.float32(0.25)
        nb = -(-n // group)
        pool_idx = np.stack([g.permutation(nb) for _ in range(3)]).astype(np.int32)
        for k in (1, 17, n):
            v, i = pooled(_gather(x, pool_idx, group), pool_idx, group, k, n, None)
            for r in range(3):
                order = np.argsort(-x[r], kind="stable")[:k]
                _same(v[r], i[r], x[r][order], order.astype(np.int32),
                      f"full pool group={group} k={k}")


def pin_pooled_slot_order_is_irrelevant(pooled):
    g = np.random.default_rng(52)
    x = np.float32(g.integers(-2, 3, size=(2, 400))) / np.float32(4.0)   # many ties
    pool_idx = np.stack([g.choice(50, size=30, replace=False) for _ in range(2)]).astype(np.int32)
    pool_idx[:, 5] = -1
    v0, i0 = pooled(_gather(x, pool_idx, 8), pool_idx, 8, 100, 400, None)
    perm = g.permutation(30)
    p2 = pool_idx[:, perm]
    v1, i1 = pooled(_gather(x, p2, 8), p2, 8, 100, 400, None)
    _same(v1, i1, v0, i0, "slot permutation")


def expected_pooled(ps_row, pi_row, group, k, L):
    keep = pi_row.size
    pos = pi_row[:, None].astype(np.int64) * group + np.arange(group)[None, :]
    ok = (pi_row[:, None] >= 0) & (pos < L)
    cand_pos = pos[ok]
    cand_val = ps_row.reshape(keep, group)[ok]
    key = total_order_key(cand_val).astype(np.int64)
    order = np.lexsort((cand_pos, -key))[:k]
    vals = np.full(k, -np.inf, dtype=np.float32)
    idx = np.full(k, -1, dtype=np.int32)
    vals[:order.size] = cand_val[order]
    idx[:order.size] = cand_pos[order]
    return vals, idx


def pin_pooled_integer_key_route(pooled):
    g = np.random.default_rng(53)
    for trial in range(40):
        n = int(g.integers(1, 400))
        group = int(g.integers(1, 9))
        nb = -(-n // group)
        keep = int(g.integers(1, nb + 3))
        rows = 3
        pool_idx = np.full((rows, keep), -1, dtype=np.int32)
        for r in range(rows):
            m = min(keep, nb)
            pool_idx[r, :m] = g.choice(nb, size=m, replace=False)
            g.shuffle(pool_idx[r])
        if trial % 2:
            ps = np.float32(g.integers(-3, 4, size=(rows, keep * group))) / np.float32(2.0)
            ps[g.random(ps.shape) < 0.1] = np.float32(-0.0)
        else:
            ps = g.standard_normal((rows, keep * group)).astype(np.float32)
        lengths = g.integers(-2, n + 3, size=rows).astype(np.int32)
        k = int(g.integers(1, keep * group + 4))
        v, i = pooled(ps, pool_idx, group, k, n, lengths)
        for r in range(rows):
            L = max(0, min(int(lengths[r]), n))
            ev, ei = expected_pooled(ps[r], pool_idx[r], group, k, L)
            _same(v[r], i[r], ev, ei, f"trial {trial} row {r}")


POOLED_PINS = [pin_pooled_golden, pin_pooled_full_pool_is_topk,
               pin_pooled_slot_order_is_irrelevant, pin_pooled_integer_key_route]
