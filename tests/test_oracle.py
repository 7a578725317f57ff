"""Pins the CPU oracle to facts that do not come from the oracle itself.

Runs on the CPU only.  See ``oracle_pins`` for the sources of truth.
"""

import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest

import oracle
import oracle_pins
import oracle_decode_pins
import oracle_pool_pins
from oracle import decode as decode_oracle
from sparse_attention_indexer_row_amd import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def _topk(scores, k, lengths):
    return oracle.topk(scores, k, lengths, threads=4)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(_topk)


def _pool(scores, group, keep, pinned, lengths):
    return oracle.block_pool(scores, group, keep, pinned, lengths)


@pytest.mark.parametrize("pin", oracle_pool_pins.POOL_PINS, ids=lambda p: p.__name__)
def test_pool_pin(pin):
    pin(_pool)


def test_pool_bad_arguments():
    x = np.zeros((1, 8), dtype=np.float32)
    for group, keep, pinned in [(0, 4, 0), (2, 0, 0), (2, 4, 5), (2, 4, -1)]:
        with pytest.raises(RuntimeError):
            oracle.block_pool(x, group, keep, pinned)
    x[0, 3] = np.nan
    with pytest.raises(oracle.OracleNaN):
        oracle.block_pool(x, 2, 4, 1)


def _pooled(pool_scores, pool_idx, group, k, n, lengths):
    return oracle.pooled_topk(pool_scores, pool_idx, group, k, n, lengths)


@pytest.mark.parametrize("pin", oracle_pool_pins.POOLED_PINS, ids=lambda p: p.__name__)
def test_pooled_pin(pin):
    pin(_pooled)


def test_pooled_bad_arguments():
    ps = np.zeros((1, 8), dtype=np.float32)
    pi = np.zeros((1, 4), dtype=np.int32)
    with pytest.raises(RuntimeError):
        oracle.pooled_topk(ps, pi, 2, 0, 8)           # k < 1
    with pytest.raises(ValueError):
        oracle.pooled_topk(ps, pi, 3, 4, 8)           # scores not [rows][keep * group]
    ps[0, 5] = np.nan
    with pytest.raises(oracle.OracleNaN):
        oracle.pooled_topk(ps, pi, 2, 4, 8)
    pi[0, 2] = -1                                     # the NaN sits in an empty slot
    oracle.pooled_topk(ps, pi, 2, 4, 8)


@pytest.mark.parametrize("pin", oracle_decode_pins.DECODE_PINS, ids=lambda p: p.__name__)
def test_decode_pin(pin):
    pin(decode_oracle.sparse_decode)


DECODE_MUTANTS = {
    "decode_no_scale": ("s = scale * (K @ q[r, h].astype(np.float64))",
                        "s = (K @ q[r, h].astype(np.float64))"),
    "decode_values_shifted": ("out[r, h] = p @ K[:, :dv]", "out[r, h] = p @ K[:, 1:dv + 1]"),
    "decode_duplicates_once": ("sel = [int(j) for j in idx[r] if 0 <= int(j) < n]",
                               "sel = sorted({int(j) for j in idx[r] if 0 <= int(j) < n})"),
    "decode_keeps_out_of_range": ("if 0 <= int(j) < n]", "if 0 <= int(j)]"),
    "decode_uniform_weights": ("p = w / w.sum()", "p = np.ones_like(w) / len(w)"),
    "decode_first_head_query": ("q[r, h].astype", "q[r, 0].astype"),
}


@pytest.mark.parametrize("name", sorted(DECODE_MUTANTS))
def test_decode_planted_mistake_is_caught(name):
    old, new = DECODE_MUTANTS[name]
    src = open(decode_oracle.__file__).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    ns = {}
    exec(compile(src.replace(old, new), "decode_mutant", "exec"), ns)
    caught = False
    for pin in oracle_decode_pins.DECODE_PINS:
        try:
            pin(ns["sparse_decode"])
        except Exception:
            caught = True
            break
    assert caught, f"mutant {name} passed every pin"


def _check_invariants(scores, lengths, k, vals, idx):
    """Properties every correct top-k output has, checked without re-sorting."""
    rows, n = scores.shape
    key_all = oracle_pins.total_order_key(scores)
    for r in range(rows):
        L = n if lengths is None else int(np.clip(lengths[r], 0, n))
        m = min(k, L)
        assert np.all(idx[r, m:] == -1)
        assert np.all(np.isneginf(vals[r, m:]))
        sel = idx[r, :m]
        assert np.all((sel >= 0) & (sel < L)), "index outside the row's valid range"
        assert np.unique(sel).size == m, "an index repeats"
        assert np.array_equal(oracle_pins.bits_of(vals[r, :m]), oracle_pins.bits_of(scores[r, sel]))
        key = key_all[r, sel].astype(np.int64)
        # sorted: key descending, equal keys by index ascending
        dk = np.diff(key)
        assert np.all(dk <= 0)
        assert np.all(np.diff(sel)[dk == 0] > 0)
        if m < L:
            mask = np.ones(L, dtype=bool)
            mask[sel] = False
            rest = key_all[r, :L][mask].astype(np.int64)
            kmin = key[-1]
            assert rest.max() <= kmin, "an excluded value beats the smallest kept one"
            # an excluded value equal to the boundary value has a higher index
            tied = np.nonzero(mask)[0][rest == kmin]
            assert np.all(tied > sel[-1])


@pytest.mark.parametrize("name", ["small", "outlier_small", "adverse_small", "ragged_small"])
def test_invariants_on_workload_shapes(name):
    if name == "small":
        w = workloads.small()
    elif name == "outlier_small":
        w = workloads.outlier(rows=6, n=20000)
    elif name == "adverse_small":
        w = workloads.adverse(rows=6, n=30000)
    else:
        w = workloads.ragged(rows=12, n=9000, k=700)
    vals, idx = oracle.topk(w.scores, w.k, w.lengths)
    _check_invariants(w.scores, w.lengths, w.k, vals, idx)


def test_thread_count_does_not_change_result():
    w = workloads.ragged(rows=9, n=5000, k=300, seed=3)
    a = oracle.topk(w.scores, w.k, w.lengths, threads=1)
    b = oracle.topk(w.scores, w.k, w.lengths, threads=7)
    assert np.array_equal(a[1], b[1])
    assert np.array_equal(oracle_pins.bits_of(a[0]), oracle_pins.bits_of(b[0]))


def test_quantized_rows_match_integer_key_route():
    # many ties at the boundary level: checked against the independent key route
    x = workloads.quantized_levels(np.random.default_rng(5).standard_normal((3, 4096)))
    vals, idx = oracle.topk(x, 200)
    for r in range(3):
        ev, ei = oracle_pins.expected_by_key(x[r], 4096, 200)
        assert np.array_equal(idx[r], ei)


def test_nan_is_rejected():
    x = np.zeros((3, 10), dtype=np.float32)
    x[2, 4] = np.nan
    with pytest.raises(oracle.OracleNaN):
        oracle.topk(x, 3)
    # NaN beyond a row's length is never looked at
    vals, idx = oracle.topk(x, 3, np.array([10, 10, 4], dtype=np.int32))
    assert idx[2].tolist() == [0, 1, 2]


def test_bad_arguments():
    lib = oracle._get()
    assert lib.oracle_topk(None, None, 1, 4, 1, None, None, 1, None) == oracle.EINVAL
    assert lib.oracle_topk(None, None, 0, 4, 1, None, None, 1, None) == oracle.OK
    x = np.zeros((1, 4), dtype=np.float32)
    o = np.zeros(4, dtype=np.float32)
    i = np.zeros(4, dtype=np.int32)
    assert lib.oracle_topk(x.ctypes.data, None, 1, 4, 0, o.ctypes.data, i.ctypes.data, 1,
                           None) == oracle.EINVAL


# Planted mistakes: each replaces one piece of the oracle's source; the pins
# above must reject every one of them.
MUTANTS = {
    "ties_to_higher_index": (
        "if (a->i < b->i) return -1;\n    if (a->i > b->i) return 1;",
        "if (a->i < b->i) return 1;\n    if (a->i > b->i) return -1;"),
    "zeros_unordered": (
        "if (a == 0.0f && !signbit(a) && signbit(b)) return 1;", ""),
    "zeros_reversed": (
        "if (a == 0.0f && !signbit(a) && signbit(b)) return 1;",
        "if (a == 0.0f && signbit(a) && !signbit(b)) return 1;"),
    "ascending_values": (
        "if (a > b) return 1;\n    if (a < b) return 0;",
        "if (a < b) return 1;\n    if (a > b) return 0;"),
    "filler_index_zero": ("out_i[j] = -1;", "out_i[j] = 0;"),
    "filler_value_zero": ("out_v[j] = -INFINITY;", "out_v[j] = 0.0f;"),
    "length_not_clamped_high": ("if (L > n) L = n;", ""),
    "length_not_clamped_low": ("if (L < 0) L = 0;", ""),
    "off_by_one_count": ("int64_t m = L < k ? L : k;", "int64_t m = L < k ? L : k - 1;"),
    "wrong_index_recorded": ("work[j].i = (int32_t)j;", "work[j].i = (int32_t)(L - 1 - j);"),
    "lengths_ignored": ("if (!lengths) return n;", "if (lengths || !lengths) return n;"),
    "pool_pins_oldest": ("        out_v[s] = work[nb - 1 - s].v;\n        out_i[s] = work[nb - 1 - s].i;",
                         "        out_v[s] = work[s].v;\n        out_i[s] = work[s].i;"),
    "pool_block_one_short": ("const int64_t hi = lo + group < L ? lo + group : L;",
                             "const int64_t hi = lo + group - 1 < L ? lo + group - 1 : L;"),
    "pool_first_not_best": ("if (value_greater(row[j], best)) best = row[j];", ""),
    "pool_pinned_reselected": ("qsort(work, (size_t)older, sizeof(pair_t), pair_cmp);",
                               "qsort(work, (size_t)nb, sizeof(pair_t), pair_cmp);"),
    "pool_keeps_one_less": ("const int64_t take = keep - P < older ? keep - P : older;",
                            "const int64_t take = keep - P - 1 < older ? keep - P - 1 : older;"),
    "pooled_ignores_length": ("                if (pos >= L) break;", ""),
    "pooled_keeps_empty_slots": ("            if (pi[s] < 0) continue;",
                                 "            if (pi[s] < -1) continue;"),
    "pooled_slot_as_index": ("                work[m].i = (int32_t)pos;",
                             "                work[m].i = (int32_t)(s * group + j);"),
    "pooled_wrong_score": ("                const float v = sc[s * group + j];",
                           "                const float v = sc[s * group + (group - 1 - j)];"),
    "pooled_group_stride": ("const int64_t pos = (int64_t)pi[s] * group + j;",
                            "const int64_t pos = (int64_t)pi[s] * (group + 1) + j;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = os.path.join(d, "libmutant.so")
        oracle.build(path, lib)
        p = subprocess.run([sys.executable, os.path.join(HERE, "_oracle_mutant_runner.py"), lib],
                           capture_output=True, text=True, timeout=300)
    assert p.returncode != 0, f"mutant {name} passed every pin:\n{p.stdout}"


def test_unmutated_oracle_passes_runner():
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "liboracle.so")
        oracle.build(oracle._SRC, lib)
        p = subprocess.run([sys.executable, os.path.join(HERE, "_oracle_mutant_runner.py"), lib],
                           capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stdout + p.stderr
