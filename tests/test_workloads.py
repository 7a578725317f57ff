"""The seeded generators produce the shapes and structure the workloads name."""

import numpy as np

from sparse_attention_indexer_row_amd import workloads


def test_small_shape_and_determinism():
    a = workloads.small()
    b = workloads.small()
    assert a.scores.shape == (4, 16384) and a.scores.dtype == np.float32 and a.k == 512
    assert np.array_equal(a.scores, b.scores)
    assert a.lengths is None and a.valid_elements() == 4 * 16384


def test_outlier_count_per_row():
    w = workloads.outlier(rows=4, n=131072)
    m = int(round(0.01 * 131072))
    assert m == 1311
    # N(4,1) draws dominate the far tail: more than ~m*0.5 values above 3
    above = (w.scores > 3.0).sum(axis=1)
    assert np.all(above > m * 0.5) and np.all(above < m * 1.2)


def test_adverse_rows():
    w = workloads.adverse(rows=4, n=1 << 16)
    assert np.all(np.diff(w.scores[0]) > 0) and np.all(np.diff(w.scores[2]) > 0)
    lv = np.unique(w.scores[1])
    assert lv.size <= 256 and lv.min() >= -4.0 and lv.max() <= 3.96875
    assert not np.any(np.signbit(w.scores[1]) & (w.scores[1] == 0))


def test_strictly_ascending_resolves_repeats():
    v = np.array([1.0, 1.0, 1.0, 2.0, 2.0], dtype=np.float32)
    out = workloads.strictly_ascending(v)
    assert np.all(np.diff(out) > 0)


def test_ragged_lengths_and_padding():
    w = workloads.ragged(rows=32, n=4096, k=300)
    assert w.lengths.dtype == np.int32 and w.lengths.min() >= 1 and w.lengths.max() <= 4096
    for r in range(32):
        L = w.lengths[r]
        assert np.all(np.isneginf(w.scores[r, L:]))
        assert np.all(np.isfinite(w.scores[r, :L]))
    assert w.valid_elements() == int(w.lengths.sum())
