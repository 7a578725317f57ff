"""GPU parity of topk_sparse_decode against the float64 oracle.

Tolerance, from the arithmetic (derived in tests/decode_tolerance.py): every
output element must lie within 2^-7 * sum_j p_j |v_jc| + 1e-6 of the exact
one, p being the exact softmax weights of the row's selected positions --
twice what bf16-rounded weights can move a convex combination, per element.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_helpers as H
from decode_tolerance import decode_error_bound, within
from oracle.decode import sparse_decode
from sparse_attention_indexer_row_amd import api, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()
    yield
    torch.cuda.synchronize()


def run(q, kv, idx, dv, scale, kv_dev=None):
    qd = torch.from_numpy(q).to("cuda", dtype=torch.bfloat16)
    kd = kv_dev if kv_dev is not None else torch.from_numpy(kv).to("cuda", dtype=torch.bfloat16)
    out = api.topk_sparse_decode(qd, kd, torch.from_numpy(idx).to("cuda"), dv, scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(q, kv, idx, dv, scale, what="", rows=None, kv_dev=None):
    print(f"[case] decode {what} q={q.shape} kv={kv.shape} k={idx.shape[1]} dv={dv} "
          f"scale={scale}", flush=True)
    got = run(q, kv, idx, dv, scale, kv_dev)
    sample = range(q.shape[0]) if rows is None else rows
    for r in sample:
        want = sparse_decode(q[r:r + 1], kv, idx[r:r + 1], scale, dv)[0]
        bound = decode_error_bound(q[r:r + 1], kv, idx[r:r + 1], scale, dv)[0]
        ok, worst = within(got[r], want, bound)
        assert ok, f"{what}: row {r} error / bound {worst:.3f}"


def test_decode_workload_sampled_rows():
    w = workloads.decode()
    rows = [0, 1, 17, 64, 127]
    check(w.q, w.kv, w.idx, w.dv, w.scale, what="decode workload", rows=rows)


@pytest.mark.parametrize("k", [1, 2, 31, 32, 33, 100, 512, 1000, 2048])
def test_selected_counts(k):
    g = np.random.Generator(np.random.PCG64(k))
    n, dqk, dv = 5000, 576, 512
    q = workloads.bf16_round(g.standard_normal((3, 16, dqk)).astype(np.float32))
    kv = workloads.bf16_round(g.standard_normal((n, dqk)).astype(np.float32))
    idx = np.stack([g.choice(n, size=k, replace=False) for _ in range(3)]).astype(np.int32)
    check(q, kv, idx, dv, 1.0 / 24.0, what=f"k={k}")


@pytest.mark.parametrize("heads,dqk,dv", [(16, 64, 64), (32, 64, 64), (16, 128, 128),
                                          (48, 576, 512), (16, 1024, 1024), (16, 1024, 64)])
def test_shapes(heads, dqk, dv):
    g = np.random.Generator(np.random.PCG64(heads * dqk + dv))
    n = 3000
    q = workloads.bf16_round(g.standard_normal((4, heads, dqk)).astype(np.float32))
    kv = workloads.bf16_round(g.standard_normal((n, dqk)).astype(np.float32))
    idx = np.stack([g.choice(n, size=200, replace=False) for _ in range(4)]).astype(np.int32)
    check(q, kv, idx, dv, float(1.0 / np.sqrt(dqk)), what=f"heads={heads} dqk={dqk} dv={dv}")


def test_filler_out_of_range_duplicates_and_empty_rows():
    g = np.random.Generator(np.random.PCG64(5))
    n, dqk, dv = 1000, 128, 64
    q = workloads.bf16_round(g.standard_normal((5, 16, dqk)).astype(np.float32))
    kv = workloads.bf16_round(g.standard_normal((n, dqk)).astype(np.float32))
    idx = g.integers(0, n, size=(5, 70)).astype(np.int32)   # repeats allowed
    idx[0, 40:] = -1                                         # the selection's filler
    idx[1, ::3] = n + 5                                      # out of range: skipped
    idx[2, :] = -1                                           # nothing selected: zeros
    idx[3, :] = 7                                            # one position, 70 times
    check(q, kv, idx, dv, 0.3, what="filler and repeats")
    out = run(q, kv, idx, dv, 0.3)
    assert np.all(out[2] == 0.0)


def test_scales_flat_and_peaked():
    g = np.random.Generator(np.random.PCG64(6))
    n, dqk, dv = 2000, 256, 128
    q = workloads.bf16_round(g.standard_normal((2, 16, dqk)).astype(np.float32))
    kv = workloads.bf16_round(g.standard_normal((n, dqk)).astype(np.float32))
    idx = np.stack([g.choice(n, size=300, replace=False) for _ in range(2)]).astype(np.int32)
    check(q, kv, idx, dv, 0.0, what="scale 0 (mean)")
    check(q, kv, idx, dv, 2.0, what="peaked softmax")


def test_many_rows_and_one_row():
    # one row spreads its positions over many splits; 600 rows use one each
    g = np.random.Generator(np.random.PCG64(8))
    n, dqk, dv = 4000, 576, 512
    kv = workloads.bf16_round(g.standard_normal((n, dqk)).astype(np.float32))
    kvd = torch.from_numpy(kv).to("cuda", dtype=torch.bfloat16)
    q1 = workloads.bf16_round(g.standard_normal((1, 16, dqk)).astype(np.float32))
    i1 = g.choice(n, size=2048, replace=False).astype(np.int32)[None, :]
    check(q1, kv, i1, dv, 1.0 / 24.0, what="one row, k=2048", kv_dev=kvd)
    qm = workloads.bf16_round(g.standard_normal((600, 16, dqk)).astype(np.float32))
    im = np.stack([g.choice(n, size=64, replace=False) for _ in range(600)]).astype(np.int32)
    check(qm, kv, im, dv, 1.0 / 24.0, what="600 rows", rows=[0, 299, 599], kv_dev=kvd)


def test_long_splits_load_positions_per_tile():
    # 300 rows of 16 heads fill the GPU with one split per row, so each split
    # walks all 1,000 positions (more than a split keeps in LDS)
    g = np.random.Generator(np.random.PCG64(9))
    n, dqk, dv = 6000, 576, 512
    kv = workloads.bf16_round(g.standard_normal((n, dqk)).astype(np.float32))
    q = workloads.bf16_round(g.standard_normal((300, 16, dqk)).astype(np.float32))
    idx = np.stack([g.choice(n, size=1000, replace=False) for _ in range(300)]).astype(np.int32)
    idx[5, 700:] = -1
    check(q, kv, idx, dv, 1.0 / 24.0, what="long splits", rows=[0, 5, 150, 299])
