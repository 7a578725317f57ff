"""GPU parity of the block-max pooled pre-selection against the oracle.

The library's topk_block_pool is compared with oracle.block_pool slot by slot:
block scores as float32 bit patterns, block indices exactly, including the
pinned slots' order and the (-inf, -1) filler.  Every case goes through the
C ABI (via the thin binding).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_helpers as H
import oracle
from sparse_attention_indexer_row_amd import api, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()
    yield
    torch.cuda.synchronize()


def check(scores_np, group, keep, pinned, lengths_np=None, what="", dev_scores=None):
    print(f"[case] pool {what} rows={scores_np.shape[0]} n={scores_np.shape[1]} group={group} "
          f"keep={keep} pinned={pinned}", flush=True)
    s = dev_scores if dev_scores is not None else H.to_dev(scores_np)
    ln = H.to_dev(lengths_np) if lengths_np is not None else None
    gv, gi = api.topk_block_pool(s, group, keep, pinned, ln)
    torch.cuda.synchronize()
    rv, ri = oracle.block_pool(scores_np, group, keep, pinned, lengths_np)
    H.assert_same(gv, gi, rv, ri, f"pool {what}")


# ---- the pooled shape: group 8, 2,000 blocks kept, the newest pinned -------

@pytest.mark.parametrize("name", ["adverse", "ragged", "outlier"])
def test_pool_full_size(name):
    w = workloads.make(name)
    check(w.scores, 8, 2000, 16, w.lengths, what=name)


def test_pool_one_row_split():
    # one row: the selection over block maxima runs split across workgroups
    w = workloads.one_row()
    check(w.scores, 8, 2000, 16, what="one_row")
    check(w.scores, 8, 512, 0, what="one_row unpinned")


# ---- edge cases ------------------------------------------------------------

@pytest.mark.parametrize("group", [1, 2, 3, 4, 5, 8, 12, 64, 1000])
def test_group_sizes(group):
    x = workloads.normal_rows(6, 20_001, seed=group)
    check(x, group, 300, 7, what=f"group={group}")
    check(x[:, :20_000].copy(), group, 300, 7, what=f"group={group} n%4==0")


@pytest.mark.parametrize("keep,pinned", [(1, 0), (1, 1), (40, 0), (40, 40), (64, 3),
                                         (2048, 0), (2100, 52), (2048, 2048)])
def test_keep_and_pinned(keep, pinned):
    x = workloads.normal_rows(5, 30_000, seed=keep + 7 * pinned)
    check(x, 8, keep, pinned, what=f"keep={keep} pinned={pinned}")


def test_short_and_ragged_rows():
    # rows shorter than the pinned blocks, than keep, empty, partial last block
    x = workloads.normal_rows(12, 4096, seed=5)
    lengths = np.array([0, 1, 7, 8, 9, 63, 64, 65, 130, 800, 4095, 4096], dtype=np.int32)
    check(x, 8, 100, 10, lengths, what="ragged")
    check(x, 8, 10, 10, lengths, what="ragged all pinned")
    check(x, 3, 100, 0, lengths, what="ragged group 3")
    # out-of-range lengths are clamped
    bad = np.array([-5, 5000, 17, 0, -1, 1 << 30, 2, 3, 4, 5, 6, 7], dtype=np.int32)
    check(x, 8, 50, 4, bad, what="clamped lengths")


def test_ties_signed_zeros_and_infinities():
    g = np.random.Generator(np.random.PCG64(9))
    levels = np.array([-np.inf, -1.0, -0.0, 0.0, 1.0, np.inf], dtype=np.float32)
    x = levels[g.integers(0, levels.size, size=(8, 8000))]
    check(x, 8, 500, 5, what="six levels")
    y = np.full((3, 4096), -np.inf, dtype=np.float32)
    check(y, 8, 600, 3, what="all -inf")
    z = np.zeros((3, 4096), dtype=np.float32)
    z[1] = -0.0
    z[2, ::2] = -0.0
    check(z, 8, 100, 2, what="signed zeros")
    q = workloads.quantized_levels(workloads.normal_rows(16, 65_536, seed=3))
    check(q, 8, 2000, 16, what="quantized rows")


def test_monotone_rows():
    # ascending rows: every older block loses to the newer ones; descending:
    # the oldest blocks win
    x = np.sort(workloads.normal_rows(4, 50_000, seed=2), axis=1)
    check(x, 8, 700, 9, what="ascending")
    check(np.ascontiguousarray(x[:, ::-1]), 8, 700, 9, what="descending")


def test_misaligned_scores_pointer():
    # a row start that is not 16-byte aligned takes the scalar path
    base = workloads.normal_rows(1, 4 * 10_000 + 8, seed=4).reshape(-1)
    dev = H.to_dev(base)
    for off in (1, 2, 3):
        view = dev[off:off + 4 * 10_000].view(4, 10_000)
        host = base[off:off + 4 * 10_000].reshape(4, 10_000)
        check(host, 8, 200, 6, what=f"offset {off}", dev_scores=view)


def test_pool_writes_only_its_rows():
    x = workloads.normal_rows(3, 10_000, seed=6)
    s = H.to_dev(x)
    keep = 300
    vals = torch.full((4, keep), 7.0, dtype=torch.float32, device="cuda")
    idx = torch.full((4, keep), 1234, dtype=torch.int32, device="cuda")
    api.topk_block_pool(s, 8, keep, 5, out=(vals[:3], idx[:3]))
    torch.cuda.synchronize()
    assert torch.all(vals[3] == 7.0) and torch.all(idx[3] == 1234)
    rv, ri = oracle.block_pool(x, 8, keep, 5)
    H.assert_same(vals[:3], idx[:3], rv, ri, "pool rows")


def test_repeated_calls_grow_and_shrink():
    # the library's buffers grow for a large call and serve a smaller one after
    for rows, n in [(2, 1000), (40, 200_000), (3, 5000)]:
        x = workloads.normal_rows(rows, n, seed=rows + n)
        check(x, 8, 1000, 8, what=f"{rows}x{n}")


# ---- selection inside a pool -------------------------------------------------

def check_pooled(pool_scores, pool_idx, group, k, n, lengths=None, what=""):
    print(f"[case] pooled {what} rows={pool_idx.shape[0]} keep={pool_idx.shape[1]} "
          f"group={group} k={k} n={n}", flush=True)
    ln = H.to_dev(lengths) if lengths is not None else None
    gv, gi = api.topk_pooled_select(H.to_dev(pool_scores), H.to_dev(pool_idx), group, k, n, ln)
    torch.cuda.synchronize()
    rv, ri = oracle.pooled_topk(pool_scores, pool_idx, group, k, n, lengths)
    H.assert_same(gv, gi, rv, ri, f"pooled {what}")


def test_pooled_full_size():
    w = workloads.pooled()
    check_pooled(w.pool_scores, w.pool_idx, w.group, w.k, w.n, w.lengths, what="pooled")


def test_pool_then_select_end_to_end():
    # pool built on the GPU from the adverse rows, then the upper layer's
    # scores (quantized, so ties between slots are common) selected inside it
    w = workloads.make("adverse")
    s = H.to_dev(w.scores)
    pv, pi = api.topk_block_pool(s, 8, 2000, 16)
    torch.cuda.synchronize()
    ov, oi = oracle.block_pool(w.scores, 8, 2000, 16)
    H.assert_same(pv, pi, ov, oi, "pool stage")
    up = workloads.quantized_levels(workloads.normal_rows(w.rows, 2000 * 8, seed=77))
    check_pooled(up, oi, 8, 512, w.n, what="end to end")


@pytest.mark.parametrize("group,keep,k", [(1, 1, 1), (1, 5000, 2048), (8, 2000, 2048),
                                          (3, 777, 100), (8, 8192, 512), (16, 64, 512)])
def test_pooled_shapes(group, keep, k):
    g = np.random.Generator(np.random.PCG64(group * 1000 + keep))
    n = 200_003
    rows = 6
    idx = np.stack([workloads.random_pool(g, n, group, keep, 4) for _ in range(rows)])
    sc = g.standard_normal((rows, keep * group)).astype(np.float32)
    check_pooled(sc, idx, group, k, n, what=f"group={group} keep={keep} k={k}")


def test_pooled_lengths_empty_slots_and_ties():
    g = np.random.Generator(np.random.PCG64(31))
    n, group, keep = 4000, 8, 300
    rows = 10
    lengths = np.array([0, 1, 7, 8, 9, 100, 2399, 3001, 4000, 5000], dtype=np.int32)
    idx = np.full((rows, keep), -1, dtype=np.int32)
    for r in range(rows):
        L = int(np.clip(lengths[r], 0, n))
        # pools drawn for the whole context, so some blocks lie past the row
        idx[r] = workloads.random_pool(g, n, group, keep, 3)
        if L:
            idx[r, -5:] = -1
    sc = np.float32(g.integers(-2, 3, size=(rows, keep * group))) / np.float32(2.0)
    sc[g.random(sc.shape) < 0.05] = np.float32(-0.0)
    sc[g.random(sc.shape) < 0.01] = np.float32(-np.inf)
    check_pooled(sc, idx, group, 512, n, lengths, what="lengths and ties")
    # scores past each row's length are +inf: any read of them would show
    bigger = sc.copy()
    for r in range(rows):
        L = int(np.clip(lengths[r], 0, n))
        pos = idx[r][:, None].astype(np.int64) * group + np.arange(group)[None, :]
        bigger[r].reshape(keep, group)[(idx[r][:, None] >= 0) & (pos >= L)] = np.inf
    check_pooled(bigger, idx, group, 512, n, lengths, what="masked +inf")
