"""GPU parity at the edges of the main calls' contract, and the schedule's
instrumentation in the pages' own setting.

- k above the streaming filter's widest list (2,049-4,096) through
  topk_select, topk_select_split and topk_select_ex, on rows shaped like the
  ragged workload and on million-score rows ("The Secret GPU Kernel Behind
  DeepSeek V4.1 Flash", transcript 5:45: the page's kernel stops near 4,000).
- A caller-owned split workspace with guard words behind it (the same page,
  12:43-12:57: writes running past the end of a tensor).
- topk_select's per-call visit order: repeated calls give identical results.
- The number of scores that ever enter a tray with the estimate off, one
  stream per row, over 16 seeds, against 1.5 x buffer x H(blocks) (4:45-5:10).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_helpers as H
from sparse_attention_indexer_row_amd import _lib, api, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()
    yield
    torch.cuda.synchronize()


def _wide_rows():
    """Ragged-shaped rows (lengths uniform in [1, 262,144], N(0,1) plus the
    log1p trend, -inf padding) and three million-score rows (N(0,1),
    strictly ascending, 256 quantized levels)."""
    rg = workloads.ragged(rows=24, n=262144, k=2048, seed=61)
    rg.lengths[:3] = np.array([1, 3000, 4096], dtype=np.int32)
    g = np.random.Generator(np.random.PCG64(62))
    big = np.empty((3, 1 << 20), dtype=np.float32)
    big[0] = g.standard_normal(1 << 20).astype(np.float32)
    big[1] = workloads.strictly_ascending(g.standard_normal(1 << 20).astype(np.float32))
    big[2] = workloads.quantized_levels(g.standard_normal(1 << 20))
    return [("ragged-shaped", rg.scores, rg.lengths), ("1M rows", big, None)]


@pytest.mark.parametrize("k", [2049, 3000, 4096])
def test_main_calls_above_the_streaming_lists(k):
    for name, x, lengths in _wide_rows():
        print(f"[case] {name} rows={x.shape[0]} n={x.shape[1]} k={k}", flush=True)
        s = H.to_dev(x)
        ln = H.to_dev(lengths) if lengths is not None else None
        rv, ri = H.oracle_topk(x, k, lengths)
        v, i = api.topk_select(s, k, ln)
        torch.cuda.synchronize()
        H.assert_same(v, i, rv, ri, f"topk_select {name} k={k}")
        ws = api.new_workspace(x.shape[0], x.shape[1], k, 4)
        v, i = api.topk_select_split(s, k, 4, ws, ln)
        torch.cuda.synchronize()
        H.assert_same(v, i, rv, ri, f"topk_select_split {name} k={k}")
        v, i = api.topk_select_ex(s, k, ln, seed=9, split=3)
        torch.cuda.synchronize()
        H.assert_same(v, i, rv, ri, f"topk_select_ex {name} k={k}")


def test_split_workspace_guard_words():
    # The caller's workspace sits inside a larger buffer whose head and tail
    # hold a pattern; every call must keep to its workspace and leave the
    # workspace itself all zero.
    guard = 4096
    pattern = 0xA5
    for split in (2, 3, 8, 17):
        rows, n, k = 6, 200_000, 700
        nbytes = api.topk_split_workspace_bytes(rows, n, k, split)
        assert nbytes > 0
        buf = torch.full((nbytes + 2 * guard,), pattern, dtype=torch.uint8, device="cuda")
        ws = buf[guard:guard + nbytes]
        assert ws.data_ptr() % 256 == 0
        api.topk_workspace_init(ws)
        for it in range(3):
            x = workloads.normal_rows(rows, n, seed=100 * split + it)
            x[1] = np.sort(x[1])        # a flooding row
            v, i = api.topk_select_split(H.to_dev(x), k, split, ws)
            torch.cuda.synchronize()
            rv, ri = H.oracle_topk(x, k)
            H.assert_same(v, i, rv, ri, f"guarded workspace split={split} call {it}")
            b = buf.cpu().numpy()
            assert np.all(b[:guard] == pattern) and np.all(b[-guard:] == pattern), split
            assert int(ws.count_nonzero()) == 0, split


def test_topk_select_visit_order_varies_per_call_result_does_not():
    # topk_select draws a new visit-order seed on every call; the result of
    # the split path (one row over many workgroups) must not change.
    w = workloads.one_row()
    s = H.to_dev(w.scores)
    rv, ri = H.oracle_topk(w.scores, w.k)
    for _ in range(6):
        v, i = api.topk_select(s, w.k)
        torch.cuda.synchronize()
        H.assert_same(v, i, rv, ri, "repeated one_row")


def test_entrant_bound_without_estimate():
    # The pages' setting: a threshold that starts at minus infinity (no
    # sampled estimate), one stream over the whole row (split 1, one streamer
    # wave), blocks in a shuffled order; the bound is on the expected number
    # of scores that ever reach the tray, 1.5 x buffer x H(number of blocks)
    # with the buffer read as the tray's capacity.  16 seeds per row.
    rows, n, k = 8, 1 << 20, 512
    g = np.random.Generator(np.random.PCG64(71))
    x = g.standard_normal((rows, n)).astype(np.float32)
    for r in range(rows // 2, rows):
        x[r] = workloads.strictly_ascending(x[r])
    s = H.to_dev(x)
    plan = api.topk_plan(rows, n, k, split=1, waves=2)
    nb = n // 1024
    h_nb = float(np.sum(1.0 / np.arange(1, nb + 1)))
    bound = 1.5 * plan["tray_words"] * h_nb
    counts = []
    rv, ri = H.oracle_topk(x, k)
    for seed in range(16):
        stats = torch.zeros((rows, 2), dtype=torch.int64, device="cuda")
        v, i = api.topk_select_ex(s, k, split=1, waves=2, stats=stats, seed=seed,
                                  flags=_lib.TOPK_FLAG_NO_ESTIMATE)
        torch.cuda.synchronize()
        H.assert_same(v, i, rv, ri, f"no-estimate seed={seed}")
        counts.append(stats.cpu().numpy()[:, 0])
    c = np.array(counts, dtype=np.float64)            # [seed][row]
    normal, ascending = c[:, : rows // 2], c[:, rows // 2:]
    print(f"[stats] bound={bound:.0f} (pages: about 29,000); N(0,1) mean={normal.mean():.0f} "
          f"max={normal.max():.0f}; ascending mean={ascending.mean():.0f} "
          f"max={ascending.max():.0f}", flush=True)
    assert np.all(c >= k)
    # the bound is on the expectation over the shuffle, for every input
    assert normal.mean(axis=0).max() <= bound
    assert ascending.mean(axis=0).max() <= bound
