"""topk_select_split_noalloc (workspace in the library's static device
array, no allocation) against topk_select_split (caller-owned workspace):
bit-identical outputs, on two calls in a row, the second smaller, and the
oracle.  Collected last so that a failure here hides no other test."""

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


CASES = [
    # rows, n, k, split: the second call is smaller than the first
    (16, 1 << 20, 512, 4),
    (3, 200_000, 1000, 3),
    (1, 1 << 20, 512, 0),      # automatic split of one long row
    (2, 50_000, 2048, 2),
]


@pytest.mark.parametrize("first,second", [(0, 1), (2, 3)])
def test_noalloc_matches_split_two_calls(first, second):
    for rows, n, k, split in (CASES[first], CASES[second]):
        print(f"[case] noalloc rows={rows} n={n} k={k} split={split}", flush=True)
        x = workloads.normal_rows(rows, n, seed=rows * 7 + k)
        x[0] = np.sort(x[0])   # one flooding row
        s = H.to_dev(x)
        ws = api.new_workspace(rows, n, k, split)
        v1, i1 = api.topk_select_split(s, k, split, ws)
        v2, i2 = api.topk_select_split_noalloc(s, k, split)
        torch.cuda.synchronize()
        assert np.array_equal(i1.cpu().numpy(), i2.cpu().numpy())
        assert np.array_equal(H.bits(v1.cpu().numpy()), H.bits(v2.cpu().numpy()))
        rv, ri = H.oracle_topk(x, k)
        H.assert_same(v2, i2, rv, ri, f"noalloc {rows}x{n} k={k} split={split}")


def test_noalloc_rejects_sizes_beyond_its_array_and_writes_nothing():
    rows, n, k = 64, 1 << 16, 2048
    need = api.topk_split_workspace_bytes(rows, n, k, 64)
    assert need > _lib.TOPK_NOALLOC_SCRATCH_BYTES
    s = H.to_dev(workloads.normal_rows(rows, n, seed=3))
    v = torch.full((rows, k), 3.0, device="cuda")
    i = torch.full((rows, k), 5, dtype=torch.int32, device="cuda")
    with pytest.raises(_lib.TopkError) as e:
        api.topk_select_split_noalloc(s, k, 64, out=(v, i))
    assert e.value.status == _lib.TOPK_EWORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(v == 3.0)) and bool(torch.all(i == 5))
