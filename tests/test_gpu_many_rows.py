"""More rows than one launch's grid takes (65,535 per launch): the host
splits the call into row chunks.  Every entry point that chunks is compared
with the oracle, the decode on rows around the chunk boundary."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_helpers as H
import oracle
from decode_tolerance import decode_error_bound, within
from oracle.decode import sparse_decode
from sparse_attention_indexer_row_amd import api, workloads

pytestmark = pytest.mark.gpu

ROWS = 70_000


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()
    yield
    torch.cuda.synchronize()


def test_radix_many_rows():
    x = workloads.normal_rows(ROWS, 100, seed=1)
    lengths = np.random.Generator(np.random.PCG64(2)).integers(0, 101, size=ROWS).astype(np.int32)
    print(f"[case] radix rows={ROWS}", flush=True)
    v, i = api.topk_select_radix(H.to_dev(x), 10, H.to_dev(lengths))
    torch.cuda.synchronize()
    rv, ri = oracle.topk(x, 10, lengths)
    H.assert_same(v, i, rv, ri, "radix many rows")


def test_block_pool_many_rows():
    x = workloads.normal_rows(ROWS, 64, seed=3)
    print(f"[case] pool rows={ROWS}", flush=True)
    v, i = api.topk_block_pool(H.to_dev(x), 8, 5, 2)
    torch.cuda.synchronize()
    rv, ri = oracle.block_pool(x, 8, 5, 2)
    H.assert_same(v, i, rv, ri, "pool many rows")


def test_pooled_select_many_rows():
    g = np.random.Generator(np.random.PCG64(4))
    idx = np.stack([workloads.random_pool(g, 64, 4, 6, 1) for _ in range(ROWS)])
    sc = g.standard_normal((ROWS, 24)).astype(np.float32)
    print(f"[case] pooled rows={ROWS}", flush=True)
    v, i = api.topk_pooled_select(H.to_dev(sc), H.to_dev(idx), 4, 5, 64)
    torch.cuda.synchronize()
    rv, ri = oracle.pooled_topk(sc, idx, 4, 5, 64)
    H.assert_same(v, i, rv, ri, "pooled many rows")


def test_decode_many_rows():
    g = np.random.Generator(np.random.PCG64(5))
    n, dqk, dv = 300, 64, 64
    q = workloads.bf16_round(g.standard_normal((ROWS, 16, dqk)).astype(np.float32))
    kv = workloads.bf16_round(g.standard_normal((n, dqk)).astype(np.float32))
    idx = g.integers(-1, n, size=(ROWS, 6)).astype(np.int32)
    print(f"[case] decode rows={ROWS}", flush=True)
    out = api.topk_sparse_decode(torch.from_numpy(q).to("cuda", dtype=torch.bfloat16),
                                 torch.from_numpy(kv).to("cuda", dtype=torch.bfloat16),
                                 torch.from_numpy(idx).to("cuda"), dv, 0.125)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for r in (0, 65_534, 65_535, 65_536, ROWS - 1):
        want = sparse_decode(q[r:r + 1], kv, idx[r:r + 1], 0.125, dv)[0]
        bound = decode_error_bound(q[r:r + 1], kv, idx[r:r + 1], 0.125, dv)[0]
        ok, worst = within(got[r], want, bound)
        assert ok, f"decode row {r}: error / bound {worst:.3f}"
