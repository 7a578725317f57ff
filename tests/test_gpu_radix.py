"""GPU parity of topk_select_radix (k up to 8,192) against the oracle.

The same result as topk_select, by per-row radix selection: values compared
as float32 bit patterns, indices exactly, slot by slot, including the
(-inf, -1) filler.  Every case calls the library through its C ABI.
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


def check(x, k, lengths=None, what="", dev=None):
    print(f"[case] radix {what} rows={x.shape[0]} n={x.shape[1]} k={k}", flush=True)
    s = dev if dev is not None else H.to_dev(x)
    ln = H.to_dev(lengths) if lengths is not None else None
    gv, gi = api.topk_select_radix(s, k, ln)
    torch.cuda.synchronize()
    rv, ri = oracle.topk(x, k, lengths)
    H.assert_same(gv, gi, rv, ri, f"radix {what}")


def test_vocab_workload_full_size():
    w = workloads.make("vocab")
    check(w.scores, w.k, w.lengths, what="vocab")


@pytest.mark.parametrize("k", [1, 2, 63, 512, 1000, 2048, 2049, 4096, 6000, 8192])
def test_k_values_on_vocab_rows(k):
    x = workloads.normal_rows(8, 129_000, seed=k)
    check(x, k, what=f"k={k}")


def test_million_long_rows():
    x = workloads.normal_rows(3, 1 << 20, seed=7)
    check(x, 8192, what="1M k=8192")
    check(x, 512, what="1M k=512")


@pytest.mark.parametrize("n", [1, 3, 5, 4097, 8191, 32_769, 129_001])
def test_unaligned_row_lengths(n):
    x = workloads.normal_rows(5, n, seed=n)
    check(x, min(4096, max(1, n // 2)), what=f"n={n}")


def test_lengths_short_ragged_and_clamped():
    x = workloads.normal_rows(12, 40_000, seed=3)
    lengths = np.array([0, 1, 2, 4095, 4096, 4097, 8191, 8192, 8193, 33_000, -3, 1 << 30],
                       dtype=np.int32)
    check(x, 4096, lengths, what="ragged k=4096")
    check(x, 8192, lengths, what="ragged k=8192")


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_misaligned_base_pointer(offset):
    base = workloads.normal_rows(1, 3 * 50_001 + 8, seed=offset).reshape(-1)
    dev = H.to_dev(base)
    host = base[offset:offset + 3 * 50_001].reshape(3, 50_001)
    view = dev[offset:offset + 3 * 50_001].view(3, 50_001)
    check(host, 3000, what=f"offset {offset}", dev=view)


def test_ties_specials_and_monotone_rows():
    g = np.random.Generator(np.random.PCG64(12))
    levels = np.array([-np.inf, -1.0, -0.0, 0.0, 1.0, np.inf], dtype=np.float32)
    check(levels[g.integers(0, levels.size, size=(4, 70_000))], 5000, what="six levels")
    check(np.zeros((2, 70_000), dtype=np.float32), 8192, what="all equal")
    q = workloads.quantized_levels(workloads.normal_rows(6, 129_000, seed=13))
    check(q, 4096, what="quantized")
    a = np.sort(workloads.normal_rows(2, 200_000, seed=14), axis=1)
    check(a, 8192, what="ascending")
    check(np.ascontiguousarray(a[:, ::-1]), 8192, what="descending")


def test_outputs_stay_in_their_rows():
    x = workloads.normal_rows(3, 20_000, seed=15)
    s = H.to_dev(x)
    k = 5000
    vals = torch.full((4, k), 7.0, dtype=torch.float32, device="cuda")
    idx = torch.full((4, k), 1234, dtype=torch.int32, device="cuda")
    api.topk_select_radix(s, k, out=(vals[:3], idx[:3]))
    torch.cuda.synchronize()
    assert torch.all(vals[3] == 7.0) and torch.all(idx[3] == 1234)
    rv, ri = oracle.topk(x, k)
    H.assert_same(vals[:3], idx[:3], rv, ri, "radix rows")


def test_topk_select_routes_wide_lists_over_many_short_rows():
    # 300 rows of 20,000 at k = 1,000 and k = 2,000 take the radix path
    # inside topk_select; the result is the same selection
    x = workloads.normal_rows(300, 20_000, seed=21)
    for k in (1000, 2000):
        print(f"[case] topk_select routed k={k}", flush=True)
        v, i = api.topk_select(H.to_dev(x), k)
        torch.cuda.synchronize()
        rv, ri = oracle.topk(x, k)
        H.assert_same(v, i, rv, ri, f"routed k={k}")
