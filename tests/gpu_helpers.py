"""Shared helpers for the GPU tests: run the HIP library, run the oracle,
compare bit-exactly."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device (run with -m 'not gpu' on a CPU-only machine)")


def bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda", dtype=dtype) if dtype is not None else t.to("cuda")


def assert_same(gpu_vals, gpu_idx, ref_vals, ref_idx, what=""):
    gv = gpu_vals.cpu().numpy() if isinstance(gpu_vals, torch.Tensor) else gpu_vals
    gi = gpu_idx.cpu().numpy() if isinstance(gpu_idx, torch.Tensor) else gpu_idx
    bad_rows = np.nonzero(np.any(gi != ref_idx, axis=1) |
                          np.any(bits(gv) != bits(ref_vals), axis=1))[0]
    if bad_rows.size:
        r = int(bad_rows[0])
        j = int(np.nonzero((gi[r] != ref_idx[r]) | (bits(gv[r]) != bits(ref_vals[r])))[0][0])
        raise AssertionError(
            f"{what}: {bad_rows.size} rows differ; first row {r} slot {j}: "
            f"gpu ({gv[r, j]!r}, {gi[r, j]}) vs oracle ({ref_vals[r, j]!r}, {ref_idx[r, j]})")


def oracle_topk(scores: np.ndarray, k: int, lengths=None):
    return oracle.topk(scores, k, lengths)
