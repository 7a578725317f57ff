"""CPU oracle for exact per-row top-k selection (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports it and
shares no code with it.

``topk`` is the plain definition of the result, written out in C
(``topk_oracle.c``): stably order each row's valid positions by value
descending in the IEEE-754 total order (so -0.0 sorts below +0.0), ties by
lower index, and emit the first ``min(k, L)``; the remaining output slots hold
``(-inf, -1)``.  The pages behind it: "The Secret GPU Kernel Behind DeepSeek
V4.1 Flash" (transcript 2:40-4:08: keep the best 512 of up to a million scores
by comparing and moving only) and kernelbench.com "DeepSeek V4.1 Flash"
(bitonic-selection paragraph: bit-exact values, indices that never repeat).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "topk_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle_topk.so")

OK, EINVAL, ENAN, ENOMEM = 0, -1, -2, -3

_lock = threading.Lock()
_lib = None


def build(src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compiles the oracle with gcc into a shared library and returns its path."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    fn = lib.oracle_topk
    fn.restype = ctypes.c_int
    fn.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
    ]
    pool = lib.oracle_block_pool
    pool.restype = ctypes.c_int
    pool.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.POINTER(ctypes.c_int64),
    ]
    pooled = lib.oracle_pooled_topk
    pooled.restype = ctypes.c_int
    pooled.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.POINTER(ctypes.c_int64),
    ]
    return lib


def _get():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                build()
            _lib = load()
        return _lib


class OracleNaN(ValueError):
    pass


def topk(scores: np.ndarray, k: int, lengths: np.ndarray | None = None,
         threads: int | None = None, lib: ctypes.CDLL | None = None):
    """Exact top-k of each row of a host fp32 array ``scores[rows][n]``.

    Returns ``(values float32 [rows][k], indices int32 [rows][k])``.
    Raises ``OracleNaN`` if a valid position holds NaN.
    """
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    if scores.ndim != 2:
        raise ValueError("scores must be 2-D [rows][n]")
    rows, n = scores.shape
    lens_arr = None
    if lengths is not None:
        lens_arr = np.ascontiguousarray(lengths, dtype=np.int32)
        if lens_arr.shape != (rows,):
            raise ValueError("lengths must have shape [rows]")
    out_v = np.empty((rows, k), dtype=np.float32)
    out_i = np.empty((rows, k), dtype=np.int32)
    if threads is None:
        threads = min(os.cpu_count() or 1, 16)
    bad = ctypes.c_int64(-1)
    lib = lib or _get()
    st = lib.oracle_topk(
        scores.ctypes.data, lens_arr.ctypes.data if lens_arr is not None else None,
        rows, n, k, out_v.ctypes.data, out_i.ctypes.data, int(threads), ctypes.byref(bad))
    if st == ENAN:
        raise OracleNaN(f"NaN in row {bad.value}")
    if st != OK:
        raise RuntimeError(f"oracle_topk failed with status {st}")
    return out_v, out_i


def block_pool(scores: np.ndarray, group: int, keep: int, pinned: int,
               lengths: np.ndarray | None = None, lib: ctypes.CDLL | None = None):
    """Block-max pooled pre-selection of each row of ``scores[rows][n]``.

    Blocks of ``group`` positions score their best value; the newest
    ``pinned`` blocks are kept, then the best older blocks up to ``keep``.
    Returns ``(block scores float32 [rows][keep], block indices int32
    [rows][keep])``, pinned blocks first (newest first), filler (-inf, -1)
    last.  Raises ``OracleNaN`` if a valid position holds NaN.
    """
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    if scores.ndim != 2:
        raise ValueError("scores must be 2-D [rows][n]")
    rows, n = scores.shape
    lens_arr = None
    if lengths is not None:
        lens_arr = np.ascontiguousarray(lengths, dtype=np.int32)
        if lens_arr.shape != (rows,):
            raise ValueError("lengths must have shape [rows]")
    out_v = np.empty((rows, keep), dtype=np.float32)
    out_i = np.empty((rows, keep), dtype=np.int32)
    bad = ctypes.c_int64(-1)
    lib = lib or _get()
    st = lib.oracle_block_pool(
        scores.ctypes.data, lens_arr.ctypes.data if lens_arr is not None else None,
        rows, n, group, keep, pinned, out_v.ctypes.data, out_i.ctypes.data, ctypes.byref(bad))
    if st == ENAN:
        raise OracleNaN(f"NaN in row {bad.value}")
    if st != OK:
        raise RuntimeError(f"oracle_block_pool failed with status {st}")
    return out_v, out_i


def pooled_topk(pool_scores: np.ndarray, pool_idx: np.ndarray, group: int, k: int, n: int,
                lengths: np.ndarray | None = None, lib: ctypes.CDLL | None = None):
    """Top-k inside a block pool.

    ``pool_idx[rows][keep]`` names the pooled blocks (negative: empty slot);
    ``pool_scores[rows][keep * group]`` holds the score of position
    ``pool_idx[r][s] * group + j`` at ``[r][s * group + j]``.  Positions at or
    beyond the row length (``lengths``, else ``n``) are not candidates.
    Returns ``(values float32 [rows][k], context positions int32 [rows][k])``,
    equal values to the lower position, filler (-inf, -1) last.
    """
    pool_idx = np.ascontiguousarray(pool_idx, dtype=np.int32)
    if pool_idx.ndim != 2:
        raise ValueError("pool_idx must be 2-D [rows][keep]")
    rows, keep = pool_idx.shape
    pool_scores = np.ascontiguousarray(pool_scores, dtype=np.float32)
    if pool_scores.shape != (rows, keep * group):
        raise ValueError("pool_scores must have shape [rows][keep * group]")
    lens_arr = None
    if lengths is not None:
        lens_arr = np.ascontiguousarray(lengths, dtype=np.int32)
        if lens_arr.shape != (rows,):
            raise ValueError("lengths must have shape [rows]")
    out_v = np.empty((rows, k), dtype=np.float32)
    out_i = np.empty((rows, k), dtype=np.int32)
    bad = ctypes.c_int64(-1)
    lib = lib or _get()
    st = lib.oracle_pooled_topk(
        pool_scores.ctypes.data, pool_idx.ctypes.data,
        lens_arr.ctypes.data if lens_arr is not None else None, rows, n, group, keep, k,
        out_v.ctypes.data, out_i.ctypes.data, ctypes.byref(bad))
    if st == ENAN:
        raise OracleNaN(f"NaN in row {bad.value}")
    if st != OK:
        raise RuntimeError(f"oracle_pooled_topk failed with status {st}")
    return out_v, out_i
