"""Python binding of the C ABI, for PyTorch device tensors.

Argument marshalling only: each function checks tensor placement, dtype and
layout, passes raw device pointers and the current HIP stream to the library,
and raises ``TopkError`` on a non-zero status.  Every step of the selection
runs in the library's HIP kernels.  Names follow include/topk_select.h.
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import TopkError, TopkOptions, TopkPlan  # noqa: F401


def _stream_handle(stream, device) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return int(s.cuda_stream)


def _check_scores(scores: torch.Tensor):
    if not isinstance(scores, torch.Tensor) or scores.dim() != 2:
        raise ValueError("scores must be a 2-D tensor [rows][n]")
    if scores.dtype != torch.float32:
        raise ValueError("scores must be float32")
    if not scores.is_cuda:
        raise ValueError("scores must be a GPU tensor")
    if not scores.is_contiguous():
        raise ValueError("scores must be contiguous (row stride n)")


def _check_lengths(lengths, scores):
    if lengths is None:
        return None
    if lengths.dtype != torch.int32 or lengths.device != scores.device:
        raise ValueError("lengths must be int32 on the scores' device")
    if lengths.shape != (scores.shape[0],) or not lengths.is_contiguous():
        raise ValueError("lengths must be a contiguous [rows] tensor")
    return lengths.data_ptr()


def _outputs(scores, k, out):
    rows = scores.shape[0]
    if out is None:
        vals = torch.empty((rows, k), dtype=torch.float32, device=scores.device)
        idx = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
        return vals, idx
    vals, idx = out
    if vals.shape != (rows, k) or idx.shape != (rows, k):
        raise ValueError("out tensors must be [rows][k]")
    if vals.dtype != torch.float32 or idx.dtype != torch.int32:
        raise ValueError("out tensors must be float32 and int32")
    if vals.device != scores.device or idx.device != scores.device:
        raise ValueError("out tensors must be on the scores' device")
    if not (vals.is_contiguous() and idx.is_contiguous()):
        raise ValueError("out tensors must be contiguous")
    return vals, idx


def topk_select(scores: torch.Tensor, k: int, lengths: torch.Tensor | None = None,
                out=None, stream=None):
    """Top-k (values, int32 indices) of every row of ``scores`` [rows][n]."""
    _check_scores(scores)
    lp = _check_lengths(lengths, scores)
    vals, idx = _outputs(scores, k, out)
    rows, n = scores.shape
    st = _lib.load().topk_select(scores.data_ptr(), lp, rows, n, k, vals.data_ptr(),
                                 idx.data_ptr(), _stream_handle(stream, scores.device))
    _lib.check(st, "topk_select")
    return vals, idx


def topk_split_workspace_bytes(rows: int, n: int, k: int, split: int = 0) -> int:
    return int(_lib.load().topk_split_workspace_bytes(rows, n, k, split))


def topk_workspace_init(workspace: torch.Tensor, stream=None) -> None:
    nbytes = workspace.numel() * workspace.element_size()
    _lib.check(_lib.load().topk_workspace_init(workspace.data_ptr(), nbytes,
                                               _stream_handle(stream, workspace.device)),
               "topk_workspace_init")


def new_workspace(rows: int, n: int, k: int, split: int = 0, device="cuda") -> torch.Tensor:
    """Allocates and zeroes a workspace for topk_select_split (uint8 tensor)."""
    nbytes = topk_split_workspace_bytes(rows, n, k, split)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("workspace allocation is not 256-byte aligned")
    topk_workspace_init(ws)
    return ws


def topk_select_split(scores: torch.Tensor, k: int, split: int, workspace: torch.Tensor,
                      lengths: torch.Tensor | None = None, out=None, stream=None):
    _check_scores(scores)
    lp = _check_lengths(lengths, scores)
    vals, idx = _outputs(scores, k, out)
    rows, n = scores.shape
    st = _lib.load().topk_select_split(
        scores.data_ptr(), lp, rows, n, k, vals.data_ptr(), idx.data_ptr(), split,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream_handle(stream, scores.device))
    _lib.check(st, "topk_select_split")
    return vals, idx


def topk_select_split_noalloc(scores: torch.Tensor, k: int, split: int = 0,
                              lengths: torch.Tensor | None = None, out=None, stream=None):
    """topk_select_split whose workspace is the library's static device array
    (no allocation in the library; calls on one GPU must not overlap)."""
    _check_scores(scores)
    lp = _check_lengths(lengths, scores)
    vals, idx = _outputs(scores, k, out)
    rows, n = scores.shape
    st = _lib.load().topk_select_split_noalloc(
        scores.data_ptr(), lp, rows, n, k, vals.data_ptr(), idx.data_ptr(), split,
        _stream_handle(stream, scores.device))
    _lib.check(st, "topk_select_split_noalloc")
    return vals, idx


def _options(seed=0, split=0, waves=0, watermark=0, stats=None, flags=0) -> TopkOptions:
    o = TopkOptions()
    o.seed = seed
    o.split = split
    o.waves = waves
    o.watermark = watermark
    o.flags = flags
    o.stats = stats.data_ptr() if stats is not None else None
    return o


def topk_select_ex(scores: torch.Tensor, k: int, lengths: torch.Tensor | None = None, *,
                   seed: int = 0, split: int = 0, waves: int = 0, watermark: int = 0,
                   stats: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   flags: int = 0, out=None, stream=None):
    """Selection with explicit options.  ``stats``: int64 [rows][2] to accumulate into."""
    _check_scores(scores)
    lp = _check_lengths(lengths, scores)
    vals, idx = _outputs(scores, k, out)
    rows, n = scores.shape
    if stats is not None and (stats.dtype != torch.int64 or stats.shape != (rows, 2)
                              or stats.device != scores.device or not stats.is_contiguous()):
        raise ValueError("stats must be a contiguous int64 [rows][2] tensor on the device")
    o = _options(seed, split, waves, watermark, stats, flags)
    wp = workspace.data_ptr() if workspace is not None else None
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.load().topk_select_ex(scores.data_ptr(), lp, rows, n, k, vals.data_ptr(),
                                    idx.data_ptr(), ctypes.byref(o), wp, wb,
                                    _stream_handle(stream, scores.device))
    _lib.check(st, "topk_select_ex")
    return vals, idx


def topk_plan(rows: int, n: int, k: int, *, split: int = 0, waves: int = 0,
              watermark: int = 0, for_select: bool = False) -> dict:
    """The launch plan.  ``for_select``: topk_select's own plan (no options,
    its routing included); otherwise topk_select_ex's with these options."""
    o = _options(0, split, waves, watermark, None)
    p = TopkPlan()
    opt = None if for_select else ctypes.byref(o)
    _lib.check(_lib.load().topk_plan(rows, n, k, opt, ctypes.byref(p)), "topk_plan")
    return {f: getattr(p, f) for f, _ in TopkPlan._fields_}


def topk_select_radix(scores: torch.Tensor, k: int, lengths: torch.Tensor | None = None,
                      out=None, stream=None):
    """Top-k by per-row radix selection, k up to 8,192 (values, int32 indices)."""
    _check_scores(scores)
    lp = _check_lengths(lengths, scores)
    vals, idx = _outputs(scores, k, out)
    rows, n = scores.shape
    st = _lib.load().topk_select_radix(scores.data_ptr(), lp, rows, n, k, vals.data_ptr(),
                                       idx.data_ptr(), _stream_handle(stream, scores.device))
    _lib.check(st, "topk_select_radix")
    return vals, idx


def topk_sparse_decode(q: torch.Tensor, kv: torch.Tensor, idx: torch.Tensor, dv: int,
                       scale: float, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Attention over selected positions: q bf16 [rows][heads][dqk], kv bf16 [n][dqk],
    idx int32 [rows][k] -> fp32 [rows][heads][dv]."""
    if q.dtype != torch.bfloat16 or kv.dtype != torch.bfloat16:
        raise ValueError("q and kv must be bfloat16")
    if q.dim() != 3 or kv.dim() != 2 or idx.dim() != 2 or idx.dtype != torch.int32:
        raise ValueError("expected q [rows][heads][dqk], kv [n][dqk], idx int32 [rows][k]")
    if not (q.is_cuda and kv.device == q.device and idx.device == q.device):
        raise ValueError("q, kv and idx must be on one GPU")
    if not (q.is_contiguous() and kv.is_contiguous() and idx.is_contiguous()):
        raise ValueError("q, kv and idx must be contiguous")
    rows, heads, dqk = q.shape
    if kv.shape[1] != dqk or idx.shape[0] != rows:
        raise ValueError("shape mismatch between q, kv and idx")
    if out is None:
        out = torch.empty((rows, heads, dv), dtype=torch.float32, device=q.device)
    elif out.shape != (rows, heads, dv) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [rows][heads][dv] tensor")
    st = _lib.load().topk_sparse_decode(q.data_ptr(), kv.data_ptr(), idx.data_ptr(), rows, heads,
                                        kv.shape[0], idx.shape[1], dqk, dv, float(scale),
                                        out.data_ptr(), _stream_handle(stream, q.device))
    _lib.check(st, "topk_sparse_decode")
    return out


def topk_block_pool(scores: torch.Tensor, group: int, keep: int, pinned: int,
                    lengths: torch.Tensor | None = None, out=None, stream=None):
    """Block-max pooled pre-selection: (block scores, int32 block indices) [rows][keep]."""
    _check_scores(scores)
    lp = _check_lengths(lengths, scores)
    vals, idx = _outputs(scores, keep, out)
    rows, n = scores.shape
    st = _lib.load().topk_block_pool(scores.data_ptr(), lp, rows, n, group, keep, pinned,
                                     vals.data_ptr(), idx.data_ptr(),
                                     _stream_handle(stream, scores.device))
    _lib.check(st, "topk_block_pool")
    return vals, idx


def topk_pooled_select(pool_scores: torch.Tensor, pool_idx: torch.Tensor, group: int, k: int,
                       n: int, lengths: torch.Tensor | None = None, out=None, stream=None):
    """Top-k inside a block pool: (values, int32 context positions) [rows][k]."""
    if not isinstance(pool_idx, torch.Tensor) or pool_idx.dim() != 2:
        raise ValueError("pool_idx must be a 2-D tensor [rows][keep]")
    if pool_idx.dtype != torch.int32 or not pool_idx.is_contiguous():
        raise ValueError("pool_idx must be a contiguous int32 tensor")
    _check_scores(pool_scores)
    rows, keep = pool_idx.shape
    if pool_scores.shape != (rows, keep * group) or pool_idx.device != pool_scores.device:
        raise ValueError("pool_scores must be [rows][keep * group] on pool_idx's device")
    lp = _check_lengths(lengths, pool_scores)
    vals, idx = _outputs(pool_scores, k, out)
    st = _lib.load().topk_pooled_select(pool_scores.data_ptr(), pool_idx.data_ptr(), lp, rows, n,
                                        group, keep, k, vals.data_ptr(), idx.data_ptr(),
                                        _stream_handle(stream, pool_scores.device))
    _lib.check(st, "topk_pooled_select")
    return vals, idx


def topk_strerror(status: int) -> str:
    return _lib.load().topk_strerror(status).decode()


def topk_visit_order(seed: int, row: int, nblocks: int) -> np.ndarray:
    out = np.empty(max(nblocks, 1), dtype=np.int32)
    _lib.check(_lib.load().topk_visit_order(seed, row, nblocks, out.ctypes.data),
               "topk_visit_order")
    return out[:nblocks]


def topk_probe_read(src: torch.Tensor, sink: torch.Tensor | None = None, stream=None):
    nbytes = src.numel() * src.element_size()
    words = int(_lib.load().topk_probe_sink_words(nbytes))
    if sink is None:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=src.device)
    _lib.check(_lib.load().topk_probe_read(src.data_ptr(), nbytes, sink.data_ptr(),
                                           _stream_handle(stream, src.device)), "topk_probe_read")
    return sink


def topk_probe_read_cfg(src: torch.Tensor, bytes_per_group: int, groups: int, threads: int,
                        loads: int, nontemporal: bool, lds_bytes: int = 0, sink=None,
                        stream=None):
    """One probe read of groups x bytes_per_group bytes of src (see the header)."""
    if groups * bytes_per_group > src.numel() * src.element_size():
        raise ValueError("the probe would read past src")
    if sink is None:
        sink = torch.empty(max(groups, 1), dtype=torch.int32, device=src.device)
    _lib.check(_lib.load().topk_probe_read_cfg(src.data_ptr(), bytes_per_group, groups, threads,
                                               loads, int(bool(nontemporal)), lds_bytes,
                                               sink.data_ptr(),
                                               _stream_handle(stream, src.device)),
               "topk_probe_read_cfg")
    return sink


def topk_probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    _lib.check(_lib.load().topk_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                                           _stream_handle(stream, src.device)), "topk_probe_copy")
