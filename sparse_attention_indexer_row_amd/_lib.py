"""ctypes declarations of the C ABI in include/topk_select.h.

Loading fails loudly when the HIP library has not been built: there is no
fallback implementation of any entry point.
"""

from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtopk_select.so")

TOPK_OK = 0
TOPK_EINVAL = -1
TOPK_EK_RANGE = -2
TOPK_EWORKSPACE = -3
TOPK_ESPLIT = -4
TOPK_ELAUNCH = -5
TOPK_EDEVICE = -6
TOPK_EALLOC = -7
TOPK_MAX_K = 4096
TOPK_MAX_K_STREAM = 2048
TOPK_MAX_K_POOLED = 2048
TOPK_PATH_STREAM = 0
TOPK_PATH_RADIX = 1
TOPK_FLAG_NO_ESTIMATE = 1
TOPK_FLAG_FORCE_RERUN = 2
TOPK_MAX_SPLIT = 1024
TOPK_MAX_POOL_SLOTS = 8192
TOPK_MAX_K_RADIX = 8192
TOPK_NOALLOC_SCRATCH_BYTES = 8 << 20

# Every function the header declares, in header order.
EXPORTS = (
    "topk_select",
    "topk_split_workspace_bytes",
    "topk_workspace_init",
    "topk_select_split",
    "topk_select_split_noalloc",
    "topk_select_ex",
    "topk_plan",
    "topk_block_pool",
    "topk_select_radix",
    "topk_sparse_decode",
    "topk_pooled_select",
    "topk_strerror",
    "topk_visit_order",
    "topk_probe_sink_words",
    "topk_probe_read",
    "topk_probe_read_cfg",
    "topk_probe_copy",
)


class TopkOptions(ctypes.Structure):
    _fields_ = [
        ("seed", ctypes.c_uint64),
        ("split", ctypes.c_int32),
        ("waves", ctypes.c_int32),
        ("watermark", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("stats", ctypes.c_void_p),
    ]


class TopkPlan(ctypes.Structure):
    _fields_ = [
        ("split", ctypes.c_int32),
        ("waves", ctypes.c_int32),
        ("list_words", ctypes.c_int32),
        ("watermark", ctypes.c_int32),
        ("tray_words", ctypes.c_int32),
        ("lds_bytes", ctypes.c_int32),
        ("compute_units", ctypes.c_int32),
        ("path", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


_vp, _i32, _u64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t

SIGNATURES = {
    "topk_select": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "topk_split_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "topk_workspace_init": (ctypes.c_int, [_vp, _sz, _vp]),
    "topk_select_split": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _sz, _vp]),
    "topk_select_split_noalloc": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _i32, _vp]),
    "topk_select_ex": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp,
                                      ctypes.POINTER(TopkOptions), _vp, _sz, _vp]),
    "topk_plan": (ctypes.c_int, [_i32, _i32, _i32, ctypes.POINTER(TopkOptions),
                                 ctypes.POINTER(TopkPlan)]),
    "topk_select_radix": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "topk_sparse_decode": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, ctypes.c_int64, _i32, _i32,
                                          _i32, ctypes.c_float, _vp, _vp]),
    "topk_block_pool": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "topk_pooled_select": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                          _vp]),
    "topk_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "topk_visit_order": (ctypes.c_int, [_u64, _i32, _i32, _vp]),
    "topk_probe_sink_words": (_sz, [_sz]),
    "topk_probe_read": (ctypes.c_int, [_vp, _sz, _vp, _vp]),
    "topk_probe_read_cfg": (ctypes.c_int, [_vp, _sz, _sz, _i32, _i32, _i32, _sz, _vp, _vp]),
    "topk_probe_copy": (ctypes.c_int, [_vp, _vp, _sz, _vp]),
}

_lock = threading.Lock()
_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads the library (once) and declares every signature."""
    global _lib
    with _lock:
        if _lib is not None and path == LIB_PATH:
            return _lib
        if not os.path.exists(path):
            raise ImportError(
                f"HIP top-k library not found at {path}; build it with "
                "`python -m sparse_attention_indexer_row_amd.build` (or __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path == LIB_PATH:
            _lib = lib
        return lib


class TopkError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = load().topk_strerror(status).decode()
        super().__init__(f"{what} failed with status {status} ({msg})")
        self.status = status


def check(status: int, what: str) -> None:
    if status != TOPK_OK:
        raise TopkError(status, what)
