"""Exact per-row top-k selection for MI355X (gfx950), hand-written HIP.

The C ABI lives in ``include/topk_select.h`` and ``libtopk_select.so``; the
functions below (same names as the C entry points) take PyTorch GPU tensors.
Importing the package does not load the library; the first call does, and
fails loudly if it has not been built.
"""

_API = (
    "topk_select", "topk_select_split", "topk_select_ex", "topk_split_workspace_bytes",
    "topk_workspace_init", "topk_plan", "topk_strerror", "topk_visit_order",
    "topk_probe_read", "topk_probe_copy", "new_workspace", "TopkError",
)


def __getattr__(name):
    if name in _API:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)


__all__ = list(_API)
