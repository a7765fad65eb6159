"""Sparse MLA paged decode for MI355X (gfx950): Python binding of libmlasd.

The decode runs in hand-written HIP kernels behind a C ABI
(include/mlasd.h); this package only marshals torch tensors to it.
"""
from ._binding import (  # noqa: F401
    MlasdError,
    Tensor,
    describe,
    library_path,
    load_library,
    mla_kv_append,
    mla_sparse_decode,
    mla_sparse_decode_noalloc,
    mla_sparse_gather_dequant,
    mla_topk_select,
    plan,
    prepare,
    release,
    reserve,
    status_string,
    topk_plan,
    workspace_bytes,
    workspace_size,
)

__all__ = ["mla_sparse_decode", "mla_sparse_decode_noalloc", "mla_sparse_gather_dequant", "mla_kv_append",
           "mla_topk_select", "topk_plan", "plan", "prepare",
           "reserve", "release", "workspace_bytes", "workspace_size", "describe", "Tensor",
           "load_library", "library_path", "status_string", "MlasdError"]
