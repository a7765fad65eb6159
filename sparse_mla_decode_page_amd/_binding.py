"""ctypes binding for libmlasd.so (argument marshalling only).

Every step of the decode runs in the HIP kernels behind the C ABI declared in
include/mlasd.h; this module only checks tensor dtypes/shapes, picks the
stream and forwards raw device pointers.  There is no fallback: if the
library is not built, or a call fails, it raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

from ._build import LIB_PATH

HEADS = 64
D_QK = 512
D_V = 448
MAX_TOPK = 512
PAGE_BYTES = 149504

_STATUS_OK = 0
_lib = None


class MlasdError(RuntimeError):
    pass


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load libmlasd.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MlasdError(f"{LIB_PATH} not found: build it first "
                         "(python -m sparse_mla_decode_page_amd._build)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    common = [vp, vp, i64, vp, i32, vp, i32, vp, i32, f32, vp, vp]
    lib.mla_sparse_decode.argtypes = common + [vp]
    lib.mla_sparse_decode.restype = ctypes.c_int
    lib.mla_sparse_decode_ex.argtypes = common + [i32, i32, vp]
    lib.mla_sparse_decode_ex.restype = ctypes.c_int
    lib.mla_sparse_plan.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                    ctypes.POINTER(i32)]
    lib.mla_sparse_plan.restype = ctypes.c_int
    lib.mla_sparse_gather_dequant.argtypes = [vp, i64, vp, i32, vp, i32, vp, i32, vp, vp, vp, vp]
    lib.mla_sparse_gather_dequant.restype = ctypes.c_int
    lib.mla_kv_append.argtypes = [vp, vp, vp, i32, vp, i32, i32, vp, i64, vp]
    lib.mla_kv_append.restype = ctypes.c_int
    lib.mlasd_prepare.argtypes = [vp, i32, i32]
    lib.mlasd_prepare.restype = ctypes.c_int
    lib.mlasd_release.argtypes = [vp]
    lib.mlasd_release.restype = ctypes.c_int
    lib.mlasd_workspace_bytes.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
    lib.mlasd_workspace_bytes.restype = ctypes.c_int
    lib.mlasd_status_string.argtypes = [ctypes.c_int]
    lib.mlasd_status_string.restype = ctypes.c_char_p
    lib.mlasd_last_hip_error.argtypes = []
    lib.mlasd_last_hip_error.restype = ctypes.c_int
    lib.mlasd_version.argtypes = []
    lib.mlasd_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().mlasd_status_string(code).decode()


def _check(rc: int, what: str):
    if rc != _STATUS_OK:
        lib = load_library()
        extra = ""
        if rc == -5:
            extra = f" (hip error {lib.mlasd_last_hip_error()})"
        raise MlasdError(f"{what}: {status_string(rc)}{extra} [{rc}]")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def plan(batch: int, topk: int, nsplit: int = 0, num_cus: int = 0):
    """(nsplit, split_len, head_groups) the library uses for this shape."""
    lib = load_library()
    a, b, c = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib.mla_sparse_plan(batch, topk, nsplit, num_cus, ctypes.byref(a), ctypes.byref(b),
                               ctypes.byref(c)), "mla_sparse_plan")
    return a.value, b.value, c.value


def prepare(max_batch: int, max_topk: int = MAX_TOPK, stream=None, device=None):
    """Reserve the split scratch of `stream` for every automatically planned
    decode with batch <= max_batch and topk <= max_topk (call before graph
    capture)."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    lib = load_library()
    with torch.cuda.device(dev):
        _check(lib.mlasd_prepare(_stream(stream, dev), max_batch, max_topk), "mlasd_prepare")


def release(stream=None, device=None):
    """Free the split scratch of `stream` (synchronises the stream)."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    lib = load_library()
    with torch.cuda.device(dev):
        _check(lib.mlasd_release(_stream(stream, dev)), "mlasd_release")


def workspace_bytes(stream=None, device=None) -> int:
    """Bytes of split scratch the library holds for `stream`."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    lib = load_library()
    n = ctypes.c_size_t(0)
    with torch.cuda.device(dev):
        _check(lib.mlasd_workspace_bytes(_stream(stream, dev), ctypes.byref(n)), "mlasd_workspace_bytes")
    return n.value


def _check_cache_args(kv_pages, page_table, topk_idx, seq_lens):
    _need(kv_pages, "kv_pages", torch.uint8, 2)
    _need(page_table, "page_table", torch.int32, 2)
    _need(topk_idx, "topk_idx", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if kv_pages.shape[1] != PAGE_BYTES:
        raise ValueError(f"kv_pages rows must be {PAGE_BYTES} bytes")
    B = seq_lens.shape[0]
    if page_table.shape[0] != B or topk_idx.shape[0] != B:
        raise ValueError("page_table / topk_idx / seq_lens batch mismatch")
    dev = kv_pages.device
    for t in (page_table, topk_idx, seq_lens):
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return B


def mla_sparse_decode(q, kv_pages, page_table, topk_idx, seq_lens, softmax_scale,
                      out=None, lse=None, stream=None, nsplit=None, head_groups=None):
    """Sparse MLA decode.  Returns (out bf16 [B,64,448], lse f32 [B,64]).

    q bf16 [B,64,512]; kv_pages uint8 [num_pages,149504]; page_table int32
    [B,max_pages]; topk_idx int32 [B,topk]; seq_lens int32 [B].  `nsplit`
    forces the number of top-k slices per query and `head_groups` (1, 2, 4)
    the number of workgroups sharing a slice's heads (None = library plan).
    """
    B = _check_cache_args(kv_pages, page_table, topk_idx, seq_lens)
    _need(q, "q", torch.bfloat16, 3)
    if tuple(q.shape) != (B, HEADS, D_QK):
        raise ValueError(f"q must be [{B},{HEADS},{D_QK}], got {tuple(q.shape)}")
    dev = q.device
    if out is None:
        out = torch.empty((B, HEADS, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, HEADS), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, 3)
    _need(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != (B, HEADS, D_V) or tuple(lse.shape) != (B, HEADS):
        raise ValueError("out / lse shape mismatch")
    lib = load_library()
    with torch.cuda.device(dev):
        args = (_ptr(q), _ptr(kv_pages), kv_pages.shape[0], _ptr(page_table), page_table.shape[1],
                _ptr(topk_idx), topk_idx.shape[1], _ptr(seq_lens), B, float(softmax_scale),
                _ptr(out), _ptr(lse))
        if nsplit is None and head_groups is None:
            rc = lib.mla_sparse_decode(*args, _stream(stream, dev))
        else:
            rc = lib.mla_sparse_decode_ex(*args, int(nsplit or 0), int(head_groups or 0),
                                          _stream(stream, dev))
    _check(rc, "mla_sparse_decode")
    return out, lse


def mla_sparse_gather_dequant(kv_pages, page_table, topk_idx, seq_lens, stream=None):
    """Test hook: (k_rows bf16 [B,topk,512], v_rows fp16 [B,topk,448], valid uint8 [B,topk])
    exactly as the decode kernel's gather + dequant stage produces them."""
    B = _check_cache_args(kv_pages, page_table, topk_idx, seq_lens)
    dev = kv_pages.device
    K = topk_idx.shape[1]
    k_rows = torch.empty((B, K, D_QK), dtype=torch.bfloat16, device=dev)
    v_rows = torch.empty((B, K, D_V), dtype=torch.float16, device=dev)
    valid = torch.empty((B, K), dtype=torch.uint8, device=dev)
    lib = load_library()
    with torch.cuda.device(dev):
        rc = lib.mla_sparse_gather_dequant(_ptr(kv_pages), kv_pages.shape[0], _ptr(page_table),
                                           page_table.shape[1], _ptr(topk_idx), K, _ptr(seq_lens), B,
                                           _ptr(k_rows), _ptr(v_rows), _ptr(valid),
                                           _stream(stream, dev))
    _check(rc, "mla_sparse_gather_dequant")
    return k_rows, v_rows, valid


def mla_kv_append(latent, seq_ids, positions, page_table, kv_pages, stream=None):
    """Quantise token latents (bf16 [N, 512]) into the paged cache in place.
    seq_ids / positions int32 [N]; page_table int32 [B, max_pages]."""
    _need(latent, "latent", torch.bfloat16, 2)
    _need(seq_ids, "seq_ids", torch.int32, 1)
    _need(positions, "positions", torch.int32, 1)
    _need(page_table, "page_table", torch.int32, 2)
    _need(kv_pages, "kv_pages", torch.uint8, 2)
    n = latent.shape[0]
    if latent.shape[1] != D_QK:
        raise ValueError(f"latent must be [N, {D_QK}]")
    if seq_ids.shape[0] != n or positions.shape[0] != n:
        raise ValueError("seq_ids / positions must have one entry per token")
    if kv_pages.shape[1] != PAGE_BYTES:
        raise ValueError(f"kv_pages rows must be {PAGE_BYTES} bytes")
    dev = kv_pages.device
    for t in (latent, seq_ids, positions, page_table):
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
    lib = load_library()
    with torch.cuda.device(dev):
        rc = lib.mla_kv_append(_ptr(latent), _ptr(seq_ids), _ptr(positions), n, _ptr(page_table),
                               page_table.shape[0], page_table.shape[1], _ptr(kv_pages),
                               kv_pages.shape[0], _stream(stream, dev))
    _check(rc, "mla_kv_append")
    return kv_pages

