"""ctypes binding for libmlasd.so (argument marshalling only).

Every step of the decode runs in the HIP kernels behind the C ABI declared in
include/mlasd.h; this module only turns torch tensors into mlasd_tensor
descriptors (pointer, dtype, shape, strides), picks the stream and forwards
the call.  Shape, stride and alignment rules are checked by the library
itself.  There is no fallback: if the library is not built, or a call
fails, it raises.
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

STATUS_WORKSPACE = -8
_STATUS_OK = 0
_lib = None

_DTYPES = {torch.uint8: 1, torch.int32: 2, torch.bfloat16: 3, torch.float32: 4}


class MlasdError(RuntimeError):
    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


class Tensor(ctypes.Structure):
    """mlasd_tensor: device pointer, dtype, ndim, shape[4], stride[4] (elements)."""
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


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
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    T = ctypes.POINTER(Tensor)
    lib.mla_sparse_decode.argtypes = [T, T, T, T, T, f32, T, T, vp]
    lib.mla_sparse_decode_ex.argtypes = [T, T, T, T, T, f32, T, T, i32, i32, vp]
    lib.mla_sparse_decode_noalloc.argtypes = [T, T, T, T, T, f32, T, T, vp]
    lib.mla_sparse_plan.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                    ctypes.POINTER(i32)]
    lib.mla_sparse_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.mla_sparse_gather_dequant.argtypes = [T, T, T, T, T, T, vp]
    lib.mla_kv_append.argtypes = [T, T, T, T, T, vp]
    lib.mla_topk_select.argtypes = [T, T, T, vp]
    lib.mla_topk_select_ex.argtypes = [T, T, T, i32, vp]
    lib.mla_topk_plan.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(sz)]
    lib.mlasd_prepare.argtypes = [vp, i32, i32]
    lib.mlasd_reserve.argtypes = [vp, sz]
    lib.mlasd_release.argtypes = [vp]
    lib.mlasd_workspace_bytes.argtypes = [vp, ctypes.POINTER(sz)]
    for name in ("mla_sparse_decode", "mla_sparse_decode_ex", "mla_sparse_decode_noalloc", "mla_sparse_plan",
                 "mla_sparse_workspace_size", "mla_sparse_gather_dequant", "mla_kv_append", "mla_topk_select",
                 "mla_topk_select_ex", "mla_topk_plan", "mlasd_prepare", "mlasd_reserve", "mlasd_release", "mlasd_workspace_bytes"):
        getattr(lib, name).restype = ctypes.c_int
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
        raise MlasdError(f"{what}: {status_string(rc)}{extra} [{rc}]", rc)


def describe(t) -> Tensor:
    """mlasd_tensor descriptor of a torch tensor (no copy, no checks: the
    library validates dtype, shape, strides and alignment)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() > 4 or t.dim() < 1:
        raise ValueError(f"tensor rank {t.dim()} not supported")
    d = Tensor()
    d.data = t.data_ptr() if t.numel() > 0 else 0
    d.dtype = _DTYPES[t.dtype]
    d.ndim = t.dim()
    for k in range(t.dim()):
        d.shape[k] = t.shape[k]
        d.stride[k] = t.stride(k)
    return d


def _same_device(*ts):
    dev = None
    for t in ts:
        if not t.is_cuda:
            raise ValueError("all tensors must be device tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _device(device):
    return torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())


def plan(batch: int, topk: int, nsplit: int = 0, num_cus: int = 0):
    """(nsplit, split_len, head_groups) the library uses for this shape."""
    lib = load_library()
    a, b, c = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib.mla_sparse_plan(batch, topk, nsplit, num_cus, ctypes.byref(a), ctypes.byref(b),
                               ctypes.byref(c)), "mla_sparse_plan")
    return a.value, b.value, c.value


def workspace_size(batch: int, topk: int, nsplit: int = 0, head_groups: int = 0, num_cus: int = 0) -> int:
    """Bytes of split scratch a decode of this shape and plan needs."""
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.mla_sparse_workspace_size(batch, topk, nsplit, head_groups, num_cus, ctypes.byref(n)),
           "mla_sparse_workspace_size")
    return n.value


def prepare(max_batch: int, max_topk: int = MAX_TOPK, stream=None, device=None):
    """Reserve the split scratch of `stream` for every automatically planned
    decode with batch <= max_batch and topk <= max_topk (before graph capture)."""
    dev = _device(device)
    lib = load_library()
    with torch.cuda.device(dev):
        _check(lib.mlasd_prepare(_stream(stream, dev), max_batch, max_topk), "mlasd_prepare")


def reserve(nbytes: int, stream=None, device=None):
    """Reserve at least `nbytes` of split scratch for `stream`."""
    dev = _device(device)
    lib = load_library()
    with torch.cuda.device(dev):
        _check(lib.mlasd_reserve(_stream(stream, dev), nbytes), "mlasd_reserve")


def release(stream=None, device=None):
    """Free the split scratch of `stream` (synchronises the stream)."""
    dev = _device(device)
    lib = load_library()
    with torch.cuda.device(dev):
        _check(lib.mlasd_release(_stream(stream, dev)), "mlasd_release")


def workspace_bytes(stream=None, device=None) -> int:
    """Bytes of split scratch the library holds for `stream`."""
    dev = _device(device)
    lib = load_library()
    n = ctypes.c_size_t(0)
    with torch.cuda.device(dev):
        _check(lib.mlasd_workspace_bytes(_stream(stream, dev), ctypes.byref(n)), "mlasd_workspace_bytes")
    return n.value


def mla_sparse_decode(q, kv_pages, page_table, topk_idx, seq_lens, softmax_scale,
                      out=None, lse=None, stream=None, nsplit=None, head_groups=None):
    """Sparse MLA decode.  Returns (out bf16 [B,64,448], lse f32 [B,64]).

    q bf16 [B,64,512]; kv_pages uint8 [num_pages,149504] (any page stride);
    page_table int32 [B,max_pages]; topk_idx int32 [B,topk]; seq_lens int32
    [B].  `nsplit` forces the number of top-k slices per query and
    `head_groups` (1, 2) the number of workgroups sharing a slice's heads
    (None = library plan).  Split plans need scratch reserved with
    prepare() / reserve() on the stream first.
    """
    dev = _same_device(q, kv_pages, page_table, topk_idx, seq_lens)
    B = seq_lens.shape[0] if seq_lens.dim() == 1 else -1
    if out is None:
        out = torch.empty((B, HEADS, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, HEADS), dtype=torch.float32, device=dev)
    _same_device(out, lse, q)
    lib = load_library()
    descs = [describe(t) for t in (q, kv_pages, page_table, topk_idx, seq_lens)]
    do, dl = describe(out), describe(lse)
    with torch.cuda.device(dev):
        args = [ctypes.byref(d) for d in descs] + [float(softmax_scale), ctypes.byref(do), ctypes.byref(dl)]
        if nsplit is None and head_groups is None:
            rc = lib.mla_sparse_decode(*args, _stream(stream, dev))
        else:
            rc = lib.mla_sparse_decode_ex(*args, int(nsplit or 0), int(head_groups or 0),
                                          _stream(stream, dev))
    _check(rc, "mla_sparse_decode")
    return out, lse


def mla_sparse_decode_noalloc(q, kv_pages, page_table, topk_idx, seq_lens, softmax_scale, out, lse,
                              stream=None):
    """mla_sparse_decode through the entry point that allocates nothing (its
    split partials live in the library's static per-GPU array).  `out` and
    `lse` must be given: this path allocates no tensors either."""
    dev = _same_device(q, kv_pages, page_table, topk_idx, seq_lens, out, lse)
    lib = load_library()
    descs = [describe(t) for t in (q, kv_pages, page_table, topk_idx, seq_lens)]
    do, dl = describe(out), describe(lse)
    with torch.cuda.device(dev):
        args = [ctypes.byref(d) for d in descs] + [float(softmax_scale), ctypes.byref(do), ctypes.byref(dl)]
        rc = lib.mla_sparse_decode_noalloc(*args, _stream(stream, dev))
    _check(rc, "mla_sparse_decode_noalloc")
    return out, lse


def mla_sparse_gather_dequant(kv_pages, page_table, topk_idx, seq_lens, stream=None):
    """Test hook: (rows f32 [B,topk,512], valid uint8 [B,topk]) exactly as the
    decode kernel's gather + dequant stage holds them."""
    dev = _same_device(kv_pages, page_table, topk_idx, seq_lens)
    B, K = topk_idx.shape[0], topk_idx.shape[1]
    rows = torch.empty((B, K, D_QK), dtype=torch.float32, device=dev)
    valid = torch.empty((B, K), dtype=torch.uint8, device=dev)
    lib = load_library()
    descs = [describe(t) for t in (kv_pages, page_table, topk_idx, seq_lens, rows, valid)]
    with torch.cuda.device(dev):
        rc = lib.mla_sparse_gather_dequant(*[ctypes.byref(d) for d in descs], _stream(stream, dev))
    _check(rc, "mla_sparse_gather_dequant")
    return rows, valid


def mla_kv_append(latent, seq_ids, positions, page_table, kv_pages, stream=None):
    """Quantise token latents (bf16 [N, 512]) into the paged cache in place.
    seq_ids / positions int32 [N]; page_table int32 [B, max_pages]."""
    dev = _same_device(latent, seq_ids, positions, page_table, kv_pages)
    lib = load_library()
    descs = [describe(t) for t in (latent, seq_ids, positions, page_table, kv_pages)]
    with torch.cuda.device(dev):
        rc = lib.mla_kv_append(*[ctypes.byref(d) for d in descs], _stream(stream, dev))
    _check(rc, "mla_kv_append")
    return kv_pages


def mla_topk_select(scores, seq_lens, k=MAX_TOPK, out=None, stream=None, parts=None):
    """Each query's top-k positions from its indexer scores (fp32 [B,
    max_len]; candidates 0 .. min(seq_len, max_len) - 1): int32 [B, k] in
    rank order (higher score first, ties by lower position), -1 padded.
    `parts` forces the workgroups per long row of the candidate pass (None:
    library plan, which cuts rows only when the stream's scratch holds
    topk_plan's bytes; a forced split needs them reserved)."""
    dev = _same_device(scores, seq_lens)
    B = scores.shape[0] if scores.dim() == 2 else -1
    if out is None:
        out = torch.empty((B, int(k)), dtype=torch.int32, device=dev)
    _same_device(out, scores)
    lib = load_library()
    descs = [describe(t) for t in (scores, seq_lens, out)]
    with torch.cuda.device(dev):
        args = [ctypes.byref(d) for d in descs]
        if parts is None:
            rc = lib.mla_topk_select(*args, _stream(stream, dev))
        else:
            rc = lib.mla_topk_select_ex(*args, int(parts), _stream(stream, dev))
    _check(rc, "mla_topk_select")
    return out


def topk_plan(batch: int, max_len: int, parts: int = 0, num_cus: int = 0):
    """(parts per row, bytes of split scratch) of a top-k selection over
    [batch, max_len] scores."""
    lib = load_library()
    a, n = ctypes.c_int32(0), ctypes.c_size_t(0)
    _check(lib.mla_topk_plan(batch, max_len, parts, num_cus, ctypes.byref(a), ctypes.byref(n)), "mla_topk_plan")
    return a.value, n.value
