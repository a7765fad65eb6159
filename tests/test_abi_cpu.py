"""C-ABI checks that need no GPU: the library loads, exports every function
include/mlasd.h declares, rejects bad descriptors on the host before touching
a device, and plans splits as documented."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_mla_decode_page_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
U8, I32, BF16, F32 = 1, 2, 3, 4


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(m\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_entry_points():
    names = _declared_functions()
    for n in ("mla_sparse_decode", "mla_sparse_decode_ex", "mla_sparse_gather_dequant",
              "mla_sparse_plan", "mla_sparse_workspace_size", "mla_kv_append", "mlasd_prepare",
              "mlasd_reserve", "mlasd_release", "mlasd_workspace_bytes", "mlasd_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = m.load_library()
    out = subprocess.run(["nm", "-D", "--defined-only", m.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for n in _declared_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_descriptor_layout_matches_header():
    """mlasd_tensor is pointer, two int32, then two int64[4]: 80 bytes."""
    assert ctypes.sizeof(m.Tensor) == 8 + 4 + 4 + 32 + 32
    assert m.Tensor.shape.offset == 16 and m.Tensor.stride.offset == 48


def test_status_strings():
    lib = m.load_library()
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        assert m.status_string(code) != "unknown status"
    assert m.status_string(-99) == "unknown status"
    assert lib.mlasd_version().decode().startswith("mlasd")


def _t(data, dtype, shape, stride=None):
    d = m.Tensor()
    d.data = data
    d.dtype = dtype
    d.ndim = len(shape)
    if stride is None:
        stride, acc = [], 1
        for s in reversed(shape):
            stride.insert(0, acc)
            acc *= s
    for k, (s, st) in enumerate(zip(shape, stride)):
        d.shape[k] = s
        d.stride[k] = st
    return d


def _decode_args(B=2, topk=4, num_pages=3, max_pages=2):
    """Descriptors of a well-formed decode call with fake (never touched) pointers."""
    return dict(
        q=_t(0x10000, BF16, [B, 64, 512]),
        kv=_t(0x20000, U8, [num_pages, 149504]),
        pt=_t(0x30000, I32, [B, max_pages]),
        idx=_t(0x40000, I32, [B, topk]),
        lens=_t(0x50000, I32, [B]),
        out=_t(0x60000, BF16, [B, 64, 448]),
        lse=_t(0x70000, F32, [B, 64]),
    )


def _decode(lib, a, scale=0.1, nsplit=None, hg=0):
    r = ctypes.byref
    args = (r(a["q"]), r(a["kv"]), r(a["pt"]), r(a["idx"]), r(a["lens"]), ctypes.c_float(scale),
            r(a["out"]), r(a["lse"]))
    if nsplit is None:
        return lib.mla_sparse_decode(*args, None)
    return lib.mla_sparse_decode_ex(*args, nsplit, hg, None)


def _mut(name, **kw):
    def f(a):
        d = a[name]
        for k, v in kw.items():
            if k in ("shape", "stride"):
                for i, x in enumerate(v):
                    getattr(d, k)[i] = x
            else:
                setattr(d, k, v)
    return f


CASES = [
    ("q null", _mut("q", data=0), -1),
    ("kv null", _mut("kv", data=0), -1),
    ("out null", _mut("out", data=0), -1),
    ("lse null", _mut("lse", data=0), -1),
    ("q dtype", _mut("q", dtype=F32), -2),
    ("q heads", _mut("q", shape=[2, 32, 512]), -2),
    ("q dim", _mut("q", shape=[2, 64, 576]), -2),
    ("q batch", _mut("q", shape=[3, 64, 512]), -2),
    ("q inner stride", _mut("q", stride=[32768, 512, 2]), -2),
    ("q misaligned", _mut("q", data=0x10008), -3),
    ("q head stride not x8", _mut("q", stride=[64 * 516, 516, 1]), -3),
    ("q batch stride padded ok-ish but not x8", _mut("q", stride=[32772, 512, 1]), -3),
    ("kv row bytes", _mut("kv", shape=[3, 147456]), -2),
    ("kv page stride < page", _mut("kv", stride=[147456, 1]), -2),
    ("kv page stride not x16", _mut("kv", stride=[149512, 1]), -3),
    ("kv misaligned", _mut("kv", data=0x20004), -3),
    ("kv empty pool", _mut("kv", shape=[0, 149504]), -2),
    ("pt batch", _mut("pt", shape=[3, 2]), -2),
    ("pt zero pages", _mut("pt", shape=[2, 0]), -2),
    ("pt dtype", _mut("pt", dtype=U8), -2),
    ("idx topk > 512", _mut("idx", shape=[2, 513]), -2),
    ("idx misaligned", _mut("idx", data=0x40002), -3),
    ("lens rank", _mut("lens", ndim=2), -2),
    ("out dims", _mut("out", shape=[2, 64, 512]), -2),
    ("out misaligned", _mut("out", data=0x60008), -3),
    ("lse shape", _mut("lse", shape=[2, 32]), -2),
    ("lse misaligned", _mut("lse", data=0x70002), -3),
    ("negative stride", _mut("pt", stride=[-2, 1]), -2),
]


@pytest.mark.parametrize("name,mutate,code", CASES, ids=[c[0] for c in CASES])
def test_host_validation_without_device(name, mutate, code):
    lib = m.load_library()
    a = _decode_args()
    mutate(a)
    assert _decode(lib, a) == code


def test_scalar_and_plan_validation_without_device():
    lib = m.load_library()
    assert _decode(lib, _decode_args(), scale=float("nan")) == -4
    assert _decode(lib, _decode_args(), scale=float("inf")) == -4
    for hg in (3, 4, 5, -1):
        assert _decode(lib, _decode_args(), nsplit=2, hg=hg) == -2


def test_empty_batch_is_a_noop_without_device():
    lib = m.load_library()
    a = _decode_args(B=0)
    assert _decode(lib, a) == 0
    for k in ("q", "out", "lse", "idx", "lens"):
        a[k].data = 0
    assert _decode(lib, a) == 0


def test_strided_views_pass_host_validation():
    """Padded page rows, a batch-strided q/out and a shared (stride 0) page
    table are accepted by the host checks; the call then needs a device
    (HIP error here, with no GPU), which proves validation went through."""
    lib = m.load_library()
    a = _decode_args()
    a["kv"] = _t(0x20000, U8, [3, 149504], [149504 + 512, 1])
    a["q"] = _t(0x10000, BF16, [2, 64, 512], [64 * 512 + 64, 512, 1])
    a["out"] = _t(0x60000, BF16, [2, 64, 448], [64 * 512, 512, 1])
    a["pt"] = _t(0x30000, I32, [2, 2], [0, 1])
    a["lens"] = _t(0x50000, I32, [2], [3])
    assert _decode(lib, a) in (-5, -6)


def test_gather_hook_validation_without_device():
    lib = m.load_library()
    r = ctypes.byref
    a = _decode_args()
    rows = _t(0x80000, F32, [2, 4, 512])
    valid = _t(0x90000, U8, [2, 4])
    f = lib.mla_sparse_gather_dequant
    assert f(r(a["kv"]), r(a["pt"]), r(a["idx"]), r(a["lens"]), r(_t(0, F32, [2, 4, 512])), r(valid), None) == -1
    assert f(r(a["kv"]), r(a["pt"]), r(a["idx"]), r(a["lens"]), r(_t(0x80000, BF16, [2, 4, 512])), r(valid),
             None) == -2
    assert f(r(a["kv"]), r(a["pt"]), r(a["idx"]), r(a["lens"]), r(_t(0x80008, F32, [2, 4, 512])), r(valid),
             None) == -3
    assert f(r(a["kv"]), r(a["pt"]), r(a["idx"]), r(a["lens"]), r(rows), r(_t(0x90000, U8, [2, 5])), None) == -2
    e = _decode_args(topk=0)
    assert f(r(e["kv"]), r(e["pt"]), r(e["idx"]), r(e["lens"]), r(_t(0, F32, [2, 0, 512])),
             r(_t(0, U8, [2, 0])), None) == 0


def test_prepare_validation_without_device():
    lib = m.load_library()
    assert lib.mlasd_prepare(None, -1, 512) == -2
    assert lib.mlasd_prepare(None, 4, 513) == -2
    assert lib.mlasd_prepare(None, 4, -1) == -2
    assert lib.mlasd_reserve(None, 0) == 0
    assert lib.mlasd_workspace_bytes(None, None) == -1


def test_workspace_size_host_only():
    """Bytes of fp32 partials (448 values + 1 lse per head, slice and query)
    for split plans, 0 for unsplit ones -- planned for a given CU count, so no
    device is needed."""
    assert m.workspace_size(16, 512, 4, 0, 256) == 16 * 4 * 64 * 449 * 4
    assert m.workspace_size(256, 512, 0, 0, 256) == 0
    ns = m.plan(1, 512, 0, 256)[0]
    assert m.workspace_size(1, 512, 0, 0, 256) == ns * 64 * 449 * 4
    with pytest.raises(m.MlasdError):
        m.workspace_size(1, 513, 0, 0, 256)
    with pytest.raises(m.MlasdError):
        m.workspace_size(1, 512, 0, 3, 256)


@pytest.mark.parametrize("cus", [256, 304, 80])
def test_prepare_bound_covers_smaller_topk(cus):
    """mlasd_prepare sizes the scratch from the automatic plans at max_topk
    for every batch up to max_batch.  That bound must hold for every smaller
    top-k too, although the plan drops a split that does not pay for its
    combine: check it over all top-k values for several max_batch."""
    for max_batch in (1, 2, 3, 8, 16, 64, 128):
        for max_topk in (64, 192, 256, 300, 512):
            bound = max(m.workspace_size(b, max_topk, 0, 0, cus) for b in range(1, max_batch + 1))
            for b in range(1, max_batch + 1):
                for k in range(1, max_topk + 1, 3):
                    assert m.workspace_size(b, k, 0, 0, cus) <= bound, (cus, max_batch, max_topk, b, k)


def _append_args(n=4, B=2, max_pages=2, num_pages=3):
    return dict(lat=_t(0x10000, BF16, [n, 512]), seq=_t(0x20000, I32, [n]), pos=_t(0x30000, I32, [n]),
                pt=_t(0x40000, I32, [B, max_pages]), kv=_t(0x50000, U8, [num_pages, 149504]))


def _append(lib, a):
    r = ctypes.byref
    return lib.mla_kv_append(r(a["lat"]), r(a["seq"]), r(a["pos"]), r(a["pt"]), r(a["kv"]), None)


ACASES = [
    ("latent null", _mut("lat", data=0), -1),
    ("latent dims", _mut("lat", shape=[4, 448]), -2),
    ("latent misaligned", _mut("lat", data=0x10008), -3),
    ("latent row stride", _mut("lat", stride=[516, 1]), -3),
    ("seq count", _mut("seq", shape=[3]), -2),
    ("pos null", _mut("pos", data=0), -1),
    ("pos misaligned", _mut("pos", data=0x30002), -3),
    ("pt empty batch", _mut("pt", shape=[0, 2]), -2),
    ("pt zero pages", _mut("pt", shape=[2, 0]), -2),
    ("kv empty", _mut("kv", shape=[0, 149504]), -2),
    ("kv misaligned", _mut("kv", data=0x50008), -3),
]


@pytest.mark.parametrize("name,mutate,code", ACASES, ids=[c[0] for c in ACASES])
def test_append_validation_without_device(name, mutate, code):
    lib = m.load_library()
    a = _append_args()
    mutate(a)
    assert _append(lib, a) == code


def test_append_zero_tokens_is_a_noop():
    lib = m.load_library()
    a = _append_args(n=0)
    a["lat"].data = 0
    a["kv"].data = 0
    assert _append(lib, a) == 0


@pytest.mark.parametrize("batch,topk,req,cus,expect", [
    (64, 512, 0, 256, (2, 256, 2)),    # 4 workgroups per query: 2 head groups x 2 slices
    (56, 512, 0, 256, (2, 256, 2)),
    (64, 512, 0, 240, (1, 512, 2)),    # 3 workgroups per query: 2 head groups, no split
    (1, 512, 0, 256, (8, 64, 2)),      # small batch: slices of at least 64 entries
    (16, 512, 0, 256, (8, 64, 2)),
    (2, 512, 0, 256, (8, 64, 2)),
    (4, 512, 0, 256, (8, 64, 2)),
    (17, 512, 0, 256, (6, 96, 2)),     # 15 workgroups per query: 7 slices -> 96-entry slices -> 6
    (32, 512, 0, 256, (4, 128, 2)),
    (128, 512, 0, 256, (1, 512, 2)),   # 2 workgroups per query: head groups, no split
    (100, 512, 0, 256, (1, 512, 2)),
    (129, 512, 0, 256, (1, 512, 1)),   # batch fills the GPU: 64 heads, no split
    (256, 512, 0, 256, (1, 512, 1)),
    (1, 64, 0, 256, (1, 64, 2)),
    (3, 300, 0, 256, (5, 64, 2)),      # ragged top-k
    (3, 45, 0, 256, (1, 64, 2)),
    (1, 0, 0, 256, (1, 32, 2)),        # empty top-k: one slice, writes zeros / -inf
    (64, 512, 1, 256, (1, 512, 2)),    # forced
    (64, 512, 3, 256, (3, 192, 2)),    # slices hold whole 32-token tiles
    (64, 512, 99, 256, (16, 32, 2)),   # clamped to ceil(topk/32)
    (8, 100, 0, 80, (1, 128, 2)),      # 10 workgroups per query, but 2 slices of 2 tiles do not pay for a split
    (64, 256, 0, 256, (1, 256, 2)),    # 2 slices would take 4 tiles off each workgroup: not worth a combine
    (64, 128, 0, 256, (1, 128, 2)),
    (1, 128, 0, 256, (1, 128, 2)),
    (1, 256, 0, 256, (4, 64, 2)),      # 6 tiles off each workgroup: split
    (16, 256, 0, 256, (4, 64, 2)),
    (48, 512, 0, 256, (2, 256, 2)),
    (32, 512, 0, 80, (1, 512, 2)),
])
def test_plan(batch, topk, req, cus, expect):
    ns, sl, hg = m.plan(batch, topk, req, cus)
    assert (ns, sl, hg) == expect
    assert sl % 32 == 0 and ns * sl >= topk and (ns - 1) * sl < max(topk, 1)
    if req == 0:
        assert batch * ns * hg <= max(cus, batch)   # one round of workgroups


def _topk(lib, scores, lens, idx):
    r = ctypes.byref
    return lib.mla_topk_select(r(scores) if scores is not None else None, r(lens), r(idx), None)


def test_topk_select_validation_without_device():
    """mla_topk_select's argument checks, all before any device work."""
    lib = m.load_library()
    ok = dict(scores=_t(0x10000, F32, [4, 1000]), lens=_t(0x20000, I32, [4]), idx=_t(0x30000, I32, [4, 512]))
    assert _topk(lib, None, ok["lens"], ok["idx"]) == -1
    assert _topk(lib, _t(0x10000, I32, [4, 1000]), ok["lens"], ok["idx"]) == -2      # scores dtype
    assert _topk(lib, _t(0x10000, F32, [4000]), ok["lens"], ok["idx"]) == -2         # scores rank
    assert _topk(lib, _t(0x10000, F32, [4, 1000], [1000, 2]), ok["lens"], ok["idx"]) == -2   # not contiguous
    assert _topk(lib, ok["scores"], _t(0x20000, I32, [3]), ok["idx"]) == -2          # seq_lens length
    assert _topk(lib, ok["scores"], ok["lens"], _t(0x30000, I32, [4, 513])) == -2    # k > 512
    assert _topk(lib, ok["scores"], ok["lens"], _t(0x30000, I32, [5, 512])) == -2    # batch mismatch
    assert _topk(lib, ok["scores"], ok["lens"], _t(0x30000, F32, [4, 512])) == -2    # out dtype
    assert _topk(lib, ok["scores"], ok["lens"], _t(0x30002, I32, [4, 512])) == -3    # out misaligned
    # empty work is a no-op
    assert _topk(lib, _t(0, F32, [0, 1000]), _t(0, I32, [0]), _t(0, I32, [0, 512])) == 0
    assert _topk(lib, ok["scores"], ok["lens"], _t(0x30000, I32, [4, 0])) == 0
    # forced parts: more than 8 refused; the argument checks come first
    r = ctypes.byref
    ex = lib.mla_topk_select_ex
    assert ex(r(ok["scores"]), r(ok["lens"]), r(ok["idx"]), 9, None) == -2
    assert ex(None, r(ok["lens"]), r(ok["idx"]), 2, None) == -1
    assert ex(r(_t(0x10000, I32, [4, 1000])), r(ok["lens"]), r(ok["idx"]), 2, None) == -2
    assert ex(r(_t(0, F32, [0, 1000])), r(_t(0, I32, [0])), r(_t(0, I32, [0, 512])), 4, None) == 0


@pytest.mark.parametrize("batch,max_len,req,cus,expect", [
    (64, 65536, 0, 256, 4),     # the indexer's B=64 x 65,536: four workgroups per row
    (1, 131072, 0, 256, 8),     # at most 8 parts
    (16, 65536, 0, 256, 4),     # parts of at least 16,384 positions
    (1, 65535, 0, 256, 1),      # fewer than 4 parts of 16,384: not cut
    (128, 131072, 0, 256, 1),   # only 2 compute units per row: not cut
    (64, 131072, 0, 256, 4),
    (256, 131072, 0, 256, 1),   # every compute unit already has a row
    (64, 32768, 0, 256, 1),
    (0, 65536, 0, 256, 1),
    (64, 65536, 8, 0, 8),       # forced: no device needed
    (3, 100, 1, 0, 1),
])
def test_topk_plan(batch, max_len, req, cus, expect):
    parts, nbytes = m.topk_plan(batch, max_len, req, cus)
    assert parts == expect
    # per row: the candidate list (16,384 composites of 8 bytes) shared by the parts, and a 32-byte
    # record per part (count, threshold, largest composite)
    assert nbytes == (0 if parts == 1 else batch * parts * ((16384 // parts) * 8 + 32))


def test_topk_plan_validation():
    with pytest.raises(m.MlasdError):
        m.topk_plan(4, 1000, 9, 256)
    with pytest.raises(m.MlasdError):
        m.topk_plan(-1, 1000, 0, 256)
    with pytest.raises(m.MlasdError):
        m.topk_plan(4, -1, 0, 256)
