"""C-ABI checks that need no GPU: the library loads, exports every function
include/mlasd.h declares, rejects bad arguments on the host before touching
a device, and plans splits as documented."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_mla_decode_page_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


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
              "mla_sparse_plan", "mla_kv_append", "mlasd_prepare", "mlasd_release",
              "mlasd_workspace_bytes", "mlasd_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = m.load_library()
    out = subprocess.run(["nm", "-D", "--defined-only", m.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for n in _declared_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_status_strings():
    lib = m.load_library()
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert m.status_string(code) != "unknown status"
    assert m.status_string(-99) == "unknown status"
    assert lib.mlasd_version().decode().startswith("mlasd")


def _decode(lib, q=0x1000, kv=0x1000, num_pages=1, pt=0x1000, max_pages=1, idx=0x1000, topk=4,
            lens=0x1000, batch=1, scale=0.1, out=0x1000, lse=0x1000, nsplit=None, hg=0):
    vp = ctypes.c_void_p
    args = (vp(q), vp(kv), num_pages, vp(pt), max_pages, vp(idx), topk, vp(lens), batch, scale,
            vp(out), vp(lse))
    if nsplit is None:
        return lib.mla_sparse_decode(*args, vp(0))
    return lib.mla_sparse_decode_ex(*args, nsplit, hg, vp(0))


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(topk=-1), -2), (dict(topk=513), -2), (dict(num_pages=0), -2),
    (dict(max_pages=0), -2), (dict(kv=0), -1), (dict(pt=0), -1), (dict(lens=0), -1),
    (dict(idx=0), -1), (dict(q=0), -1), (dict(out=0), -1), (dict(lse=0), -1),
    (dict(q=0x1008), -3), (dict(kv=0x1004), -3), (dict(out=0x1004), -3), (dict(lse=0x1002), -3),
    (dict(idx=0x1002), -3), (dict(scale=float("nan")), -4), (dict(scale=float("inf")), -4),
    (dict(batch=0), 0), (dict(batch=0, q=0, out=0, lse=0), 0),
    (dict(topk=600, nsplit=2), -2), (dict(nsplit=2, hg=3), -2), (dict(nsplit=2, hg=5), -2), (dict(nsplit=0, hg=-1), -2),
])
def test_host_validation_without_device(kw, code):
    lib = m.load_library()
    assert _decode(lib, **kw) == code


def test_gather_hook_validation_without_device():
    lib = m.load_library()
    vp = ctypes.c_void_p
    f = lib.mla_sparse_gather_dequant
    assert f(vp(0x1000), 1, vp(0x1000), 1, vp(0x1000), 4, vp(0x1000), -1, vp(0x1000), vp(0x1000),
             vp(0x1000), vp(0)) == -2
    assert f(vp(0x1000), 1, vp(0x1000), 1, vp(0x1000), 4, vp(0x1000), 1, vp(0), vp(0x1000),
             vp(0x1000), vp(0)) == -1
    assert f(vp(0x1000), 1, vp(0x1000), 1, vp(0x1000), 4, vp(0x1000), 1, vp(0x1008), vp(0x1000),
             vp(0x1000), vp(0)) == -3
    assert f(vp(0x1000), 1, vp(0x1000), 1, vp(0x1000), 0, vp(0x1000), 1, vp(0), vp(0), vp(0), vp(0)) == 0


def test_prepare_validation_without_device():
    lib = m.load_library()
    vp = ctypes.c_void_p
    assert lib.mlasd_prepare(vp(0), -1, 512) == -2
    assert lib.mlasd_prepare(vp(0), 4, 513) == -2
    assert lib.mlasd_prepare(vp(0), 4, -1) == -2
    assert lib.mlasd_workspace_bytes(vp(0), None) == -1


def _append(lib, latent=0x1000, seq=0x1000, pos=0x1000, n=4, pt=0x1000, batch=1, max_pages=1,
            kv=0x1000, num_pages=1):
    vp = ctypes.c_void_p
    return lib.mla_kv_append(vp(latent), vp(seq), vp(pos), n, vp(pt), batch, max_pages, vp(kv),
                             num_pages, vp(0))


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), -2), (dict(batch=-1), -2), (dict(batch=0), -2), (dict(max_pages=0), -2),
    (dict(num_pages=0), -2), (dict(latent=0), -1), (dict(seq=0), -1), (dict(pos=0), -1),
    (dict(pt=0), -1), (dict(kv=0), -1), (dict(latent=0x1008), -3), (dict(kv=0x1008), -3),
    (dict(pos=0x1002), -3), (dict(n=0), 0), (dict(n=0, latent=0, kv=0), 0),
])
def test_append_validation_without_device(kw, code):
    lib = m.load_library()
    assert _append(lib, **kw) == code


@pytest.mark.parametrize("batch,topk,req,cus,expect", [
    (64, 512, 0, 256, (1, 512, 4)),    # 4 workgroups per query filling the GPU: 4 head groups, no split
    (56, 512, 0, 256, (2, 256, 2)),    # 4 workgroups per query, 224 of 256 CUs: 2 slices x 2 head groups
    (64, 512, 0, 240, (1, 512, 2)),    # 3 workgroups per query: 2 head groups, no split
    (1, 512, 0, 256, (8, 64, 4)),      # small batch: slices of at least 64 entries
    (16, 512, 0, 256, (4, 128, 4)),    # >= 16 workgroups per query: 16-head workgroups
    (2, 512, 0, 256, (8, 64, 4)),      # B * nsplit * 4 <= CUs / 4: 16-head workgroups
    (4, 512, 0, 256, (8, 64, 4)),
    (17, 512, 0, 256, (6, 96, 2)),     # 15 workgroups per query: slices of 32-head groups
    (32, 512, 0, 256, (4, 128, 2)),
    (128, 512, 0, 256, (1, 512, 2)),   # 2 workgroups per query: head groups, no split
    (100, 512, 0, 256, (1, 512, 2)),
    (129, 512, 0, 256, (1, 512, 1)),   # batch fills the GPU: 64 heads, no split
    (256, 512, 0, 256, (1, 512, 1)),
    (1, 64, 0, 256, (1, 64, 4)),
    (3, 300, 0, 256, (5, 64, 4)),      # ragged top-k
    (3, 45, 0, 256, (1, 64, 4)),
    (1, 0, 0, 256, (1, 32, 4)),        # empty top-k: one slice, writes zeros / -inf
    (64, 512, 1, 256, (1, 512, 2)),    # forced
    (64, 512, 3, 256, (3, 192, 1)),    # slices hold whole 32-token tiles
    (64, 512, 99, 256, (16, 32, 1)),   # clamped to ceil(topk/32)
    (8, 100, 0, 80, (2, 64, 2)),       # 10 workgroups per query
    (32, 512, 0, 80, (1, 512, 2)),
])
def test_plan(batch, topk, req, cus, expect):
    ns, sl, hg = m.plan(batch, topk, req, cus)
    assert (ns, sl, hg) == expect
    assert sl % 32 == 0 and ns * sl >= topk and (ns - 1) * sl < max(topk, 1)
    if req == 0:
        assert batch * ns * hg <= max(cus, batch)   # one round of workgroups
