"""The decode entry point that allocates nothing (mla_sparse_decode_noalloc):
called through the C ABI, it matches mla_sparse_decode bit for bit on two
calls in a row, the second with a smaller input, both under split plans
that use its static scratch."""
import numpy as np
import pytest
import torch

import sparse_mla_decode_page_amd as mlasd
from gen import synth as G
from oracle import mla_oracle as O

from helpers import check_attention, decode, to_device

pytestmark = pytest.mark.gpu


def _noalloc(d, scale, out, lse):
    return mlasd.mla_sparse_decode_noalloc(d["q"], d["kv_pages"], d["page_table"], d["topk_idx"],
                                           d["seq_lens"], scale, out, lse)


def test_noalloc_matches_decode_twice_then_smaller():
    big = G.build_workload(6101, [5000 + 300 * b for b in range(16)], 512, name="B=16")
    small = G.build_workload(6102, [3000, 700, 40000], 200, name="B=3")
    for w in (big, small):
        ns = mlasd.plan(w.batch, w.topk)[0]
        print(f"noalloc: B={w.batch} topk={w.topk} plan nsplit={ns}", flush=True)
        assert ns > 1, "both calls must use the split scratch"
    res = []
    for w in (big, small):
        d = to_device(w)
        out = torch.full((w.batch, 64, 448), 5.0, dtype=torch.bfloat16, device="cuda")
        lse = torch.full((w.batch, 64), 5.0, dtype=torch.float32, device="cuda")
        _noalloc(d, w.softmax_scale, out, lse)
        res.append((w, d, out, lse))
    torch.cuda.synchronize()
    for w, d, out, lse in res:
        o_ref, l_ref = decode(d, w.softmax_scale)
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(lse, l_ref), f"B={w.batch}"
        ref_out, ref_lse = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx,
                                               w.seq_lens, w.softmax_scale)
        check_attention(out, lse, ref_out, ref_lse, label=f"noalloc B={w.batch}")


def test_noalloc_under_graph_capture():
    """Captured with no reservation on the capture stream, replayed three
    times with eager work between the replays."""
    w = G.make_config(1)
    assert mlasd.plan(w.batch, w.topk)[0] > 1
    d = to_device(w)
    out = torch.empty((1, 64, 448), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 64), dtype=torch.float32, device="cuda")
    _noalloc(d, w.softmax_scale, out, lse)
    torch.cuda.synchronize()
    o0, l0 = out.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    assert mlasd.workspace_bytes(stream=s) == 0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mlasd.mla_sparse_decode_noalloc(d["q"], d["kv_pages"], d["page_table"], d["topk_idx"],
                                        d["seq_lens"], w.softmax_scale, out, lse, stream=s)
    assert mlasd.workspace_bytes(stream=s) == 0
    for rep in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o0) and torch.equal(lse, l0), f"replay {rep}"
        o_e, l_e = torch.empty_like(out), torch.empty_like(lse)
        _noalloc(d, w.softmax_scale, o_e, l_e)   # eager work on the same array between replays
        torch.cuda.synchronize()
        assert torch.equal(o_e, o0)


def test_noalloc_scratch_covers_every_automatic_plan():
    """The static scratch (16 MiB) holds the partials of every automatically
    planned split on this device, for any batch and top-k width, so the
    entry point's refusal (MLASD_ERR_WORKSPACE) is never hit by an
    automatic plan."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    worst = max(mlasd.workspace_size(b, k, 0, 0, cus) for b in range(1, 1025) for k in (64, 256, 512))
    print(f"largest automatic split scratch on {cus} CUs: {worst / 2**20:.2f} MiB", flush=True)
    assert worst <= 16 << 20
