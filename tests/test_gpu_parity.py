"""Parity of the HIP path (through the C ABI) with the CPU fp64 oracle.

Gather + dequant must match bit for bit; attention outputs within
|d| <= 2e-3 + 1e-2 |ref| (out) and |d| <= 1e-3 (lse)."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import sparse_mla_decode_page_amd as mlasd
from gen import synth as G
from oracle import mla_oracle as O

from helpers import check_attention, decode, reserve_for, to_device

pytestmark = pytest.mark.gpu

_CONFIG_CACHE = {}


def config(i):
    if i not in _CONFIG_CACHE:
        w = G.make_config(i)
        ref = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx, w.seq_lens,
                                  w.softmax_scale)
        _CONFIG_CACHE[i] = (w, ref)
    return _CONFIG_CACHE[i]


def run(w, nsplit=None, stream=None):
    d = to_device(w)
    out, lse = decode(d, w.softmax_scale, nsplit=nsplit, stream=stream)
    torch.cuda.synchronize()
    return out, lse


# ----------------------------------------------------------------------------
# gather / dequant: bit-exact
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("i", [0, 1, 2, 3, 4])
def test_gather_dequant_bit_exact(i):
    w, _ = config(i)
    print(f"gather config {i}", flush=True)
    d = to_device(w)
    got, valid = mlasd.mla_sparse_gather_dequant(d["kv_pages"], d["page_table"], d["topk_idx"],
                                                 d["seq_lens"])
    torch.cuda.synchronize()
    rows, ok = O.gather_dequant(w.kv_pages, w.page_table, w.topk_idx, w.seq_lens)
    assert np.array_equal(valid.cpu().numpy().astype(bool), ok)
    gg = got.cpu().double().numpy()
    assert np.array_equal(gg, rows), np.argwhere(gg != rows)[:5]


def _all_codes_pool():
    """Two pages, 510 records: record r uses nope bytes (d + 7r) % 256 (every
    fp8 code, the NaN codes included) and scale byte r % 255 in all 7 groups,
    so every (code, finite scale byte) pair occurs."""
    rng = np.random.default_rng(11)
    pool = np.full((2, 149504), 0x7F, dtype=np.uint8)
    flat = pool.reshape(-1)
    for pos in range(510):
        pg, sl = pos // 256, pos % 256
        base = pg * 149504 + sl * 576
        flat[base:base + 448] = (np.arange(448) + 7 * pos) % 256
        flat[base + 448:base + 576] = G.bf16_bits(rng.standard_normal(64)).view(np.uint8)
        sbase = pg * 149504 + 147456 + sl * 8
        flat[sbase:sbase + 7] = pos % 255
        flat[sbase + 7] = 0xEE
    return pool


def test_gather_dequant_all_codes_all_scales():
    """Every (e4m3 code, UE8M0 byte) pair: the rows the contractions consume,
    times the row's power of two, equal the oracle's dequantised values
    exactly for scale bytes 0..246 -- the pages dequantise to bf16, exact for
    bytes 3..246 -- NaN codes included.  Bytes 247..254 scale e4m3 values
    past fp32's range: exact where the value is below 2^128, infinite (with
    its sign) where it is not."""
    pool = _all_codes_pool()
    pt = np.array([[0, 1]], dtype=np.int32)
    idx = np.arange(510, dtype=np.int32)[None][:, ::-1].copy()
    lens = np.array([510], dtype=np.int32)
    dev = lambda a: torch.from_numpy(a).cuda()
    got, valid = mlasd.mla_sparse_gather_dequant(dev(pool), dev(pt), dev(idx), dev(lens))
    torch.cuda.synchronize()
    rows, ok = O.gather_dequant(pool, pt, idx, lens)
    assert ok.all() and valid.cpu().numpy().all()
    gg = got.cpu().double().numpy()
    nan = np.isnan(rows)
    assert np.array_equal(np.isnan(gg), nan)
    byte = (510 - 1 - np.arange(510)) % 255           # scale byte of entry j (positions reversed)
    fits = np.abs(np.where(nan, 0.0, rows)) < 2.0 ** 128
    assert np.all(fits[0, byte <= 246]), "bytes 0..246 must stay inside fp32's range"
    same = ~nan & fits
    bad = np.argwhere(gg[same] != rows[same])
    assert len(bad) == 0, (len(bad), gg[same][bad[:5, 0]], rows[same][bad[:5, 0]])
    over = ~nan & ~fits
    assert np.all(np.isinf(gg[over])) and np.array_equal(np.signbit(gg[over]), np.signbit(rows[over]))


def _span_scales(spans, base_lo=-120, base_hi=110):
    """group_scale for the generator: each record gets a random base
    exponent and its 7 groups spread over the given span (binades)."""
    def f(rng, n):
        base = rng.integers(base_lo, base_hi, n)
        span = rng.choice(spans, n)
        off = np.floor(rng.random((n, 7)) * (span[:, None] + 1)).astype(np.int64)
        off[:, 0] = 0
        off[np.arange(n), rng.integers(1, 7, n)] = span        # one group at the top of the span
        return np.ldexp(1.0, base[:, None] + off)
    return f


def test_gather_dequant_rebased_tokens_exact():
    """Tokens whose 7 groups span up to 22 binades anywhere in UE8M0's range
    (scale bytes about 0..246) are held exactly: each such token is stored
    at one power of two of its own and the hook multiplies it back."""
    w = G.build_workload(77, [4000, 9000], 512, group_scale=_span_scales(np.arange(0, 23)))
    d = to_device(w)
    got, valid = mlasd.mla_sparse_gather_dequant(d["kv_pages"], d["page_table"], d["topk_idx"], d["seq_lens"])
    torch.cuda.synchronize()
    rows, ok = O.gather_dequant(w.kv_pages, w.page_table, w.topk_idx, w.seq_lens)
    assert np.array_equal(valid.cpu().numpy().astype(bool), ok)
    gg = got.cpu().double().numpy()
    fits = np.abs(rows) < 2.0 ** 128
    bad = np.argwhere((gg != rows) & fits)
    assert len(bad) == 0, (len(bad), bad[:5])


def test_gather_dequant_wider_spans_keep_the_large_groups():
    """A token whose groups span more than 22 binades keeps every group within
    22 binades of its largest exactly; smaller groups are rounded to the
    fp16 grid of that token (their values are below 2^-22 of its largest)."""
    w = G.build_workload(78, [3000], 256, group_scale=_span_scales(np.arange(23, 40), -60, 40))
    d = to_device(w)
    got, _ = mlasd.mla_sparse_gather_dequant(d["kv_pages"], d["page_table"], d["topk_idx"], d["seq_lens"])
    torch.cuda.synchronize()
    rows, ok = O.gather_dequant(w.kv_pages, w.page_table, w.topk_idx, w.seq_lens)
    gg = got.cpu().double().numpy()
    flat = w.kv_pages.reshape(-1)
    for j in range(w.topk):
        p = int(w.topk_idx[0, j])
        pg, sl = int(w.page_table[0, p // 256]), p % 256
        sb = flat[pg * 149504 + 147456 + sl * 8:][:7].astype(int) - 127
        near = np.repeat(sb >= sb.max() - 22, 64)
        assert np.array_equal(gg[0, j, :448][near], rows[0, j, :448][near]), j
        assert np.all(np.abs(gg[0, j, :448][~near] - rows[0, j, :448][~near]) <= 2.0 ** (sb.max() - 22 - 9 + 1)), j
        assert np.array_equal(gg[0, j, 448:], rows[0, j, 448:])


# ----------------------------------------------------------------------------
# attention parity
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("i", [0, 1, 2, 3, 4])
def test_decode_matches_oracle(i):
    w, (ref_out, ref_lse) = config(i)
    print(f"decode config {i} plan={mlasd.plan(w.batch, w.topk)}", flush=True)
    out, lse = run(w)
    check_attention(out, lse, ref_out, ref_lse, label=f"config {i}")


@pytest.mark.parametrize("i,nsplit", [(1, 1), (1, 2), (1, 4), (1, 16), (2, 1), (2, 3), (2, 16),
                                      (3, 1), (3, 2), (3, 8), (4, 2), (4, 4)])
def test_decode_forced_split(i, nsplit):
    w, (ref_out, ref_lse) = config(i)
    print(f"decode config {i} nsplit={nsplit}", flush=True)
    out, lse = run(w, nsplit=nsplit)
    check_attention(out, lse, ref_out, ref_lse, label=f"config {i} nsplit={nsplit}")


def _groupings_agree(r64, r32, label):
    """The 64-head and 32-head kernels run the same tiles in the same order.
    They differ in one place: the 32-head kernel splits each score's 512-dim
    dot product over two waves (nope dims [0, 192) plus rope, then
    [192, 448)) and adds the two fp32 parts, where the 64-head kernel sums it
    in one chain.  That rounding shows as lse within 1e-5 (relative) and out
    within 1 % of each query's largest |out| (measured: 4e-6 and 0.54 % at
    most over c0-c4, with 0.02-0.4 % of out elements different at all)."""
    (o1, l1), (o2, l2) = r64, r32
    fin = torch.isfinite(l1)
    assert torch.equal(fin, torch.isfinite(l2)), label
    assert torch.equal(l1[~fin], l2[~fin]), label
    if fin.any():
        dl = (l1[fin] - l2[fin]).abs()
        assert (dl <= 1e-5 * l1[fin].abs().clamp_min(1.0)).all(), f"{label}: lse {dl.max().item():.3g}"
    a, b = o1.float(), o2.float()
    mq = torch.maximum(a.abs(), b.abs()).amax(dim=(1, 2), keepdim=True)
    assert ((a - b).abs() <= 1e-2 * mq).all(), label


@pytest.mark.parametrize("i,nsplit", [(0, 1), (1, 1), (1, 8), (2, 4), (2, 8), (3, 2), (3, 1), (4, 1)])
def test_head_groups_agree(i, nsplit):
    """Two 32-head workgroups per slice against one 64-head workgroup: both
    meet the oracle bar, and they agree to the rounding of the scores'
    summation order."""
    w, (ref_out, ref_lse) = config(i)
    print(f"head groups config {i} nsplit={nsplit}", flush=True)
    d = to_device(w)
    r = [decode(d, w.softmax_scale, nsplit=nsplit, head_groups=hg) for hg in (1, 2)]
    torch.cuda.synchronize()
    _groupings_agree(r[0], r[1], f"config {i} nsplit={nsplit}")
    for hg, (o, l) in zip((1, 2), r):
        check_attention(o, l, ref_out, ref_lse, label=f"config {i} nsplit={nsplit} {64 // hg}-head groups")


def _custom(seed, lens, topk, **kw):
    """A seeded workload whose pool holds the sequences' pages plus two spare."""
    need = sum((L + 255) // 256 for L in lens)
    return G.build_workload(seed, lens, topk, num_pages=need + 2, **kw)


def _check_custom(w, nsplit=None, label="", maxnorm=False):
    ref_out, ref_lse = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx,
                                           w.seq_lens, w.softmax_scale)
    out, lse = run(w, nsplit=nsplit)
    return check_attention(out, lse, ref_out, ref_lse, label=label, maxnorm=maxnorm)


@pytest.mark.parametrize("topk", [1, 2, 31, 33, 45, 100, 257, 511])
def test_ragged_topk(topk):
    w = _custom(100 + topk, [3000, 700, 40000], topk)
    for ns in (None, 1, 3):
        _check_custom(w, nsplit=ns, label=f"topk={topk} nsplit={ns}")


def test_topk1_returns_value_row():
    w = _custom(5, [1000, 1], 1)
    out, lse = run(w)
    rows, ok = O.gather_dequant(w.kv_pages, w.page_table, w.topk_idx, w.seq_lens)
    for b in range(w.batch):
        exp_row = torch.from_numpy(rows[b, 0, :448]).to(torch.bfloat16).float().numpy()
        assert np.array_equal(out[b].float().cpu().numpy(), np.broadcast_to(exp_row, (64, 448)))
    _check_custom(w, label="topk=1")


def test_masking_and_invalid_entries():
    # every record of the pool is drawn, so re-selected positions hold data
    w = _custom(21, [5000, 300, 0, 2048], 64, fill="all")
    idx = w.topk_idx.copy()
    # query 0: -1 at arbitrary positions, idx = len-1 and len, negatives, huge
    idx[0, 3] = -1
    idx[0, 10] = 4999
    idx[0, 11] = 5000
    idx[0, 12] = -123456
    idx[0, 13] = 2 ** 31 - 1
    idx[0, 40:] = -1
    # query 3: valid positions whose page-table entries are out of range
    w.page_table[3, 2] = -1
    w.page_table[3, 5] = 10 ** 6
    idx[3, :8] = [2 * 256 + 3, 5 * 256 + 7, 1, 2, 3, 4, 2 * 256 + 100, 5 * 256]
    w.topk_idx = idx
    for ns in (None, 1, 2):
        _check_custom(w, nsplit=ns, label=f"masking nsplit={ns}")
    out, lse = run(w)
    assert np.all(out[2].float().cpu().numpy() == 0)
    assert np.all(np.isneginf(lse[2].cpu().numpy()))


def test_all_masked_and_empty():
    w = _custom(3, [0, 0, 100], 32)
    w.topk_idx[2] = -1
    for ns in (None, 1):
        out, lse = run(w, nsplit=ns)
        assert np.all(out.float().cpu().numpy() == 0)
        assert np.all(np.isneginf(lse.cpu().numpy()))


def test_topk_zero_and_batch_zero():
    w = _custom(4, [500, 20], 0)
    out, lse = run(w)
    assert np.all(out.float().cpu().numpy() == 0) and np.all(np.isneginf(lse.cpu().numpy()))
    d = to_device(_custom(4, [500], 8))
    e = {k: v[:0] for k, v in d.items() if k != "kv_pages"}
    e["kv_pages"] = d["kv_pages"]
    out, lse = decode(e, 0.1)
    assert out.shape == (0, 64, 448) and lse.shape == (0, 64)


def test_duplicates_count_each_time():
    w = _custom(8, [3000], 40)
    w.topk_idx[0, 20:30] = w.topk_idx[0, 0]
    _check_custom(w, label="duplicates")


def test_index_order_permutation():
    w = _custom(9, [9000, 4000], 200)
    base = _check_custom(w, label="order a")
    w.topk_idx = w.topk_idx[:, np.random.default_rng(0).permutation(200)].copy()
    _check_custom(w, label="order b")


@pytest.mark.parametrize("scale", [0.0, 1.0 / math.sqrt(512), 0.25, -0.1])
def test_softmax_scale_values(scale):
    w = _custom(12, [2000, 6000], 128, softmax_scale=scale)
    _check_custom(w, label=f"scale={scale}")


@pytest.mark.parametrize("q_log2", [8, -6, 20, -40, 100, -100, "tiny"])
def test_query_magnitudes(q_log2):
    """q enters Q K^T scaled per head by a power of two (its largest nope
    value lands in [2^15, 2^16)), exact over bf16's range: q scaled by 2^8,
    2^-6, 2^20 (|q| near 4e6), 2^-40 and 2^+-100, with the softmax scale
    compensating, and q with 5 % of its entries replaced by values near 1e-6
    all meet the oracle bar."""
    w = _custom(21, [5000, 30000], 256)
    q = (w.q_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if q_log2 == "tiny":
        rng = np.random.default_rng(3)
        pick = rng.random(q.shape) < 0.05
        q = np.where(pick, rng.standard_normal(q.shape) * 1e-6, q)
    else:
        q = q * 2.0 ** q_log2
        w.softmax_scale = w.softmax_scale * 2.0 ** -q_log2
    w.q_bits = G.bf16_bits(q)
    _check_custom(w, label=f"q scaled {q_log2}")


def _wide_range_workload(seed, lens, topk, q_log2):
    """Group amax log-uniform over 1e-4 .. 1e5 (scale bytes ~105 .. 135,
    independently per token and group), q times 2^q_log2, and a softmax
    scale that brings the largest score to about 30."""
    w = _custom(seed, lens, topk, group_scale=lambda r, n: 10.0 ** r.uniform(-4.0, 5.0, (n, 7)))
    q = (w.q_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64) * 2.0 ** q_log2
    w.q_bits = G.bf16_bits(q)
    rows, ok = O.gather_dequant(w.kv_pages, w.page_table, w.topk_idx, w.seq_lens)
    qd = O.bf16_value(w.q_bits)
    smax = max(np.abs(qd[b] @ rows[b][ok[b]].T).max() for b in range(w.batch) if ok[b].any())
    w.softmax_scale = 30.0 / smax
    return w


@pytest.mark.parametrize("q_log2", [0, 20])
def test_wide_dynamic_range_cache(q_log2):
    """A cache whose 64-dim groups have amax from 1e-4 to 1e5 (outside fp16's
    exact window on both sides) and q up to ~4e6, with the softmax scale
    compensating: lse meets the elementwise bar, out the per-query max-norm
    bar (values near 1e5 cancel)."""
    w = _wide_range_workload(4400 + q_log2, [3000, 20000, 700], 512, q_log2)
    print(f"wide range: softmax_scale={w.softmax_scale:.3e}", flush=True)
    for ns in (None, 1, 4):
        _check_custom(w, nsplit=ns, label=f"wide range q*2^{q_log2} nsplit={ns}", maxnorm=True)


def test_rebased_and_plain_tiles_mixed():
    """Slices whose tiles alternate between plain tokens and tokens that need
    a power-of-two rebase (tiny groups near 1e-9, large ones near 1e6), in
    both orders, so the running reference rises, stays and multiplies O
    back: the oracle bar (max-norm form: values up to 1e6) holds and 32/64-head
    workgroups agree to the rounding of the scores' summation order."""
    def gs(rng, n):
        kind = rng.integers(0, 3, n)
        scale = np.where(kind == 0, 1.0, np.where(kind == 1, 1e-9, 1e6))
        return np.repeat(scale[:, None], 7, axis=1) * 10.0 ** rng.uniform(-0.5, 0.5, (n, 7))
    w = _custom(4500, [2000, 9000, 300], 512, group_scale=gs)
    rows, ok = O.gather_dequant(w.kv_pages, w.page_table, w.topk_idx, w.seq_lens)
    qd = O.bf16_value(w.q_bits)
    w.softmax_scale = 30.0 / max(np.abs(qd[b] @ rows[b][ok[b]].T).max() for b in range(w.batch))
    d = to_device(w)
    r = [decode(d, w.softmax_scale, nsplit=1, head_groups=hg) for hg in (1, 2)]
    torch.cuda.synchronize()
    _groupings_agree(r[0], r[1], "mixed rebased tiles")
    for ns in (None, 1, 2):
        _check_custom(w, nsplit=ns, label=f"mixed rebased tiles nsplit={ns}", maxnorm=True)


def test_outliers_small_batch():
    w = _custom(13, [65536, 65536], 512, outlier_frac=0.01)
    for ns in (None, 1, 4):
        _check_custom(w, nsplit=ns, label=f"outliers nsplit={ns}")


def test_non_default_stream():
    w, (ref_out, ref_lse) = config(2)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, lse = run(w, stream=s)
    s.synchronize()
    check_attention(out, lse, ref_out, ref_lse, label="side stream")


def test_repeat_calls_deterministic():
    w, _ = config(3)
    d = to_device(w)
    outs = []
    for _ in range(3):
        o, l = decode(d, w.softmax_scale)
        outs.append((o.clone(), l.clone()))
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


def test_graph_capture_replay():
    """Decode calls captured in a HIP graph (split path with the combine, and
    the unsplit path) replay to the eager result, with eager work between
    replays."""
    ws = [config(1)[0], config(2)[0]]
    devs = [to_device(w) for w in ws]
    side = torch.cuda.Stream()
    outs = []
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for w, d in zip(ws, devs):
            for ns in (None, 1):
                o, l = decode(d, w.softmax_scale, nsplit=ns, stream=side)
                outs.append((o, l, o.clone(), l.clone(), w, d, ns))
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for o, l, _, _, w, d, ns in outs:
            decode(d, w.softmax_scale, nsplit=ns, stream=side, out=o, lse=l, reserve=False)
    for rep in range(3):
        for o, l, _, _, _, _, _ in outs:
            o.zero_()
            l.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, l, o_ref, l_ref, _, _, ns in outs:
            assert torch.equal(o, o_ref) and torch.equal(l, l_ref), f"replay {rep} nsplit={ns}"
        # eager work between replays
        w, d = ws[0], devs[0]
        decode(d, w.softmax_scale)
        torch.cuda.synchronize()


def test_graph_replay_timed_workload():
    """The full-size c3 workload (B=64, top-k 512) in the launch
    configuration the benchmark times: the planned decode captured in a HIP
    graph and replayed, with the outputs cleared between replays.  Every
    replay equals the eager result bit for bit, and the replayed output
    matches the oracle."""
    w, (ref_out, ref_lse) = config(3)
    print(f"graph replay config 3 plan={mlasd.plan(w.batch, w.topk)}", flush=True)
    d = to_device(w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o_eager, l_eager = decode(d, w.softmax_scale, stream=side)
    side.synchronize()
    o = torch.empty_like(o_eager)
    l = torch.empty_like(l_eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        decode(d, w.softmax_scale, stream=side, out=o, lse=l, reserve=False)
    for rep in range(3):
        o.zero_()
        l.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager) and torch.equal(l, l_eager), f"replay {rep}"
    check_attention(o, l, ref_out, ref_lse, label="config 3 graph replay")


def _status(fn):
    try:
        fn()
    except mlasd.MlasdError as e:
        return e.status
    return 0


def test_split_scratch_discipline():
    """The decode never allocates: a split call on a stream with no reserved
    scratch returns MLASD_ERR_WORKSPACE (outside capture too) and writes
    nothing; mlasd_prepare is the only allocator; a prepared capture replays
    to the oracle; mlasd_release frees."""
    w, (ref_out, ref_lse) = config(2)   # B=16, topk=512: a planned split
    assert mlasd.plan(w.batch, w.topk)[0] > 1
    d = to_device(w)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    out = torch.full((w.batch, 64, 448), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.batch, 64), 7.0, dtype=torch.float32, device="cuda")
    assert mlasd.workspace_bytes(stream=s) == 0
    call = lambda: decode(d, w.softmax_scale, stream=s, out=out, lse=lse, reserve=False)
    assert _status(call) == mlasd._binding.STATUS_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all()), "a refused call wrote output"
    # nor does it allocate under capture
    g0 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g0, stream=s):
        out.zero_()
        assert _status(call) == mlasd._binding.STATUS_WORKSPACE
    del g0
    assert mlasd.workspace_bytes(stream=s) == 0
    mlasd.prepare(w.batch, w.topk, stream=s)
    ns = mlasd.plan(w.batch, w.topk)[0]
    assert mlasd.workspace_bytes(stream=s) >= w.batch * ns * 64 * 449 * 4
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for rep in range(2):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_attention(out, lse, ref_out, ref_lse, label=f"prepared capture, replay {rep}")
    del g
    mlasd.release(stream=s)
    assert mlasd.workspace_bytes(stream=s) == 0
    mlasd.release(stream=s)   # nothing held: no-op


def test_graph_survives_scratch_growth():
    """A graph captured with the stream's scratch keeps working after a
    larger reservation on that stream replaced the buffer and a larger eager
    split call ran there: the superseded buffer stays allocated until
    mlasd_release, so the replay neither reads freed memory nor races the
    new buffer."""
    w_small, ref_small = config(1)       # B=1: planned split
    w_big, ref_big = config(2)           # B=16: planned split, larger scratch
    ds, db = to_device(w_small), to_device(w_big)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    mlasd.prepare(1, 512, stream=s)
    before = mlasd.workspace_bytes(stream=s)
    o = torch.empty((1, 64, 448), dtype=torch.bfloat16, device="cuda")
    l = torch.empty((1, 64), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        o_eager, l_eager = decode(ds, w_small.softmax_scale, stream=s, reserve=False)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        decode(ds, w_small.softmax_scale, stream=s, out=o, lse=l, reserve=False)
    mlasd.prepare(w_big.batch, 512, stream=s)          # grows: the old buffer is kept
    assert mlasd.workspace_bytes(stream=s) > before
    for rep in range(3):
        o.zero_()
        l.zero_()
        with torch.cuda.stream(s):
            ob, lb = decode(db, w_big.softmax_scale, stream=s, reserve=False)   # uses the new buffer
            g.replay()                                                          # uses the old one
        s.synchronize()
        assert torch.equal(o, o_eager) and torch.equal(l, l_eager), f"replay {rep}"
        check_attention(ob, lb, ref_big[0], ref_big[1], label=f"larger eager call {rep}")
    del g
    mlasd.release(stream=s)


def test_strided_views_match_contiguous():
    """Pages at a padded row stride (a [:, :149504] view of a wider pool, as
    the pages' own harness builds), q and out as views into larger buffers,
    a page table that is a column slice and strided seq_lens give bit for
    bit the contiguous call's results."""
    w, (ref_out, ref_lse) = config(2)
    d = to_device(w)
    o_ref, l_ref = decode(d, w.softmax_scale)
    B, P = w.batch, w.num_pages
    wide = torch.zeros((P, 149504 + 4096), dtype=torch.uint8, device="cuda")
    wide[:, :149504] = d["kv_pages"]
    qbig = torch.zeros((B, 66, 520), dtype=torch.bfloat16, device="cuda")
    qbig[:, 1:65, 8:520] = d["q"]
    ptbig = torch.full((B, w.max_pages + 3), -5, dtype=torch.int32, device="cuda")
    ptbig[:, 2:2 + w.max_pages] = d["page_table"]
    lbig = torch.zeros((B, 3), dtype=torch.int32, device="cuda")
    lbig[:, 1] = d["seq_lens"]
    obig = torch.full((B, 65, 456), 3.0, dtype=torch.bfloat16, device="cuda")
    lsebig = torch.full((B, 70), 3.0, dtype=torch.float32, device="cuda")
    v = dict(q=qbig[:, 1:65, 8:520], kv_pages=wide[:, :149504], page_table=ptbig[:, 2:2 + w.max_pages],
             topk_idx=d["topk_idx"], seq_lens=lbig[:, 1])
    assert not v["kv_pages"].is_contiguous() and not v["q"].is_contiguous()
    o, l = decode(v, w.softmax_scale, out=obig[:, :64, 8:456], lse=lsebig[:, 3:67])
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    assert bool((obig[:, 64] == 3.0).all()) and bool((obig[:, :, :8] == 3.0).all())
    assert bool((lsebig[:, :3] == 3.0).all()) and bool((lsebig[:, 67:] == 3.0).all())


def test_pool_reaching_past_4gib():
    """A pool view whose pages lie 1 GiB + 16 bytes apart, so pages 4-6 start
    beyond 2^32 bytes: the gathers take 64-bit offsets there (a pool within
    4 GiB of its start takes 32-bit ones), and the results equal the compact
    pool's bit for bit under both head groupings."""
    w = _custom(4600, [600, 500], 512)
    ref_out, ref_lse = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx, w.seq_lens,
                                           w.softmax_scale)
    stride = (1 << 30) + 16
    P = w.num_pages
    used = {int(x) for x in w.page_table.ravel() if x >= 0}
    assert max(used) * stride >= 1 << 32, "a selected page must start past 4 GiB"
    d = to_device(w)
    big = torch.empty(P * stride, dtype=torch.uint8, device="cuda")
    view = big.as_strided((P, 149504), (stride, 1))
    view.copy_(d["kv_pages"])
    v = dict(d, kv_pages=view)
    print(f"pool view: {P} pages at stride {stride} ({P * stride / 2**30:.1f} GiB)", flush=True)
    for hg in (1, 2):
        o_ref, l_ref = decode(d, w.softmax_scale, head_groups=hg)
        o, l = decode(v, w.softmax_scale, head_groups=hg)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref), f"head_groups={hg}"
        check_attention(o, l, ref_out, ref_lse, label=f"pool past 4 GiB, {64 // hg}-head groups")
    del big, view, v


def test_split_merge_alternating_inputs():
    """The LSE combine reads partials the decode launch just wrote to the
    stream's scratch: alternate two input sets of one shape on one stream,
    with no host synchronisation between launches, and check every result
    against the first result of its set (bitwise) and against the oracle.  A
    combine that read partials of the previous launch would differ."""
    base = config(3)[0]
    # rotation_sets writes records into the pool: work on a copy
    w, w2 = G.rotation_sets(dataclasses.replace(base, kv_pages=base.kv_pages.copy()), 2, seed=4242)
    ref_out, ref_lse = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx,
                                           w.seq_lens, w.softmax_scale)
    ref2 = O.sparse_mla_decode(w2.q_bits, w2.kv_pages, w2.page_table, w2.topk_idx, w2.seq_lens,
                               w2.softmax_scale)
    d1, d2 = to_device(w), to_device(w2)
    for ns in (4, 16):
        reserve_for(w.batch, w.topk, ns)
        res = []
        for it in range(8):
            d = d1 if it % 2 == 0 else d2
            o, l = decode(d, w.softmax_scale, nsplit=ns, reserve=False)
            res.append((o, l))
        torch.cuda.synchronize()
        for it, (o, l) in enumerate(res):
            o0, l0 = res[it % 2]
            assert torch.equal(o, o0) and torch.equal(l, l0), f"nsplit={ns} launch {it}"
        check_attention(res[0][0], res[0][1], ref_out, ref_lse, label=f"set A nsplit={ns}")
        check_attention(res[1][0], res[1][1], ref2[0], ref2[1], label=f"set B nsplit={ns}")
    # a smaller batch on the same stream afterwards
    ws = G.make_config(2)
    ref_s = O.sparse_mla_decode(ws.q_bits, ws.kv_pages, ws.page_table, ws.topk_idx, ws.seq_lens,
                                ws.softmax_scale)
    o, l = run(ws, nsplit=4)
    check_attention(o, l, ref_s[0], ref_s[1], label="smaller batch after")


def test_large_batch_several_rounds():
    """B = 1000 queries: four rounds of workgroups on 256 CUs, 64-head
    workgroups and no split; ragged lengths (some shorter than topk, so their
    lists end in -1 padding)."""
    rng = np.random.default_rng(1000)
    lens = rng.integers(20, 700, 1000)
    w = G.build_workload(5150, lens, 100, name="B=1000 topk=100")
    ns, _, hg = mlasd.plan(w.batch, w.topk)
    assert (ns, hg) == (1, 1)
    print(f"large batch: plan nsplit={ns} head_groups={hg}", flush=True)
    ref_out, ref_lse = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx,
                                           w.seq_lens, w.softmax_scale)
    out, lse = run(w)
    check_attention(out, lse, ref_out, ref_lse, label="B=1000 topk=100")


# ----------------------------------------------------------------------------
# the pages' validation matrix ("The Moment of Validation", "The Third
# Attempt"): B in {1, 4, 16, 32}, 64 heads, topk in {128, 512}
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("batch", [1, 4, 16, 32])
@pytest.mark.parametrize("topk", [128, 512])
def test_validation_matrix(batch, topk):
    lens = [4096 + 97 * b for b in range(batch)]
    w = G.build_workload(31000 + 10 * batch + topk, lens, topk, name=f"B={batch} topk={topk}")
    ref_out, ref_lse = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx,
                                           w.seq_lens, w.softmax_scale)
    d = to_device(w)
    for ns, hg in ((None, None), (1, 1), (1, 2)):
        out, lse = decode(d, w.softmax_scale, nsplit=ns, head_groups=hg)
        torch.cuda.synchronize()
        check_attention(out, lse, ref_out, ref_lse,
                        label=f"B={batch:2d} H=64 topk={topk} nsplit={ns or 'plan'} "
                              f"head_groups={hg or 'plan'}")
