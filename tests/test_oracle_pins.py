"""Pins for the CPU oracle: each test checks it against something that is not
the oracle itself -- torch's own fp8 / e8m0 / bf16 casts, torch's
scaled-dot-product attention and scipy's logsumexp, closed forms, and a
hand-computed layout example.  CPU only."""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import mla_oracle as O
from gen import synth as G

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# scalar formats
# ----------------------------------------------------------------------------

def test_e4m3_all_codes_match_torch_cast():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_value(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x80, -0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x77, 240.0), (0x7E, 448.0), (0xFE, -448.0), (0xB9, -1.125),
])
def test_e4m3_landmarks(code, value):
    got = float(O.e4m3_value(code))
    assert got == value and math.copysign(1, got) == math.copysign(1, value)


def test_e4m3_nan_codes():
    assert np.isnan(O.e4m3_value(0x7F)) and np.isnan(O.e4m3_value(0xFF))
    # exponent field 15 with mantissa < 7 is finite in the "fn" variant
    assert O.e4m3_value(0x78) == 256.0


def test_ue8m0_all_bytes_match_torch_cast():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = O.ue8m0_value(b)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert O.ue8m0_value(127) == 1.0 and O.ue8m0_value(0) == 2.0 ** -127 and O.ue8m0_value(254) == 2.0 ** 127


def test_bf16_matches_torch_view():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 65536, size=4096, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_value(bits)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


# ----------------------------------------------------------------------------
# generator encoders (inputs only), checked against torch and closed forms
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("amax,k", [(448.0, 0), (449.0, 1), (224.0, -1), (224.5, 0), (1.0, -8),
                                    (14.0, -5), (14.000001, -4), (0.0, -127), (1e-60, -127),
                                    (448.0 * 2.0 ** 127, 127), (1e300, 127)])
def test_scale_exponent_closed_form(amax, k):
    assert int(G.scale_exponent(np.float64(amax))) == k


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(2)
    y = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.uniform(-2 ** -5, 2 ** -5, 20000),
        rng.standard_normal(20000),
    ]).astype(np.float32).astype(np.float64)
    got = G.e4m3_encode(y)
    ref = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # -0 and +0 both decode to zero; compare values, then codes away from zero
    assert np.array_equal(O.e4m3_value(got), O.e4m3_value(ref))
    nz = y != 0
    assert np.array_equal(got[nz], ref[nz])


def test_quantiser_roundtrip_bound():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((500, 448)) * np.exp(rng.uniform(-5, 5, (500, 1)))
    codes, sb = G.quantize_nope(x)
    deq = O.e4m3_value(codes) * np.repeat(O.ue8m0_value(sb), 64, axis=1)
    # every group max maps into (224, 448] before rounding, [224, 448] after;
    # relative error of every normal-range value <= 2^-4
    big = np.abs(x) >= 2.0 ** -6 * np.repeat(np.exp2(sb.astype(float) - 127), 64, axis=1)
    rel = np.abs(deq - x)[big] / np.abs(x)[big]
    assert rel.max() <= 2.0 ** -4
    g = np.abs(deq.reshape(500, 7, 64)).max(-1) / np.exp2(sb.astype(float) - 127)
    assert np.all((g >= 224) & (g <= 448))


# ----------------------------------------------------------------------------
# layout: hand-computed example
# ----------------------------------------------------------------------------

def _golden_layout():
    with open(os.path.join(GOLDEN, "layout_example.json")) as f:
        return json.load(f)


def test_layout_hand_example():
    g = _golden_layout()
    pool = np.full((g["num_pages"], 256 * 584), 0x7F, dtype=np.uint8)
    ro = g["record"]["record_offset"]
    so = g["record"]["scale_offset"]
    flat = pool.reshape(-1)
    flat[ro:ro + 448] = g["nope_fill_code"]
    for d, c in g["nope_overrides"].items():
        flat[ro + int(d)] = c
    flat[ro + 448:ro + 576] = 0
    for r, bits in g["rope_bits"].items():
        flat[ro + 448 + 2 * int(r)] = bits & 0xFF
        flat[ro + 448 + 2 * int(r) + 1] = bits >> 8
    flat[so:so + 8] = g["scale_bytes"]
    rows, valid = O.gather_dequant(pool, np.array(g["page_table"]), np.array(g["topk_idx"]),
                                   np.array(g["seq_lens"]))
    assert valid.tolist() == [g["expected_valid"]]
    for d, v in g["expected_row"].items():
        assert rows[0, 0, int(d)] == v, d
    # masked entries read nothing and are zero
    assert np.all(rows[0, 1:] == 0)


def test_position_encoded_page_walk():
    """rope[0] holds the physical page, rope[1] the slot (both small integers,
    exact in bf16): gather must return exactly the record the page table and
    index select."""
    rng = np.random.default_rng(5)
    num_pages, B, max_pages = 40, 3, 12
    pool = np.full((num_pages, 256 * 584), 0x7F, dtype=np.uint8)
    flat = pool.reshape(-1)
    pt = rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    lens = np.array([max_pages * 256, 1000, 5])
    idx = np.stack([rng.choice(int(L), 16, replace=int(L) < 16) for L in lens]).astype(np.int32)
    for p in range(num_pages):
        for s in range(256):
            base = p * 149504 + s * 576
            for r, val in ((0, p), (1, s)):
                bits = int(G.bf16_bits(np.array([float(val)]))[0])
                flat[base + 448 + 2 * r] = bits & 0xFF
                flat[base + 448 + 2 * r + 1] = bits >> 8
    rows, valid = O.gather_dequant(pool, pt, idx, lens)
    for b in range(B):
        for j in range(16):
            p = idx[b, j]
            assert valid[b, j] == (p < lens[b])
            if valid[b, j]:
                assert rows[b, j, 448] == pt[b, p // 256]
                assert rows[b, j, 449] == p % 256


def _page_id_pool(num_pages):
    """Every record of page p has nope code 0x38 (1.0) at scale byte 127, so
    nope dim 0 reads 1.0, and rope[0] = p, rope[1] = slot (exact in bf16): a
    row names the record it came from."""
    pool = np.zeros((num_pages, 256 * 584), dtype=np.uint8)
    flat = pool.reshape(-1)
    for p in range(num_pages):
        for s in range(256):
            base = p * 149504 + s * 576
            flat[base:base + 448] = 0x38
            for r, val in ((0, p), (1, s)):
                bits = int(G.bf16_bits(np.array([float(val)]))[0])
                flat[base + 448 + 2 * r] = bits & 0xFF
                flat[base + 448 + 2 * r + 1] = bits >> 8
        flat[p * 149504 + 147456:(p + 1) * 149504] = np.tile(np.array([127] * 7 + [0], np.uint8), 256)
    return pool


def test_masking_branches_by_hand():
    """Reading R4 decided entry by entry (expected flags and rows written by
    hand, not computed): a position below seq_len is still masked when its
    page-table entry is -1, when its logical page lies past the page-table
    row (seq_len larger than the row covers), or when the physical page id is
    outside the pool.  A -1 page must not wrap round to the pool's last page,
    and a logical page past the row must not index outside it."""
    pool = _page_id_pool(3)
    # max_pages = 3: the row covers positions 0..767; seq_len 1000 goes past it
    pt = np.array([[2, -1, 0],
                   [5, 1, 1]], dtype=np.int32)
    lens = np.array([1000, 700], dtype=np.int32)
    idx = np.array([[5, 300, 600, 800, 999, 767],
                    [10, 256, 600, 700, -1, 699]], dtype=np.int32)
    # (valid, page, slot) by hand:
    #   q0: 5 -> lp 0 -> page 2 slot 5; 300 -> lp 1 -> page -1: masked;
    #       600 -> lp 2 -> page 0 slot 88; 800 and 999 -> lp 3 >= max_pages: masked;
    #       767 -> lp 2 -> page 0 slot 255
    #   q1: 10 -> lp 0 -> page 5 >= num_pages 3: masked; 256 -> page 1 slot 0;
    #       600 -> lp 2 -> page 1 slot 88; 700 = seq_len: masked; -1: masked;
    #       699 -> page 1 slot 187
    expect = [[(True, 2, 5), (False,), (True, 0, 88), (False,), (False,), (True, 0, 255)],
              [(False,), (True, 1, 0), (True, 1, 88), (False,), (False,), (True, 1, 187)]]
    valid, page, slot = O.resolve_entries(pt, idx, lens, 3)
    rows, valid2 = O.gather_dequant(pool, pt, idx, lens)
    assert np.array_equal(valid, valid2)
    for b in range(2):
        for j, e in enumerate(expect[b]):
            assert bool(valid[b, j]) == e[0], (b, j)
            if e[0]:
                assert (page[b, j], slot[b, j]) == e[1:], (b, j)
                assert rows[b, j, 0] == 1.0 and rows[b, j, 447] == 1.0
                assert (rows[b, j, 448], rows[b, j, 449]) == e[1:], (b, j)
            else:
                assert np.all(rows[b, j] == 0), (b, j)
    # the masked entries change nothing in the attention: query 0 over its
    # three valid records equals query 0 over exactly those records
    q = G.bf16_bits(np.random.default_rng(2).standard_normal((2, 64, 512)))
    out, lse = O.sparse_mla_decode(q, pool, pt, idx, lens, 0.05)
    out0, lse0 = O.sparse_mla_decode(q[:1], pool, pt[:1], idx[:1, [0, 2, 5]], lens[:1], 0.05)
    np.testing.assert_array_equal(out[:1], out0)
    np.testing.assert_array_equal(lse[:1], lse0)


# ----------------------------------------------------------------------------
# attention: against library routines and closed forms
# ----------------------------------------------------------------------------

def _torch_rows(pool, page_table, topk_idx, seq_lens):
    """Decode the selected records with torch's own fp8 / e8m0 / bf16 casts
    (independent of the oracle's decoders)."""
    flat = torch.from_numpy(np.ascontiguousarray(pool).reshape(-1))
    out = []
    for b in range(topk_idx.shape[0]):
        rows = []
        for p in topk_idx[b]:
            if p < 0 or p >= seq_lens[b]:
                continue
            pg = int(page_table[b, p // 256])
            base = pg * 149504 + (p % 256) * 576
            nope = flat[base:base + 448].view(torch.float8_e4m3fn).to(torch.float64)
            sb = flat[pg * 149504 + 147456 + (p % 256) * 8:][:7].view(torch.float8_e8m0fnu).to(torch.float64)
            rope = flat[base + 448:base + 576].clone().view(torch.bfloat16).to(torch.float64)
            rows.append(torch.cat([nope * sb.repeat_interleave(64), rope]))
        out.append(torch.stack(rows) if rows else torch.zeros(0, 512, dtype=torch.float64))
    return out


@pytest.mark.parametrize("i", [0, 1, 2])
def test_attention_matches_torch_sdpa_and_scipy(i):
    w = G.make_config(i)
    out, lse = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx, w.seq_lens, w.softmax_scale)
    q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    rows = _torch_rows(w.kv_pages, w.page_table, w.topk_idx, w.seq_lens)
    for b in range(w.batch):
        k = rows[b]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[b][None, :, None, :], k[None, None].expand(1, 64, -1, -1),
            k[:, :448][None, None].expand(1, 64, -1, -1), scale=w.softmax_scale)[0, :, 0]
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=1e-11, atol=1e-13)
        s = w.softmax_scale * (q[b] @ k.T).numpy()
        np.testing.assert_allclose(lse[b], logsumexp(s, axis=1), rtol=1e-13, atol=1e-13)


def _small(seed=7, lens=(700, 300), topk=24, **kw):
    need = sum((L + 255) // 256 for L in lens)
    return G.build_workload(seed, lens, topk, num_pages=need + 3, **kw)


def test_topk1_returns_dequantised_row():
    w = _small(lens=(900,), topk=1)
    out, lse = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx, w.seq_lens, w.softmax_scale)
    k = _torch_rows(w.kv_pages, w.page_table, w.topk_idx, w.seq_lens)[0][0].numpy()
    q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()[0]
    assert np.array_equal(out[0], np.broadcast_to(k[:448], (64, 448)))
    np.testing.assert_allclose(lse[0], w.softmax_scale * (q @ k), rtol=1e-14, atol=1e-14)


def test_constant_v_gives_constant_output():
    """Weights sum to one: every selected record decodes to V == 1.0."""
    w = _small()
    flat = w.kv_pages.reshape(-1)
    for b in range(w.batch):
        for p in w.topk_idx[b]:
            if 0 <= p < w.seq_lens[b]:
                pg = int(w.page_table[b, p // 256])
                base = pg * 149504 + (p % 256) * 576
                flat[base:base + 448] = 0x38
                flat[pg * 149504 + 147456 + (p % 256) * 8:][:7] = 127
    out, _ = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx, w.seq_lens, w.softmax_scale)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)


def test_zero_query_gives_log_n_and_mean():
    w = _small(lens=(5000, 17), topk=40)
    w.q_bits[:] = 0
    out, lse = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx, w.seq_lens, w.softmax_scale)
    rows = _torch_rows(w.kv_pages, w.page_table, w.topk_idx, w.seq_lens)
    for b in range(w.batch):
        n = rows[b].shape[0]
        np.testing.assert_allclose(lse[b], math.log(n), rtol=0, atol=1e-14)
        np.testing.assert_allclose(out[b], np.broadcast_to(rows[b][:, :448].mean(0).numpy(), (64, 448)),
                                   rtol=1e-13, atol=1e-15)


def test_index_order_invariance():
    w = _small(lens=(6000, 2000), topk=64)
    out, lse = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx, w.seq_lens, w.softmax_scale)
    perm = np.random.default_rng(0).permutation(64)
    out2, lse2 = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx[:, perm], w.seq_lens,
                                     w.softmax_scale)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=1e-12, atol=1e-12)


def test_masked_entries_do_not_contribute():
    w = _small(lens=(6000, 2000), topk=32)
    out, lse = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx, w.seq_lens, w.softmax_scale)
    junk = np.array([[-1, -7, 6000, 99999], [2000, -1, 2500, -2 ** 31]], dtype=np.int32)
    idx = np.concatenate([w.topk_idx[:, :10], junk, w.topk_idx[:, 10:]], axis=1)
    out2, lse2 = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, idx, w.seq_lens, w.softmax_scale)
    np.testing.assert_allclose(out2, out, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-13)


def test_split_identity():
    """Attention over disjoint subsets merged by the LSE rule equals attention
    over the union (what split top-k plus combine relies on)."""
    w = _small(lens=(6000, 2000), topk=96)
    out, lse = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx, w.seq_lens, w.softmax_scale)
    parts = [w.topk_idx[:, :10], w.topk_idx[:, 10:50], w.topk_idx[:, 50:]]
    res = [O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, p, w.seq_lens, w.softmax_scale) for p in parts]
    mo, ml = O.lse_combine([r[0] for r in res], [r[1] for r in res])
    np.testing.assert_allclose(mo, out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ml, lse, rtol=1e-13, atol=1e-13)


def test_combine_with_empty_subsets():
    o = np.random.default_rng(0).standard_normal((3, 2, 448))
    l = np.array([[0.5, -np.inf], [-np.inf, -np.inf], [1.5, -np.inf]])
    mo, ml = O.lse_combine(o, l)
    w0, w2 = math.exp(0.5), math.exp(1.5)
    np.testing.assert_allclose(mo[0], (w0 * o[0, 0] + w2 * o[2, 0]) / (w0 + w2), rtol=1e-14, atol=1e-15)
    assert ml[0] == pytest.approx(math.log(w0 + w2), rel=1e-15)
    assert np.all(mo[1] == 0) and ml[1] == -np.inf


def test_empty_query():
    w = _small(lens=(0, 300), topk=8)
    out, lse = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx, w.seq_lens, w.softmax_scale)
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.all(np.isfinite(out[1])) and np.all(np.isfinite(lse[1]))


def test_scale_multiplies_whole_score():
    """Doubling softmax_scale equals doubling Q (exact in bf16): the scale
    applies to nope and rope terms alike."""
    w = _small()
    o1, l1 = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx, w.seq_lens, 2 * w.softmax_scale)
    q2 = G.bf16_bits(2.0 * O.bf16_value(w.q_bits))
    o2, l2 = O.sparse_mla_decode(q2, w.kv_pages, w.page_table, w.topk_idx, w.seq_lens, w.softmax_scale)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-14)


def test_decimal_brute_force_tiny():
    """50-digit decimal evaluation of the definition on a tiny case."""
    getcontext().prec = 50
    w = _small(lens=(800,), topk=3)
    out, lse = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx, w.seq_lens, w.softmax_scale)
    rows = _torch_rows(w.kv_pages, w.page_table, w.topk_idx, w.seq_lens)[0].numpy()
    q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()[0]
    sc = Decimal(w.softmax_scale)
    for h in (0, 17, 63):
        s = [sc * sum(Decimal(float(q[h, d])) * Decimal(float(rows[t, d])) for d in range(512)) for t in range(3)]
        z = sum(x.exp() for x in s)
        assert abs(float(z.ln()) - lse[0, h]) < 1e-13
        for c in (0, 100, 447):
            v = sum(x.exp() / z * Decimal(float(rows[t, c])) for t, x in enumerate(s))
            assert abs(float(v) - out[0, h, c]) < 1e-13 * max(1.0, abs(float(v)))


# ----------------------------------------------------------------------------
# cache append: the quantiser (reading R13)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("amax,k", [(448.0, 0), (449.0, 1), (224.0, -1), (224.5, 0), (1.0, -8),
                                    (0.0, -127), (2.0 ** 200, 127), (2.0 ** -200, -127),
                                    (448.0 * 2.0 ** -20, -20), (448.0 * 2.0 ** -20 * (1 + 2 ** -30), -19)])
def test_append_scale_exponent_closed_form(amax, k):
    assert O.scale_exponent(amax) == k


def test_append_scale_exponent_brackets_amax():
    rng = np.random.default_rng(5)
    for amax in np.exp(rng.uniform(-60, 60, 2000)):
        k = O.scale_exponent(amax)
        assert 448.0 * 2.0 ** (k - 1) < amax <= 448.0 * 2.0 ** k


def test_append_encode_roundtrips_every_code():
    for code in range(256):
        v = O.e4m3_value(code)
        if np.isnan(v):
            continue
        y = -0.0 if code == 0x80 else float(v)
        assert O.e4m3_encode_nearest(y) == code, hex(code)


def test_append_encode_ties_to_even():
    finite = sorted({float(O.e4m3_value(c)) for c in range(127) if not np.isnan(O.e4m3_value(c))})
    for lo, hi in zip(finite, finite[1:]):
        mid = (lo + hi) / 2.0
        code = O.e4m3_encode_nearest(mid)
        assert code % 2 == 0 and float(O.e4m3_value(code)) in (lo, hi)


def test_append_encode_matches_torch_rne_cast():
    rng = np.random.default_rng(6)
    y = np.concatenate([rng.uniform(-448, 448, 3000), rng.uniform(-1, 1, 3000) * 2.0 ** -5,
                        rng.standard_normal(3000)])
    mine = np.array([O.e4m3_encode_nearest(v) for v in y], dtype=np.uint8)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def _latents(n, seed):
    """bf16 latents: N(0,1) groups, one 20-sigma group, an all-zero group, a
    tiny-magnitude group and a group with exact e4m3 values."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 512))
    x[:, 64:128] *= 20.0
    x[:, 128:192] = 0.0
    x[:, 192:256] *= 2.0 ** -30
    x[:, 256:320] = O.e4m3_value(rng.integers(0, 126, (n, 64))) * 2.0 ** 3
    return G.bf16_bits(x)


def test_append_quantize_token_error_bound_and_layout():
    bits = _latents(40, 7)
    for row in bits:
        rec, sc = O.quantize_token(row)
        x = O.bf16_value(row[:448]).reshape(7, 64)
        assert sc[7] == 0
        assert np.array_equal(rec[448:].view("<u2"), row[448:])
        dec = O.e4m3_value(rec[:448]).reshape(7, 64) * O.ue8m0_value(sc[:7])[:, None]
        for g in range(7):
            k = int(sc[g]) - 127
            amax = np.abs(x[g]).max()
            # half an e4m3 step: 2^-4 relative in the normal range, 2^-10 * 2^k below it
            bound = np.maximum(np.abs(x[g]) * 2.0 ** -4, 2.0 ** (-10 + k))
            assert np.all(np.abs(dec[g] - x[g]) <= bound)
            if amax > 0:   # the scale is tight: the largest value lands in (224, 448]
                assert 224.0 < amax * 2.0 ** -k <= 448.0
        # exactly representable values come back exactly
        assert np.array_equal(dec[4], x[4])


def test_append_quantize_agrees_with_the_generator_quantiser():
    """A second, independent implementation (frexp exponent, rint rounding)."""
    bits = _latents(60, 8)
    for row in bits:
        rec, sc = O.quantize_token(row)
        codes, scale = G.quantize_nope(O.bf16_value(row[:448])[None])
        assert np.array_equal(rec[:448], codes[0]) and np.array_equal(sc[:7], scale[0])


def test_append_writes_valid_tokens_only_and_decodes_back():
    pool = np.full((4, O.BYTES_PER_PAGE), 0x5A, dtype=np.uint8)
    pt = np.array([[2, 0], [1, -1]], dtype=np.int32)
    seq = np.array([0, 0, 1, 1, 1, 2, -1, 0], dtype=np.int32)
    pos = np.array([3, 300, 7, 256, -1, 0, 0, 600], dtype=np.int32)
    bits = _latents(len(pos), 9)
    out = O.kv_append(pool, pt, seq, pos, bits)
    # written: (0,3) -> page 2 slot 3, (0,300) -> page 0 slot 44, (1,7) -> page 1 slot 7
    written = {(2, 3): 0, (0, 44): 1, (1, 7): 2}
    for (page, slot), i in written.items():
        rows, ok = O.gather_dequant(out, np.array([[page]], dtype=np.int32),
                                    np.array([[slot]], dtype=np.int32), np.array([256], dtype=np.int32))
        rec, sc = O.quantize_token(bits[i])
        want = np.concatenate([O.e4m3_value(rec[:448]) * np.repeat(O.ue8m0_value(sc[:7]), 64),
                               O.bf16_value(bits[i][448:])])
        assert ok.all() and np.array_equal(rows[0, 0], want)
    # nothing else changed: (1,256) has no page, -1 / seq 2 / seq -1 / position 600 are invalid
    mask = np.ones_like(out, dtype=bool)
    for (page, slot) in written:
        mask[page, slot * 576:(slot + 1) * 576] = False
        mask[page, 147456 + slot * 8:147456 + slot * 8 + 8] = False
    assert np.all(out[mask] == 0x5A)


# ----------------------------------------------------------------------------
# top-k selection (reading R14)
# ----------------------------------------------------------------------------

def _golden_topk():
    with open(os.path.join(GOLDEN, "topk_example.json")) as f:
        g = json.load(f)
    scores = np.array([[float(v) for v in row] for row in g["scores"]], dtype=np.float32)
    return scores, g["cases"]


def test_topk_select_hand_worked_rows():
    """Rows worked out by hand from the ranking rule: ties by position, NaN
    as -inf after -inf's position order, -0.0 tied with +0.0, short and
    empty sequences padded with -1."""
    scores, cases = _golden_topk()
    for c in cases:
        got = O.topk_select(scores, c["seq_lens"], c["k"])
        assert got.tolist() == c["expected"], c


def _check_topk_properties(scores, seq_lens, k, got):
    """Properties that together fix the selection uniquely: the right count,
    -1 only as padding, distinct in-range positions, non-increasing scores
    with increasing positions among equal scores, every selected score >= every
    unselected one, and at the boundary score the lowest positions win."""
    B, max_len = scores.shape
    for b in range(B):
        L = min(max(int(seq_lens[b]), 0), max_len)
        n = min(k, L)
        row = got[b]
        assert (row[:n] >= 0).all() and (row[n:] == -1).all()
        sel = row[:n].astype(np.int64)
        assert len(set(sel.tolist())) == n and (sel < L).all()
        v = scores[b, :L].astype(np.float64)
        v = np.where(np.isnan(v), -np.inf, v)
        s = v[sel]
        for i in range(n - 1):
            assert s[i] > s[i + 1] or (s[i] == s[i + 1] and sel[i] < sel[i + 1])
        rest = np.setdiff1d(np.arange(L), sel)
        if n and len(rest):
            assert s.min() >= v[rest].max()
            tie = rest[v[rest] == s.min()]
            if len(tie):
                assert sel[s == s.min()].max() < tie.min()


def test_topk_select_properties_with_many_ties():
    """Random rows drawn from a handful of values (so most scores tie), with
    NaN, infinities and signed zeros sprinkled in, over every kind of
    sequence length (negative, 0, below k, above max_len)."""
    rng = np.random.default_rng(71)
    vals = np.array([-np.inf, -2.0, -0.0, 0.0, 0.5, 1.0, 1.0 + 2 ** -20, np.inf, np.nan], dtype=np.float32)
    for trial in range(40):
        B, max_len, k = int(rng.integers(1, 5)), int(rng.integers(1, 300)), int(rng.integers(1, 70))
        scores = vals[rng.integers(0, len(vals), (B, max_len))]
        seq_lens = rng.integers(-3, max_len + 10, B)
        got = O.topk_select(scores, seq_lens, k)
        assert got.shape == (B, k) and got.dtype == np.int32
        _check_topk_properties(scores, seq_lens, k, got)


def test_topk_select_distinct_scores_match_a_full_sort():
    """With distinct scores the selection is the k largest in descending
    order: compared with numpy's argsort of the negated row."""
    rng = np.random.default_rng(72)
    scores = rng.permutation(4096).astype(np.float32).reshape(4, 1024) * 0.25 - 300.0
    seq_lens = np.array([1024, 700, 5, 1024])
    got = O.topk_select(scores, seq_lens, 512)
    for b in range(4):
        L = int(seq_lens[b])
        ref = np.argsort(-scores[b, :L], kind="stable")[:512]
        assert got[b, :len(ref)].tolist() == ref.tolist()
