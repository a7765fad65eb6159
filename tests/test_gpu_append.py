"""Parity of the cache-append kernel (mla_kv_append) with the oracle's
quantiser: after the append the whole pool must match the oracle's pool
byte for byte -- written records, scale records, and every byte the append
must leave alone."""
import numpy as np
import pytest
import torch

import sparse_mla_decode_page_amd as mlasd
from gen import synth as G
from oracle import mla_oracle as O

from helpers import check_attention, decode

pytestmark = pytest.mark.gpu

PAGE = O.BYTES_PER_PAGE


def _group_mix(n, seed):
    """bf16 latents whose 64-dim groups cover the quantiser's cases: N(0,1),
    20-sigma outliers, all zero, signed zeros, tiny (2^-30) and bf16-subnormal
    magnitudes, the largest finite bf16, exact e4m3 values times a power of
    two, and amax exactly on / just past a scale boundary (448, 450, 224)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 512))
    kinds = rng.integers(0, 10, (n, 7))
    for t in range(n):
        for g in range(7):
            s = slice(64 * g, 64 * g + 64)
            k = kinds[t, g]
            if k == 1:
                x[t, s] *= 20.0
            elif k == 2:
                x[t, s] = 0.0
            elif k == 3:
                x[t, s] = np.where(rng.random(64) < 0.5, -0.0, 0.0)
                x[t, 64 * g + 5] = -3.0
            elif k == 4:
                x[t, s] *= 2.0 ** -30
            elif k == 5:   # bf16 subnormals (below 2^-126)
                x[t, s] = rng.integers(-127, 128, 64) * 2.0 ** -133
            elif k == 6:
                x[t, s] = O.e4m3_value(rng.integers(0, 255, 64) & 0xF7) * 2.0 ** int(rng.integers(-20, 20))
            elif k == 7:
                x[t, s] *= 1e37
                x[t, 64 * g + 7] = -3.3895313892515355e38   # largest finite bf16
            elif k == 8:
                x[t, s] = np.clip(x[t, s] * 100.0, -447.0, 447.0)
                x[t, 64 * g + 9] = float(rng.choice([448.0, -448.0, 450.0, 224.0, -224.0]))
    return G.bf16_bits(x)


def _pool(num_pages, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, (num_pages, PAGE), dtype=np.uint8)


def _append_gpu(pool, page_table, seq_ids, positions, bits, stream=None):
    dev = torch.device("cuda")
    kv = torch.from_numpy(pool).to(dev)
    lat = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
    mlasd.mla_kv_append(lat, torch.from_numpy(np.asarray(seq_ids, np.int32)).to(dev),
                        torch.from_numpy(np.asarray(positions, np.int32)).to(dev),
                        torch.from_numpy(np.asarray(page_table, np.int32)).to(dev), kv,
                        stream=stream)
    torch.cuda.synchronize()
    return kv.cpu().numpy()


def _assert_pool_equal(got, ref, label):
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        pg, off = bad[0]
        where = (f"record slot {off // 576} byte {off % 576}" if off < O.SCALE_REGION else
                 f"scale record slot {(off - O.SCALE_REGION) // 8} byte {(off - O.SCALE_REGION) % 8}")
        raise AssertionError(f"{label}: {len(bad)} bytes differ; first at page {pg} {where}: "
                             f"got {got[pg, off]:#04x} want {ref[pg, off]:#04x}")


def test_append_bit_exact_with_invalid_tokens():
    print("append: 3 sequences, 6 pages, mixed groups + invalid tokens", flush=True)
    rng = np.random.default_rng(5)
    num_pages = 6
    page_table = np.array([[4, 0, -1], [2, 5, 1], [3, 6, -1]], dtype=np.int32)  # 6 = out of pool
    dests = [(0, p) for p in rng.choice(512, 70, replace=False)]
    dests += [(1, p) for p in rng.choice(768, 90, replace=False)]
    dests += [(2, p) for p in rng.choice(256, 40, replace=False)]
    invalid = [(-1, 3), (3, 3), (1, -1), (0, 3 * 256), (0, 2 * 256 + 7), (2, 256 + 1),
               (2, 1 << 30), (-7, -7)]
    dests += invalid
    order = rng.permutation(len(dests))
    seq = np.array([dests[i][0] for i in order], np.int32)
    pos = np.array([dests[i][1] for i in order], np.int32)
    bits = _group_mix(len(dests), 17)
    pool = _pool(num_pages, 3)
    ref = O.kv_append(pool, page_table, seq, pos, bits)
    got = _append_gpu(pool, page_table, seq, pos, bits)
    _assert_pool_equal(got, ref, "mixed append")
    # the invalid tokens wrote nothing: the oracle pool differs from the
    # input only in the 200 valid destinations
    changed_slots = set()
    for pg, off in np.argwhere(ref != pool):
        changed_slots.add((int(pg), int(off // 576) if off < O.SCALE_REGION
                           else int((off - O.SCALE_REGION) // 8)))
    assert len(changed_slots) <= 200


@pytest.mark.parametrize("n", [1, 3, 4, 5, 127, 257])
def test_append_token_counts(n):
    """Token counts around the kernel's four tokens per workgroup."""
    print(f"append: {n} tokens", flush=True)
    rng = np.random.default_rng(100 + n)
    page_table = np.array([[1, 0]], dtype=np.int32)
    pos = rng.choice(512, n, replace=False).astype(np.int32)
    seq = np.zeros(n, np.int32)
    bits = _group_mix(n, 200 + n)
    pool = _pool(2, n)
    _assert_pool_equal(_append_gpu(pool, page_table, seq, pos, bits),
                       O.kv_append(pool, page_table, seq, pos, bits), f"n={n}")


def test_append_zero_tokens_is_noop():
    pool = _pool(1, 9)
    kv = torch.from_numpy(pool).cuda()
    empty_i = torch.empty(0, dtype=torch.int32, device="cuda")
    lat = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    mlasd.mla_kv_append(lat, empty_i, empty_i, torch.zeros((1, 1), dtype=torch.int32, device="cuda"), kv)
    torch.cuda.synchronize()
    assert np.array_equal(kv.cpu().numpy(), pool)


def test_append_overwrite_and_stream():
    """A second append to the same slots replaces the first; launched on a
    non-default stream."""
    rng = np.random.default_rng(44)
    page_table = np.array([[0], [1]], dtype=np.int32)
    seq = np.array([0] * 20 + [1] * 20, np.int32)
    pos = np.concatenate([rng.choice(256, 20, replace=False), rng.choice(256, 20, replace=False)]).astype(np.int32)
    a, b = _group_mix(40, 1), _group_mix(40, 2)
    pool = _pool(2, 4)
    dev = torch.device("cuda")
    kv = torch.from_numpy(pool).to(dev)
    s = torch.cuda.Stream()
    ids, ps, pt = (torch.from_numpy(v).to(dev) for v in (seq, pos, page_table))
    with torch.cuda.stream(s):
        for bits in (a, b):
            lat = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
            mlasd.mla_kv_append(lat, ids, ps, pt, kv, stream=s)
    s.synchronize()
    _assert_pool_equal(kv.cpu().numpy(), O.kv_append(pool, page_table, seq, pos, b), "overwrite")


def test_append_then_decode():
    """Fill two sequences through the append kernel, then decode over them:
    the pool matches the oracle's byte for byte, and the decode of it matches
    the oracle's decode within the attention tolerance."""
    rng = np.random.default_rng(808)
    lens = np.array([150, 300], np.int32)
    page_table = np.array([[3, -1], [0, 2]], dtype=np.int32)
    seq = np.concatenate([np.zeros(150, np.int32), np.ones(300, np.int32)])
    pos = np.concatenate([np.arange(150), np.arange(300)]).astype(np.int32)
    perm = rng.permutation(450)
    seq, pos = seq[perm], pos[perm]
    x = rng.standard_normal((450, 512))
    x[:, 64 * 3 + 11] *= 20.0   # an outlier channel
    bits = G.bf16_bits(x)
    pool = _pool(4, 8)
    ref_pool = O.kv_append(pool, page_table, seq, pos, bits)
    got_pool = _append_gpu(pool, page_table, seq, pos, bits)
    _assert_pool_equal(got_pool, ref_pool, "append before decode")
    topk = 128
    idx = np.full((2, topk), -1, np.int32)
    idx[0, :128] = rng.choice(150, 128, replace=False)
    idx[1] = rng.choice(300, topk, replace=False)
    q = G.bf16_bits(rng.standard_normal((2, 64, 512)))
    scale = 1.0 / np.sqrt(192.0)
    ref_out, ref_lse = O.sparse_mla_decode(q, ref_pool, page_table, idx, lens, scale)
    dev = torch.device("cuda")
    d = dict(q=torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(dev),
             kv_pages=torch.from_numpy(got_pool).to(dev), page_table=torch.from_numpy(page_table).to(dev),
             topk_idx=torch.from_numpy(idx).to(dev), seq_lens=torch.from_numpy(lens).to(dev))
    out, lse = decode(d, scale)
    torch.cuda.synchronize()
    check_attention(out, lse, ref_out, ref_lse, label="decode after append")


def test_append_large_sampled():
    """A prefill-sized append (64 sequences x 1,024 new tokens into 256 pages),
    checked on a sample of tokens against the oracle's quantiser and on the
    untouched slots of one page."""
    print("append: 65536 tokens, sampled", flush=True)
    B, per = 64, 1024
    num_pages = B * per // 256
    rng = np.random.default_rng(2026)
    page_table = rng.permutation(num_pages).astype(np.int32).reshape(B, per // 256)
    seq = np.repeat(np.arange(B, dtype=np.int32), per)
    pos = np.tile(np.arange(per, dtype=np.int32), B)
    dev = torch.device("cuda")
    g = torch.Generator(device="cpu").manual_seed(7)
    lat = (torch.randn((B * per, 512), generator=g) * torch.exp(torch.randn((B * per, 1), generator=g) * 3))
    lat = lat.to(torch.bfloat16)
    kv = torch.zeros((num_pages, PAGE), dtype=torch.uint8, device=dev)
    mlasd.mla_kv_append(lat.to(dev), torch.from_numpy(seq).to(dev), torch.from_numpy(pos).to(dev),
                        torch.from_numpy(page_table).to(dev), kv)
    torch.cuda.synchronize()
    got = kv.cpu().numpy()
    bits = lat.view(torch.int16).numpy().view(np.uint16)
    for t in rng.choice(B * per, 48, replace=False):
        s, p = int(seq[t]), int(pos[t])
        page, slot = int(page_table[s, p // 256]), p % 256
        rec, sc = O.quantize_token(bits[t])
        assert np.array_equal(got[page, slot * 576:(slot + 1) * 576], rec), f"token {t}"
        assert np.array_equal(got[page, O.SCALE_REGION + 8 * slot:O.SCALE_REGION + 8 * slot + 8], sc), \
            f"token {t} scales"


def test_append_graph_capture_replay():
    """The append captured in a HIP graph replays to the oracle's bytes: three
    replays, with the pool restored by eager work between them."""
    rng = np.random.default_rng(77)
    page_table = np.array([[2, 0], [1, -1]], dtype=np.int32)
    seq = np.array([0] * 30 + [1] * 30, np.int32)
    pos = np.concatenate([rng.choice(512, 30, replace=False), rng.choice(256, 30, replace=False)]).astype(np.int32)
    bits = _group_mix(60, 78)
    pool = _pool(3, 79)
    ref = O.kv_append(pool, page_table, seq, pos, bits)
    dev = torch.device("cuda")
    kv = torch.from_numpy(pool).to(dev)
    pool_dev = kv.clone()
    lat = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    ids, ps, pt = (torch.from_numpy(v).to(dev) for v in (seq, pos, page_table))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mlasd.mla_kv_append(lat, ids, ps, pt, kv, stream=s)
    for rep in range(3):
        kv.copy_(pool_dev)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _assert_pool_equal(kv.cpu().numpy(), ref, f"graph replay {rep}")


def test_append_strided_views():
    """Latents as a row-strided view, ids and positions with strides, a
    column-sliced page table and a pool at a padded page stride: the same
    bytes as the oracle's append into a contiguous pool, and the padding
    bytes untouched."""
    rng = np.random.default_rng(91)
    page_table = np.array([[2, 0], [1, -1]], dtype=np.int32)
    seq = np.array([0] * 20 + [1] * 20, np.int32)
    pos = np.concatenate([rng.choice(512, 20, replace=False), rng.choice(256, 20, replace=False)]).astype(np.int32)
    bits = _group_mix(40, 92)
    pool = _pool(3, 93)
    ref = O.kv_append(pool, page_table, seq, pos, bits)
    dev = torch.device("cuda")
    wide = torch.full((3, PAGE + 256), 0xA5, dtype=torch.uint8, device=dev)
    wide[:, :PAGE] = torch.from_numpy(pool).to(dev)
    latbig = torch.zeros((40, 520), dtype=torch.bfloat16, device=dev)
    latbig[:, 8:] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    ids = torch.zeros((40, 2), dtype=torch.int32, device=dev)
    ids[:, 1] = torch.from_numpy(seq).to(dev)
    ps = torch.zeros((40, 3), dtype=torch.int32, device=dev)
    ps[:, 2] = torch.from_numpy(pos).to(dev)
    ptbig = torch.full((2, 5), 7, dtype=torch.int32, device=dev)
    ptbig[:, 1:3] = torch.from_numpy(page_table).to(dev)
    mlasd.mla_kv_append(latbig[:, 8:], ids[:, 1], ps[:, 2], ptbig[:, 1:3], wide[:, :PAGE])
    torch.cuda.synchronize()
    got = wide.cpu().numpy()
    _assert_pool_equal(np.ascontiguousarray(got[:, :PAGE]), ref, "strided append")
    assert np.all(got[:, PAGE:] == 0xA5)
