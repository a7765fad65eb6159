"""Seeded synthetic inputs for sparse-MLA paged decode.

This module draws and packs inputs only.  It computes nothing that the decode
computes: no dequantisation, no scores, no softmax.  Both the CPU oracle and
the HIP library are fed from here, so neither side ever produces the other's
inputs.

Byte layout of the paged cache, as described on "The Validation Gate"
(section "The Test Design: What Gets Validated and How") and "The Moment of
Validation" (section "The Context: Building a Custom Kernel from Scratch"):

* the pool is ``uint8 [num_pages, 256 * 584]``; one page holds 256 tokens;
* the first ``256 * 576`` bytes of a page are the token records, 576 bytes
  each: 448 fp8 e4m3 "nope" bytes followed by 64 little-endian bf16 rope
  values (128 bytes);
* then come the 256 scale records, 8 bytes each: one UE8M0 exponent byte per
  64-wide nope group (7 groups) and one zero pad byte.

Value recipe (per workload description): Q ~ N(0,1) rounded to bf16; nope
~ N(0,1) quantised per 64-group with a power-of-two scale 2^k, k the least
integer with 448 * 2^k >= amax; rope ~ N(0,1) rounded to bf16.

Random numbers come from numpy's Philox counter-based generator, drawn in the
fixed order: page tables, index lists, Q, outlier channels, nope, rope.
Only the records an index list selects get drawn values; every other byte of
the pool holds a poison byte (0x7F, an fp8 NaN code), so a kernel that reads a
record it was not asked for cannot produce a finite, matching result.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

HEADS = 64
D_NOPE = 448
D_ROPE = 64
D_QK = D_NOPE + D_ROPE
GROUP = 64
N_GROUPS = D_NOPE // GROUP
PAGE_TOKENS = 256
TOKEN_BYTES = D_NOPE + 2 * D_ROPE          # 576
SCALE_BYTES = 8
PAGE_BYTES = PAGE_TOKENS * (TOKEN_BYTES + SCALE_BYTES)  # 149504
SCALE_BASE = PAGE_TOKENS * TOKEN_BYTES     # 147456
POISON = 0x7F

BASE_SEED = 20261202


# ----------------------------------------------------------------------------
# packing helpers (encoders only)
# ----------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float values to bf16 (nearest, ties to even) via float32; return
    the 16-bit patterns as uint16."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Encode finite values with |y| <= 448 as OCP fp8 e4m3 ("fn") codes,
    rounding to nearest with ties to even."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(~np.isfinite(y)) or np.any(np.abs(y) > 448.0):
        raise ValueError("e4m3_encode: input out of range")
    sign = (np.signbit(y)).astype(np.uint8) << 7
    a = np.abs(y)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal band: multiples of 2^-9; np.rint rounds half to even
    q = np.rint(a[sub] * 512.0).astype(np.int64)      # 0..8, 8 is 2^-6
    code[sub] = np.where(q == 8, 8, q)                 # 8 == exponent field 1, mantissa 0
    nrm = ~sub
    m, e = np.frexp(a[nrm])                            # a = m * 2^e, m in [0.5, 1)
    e = e - 1                                          # a = (2m) * 2^e, 2m in [1, 2)
    frac = np.rint((2.0 * m - 1.0) * 8.0).astype(np.int64)
    carry = frac == 8
    frac[carry] = 0
    e[carry] += 1
    code[nrm] = ((e + 7) << 3) | frac
    return (code.astype(np.uint8) | sign)


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Least integer k with 448 * 2^k >= amax, clamped to [-127, 127];
    amax == 0 gives -127.  Exact (frexp based, no floating log2)."""
    amax = np.asarray(amax, dtype=np.float64)
    m, e = np.frexp(amax)                  # amax = m * 2^e, m in [0.5, 1)
    # 448 = 0.875 * 2^9
    k = np.where(m <= 0.875, e - 9, e - 8)
    k = np.where(amax == 0.0, -127, k)
    return np.clip(k, -127, 127).astype(np.int64)


def quantize_nope(x: np.ndarray):
    """x: float64 [..., 448] -> (codes uint8 [..., 448], scale bytes uint8 [..., 7])."""
    g = x.reshape(*x.shape[:-1], N_GROUPS, GROUP)
    amax = np.abs(g).max(axis=-1)
    k = scale_exponent(amax)
    y = g * np.ldexp(1.0, -k)[..., None]
    codes = e4m3_encode(y).reshape(x.shape)
    return codes, (k + 127).astype(np.uint8)


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    q_bits: np.ndarray          # uint16 [B, 64, 512], bf16 bit patterns
    kv_pages: np.ndarray        # uint8  [num_pages, 149504]
    page_table: np.ndarray      # int32  [B, max_pages]
    topk_idx: np.ndarray        # int32  [B, topk]
    seq_lens: np.ndarray        # int32  [B]
    softmax_scale: float = 1.0 / math.sqrt(D_QK)
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return self.q_bits.shape[0]

    @property
    def topk(self):
        return self.topk_idx.shape[1]

    @property
    def num_pages(self):
        return self.kv_pages.shape[0]

    @property
    def max_pages(self):
        return self.page_table.shape[1]


def _rng(seed):
    return np.random.Generator(np.random.Philox(seed))


def _write_records(pool: np.ndarray, pages, slots, codes, scale_bytes, rope_bits):
    flat = pool.reshape(-1)
    pages = np.asarray(pages, dtype=np.int64)
    slots = np.asarray(slots, dtype=np.int64)
    base = pages * PAGE_BYTES + slots * TOKEN_BYTES
    rec = np.empty((len(pages), TOKEN_BYTES), dtype=np.uint8)
    rec[:, :D_NOPE] = codes
    rec[:, D_NOPE:] = np.ascontiguousarray(rope_bits.astype("<u2")).view(np.uint8).reshape(len(pages), 2 * D_ROPE)
    flat[base[:, None] + np.arange(TOKEN_BYTES)] = rec
    sbase = pages * PAGE_BYTES + SCALE_BASE + slots * SCALE_BYTES
    srec = np.zeros((len(pages), SCALE_BYTES), dtype=np.uint8)
    srec[:, :N_GROUPS] = scale_bytes
    flat[sbase[:, None] + np.arange(SCALE_BYTES)] = srec


def draw_records(rng, n, outlier_channels=None, outlier_sigma=20.0, group_scale=None):
    """Draw n token records: returns (codes [n,448], scale bytes [n,7], rope bf16 bits [n,64]).
    group_scale(rng, n) -> [n, 7] multiplies each 64-dim nope group (wide
    dynamic-range caches)."""
    x = rng.standard_normal((n, D_NOPE))
    if outlier_channels is not None and len(outlier_channels):
        x[:, outlier_channels] *= outlier_sigma
    if group_scale is not None:
        x *= np.repeat(np.asarray(group_scale(rng, n), dtype=np.float64), GROUP, axis=1)
    rope = rng.standard_normal((n, D_ROPE))
    codes, sb = quantize_nope(x)
    return codes, sb, bf16_bits(rope)


def build_workload(seed, seq_lens, topk, *, name="custom", num_pages=None, max_pages=None,
                   outlier_frac=0.0, outlier_channels=None, fill="selected",
                   index_order="random", softmax_scale=None, pool=None, page_table=None,
                   group_scale=None):
    """General seeded builder.

    seq_lens    : per-query context lengths (>= 0)
    topk        : index list width; a query with len < topk lists all of its
                  positions followed by -1 padding
    num_pages   : pool size (default: exactly the pages the sequences need)
    fill        : "selected" -> only selected records drawn, the rest poisoned;
                  "all" -> every record of every page drawn (small pools only)
    index_order : "random" (positions shuffled) or "sorted"
    pool, page_table : reuse an existing pool/page table (new index set on the
                  same cache); selected records are (re)drawn and written.
    group_scale : optional callable (rng, n) -> [n, 7] multipliers of each
                  record's nope groups before quantisation
    """
    rng = _rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = len(seq_lens)
    pages_needed = (seq_lens + PAGE_TOKENS - 1) // PAGE_TOKENS
    if page_table is None:
        total = int(pages_needed.sum())
        if num_pages is None:
            num_pages = max(total, 1)
        if num_pages < total:
            raise ValueError("pool too small")
        if max_pages is None:
            max_pages = max(int(pages_needed.max()) if B else 1, 1)
        perm = rng.permutation(num_pages)
        page_table = np.full((B, max_pages), -1, dtype=np.int32)
        off = 0
        for b in range(B):
            n = int(pages_needed[b])
            page_table[b, :n] = perm[off:off + n]
            off += n
    else:
        page_table = np.asarray(page_table, dtype=np.int32)
        num_pages = pool.shape[0]

    topk_idx = np.full((B, topk), -1, dtype=np.int32)
    for b in range(B):
        L = int(seq_lens[b])
        if L >= topk:
            sel = rng.choice(L, size=topk, replace=False)
            if index_order == "sorted":
                sel = np.sort(sel)
            topk_idx[b] = sel
        elif L > 0:
            sel = rng.permutation(L) if index_order == "random" else np.arange(L)
            topk_idx[b, :L] = sel

    q_bits = bf16_bits(rng.standard_normal((B, HEADS, D_QK)))

    if outlier_channels is not None:
        outliers = np.asarray(outlier_channels, dtype=np.int64)
    else:
        n_out = int(round(outlier_frac * D_NOPE))
        outliers = np.sort(rng.choice(D_NOPE, size=n_out, replace=False)) if n_out else None

    if pool is None:
        pool = np.full((num_pages, PAGE_BYTES), POISON, dtype=np.uint8)
    if fill == "all":
        pg = np.repeat(np.arange(num_pages), PAGE_TOKENS)
        sl = np.tile(np.arange(PAGE_TOKENS), num_pages)
    else:
        bb, jj = np.nonzero(topk_idx >= 0)
        pos = topk_idx[bb, jj].astype(np.int64)
        pg = page_table[bb, pos // PAGE_TOKENS].astype(np.int64)
        sl = pos % PAGE_TOKENS
    if len(pg):
        codes, sb, rope = draw_records(rng, len(pg), outliers, group_scale=group_scale)
        _write_records(pool, pg, sl, codes, sb, rope)

    scale = 1.0 / math.sqrt(D_QK) if softmax_scale is None else float(softmax_scale)
    return Workload(name=name, q_bits=q_bits, kv_pages=pool, page_table=page_table,
                    topk_idx=topk_idx, seq_lens=seq_lens.astype(np.int32), softmax_scale=scale,
                    meta={"seed": seed, "outlier_channels": None if outliers is None else outliers.tolist(),
                          "fill": fill})


CONFIG_NAMES = [
    "c0: B=1 topk=64 seq_len=256 (1 page)",
    "c1: B=1 topk=512 seq_len=4096 (16 pages, permuted)",
    "c2: B=16 topk=512 seq_len=32768 (pool 2048 pages)",
    "c3: B=64 topk=512 seq_len=65536 (pool 16384 pages, 1% outlier channels at 20 sigma)",
    "c4: B=256 topk=512 seq_len log-uniform in [1,131072] (-1 padded)",
]


def config_seq_lens(i, seed=None):
    """Sequence lengths of workload i (the variable-length mix for i == 4)."""
    seed = BASE_SEED + i if seed is None else seed
    if i == 0:
        return np.array([256])
    if i == 1:
        return np.array([4096])
    if i == 2:
        return np.full(16, 32768)
    if i == 3:
        return np.full(64, 65536)
    if i == 4:
        # drawn from a stream of its own so the main stream order is unchanged
        r = _rng(seed ^ 0x5EED)
        u = r.random(256)
        L = np.floor(np.exp(u * math.log(131072.0))).astype(np.int64)
        return np.clip(L, 1, 131072)
    raise ValueError(i)


def make_config(i, seed=None, fill="selected", pool=None, page_table=None):
    """Workload i of the five standard shapes, seeded with 20261202 + i."""
    seed = BASE_SEED + i if seed is None else seed
    lens = config_seq_lens(i, None)
    kw = {}
    if i == 3:
        kw["outlier_frac"] = 0.01
    if i == 4:
        kw["max_pages"] = 131072 // PAGE_TOKENS
    w = build_workload(seed, lens, 64 if i == 0 else 512, name=CONFIG_NAMES[i], fill=fill,
                       pool=pool, page_table=page_table, **kw)
    w.meta["config_index"] = i
    return w


def extra_index_set(w: Workload, seed):
    """A new Q and index list on the same pool and page tables (records drawn
    for the newly selected positions are written into the shared pool)."""
    lens = w.seq_lens.astype(np.int64)
    out = build_workload(seed, lens, w.topk, name=w.name, pool=w.kv_pages,
                         page_table=w.page_table, softmax_scale=w.softmax_scale,
                         outlier_channels=w.meta.get("outlier_channels"))
    out.meta["config_index"] = w.meta.get("config_index")
    return out


def rotation_sets(w: Workload, n_sets, seed):
    """n_sets - 1 further (Q, index list) sets on the pool of `w` for timing
    runs whose working set must exceed the caches.  Each set draws a new Q
    and new distinct positions per query (same lengths and -1 padding rule);
    the record bytes written at a newly selected slot are copied from a
    record that `w` already selected (same value distribution, no new draws),
    so only addresses change between sets.  Returns [w, set1, ...]."""
    rng = _rng(seed)
    flat = w.kv_pages.reshape(-1)
    bb, jj = np.nonzero(w.topk_idx >= 0)
    pos0 = w.topk_idx[bb, jj].astype(np.int64)
    src_pg = w.page_table[bb, pos0 // PAGE_TOKENS].astype(np.int64)
    src_sl = pos0 % PAGE_TOKENS
    src_rec = flat[(src_pg * PAGE_BYTES + src_sl * TOKEN_BYTES)[:, None] + np.arange(TOKEN_BYTES)]
    src_sc = flat[(src_pg * PAGE_BYTES + SCALE_BASE + src_sl * SCALE_BYTES)[:, None] + np.arange(SCALE_BYTES)]
    out = [w]
    B, K = w.topk_idx.shape
    lens = w.seq_lens.astype(np.int64)
    for _ in range(n_sets - 1):
        idx = np.full((B, K), -1, dtype=np.int32)
        for b in range(B):
            L = int(lens[b])
            if L >= K:
                idx[b] = rng.choice(L, size=K, replace=False)
            elif L > 0:
                idx[b, :L] = rng.permutation(L)
        q_bits = bf16_bits(rng.standard_normal((B, HEADS, D_QK)))
        nb, nj = np.nonzero(idx >= 0)
        pos = idx[nb, nj].astype(np.int64)
        pg = w.page_table[nb, pos // PAGE_TOKENS].astype(np.int64)
        sl = pos % PAGE_TOKENS
        pick = rng.integers(0, len(src_rec), size=len(pos)) if len(src_rec) else np.zeros(0, np.int64)
        if len(pos) and len(src_rec):
            flat[(pg * PAGE_BYTES + sl * TOKEN_BYTES)[:, None] + np.arange(TOKEN_BYTES)] = src_rec[pick]
            flat[(pg * PAGE_BYTES + SCALE_BASE + sl * SCALE_BYTES)[:, None] + np.arange(SCALE_BYTES)] = src_sc[pick]
        out.append(Workload(name=w.name, q_bits=q_bits, kv_pages=w.kv_pages, page_table=w.page_table,
                            topk_idx=idx, seq_lens=w.seq_lens, softmax_scale=w.softmax_scale,
                            meta=dict(w.meta, rotation=True)))
    return out


def indexer_scores(seed, batch, max_len, kind="normal"):
    """Seeded fp32 per-position scores [batch, max_len] standing in for an
    indexer's output: "normal" (standard normal, ties rare), "ties" (a
    handful of values, ties everywhere) or "special" ("ties" plus NaN,
    infinities and signed zeros)."""
    rng = _rng(seed)
    if kind == "normal":
        return rng.standard_normal((batch, max_len)).astype(np.float32)
    vals = [-1.5, -0.25, 0.5, 0.5 + 2 ** -20, 3.0]
    if kind == "special":
        vals += [np.nan, np.inf, -np.inf, -0.0, 0.0]
    vals = np.array(vals, dtype=np.float32)
    return vals[rng.integers(0, len(vals), (batch, max_len))]
