"""CPU fp64 oracle for sparse Multi-head Latent Attention decode over a paged
FP8 KV cache.

TEST INFRASTRUCTURE ONLY.  This module is the correctness reference.  Only
the test suite, the package smoke check and the CPU-baseline leg of the
benchmark may import it.  The product path (the HIP library and its Python
binding) never calls it and shares no code, table or constant with it.

Everything is computed in float64 with plain numpy.  A matrix product
(``@``) and ``exp``/``log`` are the only library primitives used; there is no
blocking, splitting or reordering beyond the definition below.

What is computed (cited by page title and section):

* Each decode query has 64 heads that share one latent KV head; the top-k
  index list belongs to the query, not to a head ("The Turning Point",
  section "Assumptions Made and Their Validity", Assumption 1; "Input
  Knowledge Required", the MLA bullet).
* The cache is a flat ``uint8 [num_pages, 256*584]`` pool.  A page holds all
  256 token records of 576 bytes (448 fp8 nope bytes, then 64 bf16 rope
  values), followed by the 256 records of 8 scale bytes ("The Validation
  Gate", section "The Test Design: What Gets Validated and How").
* The nope bytes are fp8 e4m3 with UE8M0 group scales and are dequantised
  before the matmul; data flows dequantise -> concatenate with rope ->
  matmul -> softmax -> weighted sum ("The Turning Point", "Input Knowledge
  Required", FP8/UE8M0 bullet, and "Output Knowledge Created", item 2).
* Q is ``[B, 64, 512]``: 448 nope dims followed by 64 rope dims ("The Turning
  Point", "The Reasoning Process", Step 1).  The scores use all 512 dims; the
  nope pad to 512 of the pages' Triton kernel adds only zero terms ("The
  Moment of Validation", section "Two Failures, Two Lessons").
* Only the first 448 output columns are produced ("The Moment of
  Validation", "Two Failures, Two Lessons"); with V = the 448 nope dims of the
  dequantised key.  The outputs are the attention values and a log-sum-exp
  per head ("The Validation Gate", "Output Knowledge Created", item 4).

Readings where the pages are silent (numbered as in the design notes, whose
R7-R12 cover the output format, tolerances, record order and the kernel):
  R1  7 scale bytes per token, byte g scales nope dims [64g, 64g+64); byte 7
      is padding and is ignored.
  R2  UE8M0 byte e means 2^(e-127); e = 255 is NaN.
  R3  e4m3 is the OCP "fn" variant: bias 7, subnormals, max 448, no
      infinities, 0x7F / 0xFF are NaN.
  R4  index p of query b is valid iff 0 <= p < seq_lens[b]; its logical page
      p // 256 is looked up in page_table[b]; slot p % 256.  Entries are
      masked when p is out of range, when p // 256 is beyond the page-table
      row, or when the physical page id is outside [0, num_pages).
      Every valid entry counts once, duplicates included.
  R5  lse is the natural log of the sum of exp over the *scaled* scores.
  R6  A query with no valid entry gets out = 0 and lse = -inf.
  R13 (cache append) A token latent is quantised per 64-dim group: the scale
      exponent k is the least integer with amax <= 448 * 2^k, clamped to
      [-127, 127] (amax = 0 gives -127); the scale byte is k + 127; every value
      is encoded as the e4m3 code nearest to x * 2^-k, ties to the even code,
      sign kept (also for zero).  Scale byte 7 is written as 0.  The rope
      values are stored as they are.  A token is written at position p of
      sequence s when 0 <= s < B, p >= 0, p // 256 < max_pages and the
      physical page lies in the pool; otherwise it is skipped.
  R14 (top-k selection, upstream of the decode) The indexer scores every
      position of a query's context in fp32 ("The Turning Point", "The
      Strategic Context: Why This Message Exists", item 3) and the top-k
      positions become topk_idx.  Read here: positions 0 .. L-1 with
      L = min(max(seq_len, 0), max_len) are candidates; they are ranked by
      score, higher first, equal scores by position, lower first (a NaN score
      ranks as -inf, -0.0 equals +0.0); the first min(k, L) positions in rank
      order are written, in that order, and the rest of the k slots get -1.
"""
from __future__ import annotations

import numpy as np

# Layout constants, stated from the pages (not imported from anywhere).
N_HEADS = 64
NOPE = 448
ROPE = 64
QK_DIM = NOPE + ROPE
V_DIM = NOPE
SCALE_GROUP = 64
TOKENS_PER_PAGE = 256
RECORD_BYTES = 576
SCALE_RECORD_BYTES = 8
BYTES_PER_PAGE = TOKENS_PER_PAGE * (RECORD_BYTES + SCALE_RECORD_BYTES)
SCALE_REGION = TOKENS_PER_PAGE * RECORD_BYTES


# ----------------------------------------------------------------------------
# scalar formats
# ----------------------------------------------------------------------------

def e4m3_value(code):
    """OCP fp8 E4M3 ("fn") code -> float64 (reading R3).

    sign = bit 7, exponent field E = bits 6..3, mantissa M = bits 2..0;
    E == 0: (-1)^s * M * 2^-9 (subnormal); E == 15 and M == 7: NaN;
    otherwise (-1)^s * (1 + M/8) * 2^(E - 7).
    """
    c = np.asarray(code, dtype=np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    E = (c >> 3) & 15
    M = c & 7
    normal = s * (1.0 + M / 8.0) * np.exp2(E.astype(np.float64) - 7.0)
    sub = s * M * 2.0 ** -9
    v = np.where(E == 0, sub, normal)
    return np.where((E == 15) & (M == 7), np.nan, v)


def ue8m0_value(byte):
    """UE8M0 scale byte -> float64: 2^(e-127), 255 -> NaN (reading R2)."""
    e = np.asarray(byte, dtype=np.int64)
    return np.where(e == 255, np.nan, np.exp2(e.astype(np.float64) - 127.0))


def bf16_value(bits):
    """bf16 bit pattern (uint16) -> float64 (bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


_E4M3_TABLE = e4m3_value(np.arange(256))


# ----------------------------------------------------------------------------
# index resolution and gather/dequant
# ----------------------------------------------------------------------------

def resolve_entries(page_table, topk_idx, seq_lens, num_pages):
    """Per entry (b, j): valid flag, physical page and slot (reading R4)."""
    page_table = np.asarray(page_table, dtype=np.int64)
    idx = np.asarray(topk_idx, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    B, max_pages = page_table.shape
    valid = (idx >= 0) & (idx < lens[:, None])
    logical = np.where(valid, idx // TOKENS_PER_PAGE, 0)
    valid &= logical < max_pages
    logical = np.where(valid, logical, 0)
    page = np.take_along_axis(page_table, logical, axis=1) if B else np.zeros_like(idx)
    valid &= (page >= 0) & (page < num_pages)
    page = np.where(valid, page, 0)
    slot = np.where(valid, idx % TOKENS_PER_PAGE, 0)
    return valid, page, slot


def gather_dequant(kv_pages, page_table, topk_idx, seq_lens):
    """Dequantised key rows of every entry.

    Returns (rows float64 [B, topk, 512], valid bool [B, topk]); rows of
    masked entries are 0.  Row d < 448 is e4m3(byte d) * 2^(scale[d // 64] - 127);
    rows 448.. are the 64 bf16 rope values.
    """
    kv = np.asarray(kv_pages, dtype=np.uint8)
    num_pages = kv.shape[0]
    flat = kv.reshape(-1)
    valid, page, slot = resolve_entries(page_table, topk_idx, seq_lens, num_pages)
    B, K = valid.shape
    rows = np.zeros((B, K, QK_DIM), dtype=np.float64)
    bb, jj = np.nonzero(valid)
    if len(bb):
        pg = page[bb, jj]
        sl = slot[bb, jj]
        rec = pg * BYTES_PER_PAGE + sl * RECORD_BYTES
        nope = flat[rec[:, None] + np.arange(NOPE)]
        rope_bytes = flat[rec[:, None] + NOPE + np.arange(2 * ROPE)]
        rope_bits = rope_bytes[:, 0::2].astype(np.uint16) | (rope_bytes[:, 1::2].astype(np.uint16) << 8)
        srec = pg * BYTES_PER_PAGE + SCALE_REGION + sl * SCALE_RECORD_BYTES
        groups = np.arange(NOPE) // SCALE_GROUP
        scale = ue8m0_value(flat[srec[:, None] + groups])
        rows[bb, jj, :NOPE] = _E4M3_TABLE[nope] * scale
        rows[bb, jj, NOPE:] = bf16_value(rope_bits)
    return rows, valid


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def attend(q, keys, softmax_scale):
    """Dense softmax attention of one query over exactly the given key rows.

    q: float64 [H, 512]; keys: float64 [n, 512].  V is keys[:, :448].
    Returns (out [H, 448], lse [H]); n == 0 gives (0, -inf) (reading R6).
    """
    H = q.shape[0]
    n = keys.shape[0]
    if n == 0:
        return np.zeros((H, V_DIM)), np.full(H, -np.inf)
    s = softmax_scale * (q @ keys.T)                      # [H, n]
    m = s.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))     # reading R5
    p = np.exp(s - lse[:, None])
    return p @ keys[:, :V_DIM], lse


def sparse_mla_decode(q_bits, kv_pages, page_table, topk_idx, seq_lens, softmax_scale):
    """Reference sparse MLA decode.

    q_bits: uint16 [B, 64, 512] bf16 patterns.  Returns (out float64
    [B, 64, 448], lse float64 [B, 64]).
    """
    q = bf16_value(q_bits)
    rows, valid = gather_dequant(kv_pages, page_table, topk_idx, seq_lens)
    B, H = q.shape[0], q.shape[1]
    out = np.zeros((B, H, V_DIM))
    lse = np.zeros((B, H))
    for b in range(B):
        out[b], lse[b] = attend(q[b], rows[b][valid[b]], softmax_scale)
    return out, lse


def lse_combine(outs, lses):
    """Merge attention results over disjoint entry subsets.

    outs: [S, ..., 448] per-subset normalised outputs, lses: [S, ...].  The
    merged lse is log(sum_s exp(lse_s)); the merged output weights subset s by
    exp(lse_s - lse).  All subsets empty gives (0, -inf).  This is the split
    top-k combine of "The Turning Point" (Step 5 of "The Reasoning Process").
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    m = lses.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - m_safe), 0.0)
    total = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, total, 1.0)), -np.inf)
    wn = np.where(finite, w / np.where(finite, total, 1.0), 0.0)
    out = (wn[..., None] * np.where(np.isfinite(lses)[..., None], outs, 0.0)).sum(axis=0)
    return out, lse


# ----------------------------------------------------------------------------
# cache append: quantise token latents into records (reading R13)
# ----------------------------------------------------------------------------

def scale_exponent(amax):
    """Least integer k with amax <= 448 * 2^k, clamped to [-127, 127]; amax = 0
    gives -127.  A floating log only proposes a start; the answer is settled
    by exact comparisons with the powers of two."""
    amax = float(amax)
    if amax == 0.0:
        return -127
    k = int(np.floor(np.log2(amax / 448.0))) - 2
    while 448.0 * 2.0 ** k < amax:
        k += 1
    return max(-127, min(127, k))


_FINITE_CODES = np.array([c for c in range(128) if not np.isnan(_E4M3_TABLE[c])], dtype=np.int64)


def e4m3_encode_nearest(y):
    """e4m3 code of the value nearest to y (|y| <= 448), ties to the even code,
    sign bit copied from y (so -0.0 gives 0x80).  Plain search over the table
    of all finite non-negative codes."""
    y = float(y)
    a = abs(y)
    vals = _E4M3_TABLE[_FINITE_CODES]
    d = np.abs(vals - a)
    best = d.min()
    cands = _FINITE_CODES[d == best]
    code = int(cands[0]) if len(cands) == 1 else int(cands[cands % 2 == 0][0])
    return code | (0x80 if np.signbit(y) else 0)


def quantize_token(latent_bits):
    """One token latent (bf16 bits [512]: 448 nope, 64 rope) -> (the 576-byte
    token record, the 8-byte scale record) (reading R13)."""
    bits = np.asarray(latent_bits, dtype=np.uint16)
    x = bf16_value(bits[:NOPE])
    rec = np.zeros(RECORD_BYTES, dtype=np.uint8)
    sc = np.zeros(SCALE_RECORD_BYTES, dtype=np.uint8)
    for g in range(NOPE // SCALE_GROUP):
        xs = x[g * SCALE_GROUP:(g + 1) * SCALE_GROUP]
        k = scale_exponent(np.abs(xs).max())
        sc[g] = k + 127
        for d in range(SCALE_GROUP):
            rec[g * SCALE_GROUP + d] = e4m3_encode_nearest(xs[d] * 2.0 ** -k)
    rec[NOPE:] = bits[NOPE:].astype("<u2").view(np.uint8)
    return rec, sc


def kv_append(kv_pages, page_table, seq_ids, positions, latent_bits):
    """A copy of the pool with every valid token written (reading R13)."""
    kv = np.array(kv_pages, dtype=np.uint8, copy=True)
    pt = np.asarray(page_table, dtype=np.int64)
    B, max_pages = pt.shape
    num_pages = kv.shape[0]
    for i in range(len(positions)):
        s, p = int(seq_ids[i]), int(positions[i])
        if not (0 <= s < B and p >= 0 and p // TOKENS_PER_PAGE < max_pages):
            continue
        page = int(pt[s, p // TOKENS_PER_PAGE])
        if not 0 <= page < num_pages:
            continue
        slot = p % TOKENS_PER_PAGE
        rec, sc = quantize_token(latent_bits[i])
        kv[page, slot * RECORD_BYTES:(slot + 1) * RECORD_BYTES] = rec
        kv[page, SCALE_REGION + slot * SCALE_RECORD_BYTES:SCALE_REGION + (slot + 1) * SCALE_RECORD_BYTES] = sc
    return kv


# ----------------------------------------------------------------------------
# top-k selection (reading R14)
# ----------------------------------------------------------------------------

def topk_select(scores, seq_lens, k):
    """scores fp32 [B, max_len], seq_lens [B], k -> topk_idx int32 [B, k]:
    each row's candidate positions sorted by (score descending, position
    ascending), the first min(k, L) kept, -1 after them (reading R14)."""
    sc = np.asarray(scores, dtype=np.float32)
    B, max_len = sc.shape
    out = np.full((B, k), -1, dtype=np.int32)
    for b in range(B):
        L = min(max(int(seq_lens[b]), 0), max_len)
        v = sc[b, :L].astype(np.float64)
        v = np.where(np.isnan(v), -np.inf, v)
        pos = np.arange(L)
        order = np.lexsort((pos, -v))   # primary key -v (higher score first), then position
        n = min(k, L)
        out[b, :n] = pos[order[:n]]
    return out
