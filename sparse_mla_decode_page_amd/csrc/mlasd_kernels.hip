// gfx950 (CDNA4) kernels for sparse MLA decode over a paged FP8 KV cache.
//
// Method ("The Turning Point", "The Reasoning Process", Steps 3-5): one
// program handles all heads of a query, so every selected KV row is fetched
// once and Q K^T becomes a matrix product; the top-k list may be split over
// several programs whose partial results are merged with the online-softmax
// (log-sum-exp) rule.  Data flow per tile: gather -> dequantise -> concat
// with rope -> Q K^T -> online softmax -> P V ("The Turning Point", "Output
// Knowledge Created", item 2).  The 448 nope dims are not padded here: 448 is
// a whole number of 32-wide MFMA K-steps, so the pages' pad-to-512 mask has
// nothing to do on this hardware.
//
// Workgroup = (query b, slice s of its top-k list), 512 threads = 8 waves.
// Wave w: head group hg = w & 3 owns heads [16hg, 16hg+16); half dh = w >> 2
// picks which 16 tokens of each 32-token tile it scores and which 224 of the
// 448 output dims it accumulates.  The two waves of a head group swap their
// softmax partials through LDS, so each holds P for all 32 tokens.
//   a1  the slice's entries are validated, resolved through the page table
//       and compacted (valid ones only) into an LDS list once;
//   a2  each wave gathers 4 token records (576 B + 8 B scale record) straight
//       into registers, three tiles ahead of the compute, with loads whose
//       issue never depends on data (masked slots read page 0, slot 0);
//   a3  dequantised with the gfx950 scaled fp8 conversions into an LDS K tile
//       (bf16, token-major) and V tile (fp16, token-major, rows in PV k-slot
//       order), both double-buffered;
//   a4  S^T = K Q^T on v_mfma_f32_16x16x32_bf16, Q held in registers;
//   a5  online softmax in fp32 (exp2 domain), one head per lane column;
//   a6  O^T += V^T P^T on v_mfma_f32_16x16x32_f16, the V^T operand read with
//       ds_read_b64_tr_b16 transposing loads, O^T in registers;
//   a7  epilogue: bf16 out + fp32 lse, or fp32 partials for the combine;
//   a8  the combine kernel merges slices with the LSE rule.
#include "mlasd_internal.h"

namespace mlasd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kThreads / 64;
constexpr int kKRow = kDQK + 8;     // K tile row stride (bf16 elements), +16 B pad
constexpr int kVRow = kDV + 8;      // V tile row stride (fp16 elements), +16 B pad
constexpr int kDepth = 3;           // tiles gathered ahead of the compute
constexpr int kHalfDims = kDV / 2;  // output dims per wave: 224 = 14 MFMA rows of 16

struct __align__(16) Smem {
  uint16_t k[2][kTileTokens * kKRow];   // 2 x 33,280 B
  uint16_t v[2][kTileTokens * kVRow];   // 2 x 29,184 B
  f32x4 xp[2][kWaves][64];              // softmax partial exchange (p, 4 tokens/lane)
  float xm[2][kWaves][16];              //                          (tile max per head)
  u32x4 sink[2][8];                     // write target of the scale-record lanes 56..63
  int32_t tok[kMaxTopk][2];             // compacted list: physical page, slot
  uint16_t tok_entry[kMaxTopk];         //                 entry index in the slice
  int32_t wave_cnt[kWaves];
};

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ int logical_block(int n) {
  // Workgroups are dispatched round-robin over the 8 XCDs (block i -> XCD
  // i % 8).  Renumber so that consecutive logical blocks -- the slices of one
  // query, which read the same Q -- run on the same XCD and share its L2.
  const int i = blockIdx.x;
  const int xcd = i & 7, k = i >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd < rem ? xcd * (per + 1) + k : rem * (per + 1) + (xcd - rem) * per + k;
}

template <typename V2>
__device__ __forceinline__ uint32_t pack2(V2 v) {
  static_assert(sizeof(V2) == 4, "two 16-bit lanes");
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const bf16x2 r = {(__bf16)a, (__bf16)b};   // v_cvt_pk_bf16_f32, round to nearest even
  return pack2(r);
}

// a1: one index entry -> (page, slot) if valid.  Validity: 0 <= p < seq_len,
// logical page inside the page-table row, physical page inside the pool.
__device__ __forceinline__ bool resolve_entry(int p, int seq_len, const int32_t* pt_row,
                                              int32_t max_pages, int64_t num_pages,
                                              int& page, int& slot) {
  if (p < 0 || p >= seq_len) return false;
  const int lp = p >> 8;
  if (lp >= max_pages) return false;
  const int pg = pt_row[lp];
  if (pg < 0 || (int64_t)pg >= num_pages) return false;
  page = pg;
  slot = p & (kPageTokens - 1);
  return true;
}

// a1 for a whole slice: validate, resolve and compact (stable order) the
// n_ent <= 512 entries at `idx_row` into the LDS token list, one entry per
// thread.  Returns the number of valid entries.  Ends with a barrier.
__device__ int compact_slice(Smem& sm, const int32_t* idx_row, int n_ent, int seq_len,
                             const int32_t* pt_row, int32_t max_pages, int64_t num_pages) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int p = tid < n_ent ? idx_row[tid] : -1;
  int page = 0, slot = 0;
  const bool v = resolve_entry(p, seq_len, pt_row, max_pages, num_pages, page, slot);
  const uint64_t mask = __ballot(v);
  const int in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
  if (lane == 0) sm.wave_cnt[wid] = __popcll(mask);
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int cnt = sm.wave_cnt[w];
    before += (w < wid) ? cnt : 0;
    total += cnt;
  }
  if (v) {
    const int pos = before + in_wave;
    sm.tok[pos][0] = page;
    sm.tok[pos][1] = slot;
    sm.tok_entry[pos] = (uint16_t)tid;
  }
  __syncthreads();
  return total;
}

// PV k-slot of tile token t.  Wave (hg, dh) scores tokens 16dh + 4g + r
// (g = lane group, r = accumulator row), which feed k-slots 8g + 4dh + r of
// the P^T operand; the V tile stores token t in row slot_of(t).
__device__ __forceinline__ int slot_of(int t) { return 8 * ((t >> 2) & 3) + 4 * (t >> 4) + (t & 3); }

// a2 registers of one tile for one wave: tokens 4w + j, j = 0..3.
//   rec[j]: lanes 0..55 hold nope bytes [8 lane, 8 lane + 8) of token j,
//           lanes 56..63 hold token j's 8-byte scale record;
//   rope  : rope bytes [8 (lane & 15), +8) of token lane >> 4.
struct TileRegs {
  u32x2 rec[4];
  u32x2 rope;
};

__device__ __forceinline__ void load_tile(TileRegs& r, const Smem& sm, const uint8_t* kv, int tile,
                                          int n_valid, int wid, int lane) {
  const int c0 = tile * kTileTokens + 4 * wid;
  const int cc = min(c0, kMaxTopk - 4);
  const i32x4 t01 = *(const i32x4*)&sm.tok[cc][0];      // tokens 0,1: page, slot, page, slot
  const i32x4 t23 = *(const i32x4*)&sm.tok[cc + 2][0];  // tokens 2,3
  const int pg[4] = {t01.x, t01.z, t23.x, t23.z};
  const int sl[4] = {t01.y, t01.w, t23.y, t23.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool ok = c0 + j < n_valid;
    const int64_t page = ok ? pg[j] : 0;
    const int slot = ok ? sl[j] : 0;
    const uint8_t* base = kv + page * kPageBytes;
    const uint8_t* a = lane < 56 ? base + slot * kRecordBytes + 8 * lane
                                 : base + kScaleBase + slot * kScaleRecordBytes;
    r.rec[j] = *(const u32x2*)a;
  }
  {
    const int j = lane >> 4;
    const bool ok = c0 + j < n_valid;
    const int64_t page = ok ? pg[j] : 0;
    const int slot = ok ? sl[j] : 0;
    r.rope = *(const u32x2*)(kv + page * kPageBytes + slot * kRecordBytes + kDNope + 8 * (lane & 15));
  }
}

// a3: dequantise one wave's 4 gathered tokens into LDS buffer `buf`.
// Masked tile positions are written as zeros (zero K rows, zero V rows).
__device__ __forceinline__ void store_tile(Smem& sm, const TileRegs& r, int buf, int tile, int n_valid,
                                           int wid, int lane) {
  const int c0 = tile * kTileTokens + 4 * wid;
  const int g = lane >> 3;  // scale group of nope dims [8 lane, 8 lane + 8)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool ok = c0 + j < n_valid;
    const uint32_t lo = __builtin_amdgcn_readlane(r.rec[j].x, 56);
    const uint32_t hi = __builtin_amdgcn_readlane(r.rec[j].y, 56);
    const uint32_t sb = ((g < 4) ? (lo >> (8 * g)) : (hi >> (8 * (g - 4)))) & 0xffu;
    const float scale = __uint_as_float(sb << 23);   // 2^(sb-127) as an fp32 power of two
    const uint32_t b0 = ok ? r.rec[j].x : 0u, b1 = ok ? r.rec[j].y : 0u;
    u32x4 kq, vq;
    kq.x = pack2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b0, scale, false));
    kq.y = pack2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b0, scale, true));
    kq.z = pack2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b1, scale, false));
    kq.w = pack2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b1, scale, true));
    vq.x = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b0, scale, false));
    vq.y = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b0, scale, true));
    vq.z = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b1, scale, false));
    vq.w = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b1, scale, true));
    const int t = 4 * wid + j;
    // lanes 56..63 carry the scale record, not nope bytes: their stores go to
    // a sink instead of a branch (keeps the load-wait counting exact).
    u32x4* kd = lane < 56 ? (u32x4*)&sm.k[buf][t * kKRow + 8 * lane] : &sm.sink[0][lane & 7];
    u32x4* vd = lane < 56 ? (u32x4*)&sm.v[buf][slot_of(t) * kVRow + 8 * lane] : &sm.sink[1][lane & 7];
    *kd = kq;
    *vd = vq;
  }
  const int jr = lane >> 4;
  const bool ok = c0 + jr < n_valid;
  *(u32x2*)&sm.k[buf][(4 * wid + jr) * kKRow + kDNope + 4 * (lane & 15)] =
      ok ? r.rope : u32x2{0u, 0u};
}

// ---------------------------------------------------------------------------
// a1-a7: main decode kernel
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(const DecodeParams p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int hg = wid & 3, dh = wid >> 2, partner = wid ^ 4;
  const int g = lane >> 4;         // MFMA lane group
  const int col = lane & 15;       // MFMA column: head within the head group
  const int blk = logical_block(p.batch * p.nsplit);
  const int b = blk / p.nsplit, s = blk - b * p.nsplit;
  const int e0 = s * p.split_len;
  const int n_ent = max(0, min(p.topk - e0, p.split_len));
  const int head = 16 * hg + col;

  const int n_valid = compact_slice(sm, p.topk_idx + (int64_t)b * p.topk + e0, n_ent,
                                    p.seq_lens[b], p.page_table + (int64_t)b * p.max_pages,
                                    p.max_pages, p.num_pages);
  const int ntiles = (n_valid + kTileTokens - 1) / kTileTokens;

  // Q^T operand for the wave's 16 heads, kept in registers: dims [32k + 8g, +8).
  bf16x8 qreg[16];
  {
    const uint16_t* qrow = p.q + ((int64_t)b * kHeads + head) * kDQK + 8 * g;
#pragma unroll
    for (int k = 0; k < 16; ++k) qreg[k] = *(const bf16x8*)(qrow + 32 * k);
  }

  TileRegs regs[kDepth];
#pragma unroll
  for (int u = 0; u < kDepth; ++u) load_tile(regs[u], sm, p.kv, u, n_valid, wid, lane);

  f32x4 oacc[14];
#pragma unroll
  for (int i = 0; i < 14; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int t0 = 0; t0 < ntiles; t0 += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int t = t0 + u;
      const int buf = t & 1;
      if (t < ntiles) store_tile(sm, regs[u], buf, t, n_valid, wid, lane);
      // the gather for tile t + kDepth is issued on every path, so the number
      // of loads in flight behind regs[u] is the same wherever it is consumed
      load_tile(regs[u], sm, p.kv, t + kDepth, n_valid, wid, lane);
      if (t < ntiles) {
        __syncthreads();

        // a4: S^T[token][head] for this wave's 16 tokens; two accumulation chains.
        const uint16_t* krow = &sm.k[buf][(16 * dh + col) * kKRow + 8 * g];
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 16; k += 2) {
          const bf16x8 a0 = *(const bf16x8*)(krow + 32 * k);
          const bf16x8 a1 = *(const bf16x8*)(krow + 32 * (k + 1));
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qreg[k], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qreg[k + 1], s1, 0, 0, 0);
        }
        const f32x4 sacc = s0 + s1;

        // a5: own tokens 16dh + 4g + r; tile max and exp against it.
        const int tile_valid = n_valid - t * kTileTokens;
        float x[4], m_own = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = (16 * dh + 4 * g + r) < tile_valid;
          x[r] = ok ? sacc[r] * p.scale_log2 : -INFINITY;
          m_own = fmaxf(m_own, x[r]);
        }
        m_own = fmaxf(m_own, __shfl_xor(m_own, 16));
        m_own = fmaxf(m_own, __shfl_xor(m_own, 32));
        f32x4 p_own;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          p_own[r] = (m_own == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x[r] - m_own);
        sm.xp[buf][wid][lane] = p_own;
        if (g == 0) sm.xm[buf][wid][col] = m_own;
        __syncthreads();
        const f32x4 p_part = sm.xp[buf][partner][lane];
        const float m_part = sm.xm[buf][partner][col];

        const float m_new = fmaxf(m_run, fmaxf(m_own, m_part));   // finite
        const float c_own = (m_own == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_own - m_new);
        const float c_part = (m_part == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_part - m_new);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        // P^T operand in k-slot order 8g + 4*half + r (half 0 = tokens 0..15).
        float pk[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float po = p_own[r] * c_own, pp = p_part[r] * c_part;
          pk[r] = dh == 0 ? po : pp;
          pk[4 + r] = dh == 0 ? pp : po;
        }
        float rsum = 0.f;
        f16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          rsum += pk[e];
          pb[e] = (_Float16)pk[e];
        }
        rsum += __shfl_xor(rsum, 16);
        rsum += __shfl_xor(rsum, 32);
        l_run = l_run * alpha + rsum;
        m_run = m_new;

        // a6: O^T[dim][head] = alpha O^T + V^T P^T over the tile's 32 k-slots;
        // the V^T operand comes from the token-major V tile through
        // transposing reads: lane (g, c) addresses row 8g + c/4 (+4), dims
        // d0 + 4(c%4), and receives V[8g..8g+3 (+4)][d0 + c].
        const uint16_t* vbase = &sm.v[buf][(8 * g + (col >> 2)) * kVRow + kHalfDims * dh + 4 * (col & 3)];
#pragma unroll
        for (int mb = 0; mb < 14; ++mb) {
          typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
          const f16x4 lo = __builtin_bit_cast(
              f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + 16 * mb)));
          const f16x4 hi = __builtin_bit_cast(
              f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + 4 * kVRow + 16 * mb)));
          const f16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb, oacc[mb] * alpha, 0, 0, 0);
        }
      }
    }
  }

  // a7: epilogue.  Lane holds O^T[224dh + 16mb + 4g + r][head].
  const bool empty = !(l_run > 0.f);
  const float inv = empty ? 0.f : 1.f / l_run;
  const float lse_v = empty ? -INFINITY : (m_run + __builtin_amdgcn_logf(l_run)) * 0.69314718055994531f;
  if (p.nsplit == 1) {
    uint16_t* orow = p.out + ((int64_t)b * kHeads + head) * kDV + kHalfDims * dh + 4 * g;
#pragma unroll
    for (int mb = 0; mb < 14; ++mb) {
      u32x2 w;
      w.x = bf16x2_rne(oacc[mb][0] * inv, oacc[mb][1] * inv);
      w.y = bf16x2_rne(oacc[mb][2] * inv, oacc[mb][3] * inv);
      *(u32x2*)(orow + 16 * mb) = w;
    }
    if (dh == 0 && g == 0) p.lse[(int64_t)b * kHeads + head] = lse_v;
  } else {
    const int64_t pidx = ((int64_t)b * p.nsplit + s) * kHeads + head;
    float* prow = p.part_o + pidx * kDV + kHalfDims * dh + 4 * g;
#pragma unroll
    for (int mb = 0; mb < 14; ++mb) *(f32x4*)(prow + 16 * mb) = oacc[mb] * inv;
    if (dh == 0 && g == 0) p.part_lse[pidx] = lse_v;
  }
}

// ---------------------------------------------------------------------------
// a8: LSE combine of the slices of each query.
// ---------------------------------------------------------------------------

constexpr int kCombineHeads = 4;   // heads per combine workgroup

__global__ __launch_bounds__(256) void mla_combine_kernel(const DecodeParams p) {
  __shared__ float wts[kCombineHeads][32];
  __shared__ float lse_out[kCombineHeads];
  const int b = blockIdx.x / (kHeads / kCombineHeads);
  const int h0 = (blockIdx.x % (kHeads / kCombineHeads)) * kCombineHeads;
  const int ns = p.nsplit;
  const int tid = threadIdx.x;
  if (tid < kCombineHeads) {
    const int h = h0 + tid;
    float m = -INFINITY;
    for (int s = 0; s < ns; ++s) m = fmaxf(m, p.part_lse[((int64_t)b * ns + s) * kHeads + h]);
    float tot = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float l = p.part_lse[((int64_t)b * ns + s) * kHeads + h];
      const float w = (m == -INFINITY || l == -INFINITY) ? 0.f : __expf(l - m);
      wts[tid][s] = w;
      tot += w;
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    for (int s = 0; s < ns; ++s) wts[tid][s] *= inv;
    lse_out[tid] = tot > 0.f ? m + __logf(tot) : -INFINITY;
  }
  __syncthreads();
  constexpr int kVec = kDV / 4;   // float4 per head row
  for (int e = tid; e < kCombineHeads * kVec; e += blockDim.x) {
    const int hh = e / kVec, c4 = e - hh * kVec;
    const int h = h0 + hh;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < ns; ++s) {
      const float w = wts[hh][s];
      if (w != 0.f) {
        const f32x4 o = *(const f32x4*)(p.part_o + (((int64_t)b * ns + s) * kHeads + h) * kDV + 4 * c4);
        acc += w * o;
      }
    }
    u32x2 w2;
    w2.x = bf16x2_rne(acc[0], acc[1]);
    w2.y = bf16x2_rne(acc[2], acc[3]);
    *(u32x2*)(p.out + ((int64_t)b * kHeads + h) * kDV + 4 * c4) = w2;
  }
  if (tid < kCombineHeads) p.lse[(int64_t)b * kHeads + h0 + tid] = lse_out[tid];
}

// ---------------------------------------------------------------------------
// Test hook: a1-a3 exactly as the decode kernel runs them, then the LDS tiles
// are written out per entry.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads, 1) void mla_gather_kernel(const GatherParams p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int blk = logical_block(p.batch * p.nsplit);
  const int b = blk / p.nsplit, s = blk - b * p.nsplit;
  const int e0 = s * p.split_len;
  const int n_ent = max(0, min(p.topk - e0, p.split_len));
  const int32_t* idx_row = p.topk_idx + (int64_t)b * p.topk + e0;
  const int32_t* pt_row = p.page_table + (int64_t)b * p.max_pages;
  const int seq_len = p.seq_lens[b];

  // masked entries: zero rows, valid = 0
  for (int j = tid; j < n_ent; j += kThreads) {
    int pg, sl;
    const bool v = resolve_entry(idx_row[j], seq_len, pt_row, p.max_pages, p.num_pages, pg, sl);
    const int64_t e = (int64_t)b * p.topk + e0 + j;
    p.valid[e] = v ? 1 : 0;
    if (!v) {
      for (int d = 0; d < kDQK; d += 8) *(u32x4*)(p.k_rows + e * kDQK + d) = u32x4{0, 0, 0, 0};
      for (int d = 0; d < kDV; d += 8) *(u32x4*)(p.v_rows + e * kDV + d) = u32x4{0, 0, 0, 0};
    }
  }

  const int n_valid = compact_slice(sm, idx_row, n_ent, seq_len, pt_row, p.max_pages, p.num_pages);
  const int ntiles = (n_valid + kTileTokens - 1) / kTileTokens;
  TileRegs regs;
  for (int t = 0; t < ntiles; ++t) {
    load_tile(regs, sm, p.kv, t, n_valid, wid, lane);
    store_tile(sm, regs, 0, t, n_valid, wid, lane);
    __syncthreads();
    for (int tt = wid; tt < kTileTokens; tt += kWaves) {
      const int ci = t * kTileTokens + tt;
      if (ci >= n_valid) continue;
      const int64_t e = (int64_t)b * p.topk + e0 + sm.tok_entry[ci];
      *(u32x4*)(p.k_rows + e * kDQK + 8 * lane) = *(const u32x4*)&sm.k[0][tt * kKRow + 8 * lane];
      if (lane < 56)
        *(u32x4*)(p.v_rows + e * kDV + 8 * lane) = *(const u32x4*)&sm.v[0][slot_of(tt) * kVRow + 8 * lane];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  const int nblk = p.batch * p.nsplit;
  hipLaunchKernelGGL(mla_decode_kernel, dim3(nblk), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeParams& p, hipStream_t stream) {
  const int nblk = p.batch * (kHeads / kCombineHeads);
  hipLaunchKernelGGL(mla_combine_kernel, dim3(nblk), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherParams& p, hipStream_t stream) {
  const int nblk = p.batch * p.nsplit;
  hipLaunchKernelGGL(mla_gather_kernel, dim3(nblk), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mlasd
