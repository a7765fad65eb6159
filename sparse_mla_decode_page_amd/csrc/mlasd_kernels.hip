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
// Workgroup = (query b, slice s of its top-k list), 256 threads = 4 waves.
// Wave w owns heads [16w, 16w+16).  Per tile of 32 tokens:
//   a1  entries of the slice are validated, resolved through the page table
//       and compacted (valid ones only) into an LDS list once per workgroup;
//   a2  each wave gathers 8 token records (576 B + 8 B scale record) straight
//       into registers, one tile ahead of the compute;
//   a3  dequantised with the gfx950 scaled fp8 conversions into an LDS K tile
//       (bf16, token-major) and a V^T tile (fp16, dim-major, swizzled);
//   a4  S^T = K Q^T on v_mfma_f32_16x16x32_bf16, Q held in registers;
//   a5  online softmax in fp32 (exp2 domain), one head per lane column;
//   a6  O^T += V^T P^T on v_mfma_f32_16x16x32_f16, O^T in registers;
//   a7  epilogue: bf16 out + fp32 lse, or fp32 partials for the combine;
//   a8  the combine kernel merges slices with the LSE rule.
#include "mlasd_internal.h"

namespace mlasd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kKRow = kDQK + 8;               // K tile row stride (bf16), +16 B pad
constexpr int kVRow = kTileTokens;            // V^T tile row stride (fp16), swizzled chunks
constexpr int kWaves = kThreads / 64;

struct __align__(16) Smem {
  uint16_t k[kTileTokens * kKRow];            // 33,280 B
  uint16_t v[kDV * kVRow];                    // 28,672 B
  int32_t tok_page[kMaxTopk];                 // compacted list: physical page
  int32_t tok_slot[kMaxTopk];                 //                 slot in page
  int32_t tok_entry[kMaxTopk];                //                 entry index in slice
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

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
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
// n_ent <= 512 entries starting at `idx_row` into the LDS token list.
// Returns the number of valid entries.  Ends with a barrier.
__device__ int compact_slice(Smem& sm, const int32_t* idx_row, int n_ent, int seq_len,
                             const int32_t* pt_row, int32_t max_pages, int64_t num_pages) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int p0 = -1, p1 = -1;
  if (tid < n_ent) p0 = idx_row[tid];
  if (tid + kThreads < n_ent) p1 = idx_row[tid + kThreads];
  int pg0 = 0, sl0 = 0, pg1 = 0, sl1 = 0;
  const bool v0 = resolve_entry(p0, seq_len, pt_row, max_pages, num_pages, pg0, sl0);
  const bool v1 = resolve_entry(p1, seq_len, pt_row, max_pages, num_pages, pg1, sl1);
  int base = 0;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const bool v = c ? v1 : v0;
    const uint64_t mask = __ballot(v);
    const int in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
    if (lane == 0) sm.wave_cnt[wave] = __popcll(mask);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int cnt = sm.wave_cnt[w];
      before += (w < wave) ? cnt : 0;
      total += cnt;
    }
    if (v) {
      const int pos = base + before + in_wave;
      sm.tok_page[pos] = c ? pg1 : pg0;
      sm.tok_slot[pos] = c ? sl1 : sl0;
      sm.tok_entry[pos] = tid + c * kThreads;
    }
    base += total;
    __syncthreads();
  }
  return base;
}

// Tile token t of wave w: each wave gathers the 8 tokens whose PV k-slots are
// 8w..8w+7 (slot 8w+j), i.e. tokens {4w..4w+3, 16+4w..16+4w+3}.
__device__ __forceinline__ int wave_token(int wave, int j) {
  return j < 4 ? 4 * wave + j : 16 + 4 * wave + (j - 4);
}

struct TileRegs {
  u32x2 nope[8];   // lanes 0..55: nope bytes [8*lane, 8*lane+8) of token j
  u32x4 rope;      // all lanes: rope bytes [16*(lane&7), +16) of token lane>>3
  u32x2 sc;        // lane 56+j: the 8-byte scale record of token j
};

// a2: gather one tile's records into registers (no LDS traffic).
__device__ __forceinline__ void load_tile(TileRegs& r, const Smem& sm, const uint8_t* kv,
                                          int tile, int n_valid, int wave, int lane) {
  r.sc = u32x2{0, 0};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int ci = tile * kTileTokens + wave_token(wave, j);
    r.nope[j] = u32x2{0, 0};
    if (ci < n_valid) {
      const int64_t page = sm.tok_page[ci];
      const int slot = sm.tok_slot[ci];
      const uint8_t* pg = kv + page * kPageBytes;
      if (lane < 56) r.nope[j] = *(const u32x2*)(pg + slot * kRecordBytes + 8 * lane);
      if (lane == 56 + j) r.sc = *(const u32x2*)(pg + kScaleBase + slot * kScaleRecordBytes);
    }
  }
  const int jr = lane >> 3;
  const int ci = tile * kTileTokens + wave_token(wave, jr);
  r.rope = u32x4{0, 0, 0, 0};
  if (ci < n_valid) {
    const int64_t page = sm.tok_page[ci];
    const int slot = sm.tok_slot[ci];
    r.rope = *(const u32x4*)(kv + page * kPageBytes + slot * kRecordBytes + kDNope + 16 * (lane & 7));
  }
}

template <typename V2>
__device__ __forceinline__ uint32_t pack2(V2 v) {
  static_assert(sizeof(V2) == 4, "two 16-bit lanes");
  return __builtin_bit_cast(uint32_t, v);
}

// a3: dequantise the gathered tile into LDS.
//   K tile: bf16 [32 tokens][512 (+8 pad)], natural token order.
//   V^T tile: fp16 [448 dims][32 k-slots]; token t sits at k-slot
//   8*((t%16)/4) + 4*(t/16) + t%4; 16-byte chunk c of row d is stored at
//   chunk c ^ ((d >> 2) & 3) so the PV operand reads are bank-conflict free.
// Masked tile positions carry zero records (zero K, zero V).
__device__ __forceinline__ void store_tile(Smem& sm, const TileRegs& r, int wave, int lane) {
  const int g = lane >> 3;  // scale group of nope dims [8*lane, 8*lane+8)
  float scl[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t lo = __builtin_amdgcn_readlane(r.sc.x, 56 + j);
    const uint32_t hi = __builtin_amdgcn_readlane(r.sc.y, 56 + j);
    const uint32_t sb = ((g < 4) ? (lo >> (8 * g)) : (hi >> (8 * (g - 4)))) & 0xffu;
    scl[j] = __uint_as_float(sb << 23);   // 2^(sb-127) as an fp32 power of two
    const uint32_t b0 = r.nope[j].x, b1 = r.nope[j].y;
    u32x4 kq;
    kq.x = pack2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b0, scl[j], false));
    kq.y = pack2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b0, scl[j], true));
    kq.z = pack2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b1, scl[j], false));
    kq.w = pack2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b1, scl[j], true));
    if (lane < 56) *(u32x4*)&sm.k[wave_token(wave, j) * kKRow + 8 * lane] = kq;
  }
  // V^T: for each dim pair, the 8 tokens' fp16 values form one 16-byte k-slot
  // chunk per dim (token j -> element j of chunk `wave`).
  if (lane < 56) {
#pragma unroll
    for (int ip = 0; ip < 4; ++ip) {
      uint32_t hv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t src = (ip < 2) ? r.nope[j].x : r.nope[j].y;
        hv[j] = (ip & 1) ? pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src, scl[j], true))
                         : pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src, scl[j], false));
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        u32x4 w;
#pragma unroll
        for (int jp = 0; jp < 4; ++jp) {
          const uint32_t a = hv[2 * jp], b = hv[2 * jp + 1];
          w[jp] = hf ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        const int d = 8 * lane + 2 * ip + hf;
        *(u32x4*)&sm.v[d * kVRow + ((wave ^ ((d >> 2) & 3)) * 8)] = w;
      }
    }
  }
  *(u32x4*)&sm.k[wave_token(wave, lane >> 3) * kKRow + kDNope + 8 * (lane & 7)] = r.rope;
}

// ---------------------------------------------------------------------------
// a1-a7: main decode kernel
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads, 2) void mla_decode_kernel(const DecodeParams p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4;         // MFMA lane group
  const int col = lane & 15;       // MFMA column: head within the wave
  const int blk = logical_block(p.batch * p.nsplit);
  const int b = blk / p.nsplit, s = blk - b * p.nsplit;
  const int e0 = s * p.split_len;
  const int n_ent = max(0, min(p.topk - e0, p.split_len));
  const int head = 16 * wave + col;

  // Q^T operand, kept in registers for the whole slice: dims [32k + 8g, +8).
  bf16x8 qreg[16];
  {
    const uint16_t* qrow = p.q + ((int64_t)b * kHeads + head) * kDQK + 8 * g;
#pragma unroll
    for (int k = 0; k < 16; ++k) qreg[k] = *(const bf16x8*)(qrow + 32 * k);
  }

  const int n_valid = compact_slice(sm, p.topk_idx + (int64_t)b * p.topk + e0, n_ent,
                                    p.seq_lens[b], p.page_table + (int64_t)b * p.max_pages,
                                    p.max_pages, p.num_pages);
  const int ntiles = (n_valid + kTileTokens - 1) / kTileTokens;

  f32x4 oacc[28];
#pragma unroll
  for (int i = 0; i < 28; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  TileRegs regs;
  if (ntiles > 0) load_tile(regs, sm, p.kv, 0, n_valid, wave, lane);

  for (int t = 0; t < ntiles; ++t) {
    store_tile(sm, regs, wave, lane);
    __syncthreads();
    if (t + 1 < ntiles) load_tile(regs, sm, p.kv, t + 1, n_valid, wave, lane);

    // a4: S^T[token][head] for the 32 tile tokens (two 16-token blocks).
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 a = *(const bf16x8*)&sm.k[(16 * mb + col) * kKRow + 32 * k + 8 * g];
        sacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[k], sacc[mb], 0, 0, 0);
      }
    }

    // a5: online softmax.  Lane holds tokens 16*mb + 4*g + r of head `head`.
    const int tile_valid = n_valid - t * kTileTokens;
    float x[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = (16 * mb + 4 * g + r) < tile_valid;
        x[mb][r] = ok ? sacc[mb][r] * p.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, x[mb][r]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);        // finite: the tile has a valid token
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float rsum = 0.f;
    f16x8 pb;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(x[mb][r] - m_new);
        rsum += e;
        pb[4 * mb + r] = (_Float16)e;
      }
    rsum += __shfl_xor(rsum, 16);
    rsum += __shfl_xor(rsum, 32);
    l_run = l_run * alpha + rsum;
    m_run = m_new;

    // a6: O^T[dim][head] = alpha * O^T + V^T P^T over the tile's 32 k-slots.
#pragma unroll
    for (int mb = 0; mb < 28; ++mb) {
      const int d = 16 * mb + col;
      const f16x8 a = *(const f16x8*)&sm.v[d * kVRow + ((g ^ ((d >> 2) & 3)) * 8)];
      oacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb, oacc[mb] * alpha, 0, 0, 0);
    }
    __syncthreads();
  }

  // a7: epilogue.  Lane holds O^T[16*mb + 4*g + r][head].
  const bool empty = !(l_run > 0.f);
  const float inv = empty ? 0.f : 1.f / l_run;
  const float lse_v = empty ? -INFINITY : (m_run + __builtin_amdgcn_logf(l_run)) * 0.69314718055994531f;
  if (p.nsplit == 1) {
    uint16_t* orow = p.out + ((int64_t)b * kHeads + head) * kDV + 4 * g;
#pragma unroll
    for (int mb = 0; mb < 28; ++mb) {
      u32x2 w;
      w.x = (uint32_t)f32_to_bf16_rne(oacc[mb][0] * inv) | ((uint32_t)f32_to_bf16_rne(oacc[mb][1] * inv) << 16);
      w.y = (uint32_t)f32_to_bf16_rne(oacc[mb][2] * inv) | ((uint32_t)f32_to_bf16_rne(oacc[mb][3] * inv) << 16);
      *(u32x2*)(orow + 16 * mb) = w;
    }
    if (g == 0) p.lse[(int64_t)b * kHeads + head] = lse_v;
  } else {
    const int64_t pidx = ((int64_t)b * p.nsplit + s) * kHeads + head;
    float* prow = p.part_o + pidx * kDV + 4 * g;
#pragma unroll
    for (int mb = 0; mb < 28; ++mb) *(f32x4*)(prow + 16 * mb) = oacc[mb] * inv;
    if (g == 0) p.part_lse[pidx] = lse_v;
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
    w2.x = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    w2.y = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    *(u32x2*)(p.out + ((int64_t)b * kHeads + h) * kDV + 4 * c4) = w2;
  }
  if (tid < kCombineHeads) p.lse[(int64_t)b * kHeads + h0 + tid] = lse_out[tid];
}

// ---------------------------------------------------------------------------
// Test hook: a1-a3 exactly as the decode kernel runs them, then the LDS tiles
// are written out per entry.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void mla_gather_kernel(const GatherParams p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
    load_tile(regs, sm, p.kv, t, n_valid, wave, lane);
    store_tile(sm, regs, wave, lane);
    __syncthreads();
    // one wave per tile token at a time: token tt, 64 lanes x 8 elements
    for (int tt = wave; tt < kTileTokens; tt += kWaves) {
      const int ci = t * kTileTokens + tt;
      if (ci >= n_valid) continue;
      const int64_t e = (int64_t)b * p.topk + e0 + sm.tok_entry[ci];
      *(u32x4*)(p.k_rows + e * kDQK + 8 * lane) = *(const u32x4*)&sm.k[tt * kKRow + 8 * lane];
      const int slot = 8 * ((tt & 15) >> 2) + 4 * (tt >> 4) + (tt & 3);
      for (int d = lane; d < kDV; d += 64) {
        const int c = slot >> 3;
        p.v_rows[e * kDV + d] = sm.v[d * kVRow + ((c ^ ((d >> 2) & 3)) * 8) + (slot & 7)];
      }
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
