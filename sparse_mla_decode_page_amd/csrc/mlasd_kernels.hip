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
// Workgroup = (query b, slice s of its top-k list, head group), 512 threads =
// 8 waves in two roles, meeting at one barrier per 32-token tile (waves w and
// w + 4 share a SIMD):
//   consumers: wave c owns heads [16c, 16c+16) of the workgroup's head group
//       (64, 32 or 16 heads).  With 64 heads, waves 0..3, each beside a
//       producer.  With 32, waves 0..1 run a4 and a5 only, each beside its
//       PV helper (4, 5), which runs a6 and a7 one tile behind it.  With 16,
//       wave 0 runs a4 and a5, and two PV helpers (wave 1: dims 0-223, wave
//       4: dims 224-447) run a6 and a7; wave 5 is spare.  A consumer runs
//       a4  S^T = K Q^T, Q held in registers: the 448 nope dims on
//           v_mfma_f32_16x16x32_f16 (K and Q in fp16), the 64 rope dims on
//           v_mfma_f32_16x16x32_bf16;
//       a5  online softmax in fp32 (exp2 domain), one head per lane column;
//       a6  O^T += V^T P^T on v_mfma_f32_16x16x32_f16 over all 448 dims, the
//           V^T operand read with ds_read_b64_tr_b16 transposing loads;
//       a7  epilogue: bf16 out + fp32 lse, or fp32 partials for the combine;
//   producers (waves 4..7 with 64 heads, else 2, 3, 6, 7, two per SIMD):
//       producer p owns tokens [8p, 8p+8) of every tile and
//       a2  gathers their records (576 B + 8 B scale record) into registers
//           kDepth + 1 tiles ahead, with loads whose issue never depends on
//           data (masked slots re-read the slice's last valid record);
//       a3  dequantises tile t+1 into the other LDS buffer while the
//           consumers work on tile t.  One token-major tile serves both
//           contractions: a row holds the token's 448 nope values in fp16 (the
//           K operand of the nope dims and the V operand) and its 64 rope
//           values in bf16, so every nope byte is converted and stored once.
//   a1  before that, all waves validate, resolve through the page table and
//       compact the slice's entries into an LDS list;
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
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kThreads / 64;
constexpr int kConsumers = 4;       // waves 0..3
constexpr int kRow = kDQK + 16;     // tile row stride (16-bit elements): 448 fp16 nope,
                                    // 64 bf16 rope, +32 B pad (of the pads tried, 16-64 B,
                                    // the fastest with 64 heads)
constexpr int kNopeSteps = kDNope / 32;   // 14 fp16 QK^T k-steps; 2 bf16 rope k-steps follow
constexpr int kDepth = 2;           // tiles gathered ahead by the producers
constexpr int kTokPerProducer = kTileTokens / (kWaves - kConsumers);   // 8
constexpr float kRescaleLog2 = 8.f; // lazy-rescale threshold (P <= 256)
constexpr int kPvAhead = 3;         // PV operand blocks read ahead
constexpr int kQkAhead = 3;         // QK^T operand k-steps read ahead
constexpr int kStageRowBytes = 912; // epilogue staging row: 896 B (+16 B pad)
constexpr int kStageBytes = 16 * kStageRowBytes;   // one wave's 16 rows

struct __align__(16) Smem {
  uint16_t kv[3][kTileTokens * kRow];   // 3 x 33,792 B (the 16-head kernel keeps three live)
  u32x4 pex[2][2][64];                  // per consumer wave: P^T operand handed to its PV helpers
  float aex[2][2][64];                  //                    and the rescale factor applied before it
  float lx[2][64];                      //                    final l per lane column
  int32_t tok[kMaxTopk][2];             // compacted list: physical page, slot
  uint16_t tok_entry[kMaxTopk];         //                 entry index in the slice
  int32_t wave_cnt[kWaves];
};
static_assert(kConsumers * kStageBytes <= (int)sizeof(Smem::kv), "epilogue staging must fit the tiles");

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ int logical_block(int n) {
  // Workgroups are dispatched round-robin over the 8 XCDs (block i -> XCD
  // i % 8).  Renumber so that consecutive logical blocks -- the slices of one
  // query, which read the same Q, and the combine's workgroups of that query,
  // which read what the slices wrote -- run on the same XCD and share its L2.
  // Each XCD gets one contiguous range of logical blocks, in proportion.
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

// Reductions over the 4 lane groups of a column (lanes l, l^16, l^32, l^48)
// with VALU lane swaps: each swap leaves a lane its own value and its
// partner's, so no LDS round trip is needed.
__device__ __forceinline__ float group_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float group_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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

// a2 registers of one tile for one producer wave p: tokens 8p + j, j = 0..7.
//   rec[j]: lanes 0..55 hold nope bytes [8 lane, 8 lane + 8) of token j,
//           lanes 56..63 hold token j's 8-byte scale record;
//   rope  : rope bytes [16 (lane & 7), +16) of token lane >> 3.
// Tile positions past the last valid entry re-read the slice's last valid
// record (already cached); their scores are masked, so they add nothing.
struct TileRegs {
  u32x2 rec[kTokPerProducer];
  u32x4 rope;
};

struct LastRecord {   // wave-uniform: the slice's last valid (page, slot)
  int page, slot;
};

// Per-lane record offset within a page is slot * mul + add: lanes 0..55 read
// nope bytes [8 lane, +8) of the 576-byte record, lanes 56..63 the 8-byte
// scale record in the page's scale area.
struct LaneOffset {
  uint32_t mul, add;
};

__device__ __forceinline__ LaneOffset lane_offset(int lane) {
  return lane < 56 ? LaneOffset{(uint32_t)kRecordBytes, 8u * lane}
                   : LaneOffset{(uint32_t)kScaleRecordBytes, (uint32_t)kScaleBase};
}

__device__ __forceinline__ void load_tile(TileRegs& r, const Smem& sm, const uint8_t* kv, int64_t pstride,
                                          int tile, int n_valid, LastRecord last, int pw, int lane,
                                          LaneOffset lo) {
  const int c0 = tile * kTileTokens + kTokPerProducer * pw;
  // Lane l resolves token c0 + l/8 with one LDS read; token j's page and slot
  // are then broadcast from lane 8j, so the address math is scalar and no
  // load waits on another.
  const int ci = c0 + (lane >> 3);
  const i32x2 ps = *(const i32x2*)&sm.tok[min(ci, kMaxTopk - 1)][0];
  const bool ok = ci < n_valid;
  const int page = ok ? ps.x : last.page;
  const int slot = ok ? ps.y : last.slot;
#pragma unroll
  for (int j = 0; j < kTokPerProducer; ++j) {
    const int pg = __builtin_amdgcn_readlane(page, 8 * j);
    const int sl = __builtin_amdgcn_readlane(slot, 8 * j);
    const uint8_t* base = kv + (int64_t)pg * pstride;
    r.rec[j] = *(const u32x2*)(base + (__umul24((uint32_t)sl, lo.mul) + lo.add));
  }
  r.rope = *(const u32x4*)(kv + (int64_t)page * pstride + slot * kRecordBytes + kDNope + 16 * (lane & 7));
}

// a3: dequantise one producer wave's 8 gathered tokens into LDS buffer `buf`.
// Every lane stores 16 bytes per row at 16 * lane: lanes 0..55 hold nope dims
// [8 lane, 8 lane + 8) in fp16; lanes 56..63 (the scale-record lanes) land in
// the row's rope span, which the rope store rewrites just after (LDS stores of
// one wave complete in order).  A scaled e4m3 value is exact in fp16 while
// its magnitude stays below 2^16 and it is a multiple of 2^-24.
__device__ __forceinline__ void store_tile(Smem& sm, const TileRegs& r, int buf, int pw, int lane) {
  // The lane's scale is byte lane >> 3 of the token's 8-byte scale record,
  // which lanes 56..63 hold: one v_perm_b32 picks it out of the two record
  // words broadcast from lane 56.  All 8 scales are taken first, then the
  // conversions and stores.
  const uint32_t sel = 0x0C0C0C00u | (uint32_t)(lane >> 3);   // byte g, zero-extended
  uint16_t* rb = &sm.kv[buf][8 * lane];
  float scale[kTokPerProducer];
#pragma unroll
  for (int j = 0; j < kTokPerProducer; ++j) {
    const uint32_t lo = __builtin_amdgcn_readlane(r.rec[j].x, 56);
    const uint32_t hi = __builtin_amdgcn_readlane(r.rec[j].y, 56);
    scale[j] = __uint_as_float(__builtin_amdgcn_perm(hi, lo, sel) << 23);   // 2^(sb-127) as an fp32 power of two
  }
#pragma unroll
  for (int j = 0; j < kTokPerProducer; ++j) {
    const uint32_t b0 = r.rec[j].x, b1 = r.rec[j].y;
    u32x4 vq;
    vq.x = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b0, scale[j], false));
    vq.y = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b0, scale[j], true));
    vq.z = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b1, scale[j], false));
    vq.w = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b1, scale[j], true));
    *(u32x4*)(rb + (kTokPerProducer * pw + j) * kRow) = vq;
  }
  const int tr = kTokPerProducer * pw + (lane >> 3);
  *(u32x4*)&sm.kv[buf][tr * kRow + kDNope + 8 * (lane & 7)] = r.rope;
}

// a6 over kBlocks 16-dim blocks: O^T[dim][head] += V^T P^T over the tile's 32
// tokens.  The P^T operand of lane group g holds, in k-slots 8g + 4mb + r, the
// lane's scores of tokens 16mb + 4g + r; the V^T operand comes from the
// token-major tile through transposing reads: lane (g, c) addresses row
// 4g + c/4 (+16), dims d0 + 4(c%4), and receives V[4g..4g+3 (+16)][d0 + c]
// (vbase is the lane's address for the first block).  Operands are read
// kPvAhead blocks ahead.
template <int kBlocks>
__device__ __forceinline__ void pv_blocks(f32x4* oacc, const uint16_t* vbase, f16x8 pb) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 vlo[kPvAhead + 1], vhi[kPvAhead + 1];
#pragma unroll
  for (int mb = 0; mb < kPvAhead; ++mb) {
    vlo[mb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + 16 * mb));
    vhi[mb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + 16 * kRow + 16 * mb));
  }
#pragma unroll
  for (int mb = 0; mb < kBlocks; ++mb) {
    const int nx = mb + kPvAhead;
    if (nx < kBlocks) {
      vlo[nx % (kPvAhead + 1)] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + 16 * nx));
      vhi[nx % (kPvAhead + 1)] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + 16 * kRow + 16 * nx));
    }
    const f16x4 lo = __builtin_bit_cast(f16x4, vlo[mb % (kPvAhead + 1)]);
    const f16x4 hi = __builtin_bit_cast(f16x4, vhi[mb % (kPvAhead + 1)]);
    const f16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    oacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb, oacc[mb], 0, 0, 0);
  }
  // V reads kPvAhead blocks ahead of their MFMAs (measured faster for 32
  // heads, slightly faster for 64)
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPvAhead, 1);
#pragma unroll
  for (int mb = 0; mb < kBlocks; ++mb) {
    if (mb + kPvAhead < kBlocks) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
  }
}

// a7 stores of one wave's 16 heads over dims [dim0, dim0 + 16 kBlocks):
// bf16 out, or fp32 partials for the combine.  The wave's 16 output rows are
// contiguous in memory.  They are staged through LDS (`stage`, the wave's own
// area of the tile buffers, which every wave finished reading before the last
// barrier and the producers no longer write) so each store writes whole 1 KB
// runs of cache lines instead of 16 scattered 32-byte pieces: the store rate
// is bound by write requests in flight per CU, and this cuts them four-fold.
template <int kBlocks>
__device__ __forceinline__ void store_out(const DecodeParams& p, uint8_t* stage, const f32x4* oacc, float inv,
                                          int b, int s, int head0, int dim0, int lane) {
  const int g = lane >> 4, col = lane & 15;
  if (p.nsplit == 1) {
#pragma unroll
    for (int mb = 0; mb < kBlocks; ++mb) {
      u32x2 w;
      w.x = bf16x2_rne(oacc[mb][0] * inv, oacc[mb][1] * inv);
      w.y = bf16x2_rne(oacc[mb][2] * inv, oacc[mb][3] * inv);
      *(u32x2*)(stage + col * kStageRowBytes + 2 * (16 * mb + 4 * g)) = w;
    }
    uint8_t* obase = (uint8_t*)(p.out + (int64_t)b * p.out_sb + (int64_t)head0 * p.out_sh + dim0);
    constexpr int kChunks = 2 * kBlocks;   // 16-byte chunks per row
#pragma unroll
    for (int k = 0; k < kBlocks / 2; ++k) {   // 16 rows x 32 kBlocks bytes
      const int i = lane + 64 * k, row = i / kChunks, ch = i - kChunks * row;
      *(u32x4*)(obase + row * (2 * p.out_sh) + 16 * ch) = *(const u32x4*)(stage + row * kStageRowBytes + 16 * ch);
    }
  } else {
    const int64_t prow0 = ((int64_t)b * p.nsplit + s) * kHeads + head0;
#pragma unroll
    for (int h = 0; h < kBlocks / 14; ++h) {   // fp32 partials, 224 dims per pass
#pragma unroll
      for (int mb = 0; mb < 14; ++mb)
        *(f32x4*)(stage + col * kStageRowBytes + 4 * (16 * mb + 4 * g)) = oacc[14 * h + mb] * inv;
#pragma unroll
      for (int k = 0; k < 14; ++k) {   // 16 rows x 224 floats = 14 x 1 KB
        const int i = lane + 64 * k, row = i / 56, ch = i - 56 * row;
        *(f32x4*)(p.part_o + (prow0 + row) * kDV + dim0 + kDV / 2 * h + 4 * ch) =
            *(const f32x4*)(stage + row * kStageRowBytes + 16 * ch);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// a1-a7: main decode kernel
// ---------------------------------------------------------------------------

// kHeadGroups = 1: a workgroup computes all 64 heads of its (query, slice);
// 2: 32 heads, Q K^T and the softmax on consumer waves 0..1 and P V on their
// helpers 4..5; 4: 16 heads, Q K^T and the softmax on wave 0 and P V on two
// helper waves (1: dims 0-223, 4: dims 224-447), wave 5 spare -- for
// batches too small to fill the GPU with slices alone.  The head groups of a slice run on one XCD and
// share its gathered records through L2.
template <int kHeadGroups>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(const DecodeParams p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int blk = logical_block(p.batch * p.nsplit * kHeadGroups);
  const int hg = blk % kHeadGroups, bs = blk / kHeadGroups;
  const int b = bs / p.nsplit, s = bs - b * p.nsplit;
  const int e0 = s * p.split_len;
  const int n_ent = max(0, min(p.topk - e0, p.split_len));

  const int n_valid = compact_slice(sm, p.topk_idx + (int64_t)b * p.idx_sb + e0, n_ent,
                                    p.seq_lens[(int64_t)b * p.len_s], p.page_table + (int64_t)b * p.pt_sb,
                                    p.max_pages, p.num_pages);
  const int ntiles = (n_valid + kTileTokens - 1) / kTileTokens;

  // With 16 or 32 heads, PV helper waves run P V one tile behind the
  // consumer waves, which keep only Q K^T and the softmax, so three tile
  // buffers are live and every role passes one more barrier at the end.
  constexpr bool kHelper = kHeadGroups != 1;
  constexpr int kBufs = kHelper ? 3 : 2;
  constexpr int kExtra = kHelper ? 1 : 0;

  // Roles by wave.  Waves w and w + 4 share a SIMD.  With 64 heads, waves
  // 0..3 are consumers and 4..7 producers.  With fewer heads the producers
  // are 2, 3, 6, 7 and pair up on two SIMDs.  With 32 heads, consumer waves
  // 0 and 1 each share a SIMD with their PV helper (4 and 5).  With 16, the
  // main wave 0 shares its SIMD with PV helper 4 (dims 224-447), and PV
  // helper 1 (dims 0-223) its SIMD with spare wave 5.  Other layouts
  // measured slower.
  const bool producer = kHeadGroups == 1 ? wid >= kConsumers : (wid & 2) != 0;
  const int pw = kHeadGroups == 1 ? wid - kConsumers : (wid & 1) + ((wid >> 2) << 1);   // producer index 0..3

  // Both roles pass the same barriers: one after the first tile is stored,
  // then one per tile, then kExtra.
  if (producer) {
    // ---------------- producers: a2 + a3 ----------------
    if (ntiles == 0) {   // empty slice: nothing to gather
      __syncthreads();
    } else {
      const LastRecord last = {__builtin_amdgcn_readfirstlane(sm.tok[n_valid - 1][0]),
                               __builtin_amdgcn_readfirstlane(sm.tok[n_valid - 1][1])};
      const LaneOffset lo = lane_offset(lane);
      TileRegs regs[kDepth];
#pragma unroll
      for (int u = 0; u < kDepth; ++u) load_tile(regs[u], sm, p.kv, p.page_stride, u, n_valid, last, pw, lane, lo);
      store_tile(sm, regs[0], 0, pw, lane);
      load_tile(regs[0], sm, p.kv, p.page_stride, kDepth, n_valid, last, pw, lane, lo);
      __syncthreads();
      for (int t0 = 0; t0 < ntiles; t0 += kDepth) {
#pragma unroll
        for (int u = 0; u < kDepth; ++u) {
          const int t = t0 + u;
          const int nxt = (u + 1) % kDepth;   // ring slot of tile t + 1
          if (t + 1 < ntiles) store_tile(sm, regs[nxt], (t + 1) % kBufs, pw, lane);
          // issued on every path, so the loads in flight behind each ring slot
          // are the same wherever it is consumed (past the end they re-read a
          // cached record)
          load_tile(regs[nxt], sm, p.kv, p.page_stride, t + 1 + kDepth, n_valid, last, pw, lane, lo);
          if (t < ntiles) __syncthreads();
        }
      }
    }
    if (kExtra) __syncthreads();
    return;
  }

  // ---------------- consumers: a4 - a7 ----------------
  if (kHeadGroups == 4 && wid == 5) {   // spare consumer waves only pass the barriers
    for (int t = 0; t <= ntiles + kExtra; ++t) __syncthreads();
    return;
  }
  if constexpr (kHelper) {
    if (kHeadGroups == 4 ? (wid == 1 || wid == 4) : wid >= 4) {
      // 16 heads: helpers 1 and 4 split consumer 0's dims; 32 heads: helper
      // 4 + c runs all dims of consumer c.
      constexpr int kHB = kHeadGroups == 4 ? 14 : 28;   // 16-dim blocks per helper
      const int cw = kHeadGroups == 4 ? 0 : wid - 4;     // the consumer wave served
      const int hb = kHeadGroups == 4 && wid == 4 ? 14 : 0;   // first 16-dim block
      const int slot = kHeadGroups == 4 ? (wid == 1 ? 1 : 2) : 2 + cw;   // epilogue staging area
      // PV helper: O^T over its 224 dims of the main wave's 16 heads, for
      // the tile before the one the main wave works on, with the P^T operand
      // and rescale factor the main wave left in LDS.
      const int g = lane >> 4, col = lane & 15;
      f32x4 ohi[kHB];
#pragma unroll
      for (int i = 0; i < kHB; ++i) ohi[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      __syncthreads();
      for (int t = 0; t <= ntiles; ++t) {
        if (t >= 1) {
          const int pt = t - 1;
          const f16x8 pb = __builtin_bit_cast(f16x8, sm.pex[pt & 1][cw][lane]);
          const float a = sm.aex[pt & 1][cw][lane];
          if (__ballot(a != 1.f) != 0) {
#pragma unroll
            for (int i = 0; i < kHB; ++i) ohi[i] *= a;
          }
          pv_blocks<kHB>(ohi, &sm.kv[pt % kBufs][(4 * g + (col >> 2)) * kRow + 4 * (col & 3) + 16 * hb], pb);
        }
        __syncthreads();
      }
      const float l = sm.lx[cw][lane];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const int head0 = kHeads / kHeadGroups * hg + 16 * cw;
      store_out<kHB>(p, (uint8_t*)&sm.kv[0][0] + slot * kStageBytes, ohi, inv, b, s, head0, 16 * hb, lane);
      return;
    }
  }
  const int g = lane >> 4;         // MFMA lane group
  const int col = lane & 15;       // MFMA column: head within the wave's 16
  const int head0 = kHeads / kHeadGroups * hg + 16 * wid;   // the wave's first head
  const int head = head0 + col;

  // Q^T operand for the wave's 16 heads, kept in registers: dims [32k + 8g, +8);
  // the nope k-steps in fp16 (exact for bf16 values of magnitude in
  // [2^-14, 65504]; smaller ones keep every bit down to 2^-24), the rope
  // k-steps in bf16.
  f16x8 qnope[kNopeSteps];
  bf16x8 qrope[2];
  {
    const uint16_t* qrow = p.q + (int64_t)b * p.q_sb + (int64_t)head * p.q_sh + 8 * g;
    bf16x8 qb[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) qb[k] = *(const bf16x8*)(qrow + 32 * k);
#pragma unroll
    for (int k = 0; k < kNopeSteps; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) qnope[k][i] = (_Float16)(float)qb[k][i];
    qrope[0] = qb[kNopeSteps];
    qrope[1] = qb[kNopeSteps + 1];
  }
  constexpr int kOBlocks = kHelper ? 0 : 28;   // 16-dim blocks of O^T this wave keeps
  f32x4 oacc[kOBlocks > 0 ? kOBlocks : 1];
#pragma unroll
  for (int i = 0; i < kOBlocks; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t % kBufs;
    // a4: S^T[token][head] for the tile's 32 tokens: two 16-token blocks,
    // two accumulation chains each, operands read kQkAhead k-steps ahead.
    const uint16_t* krow = &sm.kv[buf][col * kRow + 8 * g];
    u32x4 ka[kQkAhead + 1][2];   // raw operand bits: fp16 nope or bf16 rope
#pragma unroll
    for (int k = 0; k < kQkAhead; ++k)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) ka[k][mb] = *(const u32x4*)(krow + 16 * mb * kRow + 32 * k);
    f32x4 sc[2][2] = {};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k + kQkAhead < 16) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          ka[(k + kQkAhead) % (kQkAhead + 1)][mb] = *(const u32x4*)(krow + 16 * mb * kRow + 32 * (k + kQkAhead));
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const u32x4 a = ka[k % (kQkAhead + 1)][mb];
        if (k < kNopeSteps)
          sc[mb][k & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), qnope[k],
                                                                 sc[mb][k & 1], 0, 0, 0);
        else
          sc[mb][k & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                  qrope[k - kNopeSteps], sc[mb][k & 1], 0, 0, 0);
      }
    }
    {
      // Under register pressure the compiler issues each K read just before
      // its MFMA and waits out the LDS latency.  Pin the order: the prologue
      // reads, then per k-step the reads of step k + kQkAhead before the two
      // MFMAs of step k.  (Once K and V shared one tile, this order also
      // became the faster one with four consumer waves: c4 27.8 -> 25.9 us.)
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kQkAhead, 0);   // DS reads
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k + kQkAhead < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);            // MFMAs
      }
    }
    const f32x4 sacc[2] = {sc[0][0] + sc[0][1], sc[1][0] + sc[1][1]};

    // a5: online softmax.  Lane holds tokens 16mb + 4g + r of head `head`.
    const int tile_valid = n_valid - t * kTileTokens;
    float x[2][4];
    float lmax = -INFINITY;   // max over the lane's own 8 scores
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = (16 * mb + 4 * g + r) < tile_valid;
        x[mb][r] = ok ? sacc[mb][r] * p.scale_log2 : -INFINITY;
        lmax = fmaxf(lmax, x[mb][r]);
      }
    // Lazy rescale: O and l keep a reference max m_run; they are rescaled only
    // when some head of the wave sees its max rise by more than kRescaleLog2,
    // so P = exp2(x - m_run) stays <= 2^kRescaleLog2 (exact in fp16 range).
    // The quotient O / l is the same for any reference, so this changes no
    // result beyond rounding.  P is taken against the current reference
    // while the (rare) need to move it is decided from each lane's own
    // scores, so the common path has no cross-lane reduction before PV.
    float e[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) e[mb][r] = __builtin_amdgcn_exp2f(x[mb][r] - m_run);
    float alpha = 1.f;
    if (__ballot(lmax > m_run + kRescaleLog2) != 0) {   // wave-uniform
      const float tmax = group_max4(lmax);              // the head's max over the tile
      const float m_new = fmaxf(m_run, tmax);          // finite: the tile has a valid token
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < kOBlocks; ++i) oacc[i] *= alpha;
      m_run = m_new;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) e[mb][r] = __builtin_amdgcn_exp2f(x[mb][r] - m_run);
    }
    f16x8 pb;   // P^T operand, k-slot 8g + 4mb + r
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        l_run += e[mb][r];   // the lane's share of l; lane groups are summed at the end
        pb[4 * mb + r] = (_Float16)e[mb][r];
      }
    if constexpr (kHelper) {   // for the PV helpers, which run next round
      sm.pex[t & 1][wid][lane] = __builtin_bit_cast(u32x4, pb);
      sm.aex[t & 1][wid][lane] = alpha;
    }

    // a6: O^T[dim][head] += V^T P^T over the tile's 32 tokens.  The P^T
    // operand of lane group g holds, in k-slots 8g + 4mb + r, the lane's
    // scores of tokens 16mb + 4g + r; the V^T operand comes from the
    // token-major tile through transposing reads: lane (g, c) addresses row
    // 4g + c/4 (+16), dims d0 + 4(c%4), and receives V[4g..4g+3 (+16)][d0 + c].
    // Operands are read kPvAhead blocks ahead.
    if constexpr (kOBlocks > 0) pv_blocks<kOBlocks>(oacc, &sm.kv[buf][(4 * g + (col >> 2)) * kRow + 4 * (col & 3)], pb);
    __syncthreads();
  }

  // a7: epilogue.  Lane holds O^T[16mb + 4g + r][head].
  l_run = group_sum4(l_run);
  if constexpr (kHelper) {   // the helpers' last round: hand them l
    sm.lx[wid][lane] = l_run;
    __syncthreads();
  }
  const bool empty = !(l_run > 0.f);
  const float inv = empty ? 0.f : 1.f / l_run;
  const float lse_v = empty ? -INFINITY : (m_run + __builtin_amdgcn_logf(l_run)) * 0.69314718055994531f;
  if constexpr (kOBlocks > 0)
    store_out<kOBlocks>(p, (uint8_t*)&sm.kv[0][0] + wid * kStageBytes, oacc, inv, b, s, head0, 0, lane);
  if (g == 0) {
    if (p.nsplit == 1)
      p.lse[(int64_t)b * p.lse_sb + head] = lse_v;
    else
      p.part_lse[((int64_t)b * p.nsplit + s) * kHeads + head] = lse_v;
  }
}

// ---------------------------------------------------------------------------
// a8: LSE combine of the slices of each query.
// ---------------------------------------------------------------------------

constexpr int kCombineThreads = 128;   // one workgroup per (query, head); 112 float4 per row

// Every thread loads all it needs at once -- the slices' lse values of its
// head and its float4 of every slice's partial row -- so the merge costs one
// memory round trip.  Weights: w_s = exp(lse_s - max) / sum; empty slices
// (lse = -inf) get 0; a query with no valid entry gets out = 0, lse = -inf.
__global__ __launch_bounds__(kCombineThreads) void mla_combine_kernel(const DecodeParams p) {
  // Same query -> XCD placement as the decode kernel, whose slices of this
  // query wrote the partials through this XCD's L2 just before.
  const int lb = logical_block(p.batch * kHeads);
  const int b = lb / kHeads, h = lb - b * kHeads;
  const int ns = p.nsplit;   // <= kMaxTopk / kTileTokens = 16
  const int c4 = threadIdx.x;
  const float* pl = p.part_lse + (int64_t)b * ns * kHeads + h;
  const float* po = p.part_o + ((int64_t)b * ns * kHeads + h) * kDV + 4 * c4;
  float l[16];
  f32x4 o[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if (k < ns) {
      l[k] = pl[k * kHeads];
      if (c4 < kDV / 4) o[k] = *(const f32x4*)(po + (int64_t)k * kHeads * kDV);
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (k < ns) m = fmaxf(m, l[k]);
  float tot = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if (k < ns) {
      const float w = (m == -INFINITY) ? 0.f : __expf(l[k] - m);   // exp(-inf) = 0 for empty slices
      tot += w;
      acc += w * o[k];
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  if (c4 < kDV / 4) {
    u32x2 w2;
    w2.x = bf16x2_rne(acc[0] * inv, acc[1] * inv);
    w2.y = bf16x2_rne(acc[2] * inv, acc[3] * inv);
    *(u32x2*)(p.out + (int64_t)b * p.out_sb + (int64_t)h * p.out_sh + 4 * c4) = w2;
  }
  if (c4 == 0) p.lse[(int64_t)b * p.lse_sb + h] = tot > 0.f ? m + __logf(tot) : -INFINITY;
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
  const int32_t* idx_row = p.topk_idx + (int64_t)b * p.idx_sb + e0;
  const int32_t* pt_row = p.page_table + (int64_t)b * p.pt_sb;
  const int seq_len = p.seq_lens[(int64_t)b * p.len_s];
  float* rows_b = p.rows + (int64_t)b * p.rows_sb;

  // masked entries: zero rows, valid = 0
  for (int j = tid; j < n_ent; j += kThreads) {
    int pg, sl;
    const bool v = resolve_entry(idx_row[j], seq_len, pt_row, p.max_pages, p.num_pages, pg, sl);
    p.valid[(int64_t)b * p.valid_sb + e0 + j] = v ? 1 : 0;
    if (!v) {
      float* r = rows_b + (int64_t)(e0 + j) * p.rows_sj;
      for (int d = 0; d < kDQK; d += 4) *(f32x4*)(r + d) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  const int n_valid = compact_slice(sm, idx_row, n_ent, seq_len, pt_row, p.max_pages, p.num_pages);
  const int ntiles = (n_valid + kTileTokens - 1) / kTileTokens;
  TileRegs regs;
  for (int t = 0; t < ntiles; ++t) {
    if (wid >= kConsumers) {
      const LastRecord last = {sm.tok[n_valid - 1][0], sm.tok[n_valid - 1][1]};
      load_tile(regs, sm, p.kv, p.page_stride, t, n_valid, last, wid - kConsumers, lane, lane_offset(lane));
      store_tile(sm, regs, 0, wid - kConsumers, lane);
    }
    __syncthreads();
    for (int tt = wid; tt < kTileTokens; tt += kWaves) {
      const int ci = t * kTileTokens + tt;
      if (ci >= n_valid) continue;
      float* r = rows_b + (int64_t)(e0 + sm.tok_entry[ci]) * p.rows_sj;
      // the tile row as the contractions read it: fp16 nope and bf16 rope,
      // widened to fp32 (exact)
      const u32x4 raw = *(const u32x4*)&sm.kv[0][tt * kRow + 8 * lane];
      f32x4 lo4, hi4;
      if (lane < 56) {
        const f16x8 h = __builtin_bit_cast(f16x8, raw);
        lo4 = f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
        hi4 = f32x4{(float)h[4], (float)h[5], (float)h[6], (float)h[7]};
      } else {
        lo4 = f32x4{__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                    __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
        hi4 = f32x4{__uint_as_float(raw.z << 16), __uint_as_float(raw.z & 0xffff0000u),
                    __uint_as_float(raw.w << 16), __uint_as_float(raw.w & 0xffff0000u)};
      }
      *(f32x4*)(r + 8 * lane) = lo4;
      *(f32x4*)(r + 8 * lane + 4) = hi4;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  const int nblk = p.batch * p.nsplit * p.head_groups;
  if (p.head_groups == 4)
    hipLaunchKernelGGL(mla_decode_kernel<4>, dim3(nblk), dim3(kThreads), 0, stream, p);
  else if (p.head_groups == 2)
    hipLaunchKernelGGL(mla_decode_kernel<2>, dim3(nblk), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(mla_decode_kernel<1>, dim3(nblk), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeParams& p, hipStream_t stream) {
  const int nblk = p.batch * kHeads;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(nblk), dim3(kCombineThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherParams& p, hipStream_t stream) {
  const int nblk = p.batch * p.nsplit;
  hipLaunchKernelGGL(mla_gather_kernel, dim3(nblk), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mlasd

