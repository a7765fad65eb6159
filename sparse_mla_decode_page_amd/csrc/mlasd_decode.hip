// gfx950 (CDNA4) decode kernel for sparse MLA over a paged FP8 KV cache.
//
// Method ("The Turning Point", "The Reasoning Process", Steps 3-5): one
// workgroup tile holds the heads of a query, so every selected record is
// fetched once and Q K^T becomes a matrix product; the top-k list may be
// split over several workgroups whose partial results are merged with the
// log-sum-exp rule.  Data flow per tile: gather -> dequantise -> Q K^T ->
// online softmax -> P V ("The Turning Point", "Output Knowledge Created",
// item 2).  448 nope dims are 28 whole 16-wide MFMA k-steps, so the pages'
// pad-to-512 mask has nothing to do here.
//
// Workgroup = (query b, slice s of its top-k list, head group), 512 threads
// = 8 waves; wave w runs on SIMD w % 4.  Roles, meeting at one barrier per
// stage; in stage t (one 32-token tile of work each):
//   producers gather the 576-byte records and 8-byte scale records of tile
//       t + 1 (loaded two tiles ahead into registers, each lane addressing
//       only its own token) and dequantise them into an LDS tile buffer;
//   QK waves (one per 32 heads, Q^T held in registers) compute S^T[32
//       tokens][32 heads] = K Q^T of tile t on v_mfma_f32_32x32x16 (fp16 over
//       the 448 nope dims, bf16 over the 64 rope dims);
//   the online softmax (fp32, exp2 domain) of a tile turns its scores into
//       the fp16 P^T operand: in the 64-head kernel on the PV waves, one
//       stage after the scores; in the 32-head kernel on the QK wave,
//       between the next tile's MFMAs, handing P^T and the accumulator
//       rescale factor to the PV waves through LDS.  There a second wave
//       takes nope dims [192, 448) of the scores and hands its fp32 part
//       over through LDS; the QK wave adds it one stage later;
//   PV waves (two per QK wave, 224 output dims each) accumulate
//       O^T[dims][heads] += V^T P^T on v_mfma_f32_32x32x16_f16, the V^T
//       operand read from the token-major tile by ds_read_b64_tr_b16; they
//       own O and write out (or fp32 partials).
// Four tile buffers hold the tiles in flight (the 32-head kernel's PV waves
// run two tiles behind the scores, the 64-head kernel's one).  One token-major fp16 tile serves both contractions (the nope dims
// are the K operand and V).  Before the loop every thread resolves and
// compacts one index entry (a1) and converts a slice of Q to fp16.
//
// Exactness.  The pages dequantise to bf16 ("The Turning Point", "Input
// Knowledge Required", FP8/UE8M0 bullet); here the shared tile is fp16, whose
// 11-bit significand also holds P to the precision PV needs, and both
// operands are kept exact over bf16's range by powers of two folded back in
// fp32:
//   - a token whose 7 scale bytes all lie in [112, 134] is stored as is
//     (e4m3 * 2^k is exact in fp16 for k in [-15, 7]); otherwise the tile
//     stores e4m3 * 2^(k_g - r_t) with one exponent r_t per token chosen so
//     every group is exact (possible whenever the token's groups span at
//     most 22 binades), the score gets 2^r_t back in fp32, and P V takes
//     2^(r_t - R) into P (R: running maximum of r_t, O rescaled when it
//     grows).  Tiles without such tokens run the plain path;
//   - each head's q is scaled by 2^-e_h, e_h placing its largest nope value
//     in [2^15, 2^16), so every value within 2^29 of the largest is exact in
//     fp16; the softmax scale takes 2^e_h back.
// Products of fp16 (or bf16) operands are exact in the fp32 accumulators.
#include "mlasd_internal.h"

namespace mlasd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = kThreads / 64;
constexpr int kRowB = 1024;               // tile row: 448 fp16 nope, 64 bf16 rope; 16-byte chunks swizzled
constexpr int kChunkH = 8;                // 16-bit values per 16-byte chunk
constexpr int kRowH = kRowB / 2;          // in 16-bit units
constexpr int kNopeSteps = kDNope / 16;   // 28 fp16 k-steps of Q K^T; 4 bf16 rope k-steps follow
constexpr int kQkAhead = 2;               // Q K^T operand k-steps read ahead
constexpr int kPvAhead = 2;               // P V operand blocks read ahead
constexpr int kDepth = 2;                 // tiles gathered ahead by the producers
constexpr int kBufs = 4;                  // tile buffers: producers t + 1, Q K^T t, P V t - 1 (64 heads) or t - 2
constexpr int kPtStaged = kTileTokens * kRowB / 4;   // page-table entries staged in tile buffer 0
constexpr float kRescaleLog2 = 8.f;       // lazy-rescale threshold: P <= 2^8
constexpr int kQRowH = 520;               // Q staging row (16-bit units): 512 + 8 pad
constexpr int kStageRowB = 464;           // epilogue staging row: 224 bf16 (448 B) + 16 B
constexpr int kNoRebase = -100000;        // R before any tile
constexpr int kQkSplit = 12;              // 32-head kernel: nope k-steps of the QK wave; wave 7 takes the rest

struct __align__(16) Smem {
  uint16_t kv[kBufs][kTileTokens * kRowH];   // 4 x 32 KiB tile buffers
  alignas(16) int32_t tflag[kBufs][4];    // [buffer][producer]: mask of rebased tokens
  alignas(16) int32_t rmax[kBufs][4];     // [buffer][producer]: largest rebase exponent
  alignas(16) int8_t rt[kBufs][kTileTokens];   // [buffer][row]: rebase exponent r_t of each row
  int32_t eh[kHeads];                     // per head of the workgroup: q prescale exponent
  u64x2 tok[kMaxTopk];                    // compacted list: byte offsets of the token's record and scale record
  uint16_t tok_entry[kMaxTopk];           //                 entry index in the slice
  int32_t wave_cnt[kWaves];
  alignas(16) float sf[4][16][8];        // [producer][token][group]: 2^(k_g - r_t) of the share's tokens
  union {
    // 64-head kernel: each QK wave hands a tile's raw scores S^T (fp32, in the
    // QK MFMAs' layout) to its PV waves: [tile & 1][QK wave][register quad][lane]
    f32x4 sx[2][2][4][64];
    // 32-head kernel: the QK wave runs the softmax and hands P to its PV waves
    struct {
      u32x4 pex[2][2][64];   // [tile & 1][k-step][lane]: P^T operand (fp16 x 8)
      float aex[2][64];      // [tile & 1][lane]: O rescale factor
      float lx[64];          // [lane]: final softmax sum
      int32_t rx;            // final rebase reference R
      alignas(16) f32x4 sx2[2][4][64];   // [tile & 1][register quad][lane]: wave 7's part of the scores
    } e;
  } h;
};
static_assert(kHeads * kQRowH * 2 <= 3 * kTileTokens * kRowB, "q staging must fit tile buffers 1-3");
static_assert(4 * 32 * kStageRowB <= 2 * kTileTokens * kRowB, "epilogue staging must fit two tile buffers");

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ int logical_block(int n) {
  // Workgroups are dispatched round-robin over the 8 XCDs (block i -> XCD
  // i % 8).  Renumber so that consecutive logical blocks -- the slices and
  // head groups of one query, which share Q and the gathered records -- run
  // on the same XCD and share its L2.
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
  const bf16x2_t r = {(__bf16)a, (__bf16)b};
  return pack2(r);
}

// max of x over lanes l and l ^ 32 (the two halves of a 32x32 result column)
__device__ __forceinline__ float pair_max(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __attribute__((noinline)) int page_entry_global(const int32_t* pt_row, int lp) { return pt_row[lp]; }

// a1: one index entry -> (page, slot) if valid.  Valid: 0 <= p < seq_len,
// logical page inside the page-table row, physical page inside the pool.
// Page-table entries below n_staged are read from the LDS copy `pt_lds`.
__device__ __forceinline__ bool resolve_entry(int p, int seq_len, const int32_t* pt_row, int32_t max_pages,
                                              int64_t num_pages, const int32_t* pt_lds, int n_staged, int& page,
                                              int& slot) {
  if (p < 0 || p >= seq_len) return false;
  const int lp = p >> 8;
  if (lp >= max_pages) return false;
  // pages past the staged part (rows over kPtStaged pages) come from the
  // page table itself, in a function of their own so the compiler does not
  // merge the two loads into one through a generic pointer
  const int pg = lp < n_staged ? pt_lds[lp] : page_entry_global(pt_row, lp);
  if (pg < 0 || (int64_t)pg >= num_pages) return false;
  page = pg;
  slot = p & (kPageTokens - 1);
  return true;
}

// a1 for a slice: stable compaction of its valid entries (one per thread)
// into the LDS token list, as the byte offsets in the pool of each token's
// 576-byte record and 8-byte scale record.  `p` is the thread's index entry (or -1).
// Returns the number of valid entries.  Ends with a barrier.
__device__ int compact_slice(Smem& sm, int p, int seq_len, const int32_t* pt_row, int32_t max_pages,
                             int64_t num_pages, int64_t pstride, const int32_t* pt_lds, int n_staged) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int page = 0, slot = 0;
  const bool v = resolve_entry(p, seq_len, pt_row, max_pages, num_pages, pt_lds, n_staged, page, slot);
  const uint64_t mask = __ballot(v);
  const int in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
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
    const uint64_t pg = (uint64_t)page * (uint64_t)pstride;
    sm.tok[pos] = u64x2{pg + slot * kRecordBytes, pg + kScaleBase + slot * kScaleRecordBytes};
    sm.tok_entry[pos] = (uint16_t)tid;
  }
  __syncthreads();
  return total;
}

// ---------------------------------------------------------------------------
// producers: a2 gather + a3 dequantise, 8 tokens per batch
// ---------------------------------------------------------------------------

// Tile rows are 64 chunks of 16 bytes (56 fp16 nope, 8 bf16 rope).  Chunk c
// of row r is stored at chunk (c & ~15) | ((c & 15) ^ swz(r)): with this
// permutation the three access patterns of a tile -- the producers' writes
// (two rows of 512 contiguous bytes per instruction), the Q K^T reads (32
// rows, one chunk each) and the transposing V reads (4 rows x 4 chunks per
// 16 lanes) -- each spread over all 64 LDS banks.
__device__ __forceinline__ int swz(int r) { return ((r & 1) << 3) | ((r & 2) << 1) | ((r >> 2) & 3); }
__device__ __forceinline__ int chunk_at(int r, int c) { return (c & ~15) | ((c & 15) ^ swz(r)); }

// The rebase exponent of a token from its largest and smallest group
// exponent: 0 when every group is exact in fp16 as stored (k in [-15, 7],
// bytes 112..134); else the value closest to 0 that keeps every group within
// fp16's exact range (k_g - r in [-15, 7]); if the groups span more than 22
// binades, the one that keeps the largest group exact.
__device__ __forceinline__ int rebase_exponent(int kmax, int kmin) {
  const int lo_r = kmax - 7, hi_r = kmin + 15;
  return lo_r > hi_r ? lo_r : min(max(0, lo_r), hi_r);
}

// A producer's share of one tile: kTok consecutive list entries starting at
// list0.  sc: lane l (< kTok) holds token l's 8-byte scale record.  b[h],
// the 2-token batch h: lane (t = lane / 32, p = lane % 32) owns token 2 h + t
// and chunks p and 32 + p of its tile row: n0 holds fp8 bytes [8 p, +8)
// (group p / 8); n1 holds, for p < 24, fp8 bytes [256 + 8 p, +8) in .xy
// (group 4 + p / 8), for p >= 24 rope bytes [16 (p - 24), +16).  Every lane
// addresses only its own token, so no value crosses lanes.
struct Batch {
  u32x2 n0;
  u32x4 n1;
};
template <int kTok>
struct Share {
  Batch b[kTok / 2];
  u32x2 sc;
};

// Loads of a share.  Entries past the last valid one re-read the slice's
// last valid record (already cached); their scores are masked.  n_valid >= 1.
// !kWide (the pool lies within 4 GiB of kv): each address is kv plus a
// zero-extended 32-bit offset, which the loads take as an SGPR base and a
// VGPR offset, with no 64-bit address arithmetic per load.
template <int kTok, bool kWide>
__device__ __forceinline__ void load_share(Share<kTok>& r, const Smem& sm, const uint8_t* kv, int list0, int n_valid,
                                           int lane) {
  const int p = lane & 31;
  // p < 24: the 8 bytes of chunk 32 + p (the load's upper half is unused and
  // stays inside the record); p >= 24: 16 rope bytes
  const int off1 = p < 24 ? 256 + 8 * p : kDNope + 16 * (p - 24);
  const bool full = list0 + kTok <= n_valid;   // wave-uniform: no entry past the end
  const int e_sc = list0 + (lane & (kTok - 1));
  const u64x2 a_sc = sm.tok[full ? e_sc : min(e_sc, n_valid - 1)];
#pragma unroll
  for (int h = 0; h < kTok / 2; ++h) {
    const int e = list0 + 2 * h + (lane >> 5);
    const u64x2 a = sm.tok[full ? e : min(e, n_valid - 1)];
    if constexpr (kWide) {
      const uint8_t* rec = kv + a.x;
      r.b[h].n0 = *(const u32x2*)(rec + 8 * p);
      r.b[h].n1 = *(const u32x4*)(rec + off1);
    } else {
      const uint32_t o = (uint32_t)a.x;
      r.b[h].n0 = *(const u32x2*)(kv + (uint32_t)(o + 8 * p));
      r.b[h].n1 = *(const u32x4*)(kv + (uint32_t)(o + off1));
    }
  }
  r.sc = *(const u32x2*)(kv + (kWide ? a_sc.y : (uint64_t)(uint32_t)a_sc.y));
}

// Lane byte offsets, from the share's first row, of the 16-byte chunk p of
// row 2 h + t (the batch rows); chunk 32 + p is 512 bytes further.
template <int kTok>
struct ShareAddr {
  int wo[kTok / 2];
};
template <int kTok>
__device__ __forceinline__ void share_addr(ShareAddr<kTok>& w, int row0, int lane) {
  const int t = lane >> 5, p = lane & 31;
#pragma unroll
  for (int h = 0; h < kTok / 2; ++h) {
    const int r = row0 + 2 * h + t;
    w.wo[h] = (2 * h + t) * kRowB + 16 * chunk_at(r, p);
  }
}

// a3: dequantise a share into rows [row0, row0 + kTok) of tile buffer `buf`
// (nope in fp16, rope as stored), with the rows' rebase exponents; producer
// pw's flags: mask of rebased rows and their largest exponent (0 if none).
// First, per token (lane l < kTok: token l): r_t and the 7 group scales
// 2^(k_g - r_t) as fp32 (0 below fp32's normal range), through LDS to the
// lanes of the token's batch.
template <int kTok>
__device__ __forceinline__ void store_share(Smem& sm, const Share<kTok>& r, const ShareAddr<kTok>& wa, int buf,
                                            int row0, int pw, int lane) {
  uint32_t bmax = 0, bmin = 255;
  uint32_t bs[7];
#pragma unroll
  for (int g = 0; g < 7; ++g) {
    bs[g] = ((g < 4 ? r.sc.x >> (8 * g) : r.sc.y >> (8 * (g - 4)))) & 0xFFu;
    bmax = max(bmax, bs[g]);
    bmin = min(bmin, bs[g]);
  }
  const int rt = rebase_exponent((int)bmax - 127, (int)bmin - 127);
  const uint32_t slow = (uint32_t)__ballot(rt != 0 && lane < kTok);
  if (lane < kTok) {
    u32x4 f0, f1;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const uint32_t v = g < 7 ? (uint32_t)max((int)bs[g] - rt, 0) << 23 : 0u;
      if (g < 4) f0[g] = v; else f1[g - 4] = v;
    }
    *(u32x4*)&sm.sf[pw][lane][0] = f0;
    *(u32x4*)&sm.sf[pw][lane][4] = f1;
    sm.rt[buf][row0 + lane] = (int8_t)rt;
  }
  int rm = 0;
  if (slow != 0) {   // rare: largest r_t of the share
#pragma unroll
    for (int l = 0; l < kTok; ++l) rm = max(rm, __builtin_amdgcn_readlane(rt, l));
  }
  if (lane == 0) {
    sm.tflag[buf][pw] = (int32_t)slow;
    sm.rmax[buf][pw] = rm;
  }
  const int t = lane >> 5, p = lane & 31, g0 = p >> 3;
  float sc0[kTok / 2], sc1[kTok / 2];   // read together: one LDS round trip for the share
#pragma unroll
  for (int h = 0; h < kTok / 2; ++h) {
    sc0[h] = sm.sf[pw][2 * h + t][g0];
    sc1[h] = sm.sf[pw][2 * h + t][4 + g0];   // group 7 (pad) for the rope lanes: unused
  }
  uint8_t* base = reinterpret_cast<uint8_t*>(&sm.kv[buf][row0 * kRowH]);
#pragma unroll
  for (int h = 0; h < kTok / 2; ++h) {
    const Batch& bt = r.b[h];
    u32x4 v0, v1;
    v0.x = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bt.n0.x, sc0[h], false));
    v0.y = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bt.n0.x, sc0[h], true));
    v0.z = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bt.n0.y, sc0[h], false));
    v0.w = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bt.n0.y, sc0[h], true));
    v1.x = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bt.n1.x, sc1[h], false));
    v1.y = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bt.n1.x, sc1[h], true));
    v1.z = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bt.n1.y, sc1[h], false));
    v1.w = pack2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bt.n1.y, sc1[h], true));
    uint8_t* dst = base + wa.wo[h];
    *(u32x4*)dst = v0;
    if (p < 24)
      *(u32x4*)(dst + 512) = v1;
    else
      *(u32x4*)(dst + 512) = bt.n1;   // rope chunks, as stored
  }
}

// ---------------------------------------------------------------------------
// Q: loaded and converted by all threads before the loop
// ---------------------------------------------------------------------------

// Thread (head h, chunk c) of the workgroup's heads: 64 dims [64 c, 64 c + 64)
// of q; chunks 0..6 are nope, chunk 7 is rope.
struct QChunk {
  u32x4 v[8];
};

__device__ __forceinline__ void load_q(QChunk& q, const DecodeParams& p, int b, int head, int chunk) {
  const uint16_t* row = p.q + (int64_t)b * p.q_sb + (int64_t)head * p.q_sh + 64 * chunk;
#pragma unroll
  for (int i = 0; i < 8; ++i) q.v[i] = *(const u32x4*)(row + 8 * i);
}

// e_h: the head's largest |q| over the 448 nope dims, m * 2^E with m in [1, 2),
// gives e_h = E - 15 (largest value in [2^15, 2^16)); all-zero heads get 0.
// The 8 threads of a head are 8 consecutive lanes.  Writes the head's q,
// times 2^-e_h (and -1 if `neg`), to the staging rows: nope in fp16, rope in
// bf16.
__device__ __forceinline__ void stage_q(Smem& sm, const QChunk& q, int hl, int chunk, bool neg, int lane) {
  uint32_t mx = 0;
  if (chunk < 7) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w = q.v[i][k];   // two bf16: |.| of each as an integer is monotonic in magnitude
        mx = max(mx, max(w & 0x7FFFu, (w >> 16) & 0x7FFFu));
      }
  }
  // max over the head's 8 lanes: xor 1 and xor 2 (quad permutes), then
  // each lane with its mirror in the 8-lane half row (the other quad)
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0xB1, 0xF, 0xF, false));
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x4E, 0xF, 0xF, false));
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x141, 0xF, 0xF, false));
  const int E = (int)(mx >> 7) - 127;
  const int eh = mx == 0 ? 0 : min(max(E - 15, -100), 100);
  // 2^-e_h, negated for a negative softmax scale (the scores change sign,
  // the exp2-domain factor c_h stays >= 0)
  const float down = __uint_as_float(((uint32_t)(127 - eh) << 23) | (neg ? 0x80000000u : 0u));
  uint16_t* dst = reinterpret_cast<uint16_t*>(&sm.kv[1][0]) + hl * kQRowH + 64 * chunk;
  auto convert = [&](auto cvt2) {   // one branch per thread: a thread's 64 dims are all nope or all rope
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w = q.v[i][k];
        o[k] = cvt2(__uint_as_float(w << 16) * down, __uint_as_float(w & 0xffff0000u) * down);
      }
      *(u32x4*)(dst + 8 * i) = o;
    }
  };
  if (chunk < 7)
    convert([](float f0, float f1) { return pack2(__builtin_amdgcn_cvt_pkrtz(f0, f1)); });
  else
    convert([](float f0, float f1) { return bf16x2_rne(f0, f1); });
  if (chunk == 0) sm.eh[hl] = eh;
  (void)lane;
}

// ---------------------------------------------------------------------------
// QK waves
// ---------------------------------------------------------------------------

// Q^T operands of a wave: nope k-steps [kA, kB) and, if kRope, the 4 rope
// k-steps.
template <int kA, int kB, bool kRope>
struct QRegs {
  f16x8 n[kB - kA];
  bf16x8 r[kRope ? 4 : 1];
};

// Rebase exponent of tile row 8 (i / 4) + 4 half + i % 4 (the row a QK
// lane holds in result register i), from the tile's 32 packed bytes.
__device__ __forceinline__ int row_rebase(const u32x4& rr0, const u32x4& rr1, int i, int half) {
  const int row = 8 * (i >> 2) + 4 * half + (i & 3);
  const uint32_t w = row < 16 ? rr0[row >> 2] : rr1[(row - 16) >> 2];
  return (int)(int8_t)(w >> (8 * (row & 3)));
}

// a5, the online softmax of one tile, as pieces a QK wave can issue between
// its MFMAs.  Input: the tile's scores acc (lane l: head l % 32, rows
// 8 (i / 4) + 4 (l / 32) + i % 4) and the factor c that takes them to the
// exp2 domain (c_h >= 0 for a full tile; 1 for the last tile, whose scores
// arrive scaled, with rows past the end at -inf).  Lazy rescale: m_run is a reference, not the
// running max; it moves only when some head of the wave sees its tile max
// exceed it by more than kRescaleLog2, so P = exp2(x - m_run) <=
// 2^kRescaleLog2 and alpha (the factor O and l take) is 1 on most tiles.
// O / l does not depend on the reference.  Every tile holds a valid token,
// so the new reference is finite.
struct Softmax {
  float lmax, m_new, sum, e_even;
};
// piece k of 19 (k = 0: tile max; 1: reference and alpha; 2..17: P of row
// register k - 2; 18: l and m)
__device__ __forceinline__ void softmax_piece(int k, Softmax& st, const f32x16& acc, float c_h, float& m_run,
                                              float& l_run, float& alpha, u32x4* pk) {
  if (k == 0) {   // c >= 0: the largest c * acc is c times the largest acc
    st.lmax = acc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) st.lmax = fmaxf(st.lmax, acc[i]);
    st.sum = 0.f;
  } else if (k == 1) {
    const float tmax = st.lmax * c_h;
    const float pm = pair_max(tmax);
    const bool up = __ballot(tmax > m_run + kRescaleLog2) != 0;   // wave-uniform
    st.m_new = up ? fmaxf(m_run, pm) : m_run;
    alpha = __builtin_amdgcn_exp2f(m_run - st.m_new);   // 0 on the first tile (m_run = -inf)
  } else if (k < 18) {
    const int i = k - 2;
    const float ei = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], c_h, -st.m_new));
    st.sum += ei;
    if (i & 1) {
      const f16x2_t h = {(_Float16)st.e_even, (_Float16)ei};
      pk[i >> 3][(i >> 1) & 3] = __builtin_bit_cast(uint32_t, h);
    } else {
      st.e_even = ei;
    }
  } else if (k == 18) {
    l_run = l_run * alpha + st.sum;   // the lane's share; the two halves are summed at the end
    m_run = st.m_new;
  }
}

// One QK-wave stage: S^T[token][head] for the tile row at krow over nope
// k-steps [kA, kB) and, if kRope, the 4 rope k-steps (k-step k reads chunk
// 2 k + l / 32, at krow + koff[k % 8] + 128 (k / 8)) into acc; in a tile
// with rebased rows (flag word `tflag` nonzero) the nope part of row r is
// multiplied by 2^r_t (exact in fp32; exponents from `rt`) before the rope
// k-steps are added.  kSM: also the softmax of the previous tile (scores in
// prev), cut into pieces issued between the MFMAs so the VALU work runs
// while the matrix core is busy.  Scheduling barriers keep each k-step's
// read (kQkAhead steps ahead), MFMA and piece together.
template <bool kSM, int kProd, int kA, int kB, bool kRope>
__device__ __forceinline__ void qk_stage(const uint16_t* krow, const int* koff, const QRegs<kA, kB, kRope>& q,
                                         f32x16& acc, const int32_t* tflags, const int8_t* rt, int half,
                                         const f32x16& prev, float c_h, float& m_run, float& l_run, float& alpha,
                                         u32x4* pk) {
  constexpr int kRing = kQkAhead + 1;
  constexpr int kNn = kB - kA;                      // nope k-steps
  constexpr int kSteps = kNn + (kRope ? 4 : 0);
  auto kread = [&](int j) {
    const int k = j < kNn ? kA + j : kNopeSteps + (j - kNn);   // the j-th k-step
    return *(const u32x4*)(krow + koff[k & 7] + 128 * (k >> 3));
  };
  const i32x4 fl = *(const i32x4*)tflags;   // consumed after the nope steps
  auto rebase_rows = [&]() {
    const int tf = kProd == 2 ? fl.x | fl.y : fl.x | fl.y | fl.z | fl.w;
    if (__builtin_amdgcn_readfirstlane(tf) != 0) {   // rare
      const u32x4 rr0 = *(const u32x4*)rt;
      const u32x4 rr1 = *(const u32x4*)(rt + 16);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = __builtin_ldexpf(acc[i], row_rebase(rr0, rr1, i, half));
    }
  };
  u32x4 ka[kRing];
#pragma unroll
  for (int j = 0; j < kQkAhead; ++j) ka[j] = kread(j);
  acc = f32x16{};
  Softmax st{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kSteps; ++j) {
    if (j + kQkAhead < kSteps) ka[(j + kQkAhead) % kRing] = kread(j + kQkAhead);
    if (j == kNn) rebase_rows();
    if (j < kNn)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, ka[j % kRing]), q.n[j], acc, 0, 0, 0);
    else
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[j % kRing]), q.r[j - kNn], acc,
                                                    0, 0, 0);
    if constexpr (kSM) {
      if (j <= 18) {
        softmax_piece(j, st, prev, c_h, m_run, l_run, alpha, pk);
        // keep the piece here (the compiler would sink it to its use)
        if (j == 1) asm volatile("" ::"v"(alpha), "v"(st.m_new));
        if (j >= 2 && j < 18) asm volatile("" ::"v"(st.sum), "v"(st.e_even), "v"(pk[(j - 2) >> 3][((j - 2) >> 1) & 3]));
        if (j == 18) asm volatile("" ::"v"(l_run));
      }
    }
    if (j < kNn || (kSM && j <= 18)) __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (kSM) {
#pragma unroll
    for (int j = kSteps; j <= 18; ++j) softmax_piece(j, st, prev, c_h, m_run, l_run, alpha, pk);
  }
  if constexpr (!kRope) rebase_rows();
}

// ---------------------------------------------------------------------------
// PV waves
// ---------------------------------------------------------------------------

// O^T[dims][heads] += V^T P^T over a tile's 32 tokens for kBlocks 32-dim
// blocks.  k-step s covers tile rows 16 s .. 16 s + 15 in the order the QK
// result hands them over: the P^T operand of lane l holds the lane's P of
// rows 8 (j / 4) + 4 (l / 32) + j % 4 (+16 s), j = 0..7.  The V^T operand
// comes from two transposing reads per k-step: the 16 lanes of group G
// address rows 16 s + 8 h + 4 (G / 2) + c / 4 (h = 0, 1; c = lane % 16) at
// dims d + 16 (G % 2) + 4 (c % 4) and receive V[those 4 rows][d + 16 (G % 2) + c].
// `voff[2 m + h]` is the lane's offset in the tile for block m, k-step 0,
// half h (k-step 1 is 16 rows further).
template <int kBlocks>
__device__ __forceinline__ void pv_tile(f32x16* o, const uint16_t* tile, const int* voff, const f16x8 pb[2]) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  constexpr int kN = 2 * kBlocks;   // (block, k-step) pairs
  i16x4 va[kPvAhead + 1][2];
  auto addr = [&](int i, int h) { return tile + voff[2 * (i >> 1) + h] + (i & 1) * 16 * kRowH; };
#pragma unroll
  for (int i = 0; i < kPvAhead; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) va[i][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)addr(i, h));
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    if (i + kPvAhead < kN)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        va[(i + kPvAhead) % (kPvAhead + 1)][h] =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)addr(i + kPvAhead, h));
    const f16x4 lo = __builtin_bit_cast(f16x4, va[i % (kPvAhead + 1)][0]);
    const f16x4 hi = __builtin_bit_cast(f16x4, va[i % (kPvAhead + 1)][1]);
    const f16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    o[i >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[i & 1], o[i >> 1], 0, 0, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPvAhead, 1);
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    if (i + kPvAhead < kN) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
  }
}

// a7 for one PV wave: its 32 heads x 224 dims, O^T in o[7] (lane l: head
// l % 32, dims 32 blk + 8 (i / 4) + 4 (l / 32) + i % 4), scaled by `mul`
// (2^R / l).  bf16 out (nsplit == 1) or fp32 partials, staged through LDS
// (`stage`, 32 rows of kStageRowB bytes) so the stores write whole runs of
// cache lines.
__device__ __forceinline__ void store_pv(const DecodeParams& p, uint8_t* stage, const f32x16* o, float mul, int b,
                                         int s, int head0, int dim0, int lane) {
  const int col = lane & 31, half = lane >> 5;
  if (p.nsplit == 1) {
#pragma unroll
    for (int blk = 0; blk < 7; ++blk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w;
        w.x = bf16x2_rne(o[blk][4 * j] * mul, o[blk][4 * j + 1] * mul);
        w.y = bf16x2_rne(o[blk][4 * j + 2] * mul, o[blk][4 * j + 3] * mul);
        *(u32x2*)(stage + col * kStageRowB + 2 * (32 * blk + 8 * j + 4 * half)) = w;
      }
    uint8_t* obase = (uint8_t*)(p.out + (int64_t)b * p.out_sb + (int64_t)head0 * p.out_sh + dim0);
#pragma unroll
    for (int k = 0; k < 14; ++k) {   // 32 rows x 28 chunks of 16 B
      const int i = lane + 64 * k, row = i / 28, ch = i - 28 * row;
      *(u32x4*)(obase + (int64_t)row * (2 * p.out_sh) + 16 * ch) = *(const u32x4*)(stage + row * kStageRowB + 16 * ch);
    }
  } else {
    const int64_t prow0 = ((int64_t)b * p.nsplit + s) * kHeads + head0;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {   // fp32: 112 dims (3.5 blocks) per pass through the 464-byte rows
#pragma unroll
      for (int blk = 0; blk < 7; ++blk)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 32 * blk + 8 * j + 4 * half;   // 0..223
          if ((d >= 112) == (hh == 1))
            *(f32x4*)(stage + col * kStageRowB + 4 * (d - 112 * hh)) =
                f32x4{o[blk][4 * j] * mul, o[blk][4 * j + 1] * mul, o[blk][4 * j + 2] * mul, o[blk][4 * j + 3] * mul};
        }
#pragma unroll
      for (int k = 0; k < 14; ++k) {   // 32 rows x 28 chunks of 16 B
        const int i = lane + 64 * k, row = i / 28, ch = i - 28 * row;
        *(f32x4*)(p.part_o + (prow0 + row) * kDV + dim0 + 112 * hh + 4 * ch) =
            *(const f32x4*)(stage + row * kStageRowB + 16 * ch);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// the decode kernel
// ---------------------------------------------------------------------------

// kHG = 1: a workgroup computes all 64 heads of its (query, slice): QK
// waves 0 and 1 (SIMDs 0, 1), producers 2 and 3 (16 tokens each, SIMDs 2,
// 3), PV waves 4, 6 (heads 0-31, dims 0-223 / 224-447) and 5, 7 (heads
// 32-63): each SIMD runs one MFMA-heavy wave and one lighter one.  Stage t
// (between barriers B_t and B_t+1, t = 0..ntiles): producers dequantise
// tile t + 1, QK waves compute the scores of tile t and hand them over raw,
// PV waves run the online softmax of tile t - 1 and accumulate it (each of
// a QK wave's two PV waves computes the same P for its 32 heads).
// kHG = 2: 32 heads: QK wave 0 (nope dims [0, 192) and rope), second QK
// wave 7 (nope dims [192, 448)), PV waves 2 and 3, producers 1, 4, 5, 6 (8
// tokens each).  Stage t (t = 0..ntiles + 1): producers dequantise tile
// t + 1, the QK wave computes the scores of tile t and the softmax of tile
// t - 1 between its MFMAs, PV waves accumulate tile t - 2.  (With the
// softmax on the PV waves as in the 64-head kernel, the last tile's serial
// softmax and P V cost more on short slices than the stage it saves.)
// Tile t lives in buffer t % 4.
template <int kHG, bool kWide>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(const DecodeParams p) {
  __shared__ Smem sm;
  constexpr int kHeadsWG = kHeads / kHG;
  constexpr int kProd = kHG == 1 ? 2 : 4;
  constexpr int kTokP = kTileTokens / kProd;   // 16 or 8
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int blk = logical_block(p.batch * p.nsplit * kHG);
  const int hg = blk % kHG, bs = blk / kHG;
  const int b = bs / p.nsplit, s = bs - b * p.nsplit;
  const int e0 = s * p.split_len;
  const int n_ent = max(0, min(p.topk - e0, p.split_len));
  const int head_base = kHeadsWG * hg;

  // ---- prologue: index entry, page-table entry, q; compaction ----
  const int32_t* pt_row = p.page_table + (int64_t)b * p.pt_sb;
  const int seq_len = p.seq_lens[(int64_t)b * p.len_s];
  // Loads without branches (clamped indices, results discarded where out of
  // range), so the wait for the index and page-table entries does not also
  // wait for Q, whose loads are issued after them and complete in order.
  int idx = n_ent > 0 ? p.topk_idx[(int64_t)b * p.idx_sb + e0 + min(tid, n_ent - 1)] : -1;
  idx = tid < n_ent ? idx : -1;
  // The query's page-table row (its first kPtStaged entries) goes to LDS in
  // the same round trip as the index entries, so resolving an entry costs
  // no dependent global load.  Tile buffer 0 holds it until compaction ends.
  int32_t* pt_lds = reinterpret_cast<int32_t*>(&sm.kv[0][0]);
  const int n_staged = min(p.max_pages, kPtStaged);
  int ptv[4];
  const int32_t* pt_src = n_staged > 0 ? pt_row : p.seq_lens;   // an empty row reads a harmless word
#pragma unroll
  for (int j = 0; j < 4; ++j) ptv[j] = pt_src[max(0, min(j * kThreads + tid, n_staged - 1))];
  __builtin_amdgcn_sched_barrier(0);
  const int q_hl = tid >> 3, q_chunk = tid & 7;   // q staging: 8 threads per head
  const bool q_thread = q_hl < kHeadsWG;
  QChunk qc;
  // every thread of the 64-head kernel loads q; in the 32-head kernel the
  // waves past the group's heads skip it (wave-uniform)
  if (kHG == 1 || q_thread) load_q(qc, p, b, head_base + (q_hl & (kHeadsWG - 1)), q_chunk);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 4; ++j) pt_lds[j * kThreads + tid] = ptv[j];   // entries past n_staged are never read
  for (int i = 4 * kThreads + tid; i < n_staged; i += kThreads) pt_lds[i] = pt_row[i];   // rows past 2048 pages
  __syncthreads();
  const int n_valid =
      compact_slice(sm, idx, seq_len, pt_row, p.max_pages, p.num_pages, p.page_stride, pt_lds, n_staged);
  const int ntiles = (n_valid + kTileTokens - 1) / kTileTokens;
  // barriers B_0 .. B_nstages-1: the 64-head kernel's PV waves run one stage
  // behind the scores, the 32-head kernel's two (the softmax in between)
  constexpr int kLag = kHG == 1 ? 1 : 2;
  const int nstages = ntiles > 0 ? ntiles + kLag : 0;

  // 0 QK, 1 PV, 2 producer, 3 second QK wave (32-head kernel)
  const int role = kHG == 1 ? (wid < 2 ? 0 : (wid == 2 || wid == 3) ? 2 : 1)
                            : (wid == 0 ? 0 : (wid == 2 || wid == 3) ? 1 : wid == 7 ? 3 : 2);
  const int pw = kHG == 1 ? wid - 2 : (wid == 1 ? 0 : wid - 3);   // producer index

  // ---- producers: a2 (gather) and a3 (dequantise) ----
  if (role == 2) {
    Share<kTokP> regs[kDepth];
    ShareAddr<kTokP> wa;
    share_addr(wa, kTokP * pw, lane);
    if (ntiles > 0) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) load_share<kTokP, kWide>(regs[u], sm, p.kv, u * kTileTokens + kTokP * pw, n_valid, lane);
    }
    if (q_thread) stage_q(sm, qc, q_hl, q_chunk, p.scale_log2 < 0.f, lane);
    __syncthreads();   // q staged
    if (ntiles == 0) return;
    store_share(sm, regs[0], wa, 0, kTokP * pw, pw, lane);
    load_share<kTokP, kWide>(regs[0], sm, p.kv, kDepth * kTileTokens + kTokP * pw, n_valid, lane);
    __syncthreads();   // B_0
    for (int t0 = 0; t0 + 1 < nstages; t0 += kDepth) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const int t = t0 + u;                // stage
        const int nxt = (u + 1) % kDepth;   // ring slot of tile t + 1
        if (t + 1 < ntiles) store_share(sm, regs[nxt], wa, (t + 1) % kBufs, kTokP * pw, pw, lane);
        // issued on every path so the loads behind each ring slot are the
        // same wherever it is consumed (past the end they re-read a cached record)
        load_share<kTokP, kWide>(regs[nxt], sm, p.kv, (t + 1 + kDepth) * kTileTokens + kTokP * pw, n_valid, lane);
        if (t + 1 < nstages) __syncthreads();   // B_{t+1}
      }
    }
    return;
  }

  if (q_thread) stage_q(sm, qc, q_hl, q_chunk, p.scale_log2 < 0.f, lane);
  __syncthreads();   // q staged
  if (ntiles == 0) {
    if (role == 1) {   // no valid entry: zero output, lse -inf
      const int qk = kHG == 1 ? (wid & 1) : 0;
      const int dhalf = kHG == 1 ? ((wid >> 1) & 1) : (wid & 1);
      f32x16 o[7];
#pragma unroll
      for (int i = 0; i < 7; ++i) o[i] = f32x16{};
      const int slot = kHG == 1 ? wid - 4 : dhalf;
      uint8_t* stage = (uint8_t*)&sm.kv[slot >> 1][0] + (slot & 1) * (32 * kStageRowB);
      store_pv(p, stage, o, 0.f, b, s, head_base + 32 * qk, 224 * dhalf, lane);
    } else if (role == 0 && (lane >> 5) == 0) {
      const int head = head_base + 32 * (kHG == 1 ? wid : 0) + lane;
      if (p.nsplit == 1)
        p.lse[(int64_t)b * p.lse_sb + head] = -INFINITY;
      else
        p.part_lse[((int64_t)b * p.nsplit + s) * kHeads + head] = -INFINITY;
    }
    return;
  }

  if (role == 3) {
    // 32-head kernel, wave 7: the nope k-steps [kQkSplit, 28) of each tile's
    // scores, handed to the QK wave through LDS (it adds them one stage later)
    const int col = lane & 31, half = lane >> 5;
    QRegs<kQkSplit, kNopeSteps, false> q;
    {
      const uint16_t* qs = reinterpret_cast<const uint16_t*>(&sm.kv[1][0]) + col * kQRowH + 8 * half;
#pragma unroll
      for (int k = kQkSplit; k < kNopeSteps; ++k) q.n[k - kQkSplit] = *(const f16x8*)(qs + 16 * k);
    }
    int koff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) koff[j] = kChunkH * chunk_at(col, 2 * j + half);
    __syncthreads();   // B_0
    f32x16 acc;
    float m_unused = 0.f, l_unused = 0.f, a_unused = 1.f;
    for (int t = 0; t + 1 < nstages; ++t) {
      if (t < ntiles) {
        const int buf = t % kBufs;
        qk_stage<false, kProd, kQkSplit, kNopeSteps, false>(&sm.kv[buf][col * kRowH], koff, q, acc, sm.tflag[buf],
                                                             sm.rt[buf], half, acc, 0.f, m_unused, l_unused,
                                                             a_unused, nullptr);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          sm.h.e.sx2[t & 1][c][lane] = f32x4{acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]};
      }
      __syncthreads();   // B_{t+1}
    }
    return;
  }

  if (role == 1) {
    if constexpr (kHG == 1) {
      // ---- PV waves (64 heads): a5 (online softmax) and a6 (P V), one stage behind the scores ----
      const int qk = kHG == 1 ? (wid & 1) : 0;   // the QK wave served (its 32 heads)
      const int dhalf = kHG == 1 ? ((wid >> 1) & 1) : (wid & 1);
      const int dim0 = 224 * dhalf;
      const int col = lane & 31, half = lane >> 5;
      const int hl = 32 * qk + col;   // head within the workgroup
      const float c_h = __builtin_ldexpf(fabsf(p.scale_log2), sm.eh[hl]);   // |scale| * log2(e) * 2^e_h
      f32x16 o[7];
#pragma unroll
      for (int i = 0; i < 7; ++i) o[i] = f32x16{};
      const int G = lane >> 4, c = lane & 15;
      int voff[14];
#pragma unroll
      for (int m = 0; m < 7; ++m)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = 4 * (G >> 1) + (c >> 2) + 8 * h;
          const int d = dim0 + 16 * (G & 1) + 4 * (c & 3) + 32 * m;
          voff[2 * m + h] = r * kRowH + kChunkH * chunk_at(r, d >> 3) + (d & 7);
        }
      float m_run = -INFINITY, l_run = 0.f;
      int R = kNoRebase;
      __syncthreads();   // B_0
      for (int t = 1; t < nstages; ++t) {
        __syncthreads();   // B_t: the scores of tile t - 1 are in LDS
        const int pt = t - 1, pbuf = pt % kBufs;
        // S^T of tile pt, laid out as the QK MFMAs left it (lane l: head l % 32,
        // rows 8 (i / 4) + 4 (l / 32) + i % 4); the 32-head kernel adds wave 7's part
        f32x16 sc;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 x = sm.h.sx[pt & 1][qk][q4][lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[4 * q4 + e] = x[e];
        }
        float cs = c_h;
        if (pt == ntiles - 1) {   // the last tile, possibly partial: scaled here, rows past the end -inf
          const int tile_valid = n_valid - pt * kTileTokens;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = 8 * (i >> 2) + 4 * half + (i & 3);
            sc[i] = row < tile_valid ? sc[i] * c_h : -INFINITY;
          }
          cs = 1.f;
        }
        float alpha = 1.f;
        u32x4 pk[2];
        Softmax st{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k <= 18; ++k) softmax_piece(k, st, sc, cs, m_run, l_run, alpha, pk);
        // P V takes 2^(r_t - R) into P, R the running largest r_t (O rescaled
        // by 2^(R_old - R_new) when it grows).
        const i32x4 pf = *(const i32x4*)sm.tflag[pbuf];
        const i32x4 pr = *(const i32x4*)sm.rmax[pbuf];
        const uint32_t pflag = __builtin_amdgcn_readfirstlane(kProd == 2 ? pf.x | pf.y : pf.x | pf.y | pf.z | pf.w);
        const int prt = __builtin_amdgcn_readfirstlane(
            max(0, kProd == 2 ? max(pr.x, pr.y) : max(max(pr.x, pr.y), max(pr.z, pr.w))));
        const int R_new = max(R, prt);
        if (R_new != R) {
          alpha = R == kNoRebase ? alpha : __builtin_ldexpf(alpha, R - R_new);
          R = R_new;
        }
        if (pflag != 0 || R != 0) {   // rare: P takes 2^(r_t - R) per row (r_t - R <= 0)
          const u32x4 pr0 = *(const u32x4*)&sm.rt[pbuf][0];
          const u32x4 pr1 = *(const u32x4*)&sm.rt[pbuf][16];
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              f16x8& v = reinterpret_cast<f16x8*>(pk)[j];
              v[i] = (_Float16)__builtin_ldexpf((float)v[i], row_rebase(pr0, pr1, 8 * j + i, half) - R);
            }
        }
        if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
          for (int i = 0; i < 7; ++i) o[i] *= alpha;
        }
        const f16x8 pb[2] = {__builtin_bit_cast(f16x8, pk[0]), __builtin_bit_cast(f16x8, pk[1])};
        pv_tile<7>(o, sm.kv[pbuf], voff, pb);
      }
      const float l = pair_sum(l_run);
      const float mul = l > 0.f ? __builtin_ldexpf(1.f / l, R == kNoRebase ? 0 : R) : 0.f;
      // staging: two slots in each of the tile buffers the last P V does not read
      const int slot = kHG == 1 ? wid - 4 : dhalf;
      const int sbuf = (ntiles + (slot >> 1)) % kBufs;
      uint8_t* stage = (uint8_t*)&sm.kv[sbuf][0] + (slot & 1) * (32 * kStageRowB);
      store_pv(p, stage, o, mul, b, s, head_base + 32 * qk, dim0, lane);
      // a7 (lse): lanes 0..31 of the wave with the first 224 dims write their head
      if (dhalf == 0 && half == 0) {
        const float lse_v = l > 0.f ? (m_run + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
        const int head = head_base + hl;
        if (p.nsplit == 1)
          p.lse[(int64_t)b * p.lse_sb + head] = lse_v;
        else
          p.part_lse[((int64_t)b * p.nsplit + s) * kHeads + head] = lse_v;
      }

    } else {
      // ---- PV waves (32 heads): a6, two stages behind the scores ----
      const int qk = kHG == 1 ? (wid & 1) : 0;   // the QK wave served (its 32 heads)
      const int dhalf = kHG == 1 ? ((wid >> 1) & 1) : (wid & 1);
      const int dim0 = 224 * dhalf;
      f32x16 o[7];
#pragma unroll
      for (int i = 0; i < 7; ++i) o[i] = f32x16{};
      const int G = lane >> 4, c = lane & 15;
      int voff[14];
#pragma unroll
      for (int m = 0; m < 7; ++m)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = 4 * (G >> 1) + (c >> 2) + 8 * h;
          const int d = dim0 + 16 * (G & 1) + 4 * (c & 3) + 32 * m;
          voff[2 * m + h] = r * kRowH + kChunkH * chunk_at(r, d >> 3) + (d & 7);
        }
      __syncthreads();   // B_0
      __syncthreads();   // B_1
      for (int t = 2; t < nstages; ++t) {
        __syncthreads();   // B_t: P of tile t - 2 is in LDS
        const int pt = t - 2;
        f16x8 pb[2];
        pb[0] = __builtin_bit_cast(f16x8, sm.h.e.pex[pt & 1][0][lane]);
        pb[1] = __builtin_bit_cast(f16x8, sm.h.e.pex[pt & 1][1][lane]);
        const float a = sm.h.e.aex[pt & 1][lane];
        if (__ballot(a != 1.f) != 0) {
#pragma unroll
          for (int i = 0; i < 7; ++i) o[i] *= a;
        }
        pv_tile<7>(o, sm.kv[pt % kBufs], voff, pb);
      }
      // the QK wave wrote the final l and R before the last barrier
      const float l = sm.h.e.lx[lane];
      const int R = sm.h.e.rx;
      const float mul = l > 0.f ? __builtin_ldexpf(1.f / l, R == kNoRebase ? 0 : R) : 0.f;
      // staging: two slots in each of the tile buffers the last P V does not read
      const int slot = kHG == 1 ? wid - 4 : dhalf;
      const int sbuf = (ntiles + (slot >> 1)) % kBufs;
      uint8_t* stage = (uint8_t*)&sm.kv[sbuf][0] + (slot & 1) * (32 * kStageRowB);
      store_pv(p, stage, o, mul, b, s, head_base + 32 * qk, dim0, lane);

    }
    return;
  }

  if constexpr (kHG == 1) {
    // ---- QK waves: a4 (scores), handed to the PV waves through LDS ----
    const int qk = wid;
    const int col = lane & 31, half = lane >> 5;
    const int hl = 32 * qk + col;                      // head within the workgroup
    constexpr int kQkN = kNopeSteps;                   // nope k-steps of this wave
    QRegs<0, kQkN, true> q;
    {
      const uint16_t* qs = reinterpret_cast<const uint16_t*>(&sm.kv[1][0]) + hl * kQRowH + 8 * half;
#pragma unroll
      for (int k = 0; k < kQkN; ++k) q.n[k] = *(const f16x8*)(qs + 16 * k);
#pragma unroll
      for (int k = 0; k < 4; ++k) q.r[k] = *(const bf16x8*)(qs + kDNope + 16 * k);
    }
    int koff[8];   // k-step k % 8 -> the lane's chunk in its row's 16-chunk block k / 8
#pragma unroll
    for (int j = 0; j < 8; ++j) koff[j] = kChunkH * chunk_at(col, 2 * j + half);
    __syncthreads();   // B_0
    f32x16 acc;
    float m_unused = 0.f, l_unused = 0.f, a_unused = 1.f;
    for (int t = 0; t + 1 < nstages; ++t) {   // stage t: Q K^T of tile t
      const int buf = t % kBufs;
      qk_stage<false, kProd, 0, kQkN, true>(&sm.kv[buf][col * kRowH], koff, q, acc, sm.tflag[buf], sm.rt[buf], half,
                                            acc, 0.f, m_unused, l_unused, a_unused, nullptr);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        sm.h.sx[t & 1][qk][c][lane] = f32x4{acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]};
      __syncthreads();   // B_{t+1}
    }
  } else {
    // ---- QK wave: a4 (scores) and a5 (online softmax) ----
    const int qk = 0;
    const int col = lane & 31, half = lane >> 5;
    const int hl = col;                                // head within the workgroup
    constexpr int kQkN = kQkSplit;                     // nope k-steps of this wave; wave 7 has the rest
    QRegs<0, kQkN, true> q;
    {
      const uint16_t* qs = reinterpret_cast<const uint16_t*>(&sm.kv[1][0]) + hl * kQRowH + 8 * half;
#pragma unroll
      for (int k = 0; k < kQkN; ++k) q.n[k] = *(const f16x8*)(qs + 16 * k);
#pragma unroll
      for (int k = 0; k < 4; ++k) q.r[k] = *(const bf16x8*)(qs + kDNope + 16 * k);
    }
    const float c_h = __builtin_ldexpf(fabsf(p.scale_log2), sm.eh[hl]);   // |scale| * log2(e) * 2^e_h
    int koff[8];   // k-step k % 8 -> the lane's chunk in its row's 16-chunk block k / 8
#pragma unroll
    for (int j = 0; j < 8; ++j) koff[j] = kChunkH * chunk_at(col, 2 * j + half);
    float m_run = -INFINITY, l_run = 0.f;
    int R = kNoRebase;
    __syncthreads();   // B_0

    // stage t: Q K^T of tile t (t < ntiles) into `cur`, softmax of tile t - 1
    // from `prev` (the two accumulators alternate, so the next stage's MFMAs
    // never wait for this one's softmax to have read its scores)
    auto stage = [&](int t, f32x16& cur, f32x16& prev) {
      const int buf = t % kBufs, pbuf = (t + kBufs - 1) % kBufs;
      const uint16_t* krow = &sm.kv[buf][col * kRowH];
      const i32x4 pf = *(const i32x4*)sm.tflag[pbuf];   // the previous tile's flags, used after the MFMAs
      const i32x4 pr = *(const i32x4*)sm.rmax[pbuf];
      float alpha = 1.f;
      u32x4 pk[2];
      if constexpr (kHG == 2) {
        if (t > 0) {   // wave 7's part of the previous tile's scores
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const f32x4 x = sm.h.e.sx2[(t - 1) & 1][c][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) prev[4 * c + e] += x[e];
          }
        }
      }
      if (t == 0) {
        qk_stage<false, kProd, 0, kQkN, true>(krow, koff, q, cur, sm.tflag[buf], sm.rt[buf], half, prev, c_h, m_run,
                                              l_run, alpha, pk);
      } else if (t < ntiles) {
        qk_stage<true, kProd, 0, kQkN, true>(krow, koff, q, cur, sm.tflag[buf], sm.rt[buf], half, prev, c_h, m_run,
                                             l_run, alpha, pk);
      } else {
        // the last tile, possibly partial: scaled here, rows past the end -inf
        const int tile_valid = n_valid - (t - 1) * kTileTokens;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = 8 * (i >> 2) + 4 * half + (i & 3);
          prev[i] = row < tile_valid ? prev[i] * c_h : -INFINITY;
        }
        Softmax st{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k <= 18; ++k) softmax_piece(k, st, prev, 1.f, m_run, l_run, alpha, pk);
      }
      if (t > 0) {
        const uint32_t pflag =
            __builtin_amdgcn_readfirstlane(kProd == 2 ? pf.x | pf.y : pf.x | pf.y | pf.z | pf.w);
        const int prt = __builtin_amdgcn_readfirstlane(
            max(0, kProd == 2 ? max(pr.x, pr.y) : max(max(pr.x, pr.y), max(pr.z, pr.w))));
        // P V takes 2^(r_t - R) into P, R the running largest r_t (O rescaled
        // by 2^(R_old - R_new) when it grows).
        const int R_new = max(R, prt);
        if (R_new != R) {
          alpha = R == kNoRebase ? alpha : __builtin_ldexpf(alpha, R - R_new);
          R = R_new;
        }
        if (pflag != 0 || R != 0) {   // rare: P takes 2^(r_t - R) per row (r_t - R <= 0)
          const u32x4 pr0 = *(const u32x4*)&sm.rt[pbuf][0];
          const u32x4 pr1 = *(const u32x4*)&sm.rt[pbuf][16];
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              f16x8& v = reinterpret_cast<f16x8*>(pk)[j];
              v[i] = (_Float16)__builtin_ldexpf((float)v[i], row_rebase(pr0, pr1, 8 * j + i, half) - R);
            }
        }
        const int pt = t - 1;
        sm.h.e.pex[pt & 1][0][lane] = pk[0];
        sm.h.e.pex[pt & 1][1][lane] = pk[1];
        sm.h.e.aex[pt & 1][lane] = alpha;
        if (t == ntiles) {   // the PV waves' epilogue reads the final l and R
          sm.h.e.lx[lane] = pair_sum(l_run);
          if (lane == 0) sm.h.e.rx = R;
        }
      }
      __syncthreads();   // B_{t+1}
    };
    f32x16 acc0, acc1;
    acc1 = f32x16{};
    for (int t = 0; t + 1 < nstages; t += 2) {
      stage(t, acc0, acc1);
      if (t + 2 < nstages) stage(t + 1, acc1, acc0);
    }
    // a7 (lse): lanes 0..31 write their head
    const float l = pair_sum(l_run);
    const float lse_v = l > 0.f ? (m_run + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
    if (half == 0) {
      const int head = head_base + hl;
      if (p.nsplit == 1)
        p.lse[(int64_t)b * p.lse_sb + head] = lse_v;
      else
        p.part_lse[((int64_t)b * p.nsplit + s) * kHeads + head] = lse_v;
    }
  }
}

// ---------------------------------------------------------------------------
// test hook: a1-a3 exactly as the decode runs them, rows written per entry
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

  for (int j = tid; j < n_ent; j += kThreads) {   // masked entries: zero rows, valid = 0
    int pg, sl;
    const bool v = resolve_entry(idx_row[j], seq_len, pt_row, p.max_pages, p.num_pages, nullptr, 0, pg, sl);
    p.valid[(int64_t)b * p.valid_sb + e0 + j] = v ? 1 : 0;
    if (!v) {
      float* r = rows_b + (int64_t)(e0 + j) * p.rows_sj;
      for (int d = 0; d < kDQK; d += 4) *(f32x4*)(r + d) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const int n_valid = compact_slice(sm, tid < n_ent ? idx_row[tid] : -1, seq_len, pt_row, p.max_pages, p.num_pages,
                                    p.page_stride, nullptr, 0);
  const int ntiles = (n_valid + kTileTokens - 1) / kTileTokens;
  for (int t = 0; t < ntiles; ++t) {
    if (wid >= 4) {   // 4 producer waves of 8 tokens, the decode's own code
      Share<8> r;
      ShareAddr<8> wa;
      share_addr(wa, 8 * (wid - 4), lane);
      load_share<8, true>(r, sm, p.kv, t * kTileTokens + 8 * (wid - 4), n_valid, lane);
      store_share(sm, r, wa, 0, 8 * (wid - 4), wid - 4, lane);
    }
    __syncthreads();
    for (int tt = wid; tt < kTileTokens; tt += kWaves) {
      const int ci = t * kTileTokens + tt;
      if (ci >= n_valid) continue;
      float* r = rows_b + (int64_t)(e0 + sm.tok_entry[ci]) * p.rows_sj;
      // the row as the contractions read it, times the row's 2^r_t: fp16
      // nope and bf16 rope, widened to fp32 (exact)
      const int rexp = sm.rt[0][tt];
      const u32x4 raw = *(const u32x4*)&sm.kv[0][tt * kRowH + kChunkH * chunk_at(tt, lane)];
      f32x4 lo4, hi4;
      if (lane < 56) {
        const f16x8 h = __builtin_bit_cast(f16x8, raw);
        lo4 = f32x4{__builtin_ldexpf((float)h[0], rexp), __builtin_ldexpf((float)h[1], rexp),
                    __builtin_ldexpf((float)h[2], rexp), __builtin_ldexpf((float)h[3], rexp)};
        hi4 = f32x4{__builtin_ldexpf((float)h[4], rexp), __builtin_ldexpf((float)h[5], rexp),
                    __builtin_ldexpf((float)h[6], rexp), __builtin_ldexpf((float)h[7], rexp)};
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

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  const int nblk = p.batch * p.nsplit * p.head_groups;
  // gathers take 32-bit offsets when every byte of the pool lies within 4 GiB of its start
  const bool wide = (uint64_t)p.num_pages * (uint64_t)p.page_stride > (1ull << 32);
  if (p.head_groups == 2) {
    if (wide)
      hipLaunchKernelGGL((mla_decode_kernel<2, true>), dim3(nblk), dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((mla_decode_kernel<2, false>), dim3(nblk), dim3(kThreads), 0, stream, p);
  } else {
    if (wide)
      hipLaunchKernelGGL((mla_decode_kernel<1, true>), dim3(nblk), dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((mla_decode_kernel<1, false>), dim3(nblk), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_gather(const GatherParams& p, hipStream_t stream) {
  const int nblk = p.batch * p.nsplit;
  hipLaunchKernelGGL(mla_gather_kernel, dim3(nblk), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mlasd
