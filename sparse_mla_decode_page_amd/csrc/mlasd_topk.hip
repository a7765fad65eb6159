// gfx950 (CDNA4) top-k selection: the step upstream of the decode that
// turns a query's per-position indexer scores (fp32, "The Turning Point",
// "The Strategic Context: Why This Message Exists", item 3) into its top-k
// index list.  Candidates are positions 0 .. L-1, L = min(max(seq_len, 0),
// max_len); they rank by score, higher first, equal scores by position,
// lower first (NaN ranks as -inf, -0.0 equals +0.0); the first min(k, L)
// positions in rank order are written in that order, then -1.
//
// One workgroup per query.  Each score maps to a 32-bit key whose unsigned
// order is the rank order of the scores.  A three-digit radix select (11,
// 11 and 10 bits, histograms in LDS) finds the k-th largest key T; one more
// pass in position order collects every key above T and, of the keys equal
// to T, the lowest positions that complete k (block-wide prefix sums keep
// position order); a bitonic sort of the <= 512 picks by (key, -position)
// gives the output order.  Rows of at most k candidates skip the select.
#include "mlasd_internal.h"

namespace mlasd {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBins = 2048;

struct TopkSmem {
  uint32_t hist[kBins];
  uint64_t sel[kMaxTopk];      // (key << 32) | (0xffffffff - position): larger = earlier in rank order
  uint32_t wave_sum[kTopkWaves];
  uint32_t found[2];           // digit, count of keys above it
};

// Unsigned order of the key = rank order of the score.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (x != x) u = 0xFF800000u;        // NaN ranks as -inf
  if (u == 0x80000000u) u = 0u;        // -0.0 ties with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of v over the workgroup (thread order); *total gets
// the sum.  Ends with a barrier, so LDS it used may be reused at once.
__device__ __forceinline__ uint32_t block_exclusive_sum(TopkSmem& sm, uint32_t v, uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) sm.wave_sum[wid] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t c = sm.wave_sum[w];
    before += w < wid ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// The digit d of a histogram over nbins digits with
// count(digits > d) < need <= count(digits >= d), and count(digits > d).
__device__ __forceinline__ void find_digit(TopkSmem& sm, int nbins, uint32_t need, uint32_t* digit,
                                           uint32_t* above) {
  const int per = nbins / kTopkThreads;   // 2 or 1 bins per thread, highest digits first
  const int t = threadIdx.x;
  uint32_t v = 0;
  for (int j = 0; j < per; ++j) v += sm.hist[nbins - 1 - (t * per + j)];
  uint32_t total;
  uint32_t run = block_exclusive_sum(sm, v, &total);
  for (int j = 0; j < per; ++j) {
    const int d = nbins - 1 - (t * per + j);
    const uint32_t c = sm.hist[d];
    if (run < need && need <= run + c) {
      sm.found[0] = (uint32_t)d;
      sm.found[1] = run;
    }
    run += c;
  }
  __syncthreads();
  *digit = sm.found[0];
  *above = sm.found[1];
  __syncthreads();
}

__device__ __forceinline__ void clear_hist(TopkSmem& sm) {
  for (int i = threadIdx.x; i < kBins; i += kTopkThreads) sm.hist[i] = 0;
  __syncthreads();
}

__global__ __launch_bounds__(kTopkThreads, 1) void mla_topk_kernel(const TopkParams p) {
  __shared__ TopkSmem sm;
  const int b = blockIdx.x, tid = threadIdx.x;
  const float* row = p.scores + (int64_t)b * p.sc_sb;
  int32_t* dst = p.topk_idx + (int64_t)b * p.idx_sb;
  const int L = min(max(p.seq_lens[(int64_t)b * p.len_s], 0), p.max_len);
  const int k = p.k;
  const int n = min(k, L);

  // The threshold: keys above T are all taken, keys equal to T fill the
  // remaining `eq_take` slots in position order.  With L <= k every
  // candidate is taken.
  const bool all = L <= k;
  uint32_t T = 0, n_above = 0;
  if (!all) {
    clear_hist(sm);
    for (int i = tid; i < L; i += kTopkThreads) atomicAdd(&sm.hist[score_key(row[i]) >> 21], 1u);
    __syncthreads();
    uint32_t d1, a1, d2, a2, d3, a3;
    find_digit(sm, kBins, (uint32_t)k, &d1, &a1);
    clear_hist(sm);
    for (int i = tid; i < L; i += kTopkThreads) {
      const uint32_t key = score_key(row[i]);
      if ((key >> 21) == d1) atomicAdd(&sm.hist[(key >> 10) & 0x7FFu], 1u);
    }
    __syncthreads();
    find_digit(sm, kBins, (uint32_t)k - a1, &d2, &a2);
    clear_hist(sm);
    const uint32_t hi = (d1 << 11) | d2;
    for (int i = tid; i < L; i += kTopkThreads) {
      const uint32_t key = score_key(row[i]);
      if ((key >> 10) == hi) atomicAdd(&sm.hist[key & 0x3FFu], 1u);
    }
    __syncthreads();
    find_digit(sm, 1024, (uint32_t)k - a1 - a2, &d3, &a3);
    T = (hi << 10) | d3;
    n_above = a1 + a2 + a3;
  }
  const uint32_t eq_take = (uint32_t)n - n_above;

  // collect in position order
  uint32_t cnt_above = 0, cnt_eq = 0;
  for (int base = 0; base < L; base += kTopkThreads) {
    const int i = base + tid;
    const uint32_t key = i < L ? score_key(row[i]) : 0u;
    const bool take_above = i < L && (all || key > T);
    const bool is_eq = i < L && !all && key == T;
    uint32_t total;
    const uint32_t ex = block_exclusive_sum(sm, (take_above ? 1u : 0u) | (is_eq ? 0x10000u : 0u), &total);
    const uint64_t comp = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
    if (take_above) sm.sel[cnt_above + (ex & 0xFFFFu)] = comp;
    const uint32_t eq_rank = cnt_eq + (ex >> 16);
    if (is_eq && eq_rank < eq_take) sm.sel[n_above + eq_rank] = comp;
    cnt_above += total & 0xFFFFu;
    cnt_eq += total >> 16;
    if (!all && cnt_above >= n_above && cnt_eq >= eq_take) break;   // uniform: the rest is not taken
  }
  for (int i = n + tid; i < kMaxTopk; i += kTopkThreads) sm.sel[i] = 0;   // below every real pick
  __syncthreads();

  // bitonic sort, descending
  for (int size = 2; size <= kMaxTopk; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (tid < kMaxTopk / 2) {
        const int i = 2 * tid - (tid & (stride - 1)), j = i + stride;
        const uint64_t a = sm.sel[i], c = sm.sel[j];
        const bool desc = (i & size) == 0;
        if ((a < c) == desc) {
          sm.sel[i] = c;
          sm.sel[j] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < k; i += kTopkThreads)
    dst[i] = i < n ? (int32_t)(0xFFFFFFFFu - (uint32_t)(sm.sel[i] & 0xFFFFFFFFu)) : -1;
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(mla_topk_kernel, dim3(p.batch), dim3(kTopkThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mlasd
