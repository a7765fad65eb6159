// gfx950 (CDNA4) LSE combine for a decode whose top-k lists were split into
// slices ("The Turning Point", "The Reasoning Process", Step 5): each slice
// left fp32 partial rows (already divided by its own softmax sum) and its
// log-sum-exp; out = sum_s w_s o_s with w_s = exp(lse_s - lse), lse = log
// sum_s exp(lse_s).
#include "mlasd_internal.h"

namespace mlasd {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int logical_block(int n) {
  // Workgroups are dispatched round-robin over the 8 XCDs (block i -> XCD
  // i % 8).  Renumbered as the decode kernel numbers its blocks, so the
  // workgroups of one query run on the XCD whose L2 holds its partials.
  const int i = blockIdx.x;
  const int xcd = i & 7, k = i >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd < rem ? xcd * (per + 1) + k : rem * (per + 1) + (xcd - rem) * per + k;
}

__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const bf16x2 r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
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

}  // namespace

hipError_t launch_combine(const DecodeParams& p, hipStream_t stream) {
  const int nblk = p.batch * kHeads;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(nblk), dim3(kCombineThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mlasd
