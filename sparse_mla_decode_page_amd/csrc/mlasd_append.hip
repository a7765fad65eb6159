// gfx950 kernel for the step before the decode: appending token latents to
// the paged FP8 cache.  Each 448-dim nope vector is quantised per 64-dim
// group to fp8 e4m3 with one UE8M0 scale byte per group, and stored with its
// 64 bf16 rope values in the 584-byte token layout the decode reads ("The
// Turning Point", "Input Knowledge Required", FP8/UE8M0 bullet; "The
// Validation Gate", "The Test Design: What Gets Validated and How").
//
// Quantiser (the pages name the format, not the rule; this is the plainest
// reading): the group's scale exponent k is the least integer with
// amax <= 448 * 2^k, clamped to [-127, 127] (amax = 0 gives -127); the scale
// byte is k + 127 and every value becomes the e4m3 code nearest to
// x * 2^-k, ties to even.  Scale byte 7 is written as 0.
//
// One wave per token: lanes 0..55 own nope dims [8 l, 8 l + 8) (group l / 8),
// lanes 56..63 copy 16 rope bytes each.  Loads and stores are contiguous.
#include "mlasd_internal.h"

namespace mlasd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kAppendWaves = 4;   // tokens per workgroup

// Least k with a <= 448 * 2^k for a finite a > 0: with a = m 2^e, m in
// [0.5, 1), and 448 = 0.875 * 2^9, k = e - 9 if m <= 0.875, else e - 8.
__device__ __forceinline__ int scale_exponent(float amax) {
  if (!(amax > 0.f)) return -127;
  int e;
  const float m = __builtin_frexpf(amax, &e);
  const int k = m <= 0.875f ? e - 9 : e - 8;
  return min(max(k, -127), 127);
}

__global__ __launch_bounds__(64 * kAppendWaves) void mla_kv_append_kernel(const AppendParams p) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * kAppendWaves + (threadIdx.x >> 6);
  if (tok >= p.n_tokens) return;   // wave-uniform
  // The latent row is issued first so its latency overlaps the dependent
  // seq id -> page table lookups.  Lanes 0..55: 8 nope values; lanes 56..63:
  // 8 rope values (bf16 bits).  Nothing here is read again: stream it.
  const u32x4 w = __builtin_nontemporal_load((const u32x4*)(p.latent + (int64_t)tok * p.lat_s) + lane);
  // Validity, wave-uniform and branch-free up to one exit so the compiler
  // keeps the latent load above it: the page-table lookup is clamped to
  // entry 0 (batch >= 1 and max_pages >= 1) when the token is out of range.
  const int s = p.seq_ids[(int64_t)tok * p.seq_s], pos = p.positions[(int64_t)tok * p.pos_s];
  const bool in_table = s >= 0 && s < p.batch && pos >= 0 && (pos >> 8) < p.max_pages;
  const int64_t entry = in_table ? (int64_t)s * p.pt_sb + (pos >> 8) : 0;
  const int looked_up = p.page_table[entry];
  const int page = in_table ? looked_up : -1;
  if (page < 0 || (int64_t)page >= p.num_pages) return;
  const int slot = pos & (kPageTokens - 1);
  uint8_t* pbase = p.kv + (int64_t)page * p.page_stride;

  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // group max over the 8 lanes of the group (aligned blocks of 8 lanes)
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  const int k = scale_exponent(amax);

  if (lane < kDNope / 8) {
    // x * 2^-k is exact (|x * 2^-k| <= 448); the conversion rounds to
    // nearest even onto the e4m3 grid, subnormals included.
    u32x2 codes;
    uint32_t lo = 0, hi = 0;
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[0], -k), ldexpf(v[1], -k), lo, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[2], -k), ldexpf(v[3], -k), lo, true);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4], -k), ldexpf(v[5], -k), hi, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[6], -k), ldexpf(v[7], -k), hi, true);
    codes.x = lo;
    codes.y = hi;
    __builtin_nontemporal_store(codes, (u32x2*)(pbase + slot * kRecordBytes + 8 * lane));
  } else {
    __builtin_nontemporal_store(w, (u32x4*)(pbase + slot * kRecordBytes + kDNope + 16 * (lane - kDNope / 8)));
  }
  // scale record: bytes 0..6 = k + 127 of groups 0..6 (lanes 0, 8, .., 48), byte 7 = 0
  uint32_t sb[7];
#pragma unroll
  for (int g = 0; g < 7; ++g) sb[g] = (uint32_t)(__builtin_amdgcn_readlane(k, 8 * g) + 127);
  if (lane == 0) {
    u32x2 rec;
    rec.x = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
    rec.y = sb[4] | (sb[5] << 8) | (sb[6] << 16);
    __builtin_nontemporal_store(rec, (u32x2*)(pbase + kScaleBase + slot * kScaleRecordBytes));
  }
}

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  const int nblk = (p.n_tokens + kAppendWaves - 1) / kAppendWaves;
  hipLaunchKernelGGL(mla_kv_append_kernel, dim3(nblk), dim3(64 * kAppendWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mlasd
