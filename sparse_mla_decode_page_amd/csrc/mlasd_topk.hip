// gfx950 (CDNA4) top-k selection: the step upstream of the decode that
// turns a query's per-position indexer scores (fp32, "The Turning Point",
// "The Strategic Context: Why This Message Exists", item 3) into its top-k
// index list.  Candidates are positions 0 .. L-1, L = min(max(seq_len, 0),
// max_len); they rank by score, higher first, equal scores by position,
// lower first (NaN ranks as -inf, -0.0 equals +0.0); the first min(k, L)
// positions in rank order are written in that order, then -1.
//
// Steps 3-4 run in one workgroup per query.  Each candidate becomes a
// 64-bit composite, (key << 32) | (2^32 - 1 - position), key a 32-bit map
// of the score whose unsigned order is the score order: composites are
// distinct and their unsigned order is the rank order, so the picks are
// exactly the min(k, L) largest composites.
//   1. Threshold guess (rows over kSmallRow positions): the composites of 512
//      positions spread over the row; t0, the lower edge of the 22-bit bin
//      holding their r-th largest, r set so about 3 k of the row's
//      composites lie at or above t0.
//   2. One pass over the row (its only read from HBM) appends every
//      composite >= t0 to an LDS candidate list, one LDS atomic per wave
//      and batch.  Since t0's low 42 bits are 0, the test is a float
//      comparison with the score whose key t0 holds, unless that score is
//      zero or denormal.  Shorter rows go to the list whole.
//   3. If the list holds at least k and at most kCand composites, a radix
//      select over it (11/11/10-bit digits over the 64 bits, LDS
//      histograms, stopping once a digit's bin is taken whole) gives the
//      k-th largest composite Tc, and the picks are the list's composites
//      >= Tc.  Otherwise (guess too high or too low, e.g. long rows of
//      equal scores) the same select and collection run over the row.
//   4. Output order: each wave sorts its 64 of the <= 512 picks by
//      bitonic stages within the wave (DPP and lane swizzles); a pick's
//      place is the number of picks above it, its lane plus a binary search
//      in each other wave's sorted run (composites are distinct).
// At small batch, steps 1-2 of long rows can run in a launch of their own,
// one workgroup per (part, row), each part of the row appending its
// composites >= the row's t0 (the same sample, so the same t0 in every
// part) to its own region of a workspace; the per-row launch then joins the
// parts' lists in LDS and runs steps 3-4.  The picks, and so the output,
// are the same as with one workgroup per row.
// A row is read as a head of up to 3 positions before its first 16-byte
// boundary, a body of float4 vectors and a tail of up to 3 positions.
#include "mlasd_internal.h"

namespace mlasd {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / 64;
static_assert(kTopkThreads == kMaxTopk, "one pick per thread in the output step");
constexpr int kBins = 2048;
constexpr int kCand = 16384;       // LDS candidate list (128 KiB)
constexpr int kSmallRow = 4096;    // rows up to this length go to the list whole
constexpr int kSample = kTopkThreads;
constexpr int kUnroll = 8;         // float4 loads in flight per thread in a compaction pass
constexpr int kSweepUnroll = 2;    // and in a histogram pass over the row (the rare path)
constexpr int kMaxParts = 8;       // workgroups per row in the candidate pass, at most

struct TopkSmem {
  uint64_t cand[kCand];
  uint64_t sel[kMaxTopk];
  uint32_t hist[kBins];
  uint32_t wave_tot[kTopkWaves];
  uint32_t found[3];   // digit, count above it, count in its bin
  uint32_t n_cand, n_sel;
  uint32_t kmax;       // largest key appended to the candidate list
};

// Unsigned order of the key = rank order of the score.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (x != x) u = 0xFF800000u;        // NaN ranks as -inf
  if (u == 0x80000000u) u = 0u;        // -0.0 ties with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Every key is >= score_key(-inf) = 0x007fffff, so 0 is below every composite.
__device__ __forceinline__ uint64_t composite(float x, int pos) {
  return ((uint64_t)score_key(x) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)pos);
}

// Inclusive prefix sum of v over the wave's lanes: shifts within rows of
// 16 lanes, then each row's total carried to the rows above it.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2, 3
  return x;
}

// The digit d of the histogram's 2^kW digits with count(digits > d) <
// need <= count(digits >= d); count(digits > d) and count(digit d).
// Thread t holds the t-th highest group of kPer digits (wave 0 the
// highest); a prefix sum over the threads finds the group that crosses
// `need`, its thread the digit.  Each thread zeroes its bins, so the next
// level starts from a clear histogram.  need >= 1 and at most the
// histogram's total.  Called by every thread, after a barrier that follows
// the histogram's last update; ends with a barrier.
template <int kW>
__device__ __forceinline__ void find_digit(TopkSmem& sm, uint32_t need, uint32_t* digit, uint32_t* above,
                                           uint32_t* in_bin) {
  constexpr int kPer = (1 << kW) / kTopkThreads;   // 4 or 2
  static_assert(kPer == 2 || kPer == 4, "digits per thread");
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lo = (1 << kW) - kPer * (tid + 1);   // the thread's lowest digit
  uint32_t h[kPer];
  if constexpr (kPer == 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(&sm.hist[lo]);
    h[0] = v[0], h[1] = v[1], h[2] = v[2], h[3] = v[3];
    *reinterpret_cast<u32x4*>(&sm.hist[lo]) = u32x4{0u, 0u, 0u, 0u};
  } else {
    const u32x2 v = *reinterpret_cast<const u32x2*>(&sm.hist[lo]);
    h[0] = v[0], h[1] = v[1];
    *reinterpret_cast<u32x2*>(&sm.hist[lo]) = u32x2{0u, 0u};
  }
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) s += h[j];
  const uint32_t incl = wave_incl_sum(s);
  if (lane == 63) sm.wave_tot[wid] = incl;
  __syncthreads();
  uint32_t run = incl - s;   // count of the digits above this thread's
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) run += w < wid ? sm.wave_tot[w] : 0u;
  if (run < need && need <= run + s) {   // exactly one thread: walk its digits downwards
#pragma unroll
    for (int j = kPer - 1; j >= 0; --j) {
      if (run < need && need <= run + h[j]) {
        sm.found[0] = (uint32_t)(lo + j);
        sm.found[1] = run;
        sm.found[2] = h[j];
      }
      run += h[j];
    }
  }
  __syncthreads();
  *digit = sm.found[0];
  *above = sm.found[1];
  *in_bin = sm.found[2];
}

// hist[bin] += 1 for every active lane.  Lanes of one wave often share a
// bin (scores cluster in a few exponents): up to four rounds add each
// shared bin's count once, while the bins found are shared by more than
// two lanes; the remaining lanes add singly.
__device__ __forceinline__ void hist_add(TopkSmem& sm, uint32_t bin, bool active) {
  const int lane = threadIdx.x & 63;
  uint64_t todo = __ballot(active);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    if (todo == 0) return;   // wave-uniform
    const int leader = __builtin_ctzll(todo);
    const uint32_t lb = __builtin_amdgcn_readlane(bin, leader);
    const uint64_t same = __ballot(bin == lb) & todo;
    const uint32_t c = (uint32_t)__popcll(same);
    if (lane == leader) atomicAdd(&sm.hist[lb], c);
    todo &= ~same;
    if (c <= 2) break;   // wave-uniform
  }
  if ((todo >> lane) & 1) atomicAdd(&sm.hist[bin], 1u);
}

// First slot of this lane's `mine` appends: one LDS atomic per wave on
// *count, lanes in order after it.
__device__ __forceinline__ uint32_t wave_reserve(uint32_t* count, uint32_t mine) {
  const uint32_t incl = wave_incl_sum(mine);
  const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
  uint32_t base = 0;
  if (total != 0) {   // uniform
    if ((threadIdx.x & 63) == 0) base = atomicAdd(count, total);
    base = __builtin_amdgcn_readlane(base, 0);
  }
  return base + incl - mine;
}

// L >= 1 consecutive positions of a row, the first at row position pos0:
// head [0, hh) before the first 16-byte boundary, body of nv float4
// vectors (elements hh + 4 j + e), tail [hh + 4 nv, L).  Composites and
// takes see row positions, pos0 + element.
struct RowView {
  const float* row;
  const f32x4* body;
  int L, hh, nv, pos0;
};

__device__ __forceinline__ RowView view_row(const float* row, int L, int pos0 = 0) {
  RowView rv;
  rv.row = row;
  rv.L = L;
  rv.pos0 = pos0;
  rv.hh = min(L, (int)(((16u - (uint32_t)(reinterpret_cast<uintptr_t>(row) & 15u)) & 15u) >> 2));
  rv.body = reinterpret_cast<const f32x4*>(row + rv.hh);
  rv.nv = (L - rv.hh) >> 2;
  return rv;
}

// f(valid, x, position) for the head's and the tail's positions, one per
// thread; every lane makes the same calls.
template <class F>
__device__ __forceinline__ void for_singles(const RowView& rv, F&& f) {
  const int tid = threadIdx.x;
  if (rv.hh > 0) f(tid < rv.hh, rv.row[min(tid, rv.hh - 1)], rv.pos0 + tid);   // uniform
  const int t0 = rv.hh + 4 * rv.nv;
  if (t0 < rv.L) f(t0 + tid < rv.L, rv.row[min(t0 + tid, rv.L - 1)], rv.pos0 + t0 + tid);   // uniform
}

// Body vectors base + u * kTopkThreads + tid into x[u] (clamped to the last one); nv >= 1.
template <int kN>
__device__ __forceinline__ void load_batch(const RowView& rv, int base, f32x4 (&x)[kN]) {
#pragma unroll
  for (int u = 0; u < kN; ++u) x[u] = rv.body[min(base + u * kTopkThreads + (int)threadIdx.x, rv.nv - 1)];
}

// Appends composite(x) of the batch's positions with take(x, position) to
// list[0 .. cap) (counted past cap, not stored), one LDS atomic per wave.
// The takes are kept as one bit each between the count and the writes.
template <class Take>
__device__ __forceinline__ void emit_batch(const RowView& rv, const f32x4 (&x)[kUnroll], int base, Take&& take,
                                           uint64_t* list, uint32_t* count, int cap, uint32_t& mk) {
  static_assert(4 * kUnroll <= 64, "one bit per position of a batch");
  const int tid = threadIdx.x;
  uint64_t m = 0;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int j = base + u * kTopkThreads + tid;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      m |= (j < rv.nv && take(x[u][e], rv.pos0 + rv.hh + 4 * j + e)) ? 1ull << (4 * u + e) : 0ull;
  }
  uint32_t slot = wave_reserve(count, (uint32_t)__popcll(m));
  // each lane walks its set bits (few: the takes are sparse), two at a
  // time, reading those scores again (the batch was just read: L2 hits)
  while (__ballot(m != 0) != 0) {   // wave-uniform
    const bool h0 = m != 0;
    const int b0 = h0 ? __builtin_ctzll(m) : 0;
    m &= m - 1;
    const bool h1 = m != 0;
    const int b1 = h1 ? __builtin_ctzll(m) : 0;
    m &= m - 1;
    const int p0 = rv.hh + 4 * (base + (b0 >> 2) * kTopkThreads + tid) + (b0 & 3);
    const int p1 = rv.hh + 4 * (base + (b1 >> 2) * kTopkThreads + tid) + (b1 & 3);
    const float x0 = rv.row[h0 ? p0 : 0];
    const float x1 = rv.row[h1 ? p1 : 0];
    if (h0) {
      const uint64_t c = composite(x0, rv.pos0 + p0);
      if (slot < (uint32_t)cap) list[slot] = c;
      mk = max(mk, (uint32_t)(c >> 32));
      ++slot;
    }
    if (h1) {
      const uint64_t c = composite(x1, rv.pos0 + p1);
      if (slot < (uint32_t)cap) list[slot] = c;
      mk = max(mk, (uint32_t)(c >> 32));
      ++slot;
    }
  }
}

// Largest of x over lanes 0 .. i, in lane i (lane 63: the wave's largest):
// the prefix pattern of wave_incl_sum with max in place of the sum.
__device__ __forceinline__ uint32_t wave_incl_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false));   // row_shr:1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false));   // row_shr:2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false));   // row_shr:4
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false));   // row_shr:8
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false));   // row_bcast:15
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false));   // row_bcast:31
  return x;
}

// Appends composite(x) of every position of the row with take(x,
// position), in no particular order; if kmax is not null, the largest
// appended key is max-ed into *kmax (LDS).  x0 holds the body's first
// batch.
template <class Take>
__device__ __forceinline__ void compact_row(const RowView& rv, const f32x4 (&x0)[kUnroll], Take&& take,
                                            uint64_t* list, uint32_t* count, int cap, uint32_t* kmax = nullptr) {
  constexpr int kStep = kUnroll * kTopkThreads;
  uint32_t mk = 0;
  if (rv.nv > 0) {
    // two batches in flight: the next is requested before this one's appends
    f32x4 xa[kUnroll], xb[kUnroll];
    for (int u = 0; u < kUnroll; ++u) xa[u] = x0[u];
    for (int base = 0; base < rv.nv; base += 2 * kStep) {
      if (base + kStep < rv.nv) load_batch(rv, base + kStep, xb);   // uniform
      emit_batch(rv, xa, base, take, list, count, cap, mk);
      if (base + kStep < rv.nv) {
        if (base + 2 * kStep < rv.nv) load_batch(rv, base + 2 * kStep, xa);
        emit_batch(rv, xb, base + kStep, take, list, count, cap, mk);
      }
    }
  }
  for_singles(rv, [&](bool ok, float x, int pos) {
    const bool t = ok && take(x, pos);
    const uint32_t slot = wave_reserve(count, t ? 1u : 0u);
    const uint64_t c = composite(x, pos);
    if (t && slot < (uint32_t)cap) list[slot] = c;
    if (t) mk = max(mk, (uint32_t)(c >> 32));
  });
  if (kmax != nullptr) {   // uniform
    mk = wave_incl_max(mk);
    if ((threadIdx.x & 63) == 63 && mk != 0) atomicMax(kmax, mk);
  }
}

// f(valid, composite) over the row's positions; every lane makes the same
// number of calls (f uses wave ballots).
template <class F>
__device__ __forceinline__ void sweep_row(const RowView& rv, F&& f) {
  const int tid = threadIdx.x;
  for (int base = 0; base < rv.nv; base += kSweepUnroll * kTopkThreads) {
    f32x4 x[kSweepUnroll];
    load_batch(rv, base, x);
#pragma unroll
    for (int u = 0; u < kSweepUnroll; ++u) {
      const int j = base + u * kTopkThreads + tid;
#pragma unroll
      for (int e = 0; e < 4; ++e) f(j < rv.nv, composite(x[u][e], rv.pos0 + rv.hh + 4 * j + e));
    }
  }
  for_singles(rv, [&](bool ok, float x, int pos) { f(ok, composite(x, pos)); });
}

// f(valid, composite) over the candidate list list[0 .. n), n >= 1, four
// loads in flight per thread
template <class F>
__device__ __forceinline__ void sweep_list(const uint64_t* list, int n, F&& f) {
  constexpr int kL = 4;
  const int tid = threadIdx.x;
  for (int base = 0; base < n; base += kL * kTopkThreads) {
    uint64_t c[kL];
#pragma unroll
    for (int q = 0; q < kL; ++q) c[q] = list[min(base + q * kTopkThreads + tid, n - 1)];
#pragma unroll
    for (int q = 0; q < kL; ++q) f(base + q * kTopkThreads + tid < n, c[q]);
  }
}

// Radix select over the composites a sweep visits: the largest threshold
// Tc with count(composites >= Tc) >= need, using at most max_levels digits
// (11, 11, 10, 11, 11, 10 bits from the top).  It stops early once `need`
// takes a digit's bin whole, and then count(>= Tc) == need exactly; so it
// does after six levels (the bin holds one composite).  With max_levels 2,
// count(>= Tc) >= need and Tc is the lower edge of a 22-bit bin.  1 <= need
// <= number of composites; the histogram is clear on entry and on exit.
template <class Sweep>
__device__ __forceinline__ uint64_t radix_threshold(TopkSmem& sm, uint32_t need, int max_levels, Sweep&& sweep) {
  uint64_t prefix = 0;
  int bits = 0;
  for (int lvl = 0; lvl < max_levels; ++lvl) {
    const int w = lvl % 3 == 2 ? 10 : 11;
    const int shift = 64 - bits - w;
    const uint32_t dmask = (1u << w) - 1;
    sweep([&](bool ok, uint64_t c) {
      const bool in = ok && ((c >> 1) >> (63 - bits)) == prefix;   // bits = 0: 0 == 0
      hist_add(sm, (uint32_t)(c >> shift) & dmask, in);
    });
    __syncthreads();
    uint32_t d, above, cnt;
    if (w == 11)
      find_digit<11>(sm, need, &d, &above, &cnt);
    else
      find_digit<10>(sm, need, &d, &above, &cnt);
    need -= above;
    prefix = (prefix << w) | d;
    bits += w;
    if (cnt == need) break;   // uniform
  }
  return prefix << (64 - bits);
}

// Step 3's select over the candidate list sm.cand[0 .. nc), whose
// composites all lie in [lo, hi]: the largest Tc with count(>= Tc) == need.
// The first digit is (c >> s) - (lo >> s), s the least shift that fits
// [lo, hi] into 2^11 bins, each bin the composites that share their top
// 64 - s bits; then 11-bit digits below it (a last narrower one placed high
// in a 10-bit histogram) until `need` takes a bin whole, which it does at
// the latest when the bin holds one composite.  1 <= need <= nc; the
// histogram is clear on entry and on exit.
__device__ __forceinline__ uint64_t list_threshold(TopkSmem& sm, uint32_t need, uint64_t lo, uint64_t hi, int nc) {
  // (hi - lo) >> s < 2^11, so (hi >> s) - (lo >> s) <= 2^11; one more bit if it is 2^11
  int s = hi - lo < 2048u ? 0 : 53 - __builtin_clzll(hi - lo);
  if ((hi >> s) - (lo >> s) > 2047u) ++s;
  const uint64_t base = lo >> s;
  sweep_list(sm.cand, nc, [&](bool ok, uint64_t c) {
    hist_add(sm, (uint32_t)min((c >> s) - base, (uint64_t)2047u), ok);
  });
  __syncthreads();
  uint32_t d, above, cnt;
  find_digit<11>(sm, need, &d, &above, &cnt);
  need -= above;
  uint64_t prefix = base + d;
  int bits = 64 - s;
  while (cnt != need && bits < 64) {   // uniform
    const int rem = 64 - bits;                 // 1 .. 63 bits below the prefix
    const int used = rem < 11 ? rem : 11;
    const int sh = rem - used;
    const int pad = used < 10 ? 10 - used : 0;
    sweep_list(sm.cand, nc, [&](bool ok, uint64_t c) {
      const bool in = ok && (c >> rem) == prefix;
      hist_add(sm, (uint32_t)((c >> sh) & ((1ull << used) - 1)) << pad, in);
    });
    __syncthreads();
    if (used == 11)
      find_digit<11>(sm, need, &d, &above, &cnt);
    else
      find_digit<10>(sm, need, &d, &above, &cnt);
    need -= above;
    prefix = (prefix << used) | (d >> pad);
    bits += used;
  }
  return prefix << (64 - bits);
}

// r for a sample of kSample out of L > kSmallRow positions: about 3 k of the
// row's composites lie at or above the sample's r-th largest.
__device__ __forceinline__ uint32_t sample_rank(int L, int k) {
  return (uint32_t)min(kSample, max(8, (int)((3ll * k * kSample + L - 1) / L)));
}

// Step 1 for a row of L > kSmallRow positions: t0 from the sample of
// kSample positions spread over the whole row (every workgroup of a row
// that is cut into parts computes the same t0).
__device__ __forceinline__ uint64_t row_threshold(TopkSmem& sm, const float* row, int L, int k) {
  const int sp = (int)(((int64_t)threadIdx.x * L) / kSample);
  const uint64_t sc = composite(row[sp], sp);
  return radix_threshold(sm, sample_rank(L, k), 2, [&](auto&& f) { f(true, sc); });
}

// Step 2 over the positions of rv: appends their composites >= t0 to
// list[0 .. cap), counting in *count (past cap: counted, not stored).
// t0's low 42 bits are 0, so composite >= t0 is key >= kt.  Below
// key(-inf) every position qualifies: all of rv is appended, or only
// counted if it cannot fit.  Otherwise kt is the key of a float f0; when f0
// is normal or infinite, key(x) >= kt is x >= f0 in float order (NaN is
// below f0 on both sides, -0 equals +0, and a denormal x lies on the same
// side of f0 whether flushed or not).  The largest appended key is max-ed
// into *kmax (LDS).  x0 holds rv's first body batch.
__device__ __forceinline__ void compact_above(const RowView& rv, const f32x4 (&x0)[kUnroll], uint64_t t0,
                                              uint64_t* list, uint32_t* count, int cap, uint32_t* kmax) {
  const uint32_t kt = (uint32_t)(t0 >> 32);
  const uint32_t fb = kt >= 0x80000000u ? kt ^ 0x80000000u : ~kt;
  if (kt <= 0x007FFFFFu) {
    if (rv.L <= cap)
      compact_row(rv, x0, [](float, int) { return true; }, list, count, cap, kmax);
    else if (threadIdx.x == 0)
      *count = (uint32_t)rv.L;
  } else if ((fb & 0x7F800000u) != 0) {
    const float f0 = __uint_as_float(fb);
    compact_row(rv, x0, [f0](float x, int) { return x >= f0; }, list, count, cap, kmax);
  } else {
    compact_row(rv, x0, [kt](float x, int) { return score_key(x) >= kt; }, list, count, cap, kmax);
  }
}

// Step 3 with the candidate list in sm.cand[0 .. sm.n_cand) (n_cand past
// kCand: the list overflowed), every composite of it at least lo and with
// a key at most sm.kmax: the k picks appended to sm.sel.  Called by every
// thread after a barrier that follows the list's last write.
__device__ __forceinline__ void select_picks(TopkSmem& sm, const RowView& rv, int k, uint64_t lo) {
  const uint32_t nc = sm.n_cand;
  if (nc >= (uint32_t)k && nc <= (uint32_t)kCand) {
    const uint64_t hi = ((uint64_t)sm.kmax << 32) | 0xFFFFFFFFull;
    const uint64_t tc = list_threshold(sm, (uint32_t)k, lo, hi, (int)nc);
    sweep_list(sm.cand, (int)nc, [&](bool ok, uint64_t c) {
      const bool take = ok && c >= tc;
      const uint32_t slot = wave_reserve(&sm.n_sel, take ? 1u : 0u);
      if (take && slot < (uint32_t)kMaxTopk) sm.sel[slot] = c;
    });
  } else {   // the guess left too few or too many: select over the row
    const uint64_t tc = radix_threshold(sm, (uint32_t)k, 6, [&](auto&& f) { sweep_row(rv, f); });
    f32x4 x0[kUnroll];
    if (rv.nv > 0) load_batch(rv, 0, x0);
    compact_row(rv, x0, [tc](float x, int pos) { return composite(x, pos) >= tc; }, sm.sel, &sm.n_sel, kMaxTopk);
  }
  __syncthreads();
}

// Steps 1-3 for one row in one workgroup: the min(k, L) picks appended to sm.sel.
__device__ __forceinline__ void select_row(TopkSmem& sm, const RowView& rv, int k) {
  const int L = rv.L;
  // the body's first batch is requested before the sample's select runs
  f32x4 x0[kUnroll];
  if (rv.nv > 0) load_batch(rv, 0, x0);
  if (L <= k) {   // every candidate is picked
    compact_row(rv, x0, [](float, int) { return true; }, sm.sel, &sm.n_sel, kMaxTopk);
    __syncthreads();
    return;
  }
  uint64_t t0 = 0;
  if (L <= kSmallRow) {   // the whole row is the list
    compact_row(rv, x0, [](float, int) { return true; }, sm.cand, &sm.n_cand, kCand, &sm.kmax);
  } else {
    t0 = row_threshold(sm, rv.row, L, k);
    compact_above(rv, x0, t0, sm.cand, &sm.n_cand, kCand, &sm.kmax);
  }
  __syncthreads();
  select_picks(sm, rv, k, t0);
}

// v of lane (lane ^ kS), kS < 64, within the wave
template <int kS>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (kS == 1) {
    return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1, 0, 3, 2]
  } else if constexpr (kS == 2) {
    return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2, 3, 0, 1]
  } else if constexpr (kS == 4 || kS == 8) {
    const uint32_t up = __builtin_amdgcn_update_dpp(0u, v, 0x100 + kS, 0xF, 0xF, false);   // row_shl: lane + kS
    const uint32_t dn = __builtin_amdgcn_update_dpp(0u, v, 0x110 + kS, 0xF, 0xF, false);   // row_shr: lane - kS
    return (threadIdx.x & kS) ? dn : up;
  } else if constexpr (kS == 16) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (16 << 10));   // xor 16 within 32 lanes
  } else {
    return __shfl_xor(v, kS);
  }
}

// One bitonic stage (kSize, kStride) over one composite per lane i of a
// wave: pairs (i, i ^ kStride); segments of kSize alternate in direction,
// so after the last stage (64, 1) the wave's 64 entries are descending.
template <int kSize, int kStride>
__device__ __forceinline__ void wave_bitonic_stage(uint64_t& v) {
  const int i = threadIdx.x & 63;
  const uint32_t lo = lane_xor<kStride>((uint32_t)v);
  const uint32_t hi = lane_xor<kStride>((uint32_t)(v >> 32));
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  const bool keep_max = ((i & kStride) == 0) == ((i & kSize) == 0);
  const uint64_t mx = v > o ? v : o, mn = v > o ? o : v;
  v = keep_max ? mx : mn;
}

// Stages (kSize, kStride), (kSize, kStride / 2), .., then the next sizes up to 64.
template <int kSize, int kStride>
__device__ __forceinline__ void wave_bitonic_from(uint64_t& v) {
  wave_bitonic_stage<kSize, kStride>(v);
  if constexpr (kStride > 1)
    wave_bitonic_from<kSize, kStride / 2>(v);
  else if constexpr (kSize < 64)
    wave_bitonic_from<kSize * 2, kSize>(v);
}

// Number of entries of run[0 .. 64), descending, above v: a binary search.
__device__ __forceinline__ uint32_t count_above(const uint64_t* run, uint64_t v) {
  uint32_t pos = 0;
#pragma unroll
  for (uint32_t st = 32; st >= 1; st >>= 1) pos += run[pos + st - 1] > v ? st : 0u;
  return pos + (run[pos] > v ? 1u : 0u);
}

// 4. Thread i holds pick i (i < n) or 0 (below every pick).  The picks are
// distinct, so each one's place in the output is the number of picks above
// it: each wave sorts its 64 entries (its run), and a pick counts the
// entries above it in every run by binary search (in its own run that is
// its lane).  Picks go to dst[place]; places n .. k-1 get -1.
__device__ __forceinline__ void write_ranked(uint64_t v, uint64_t* runs, int n, int k, int32_t* dst) {
  const int tid = threadIdx.x;
  wave_bitonic_from<2, 1>(v);
  runs[tid] = v;
  __syncthreads();
  uint32_t place = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) place += count_above(runs + 64 * w, v);
  if (v != 0) dst[place] = (int32_t)(0xFFFFFFFFu - (uint32_t)(v & 0xFFFFFFFFu));
  if (tid >= n && tid < k) dst[tid] = -1;
}

// A row of L positions that is cut into parts (L > k and L > kSmallRow):
// part i covers [i c, min(L, (i + 1) c)), c = ceil(L / parts) rounded up
// to a multiple of 4.
__device__ __forceinline__ bool row_in_parts(int L, int k) { return L > k && L > kSmallRow; }
__device__ __forceinline__ int part_len(int L, int parts) { return ((L + parts - 1) / parts + 3) & ~3; }

// Rows cut into parts, one workgroup per (part, row): steps 1-2 over the
// part, with the row's t0, into the part's region of the workspace.  Its
// record in ws_meta: the count (past cap_part: overflowed, nothing
// usable), t0, and the largest key in its list.
__global__ __launch_bounds__(kTopkThreads, 1) void mla_topk_parts_kernel(const TopkParams p) {
  __shared__ TopkSmem sm;
  const int b = blockIdx.x % p.batch, part = blockIdx.x / p.batch, tid = threadIdx.x;
  const int L = min(max(p.seq_lens[(int64_t)b * p.len_s], 0), p.max_len);
  if (!row_in_parts(L, p.k)) return;   // the row is selected whole by mla_topk_kernel
  const float* row = p.scores + (int64_t)b * p.sc_sb;
  const int c = part_len(L, p.parts);
  const int lo = min(L, part * c), n = min(L, lo + c) - lo;
  uint64_t* meta = p.ws_meta + ((int64_t)b * p.parts + part) * 4;
  if (n == 0) {
    if (tid == 0) meta[0] = meta[1] = meta[2] = 0;
    return;
  }
  for (int i = tid; i < kBins; i += kTopkThreads) sm.hist[i] = 0;
  if (tid == 0) {
    sm.n_cand = 0;
    sm.kmax = 0;
  }
  const RowView rv = view_row(row + lo, n, lo);
  f32x4 x0[kUnroll];
  if (rv.nv > 0) load_batch(rv, 0, x0);
  __syncthreads();
  const uint64_t t0 = row_threshold(sm, row, L, p.k);
  compact_above(rv, x0, t0, p.ws_list + ((int64_t)b * p.parts + part) * p.cap_part, &sm.n_cand, p.cap_part,
                &sm.kmax);
  __syncthreads();
  if (tid == 0) {
    meta[0] = sm.n_cand;
    meta[1] = t0;
    meta[2] = sm.kmax;
  }
}

// One workgroup per row: steps 1-3 (or, for a row cut into parts, the
// parts' lists joined into the candidate list, then step 3), then step 4.
__global__ __launch_bounds__(kTopkThreads, 1) void mla_topk_kernel(const TopkParams p) {
  __shared__ TopkSmem sm;
  const int b = blockIdx.x, tid = threadIdx.x;
  const float* row = p.scores + (int64_t)b * p.sc_sb;
  int32_t* dst = p.topk_idx + (int64_t)b * p.idx_sb;
  const int L = min(max(p.seq_lens[(int64_t)b * p.len_s], 0), p.max_len);
  const int k = p.k;
  const int n = min(k, L);

  for (int i = tid; i < kBins; i += kTopkThreads) sm.hist[i] = 0;
  if (tid == 0) {
    sm.n_cand = 0;
    sm.n_sel = 0;
    sm.kmax = 0;
  }
  __syncthreads();
  if (p.parts > 1 && row_in_parts(L, k)) {
    // the parts' records, all requested at once (the same words for every
    // thread); a part past its region, or a total the list cannot hold,
    // sends step 3 to the row
    const uint64_t* meta = p.ws_meta + (int64_t)b * p.parts * 4;
    uint32_t c[kMaxParts], kmax = 0;
#pragma unroll
    for (int i = 0; i < kMaxParts; ++i) {
      c[i] = i < p.parts ? (uint32_t)min(meta[4 * i], (uint64_t)0xFFFFFFFFu) : 0u;
      kmax = max(kmax, i < p.parts ? (uint32_t)meta[4 * i + 2] : 0u);
    }
    const uint64_t t0 = meta[1];   // part 0 (never empty) holds the row's t0
    // list entry f of the joined list is workspace entry f + gap[i] of the
    // row's lists, i the part holding f: gap[i] = i * cap_part - (entries
    // of the parts before i)
    uint32_t total = 0, start[kMaxParts], gap[kMaxParts];
    bool over = false;
#pragma unroll
    for (int i = 0; i < kMaxParts; ++i) {
      start[i] = total;
      gap[i] = (uint32_t)(i * p.cap_part) - total;
      over |= c[i] > (uint32_t)p.cap_part;
      total += c[i];
    }
    if (over || total > (uint32_t)kCand) {
      total = kCand + 1;
    } else if (total >= (uint32_t)k) {
      const uint64_t* src = p.ws_list + (int64_t)b * p.parts * p.cap_part;
      constexpr int kJ = 8;   // loads in flight per thread
      for (uint32_t f0 = 0; f0 < total; f0 += kJ * kTopkThreads) {
        uint64_t v[kJ];
#pragma unroll
        for (int u = 0; u < kJ; ++u) {
          const uint32_t f = f0 + u * kTopkThreads + tid;
          uint32_t g = 0;
#pragma unroll
          for (int i = 1; i < kMaxParts; ++i) g = (i < p.parts && f >= start[i]) ? gap[i] : g;
          v[u] = src[f < total ? f + g : 0];
        }
#pragma unroll
        for (int u = 0; u < kJ; ++u) {
          const uint32_t f = f0 + u * kTopkThreads + tid;
          if (f < total) sm.cand[f] = v[u];
        }
      }
    }
    if (tid == 0) {
      sm.n_cand = total;
      sm.kmax = kmax;
    }
    __syncthreads();
    select_picks(sm, view_row(row, L), k, t0);
  } else if (L > 0) {
    select_row(sm, view_row(row, L), k);
  }

  // 4. the n picks (exactly n were appended) in rank order; the candidate
  // list is free by now and holds the sorted runs
  write_ranked(tid < n ? sm.sel[tid] : 0ull, sm.cand, n, k, dst);
}

}  // namespace

size_t topk_workspace_bytes(int32_t batch, int32_t parts) {
  if (parts <= 1) return 0;
  const size_t cap = (size_t)(kCand / parts);
  return (size_t)batch * parts * (cap + 4) * sizeof(uint64_t);
}

hipError_t launch_topk(TopkParams p, void* ws, hipStream_t stream) {
  if (p.parts > 1) {
    p.cap_part = kCand / p.parts;
    p.ws_list = (uint64_t*)ws;
    p.ws_meta = p.ws_list + (size_t)p.batch * p.parts * p.cap_part;
    hipLaunchKernelGGL(mla_topk_parts_kernel, dim3(p.batch * p.parts), dim3(kTopkThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(mla_topk_kernel, dim3(p.batch), dim3(kTopkThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mlasd
