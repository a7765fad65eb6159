// C-ABI entry points: argument validation, split planning, scratch, launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "../../include/mlasd.h"
#include "mlasd_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return MLASD_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Compute-unit count of the current device, cached per device id.
int device_cus(int* cus) {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= 64) return MLASD_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e);
    if (std::string(prop.gcnArchName).rfind("gfx950", 0) != 0) return MLASD_ERR_DEVICE;
    cache[dev] = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  }
  *cus = cache[dev];
  return MLASD_OK;
}

// Split scratch: one buffer per (device, stream) for the fp32 partials of
// the slices, grown on demand and kept for the life of the process.
// Growing synchronises the stream and frees the old buffer, so it is refused
// while the stream is capturing: a first call with the largest shape outside
// capture sizes it.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

int stream_workspace(hipStream_t stream, size_t bytes, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lock(g_ws_mu);
  Workspace& w = g_ws[{dev, stream}];
  if (w.bytes < bytes) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_fail(e);
    if (cs != hipStreamCaptureStatusNone) return MLASD_ERR_CAPTURE;
    if (w.ptr) {
      e = hipStreamSynchronize(stream);
      if (e != hipSuccess) return hip_fail(e);
      e = hipFree(w.ptr);
      if (e != hipSuccess) return hip_fail(e);
      w.ptr = nullptr;
      w.bytes = 0;
    }
    const size_t want = (bytes + (1u << 20) - 1) & ~(size_t)((1u << 20) - 1);
    e = hipMalloc(&w.ptr, want);
    if (e != hipSuccess) return hip_fail(e);
    w.bytes = want;
  }
  *out = w.ptr;
  return MLASD_OK;
}

// Plan: one workgroup per (query, top-k slice, head group).  Without a
// request the workgroups of a query are floor(cus / batch), so one round of
// workgroups covers the GPU:
//   - two head groups of 32 heads whenever batch * nsplit * 2 fits the CUs:
//     a 32-head workgroup reads each LDS tile with two head-group waves
//     instead of four and loads half of Q, and its sibling shares the
//     gathered records through L2 (measured: c1 12.8 -> 11.2 us, c2 15.6 ->
//     13.9 us, c3 with 2 slices of 32-head groups 23.8 us against 24.9 us
//     with 4 slices of 64 heads);
//   - four head groups of 16 heads instead when a query gets at least 16
//     workgroups (batch <= cus / 16), and for forced slice counts when
//     batch * nsplit * 4 still leaves three quarters of the CUs idle: fewer
//     slices then means fewer fp32 partials to write and merge (measured at
//     topk 512: B=16 with (4 slices, 4 groups) 12.8 us against 13.2 us with
//     (8, 2); B=4 10.6 against 11.1 us; but B=32 prefers (4, 2) 15.5 us over
//     (2, 4) 17.0 us and B=48 (2, 2) 18.8 us over (1, 4) 20.0 us, where a
//     16-head workgroup has too many tiles to walk alone);
//   - four head groups and no split when they alone fill the GPU (4 * batch
//     above 7/8 of the CUs, B = 57..64 on 256): the longer tile walk then costs
//     less than the split's fp32 partials and combine launch (B=64, 65,536-
//     token sequences: 20.4 us against 20.7-20.9 us for (2, 2), and 62.8 ->
//     ~33 MB of HBM traffic per step; B=56: (2, 2) 19.5 us against 20.0 us);
//   - the rest of the budget in top-k slices, none cut below kMinAutoSlice
//     entries: every extra slice costs a partial write and read, and below
//     two tiles a workgroup's fixed start-up cost (index resolution, first
//     gather) dominates.
// A slice holds a whole number of 32-token tiles.
constexpr int kMinAutoSlice = 64;

void make_plan(int32_t batch, int32_t topk, int32_t ns_request, int32_t hg_request, int cus,
               int32_t* nsplit, int32_t* split_len, int32_t* head_groups) {
  const int tile = mlasd::kTileTokens;
  const int max_split = topk > 0 ? (topk + tile - 1) / tile : 1;
  const int per_query = batch > 0 ? cus / batch : cus;   // workgroups per query in one round
  const bool fill_by_groups = ns_request <= 0 && per_query == 4 && (int64_t)batch * 4 * 8 > (int64_t)cus * 7;
  const bool four_groups = ns_request <= 0 && (per_query >= 16 || fill_by_groups);
  int ns;
  if (ns_request > 0) {
    ns = ns_request;
  } else {
    ns = four_groups ? per_query / 4 : per_query >= 2 ? per_query / 2 : 1;   // fill_by_groups: 1
    const int by_len = topk > 0 ? (topk + kMinAutoSlice - 1) / kMinAutoSlice : 1;
    if (ns > by_len) ns = by_len;
  }
  if (ns > max_split) ns = max_split;
  if (ns < 1) ns = 1;
  int len = topk > 0 ? (topk + ns - 1) / ns : tile;
  len = (len + tile - 1) / tile * tile;
  ns = topk > 0 ? (topk + len - 1) / len : 1;
  *nsplit = ns;
  *split_len = len;
  if (hg_request > 0)
    *head_groups = hg_request;
  else if (four_groups || (int64_t)batch * ns * 4 <= cus / 4)
    *head_groups = 4;
  else
    *head_groups = (int64_t)batch * ns * 2 <= cus ? 2 : 1;
}

// Bytes of split scratch for one call: fp32 partial rows, then fp32 lse values.
size_t split_scratch_bytes(int32_t batch, int32_t nsplit) {
  const size_t n_o = (size_t)batch * nsplit * mlasd::kHeads * mlasd::kDV;
  const size_t n_l = (size_t)batch * nsplit * mlasd::kHeads;
  return (n_o + n_l) * sizeof(float);
}

int check_common(const void* kv, int64_t num_pages, const int32_t* page_table, int32_t max_pages,
                 const int32_t* topk_idx, int32_t topk, const int32_t* seq_lens, int32_t batch) {
  if (batch < 0 || topk < 0 || topk > MLASD_MAX_TOPK) return MLASD_ERR_SHAPE;
  if (batch == 0) return MLASD_OK;
  if (num_pages < 1 || max_pages < 1) return MLASD_ERR_SHAPE;
  if (!kv || !page_table || !seq_lens) return MLASD_ERR_NULL;
  if (topk > 0 && !topk_idx) return MLASD_ERR_NULL;
  if (!aligned(kv, 16) || !aligned(page_table, 4) || !aligned(seq_lens, 4) ||
      (topk_idx && !aligned(topk_idx, 4)))
    return MLASD_ERR_ALIGN;
  return MLASD_OK;
}

int decode_impl(const void* q, const void* kv_pages, int64_t num_pages, const int32_t* page_table,
                int32_t max_pages, const int32_t* topk_idx, int32_t topk, const int32_t* seq_lens,
                int32_t batch, float softmax_scale, void* out, float* lse, int32_t nsplit_req,
                int32_t hg_req, hipStream_t stream) {
  int rc = check_common(kv_pages, num_pages, page_table, max_pages, topk_idx, topk, seq_lens, batch);
  if (rc != MLASD_OK) return rc;
  if (!std::isfinite(softmax_scale)) return MLASD_ERR_VALUE;
  if (hg_req < 0 || hg_req > 4 || hg_req == 3) return MLASD_ERR_SHAPE;
  if (batch == 0) return MLASD_OK;
  if (!q || !out || !lse) return MLASD_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 8) || !aligned(lse, 4)) return MLASD_ERR_ALIGN;
  int cus = 0;
  rc = device_cus(&cus);
  if (rc != MLASD_OK) return rc;

  mlasd::DecodeParams p{};
  p.q = (const uint16_t*)q;
  p.kv = (const uint8_t*)kv_pages;
  p.num_pages = num_pages;
  p.page_table = page_table;
  p.max_pages = max_pages;
  p.topk_idx = topk_idx;
  p.topk = topk;
  p.seq_lens = seq_lens;
  p.batch = batch;
  p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  p.out = (uint16_t*)out;
  p.lse = lse;
  make_plan(batch, topk, nsplit_req, hg_req, cus, &p.nsplit, &p.split_len, &p.head_groups);

  if (p.nsplit > 1) {
    const size_t n_o = (size_t)batch * p.nsplit * mlasd::kHeads * mlasd::kDV;
    void* scratch = nullptr;
    rc = stream_workspace(stream, split_scratch_bytes(batch, p.nsplit), &scratch);
    if (rc != MLASD_OK) return rc;
    p.part_o = (float*)scratch;
    p.part_lse = (float*)scratch + n_o;
  }
  hipError_t e = mlasd::launch_decode(p, stream);
  if (e == hipSuccess && p.nsplit > 1) e = mlasd::launch_combine(p, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MLASD_OK;
}

}  // namespace

extern "C" {

int mla_sparse_decode(const void* q, const void* kv_pages, int64_t num_pages,
                      const int32_t* page_table, int32_t max_pages, const int32_t* topk_idx,
                      int32_t topk, const int32_t* seq_lens, int32_t batch, float softmax_scale,
                      void* out, float* lse, mlasd_stream_t stream) {
  return decode_impl(q, kv_pages, num_pages, page_table, max_pages, topk_idx, topk, seq_lens, batch,
                     softmax_scale, out, lse, 0, 0, (hipStream_t)stream);
}

int mla_sparse_decode_ex(const void* q, const void* kv_pages, int64_t num_pages,
                         const int32_t* page_table, int32_t max_pages, const int32_t* topk_idx,
                         int32_t topk, const int32_t* seq_lens, int32_t batch, float softmax_scale,
                         void* out, float* lse, int32_t nsplit, int32_t head_groups,
                         mlasd_stream_t stream) {
  return decode_impl(q, kv_pages, num_pages, page_table, max_pages, topk_idx, topk, seq_lens, batch,
                     softmax_scale, out, lse, nsplit, head_groups, (hipStream_t)stream);
}

int mla_sparse_plan(int32_t batch, int32_t topk, int32_t nsplit_request, int32_t num_cus,
                    int32_t* nsplit, int32_t* split_len, int32_t* head_groups) {
  if (!nsplit || !split_len) return MLASD_ERR_NULL;
  if (batch < 0 || topk < 0 || topk > MLASD_MAX_TOPK) return MLASD_ERR_SHAPE;
  int cus = num_cus;
  if (cus <= 0) {
    int rc = device_cus(&cus);
    if (rc != MLASD_OK) return rc;
  }
  int32_t hg = 1;
  make_plan(batch, topk, nsplit_request, 0, cus, nsplit, split_len, &hg);
  if (head_groups) *head_groups = hg;
  return MLASD_OK;
}

int mla_sparse_gather_dequant(const void* kv_pages, int64_t num_pages, const int32_t* page_table,
                              int32_t max_pages, const int32_t* topk_idx, int32_t topk,
                              const int32_t* seq_lens, int32_t batch, void* k_rows, void* v_rows,
                              uint8_t* valid, mlasd_stream_t stream) {
  int rc = check_common(kv_pages, num_pages, page_table, max_pages, topk_idx, topk, seq_lens, batch);
  if (rc != MLASD_OK) return rc;
  if (batch == 0 || topk == 0) return MLASD_OK;
  if (!k_rows || !v_rows || !valid) return MLASD_ERR_NULL;
  if (!aligned(k_rows, 16) || !aligned(v_rows, 16)) return MLASD_ERR_ALIGN;
  int cus = 0;
  rc = device_cus(&cus);
  if (rc != MLASD_OK) return rc;
  mlasd::GatherParams p{};
  p.kv = (const uint8_t*)kv_pages;
  p.num_pages = num_pages;
  p.page_table = page_table;
  p.max_pages = max_pages;
  p.topk_idx = topk_idx;
  p.topk = topk;
  p.seq_lens = seq_lens;
  p.batch = batch;
  p.k_rows = (uint16_t*)k_rows;
  p.v_rows = (uint16_t*)v_rows;
  p.valid = valid;
  int32_t hg_unused = 1;
  make_plan(batch, topk, 0, 0, cus, &p.nsplit, &p.split_len, &hg_unused);
  hipError_t e = mlasd::launch_gather(p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e);
  return MLASD_OK;
}

int mla_kv_append(const void* latent, const int32_t* seq_ids, const int32_t* positions,
                  int32_t n_tokens, const int32_t* page_table, int32_t batch, int32_t max_pages,
                  void* kv_pages, int64_t num_pages, mlasd_stream_t stream) {
  if (n_tokens < 0 || batch < 0) return MLASD_ERR_SHAPE;
  if (n_tokens == 0) return MLASD_OK;
  if (batch < 1 || max_pages < 1 || num_pages < 1) return MLASD_ERR_SHAPE;
  if (!latent || !seq_ids || !positions || !page_table || !kv_pages) return MLASD_ERR_NULL;
  if (!aligned(latent, 16) || !aligned(kv_pages, 16) || !aligned(seq_ids, 4) || !aligned(positions, 4) ||
      !aligned(page_table, 4))
    return MLASD_ERR_ALIGN;
  int cus = 0;
  int rc = device_cus(&cus);
  if (rc != MLASD_OK) return rc;
  mlasd::AppendParams p{};
  p.latent = (const uint16_t*)latent;
  p.seq_ids = seq_ids;
  p.positions = positions;
  p.n_tokens = n_tokens;
  p.page_table = page_table;
  p.batch = batch;
  p.max_pages = max_pages;
  p.kv = (uint8_t*)kv_pages;
  p.num_pages = num_pages;
  hipError_t e = mlasd::launch_append(p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e);
  return MLASD_OK;
}

int mlasd_prepare(mlasd_stream_t stream_, int32_t max_batch, int32_t max_topk) {
  if (max_batch < 0 || max_topk < 0 || max_topk > MLASD_MAX_TOPK) return MLASD_ERR_SHAPE;
  int cus = 0;
  int rc = device_cus(&cus);
  if (rc != MLASD_OK) return rc;
  // The automatic plan's slice count grows with topk, so planning at
  // max_topk for every batch size up to max_batch bounds every call.
  size_t need = 0;
  for (int32_t b = 1; b <= max_batch; ++b) {
    int32_t ns = 1, len = 0, hg = 1;
    make_plan(b, max_topk, 0, 0, cus, &ns, &len, &hg);
    if (ns > 1 && split_scratch_bytes(b, ns) > need) need = split_scratch_bytes(b, ns);
  }
  if (need == 0) return MLASD_OK;
  void* scratch = nullptr;
  return stream_workspace((hipStream_t)stream_, need, &scratch);
}

int mlasd_release(mlasd_stream_t stream_) {
  hipStream_t stream = (hipStream_t)stream_;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lock(g_ws_mu);
  auto it = g_ws.find({dev, stream});
  if (it == g_ws.end() || it->second.ptr == nullptr) return MLASD_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return hip_fail(e);
  if (cs != hipStreamCaptureStatusNone) return MLASD_ERR_CAPTURE;
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e);
  e = hipFree(it->second.ptr);
  g_ws.erase(it);
  if (e != hipSuccess) return hip_fail(e);
  return MLASD_OK;
}

int mlasd_workspace_bytes(mlasd_stream_t stream_, size_t* bytes) {
  if (bytes == nullptr) return MLASD_ERR_NULL;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lock(g_ws_mu);
  auto it = g_ws.find({dev, (hipStream_t)stream_});
  *bytes = it == g_ws.end() ? 0 : it->second.bytes;
  return MLASD_OK;
}

const char* mlasd_status_string(int status) {
  switch (status) {
    case MLASD_OK: return "ok";
    case MLASD_ERR_NULL: return "null pointer argument";
    case MLASD_ERR_SHAPE: return "size out of range";
    case MLASD_ERR_ALIGN: return "misaligned pointer";
    case MLASD_ERR_VALUE: return "invalid scalar argument";
    case MLASD_ERR_HIP: return "HIP runtime error";
    case MLASD_ERR_DEVICE: return "current device is not gfx950";
    case MLASD_ERR_CAPTURE: return "split scratch would have to grow while the stream is capturing";
    default: return "unknown status";
  }
}

int mlasd_last_hip_error(void) { return g_last_hip_error; }

const char* mlasd_version(void) { return "mlasd 0.1.0 (gfx950)"; }

}  // extern "C"
