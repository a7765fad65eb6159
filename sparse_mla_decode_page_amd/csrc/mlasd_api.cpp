// C-ABI entry points: descriptor validation, split planning, split scratch,
// launches.  No compute entry point allocates or synchronises: split scratch
// is created only by mlasd_prepare / mlasd_reserve and freed only by
// mlasd_release.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/mlasd.h"
#include "mlasd_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return MLASD_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Compute-unit count of the current device, cached per device id; refuses
// devices other than gfx950.
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

// ---------------------------------------------------------------------------
// tensor descriptors
// ---------------------------------------------------------------------------

// Checks dtype, rank, shape (want[k] >= 0 fixes dim k; -1 leaves it free)
// and, if `inner_contiguous`, that the innermost dim has stride 1.  A NULL
// descriptor or data pointer is MLASD_ERR_NULL unless the tensor is empty
// and `empty_ok`.
int check_tensor(const mlasd_tensor* t, int dtype, int ndim, const int64_t* want, bool empty_ok,
                 bool inner_contiguous = true) {
  if (t == nullptr) return MLASD_ERR_NULL;
  if (t->dtype != dtype || t->ndim != ndim) return MLASD_ERR_SHAPE;
  int64_t n = 1;
  for (int k = 0; k < ndim; ++k) {
    if (t->shape[k] < 0 || t->stride[k] < 0) return MLASD_ERR_SHAPE;
    if (want[k] >= 0 && t->shape[k] != want[k]) return MLASD_ERR_SHAPE;
    n *= t->shape[k];
  }
  if (inner_contiguous && n > 0 && t->shape[ndim - 1] > 1 && t->stride[ndim - 1] != 1) return MLASD_ERR_SHAPE;
  if (t->data == nullptr && !(empty_ok && n == 0)) return MLASD_ERR_NULL;
  return MLASD_OK;
}

// Element strides that must keep 16-byte vector accesses aligned.
bool strides_multiple(const mlasd_tensor* t, int upto, int64_t m) {
  for (int k = 0; k < upto; ++k)
    if (t->stride[k] % m != 0) return false;
  return true;
}

// Cache-side tensors shared by the decode, the gather hook and the append.
struct Cache {
  const uint8_t* kv;
  int64_t num_pages, page_stride;
  const int32_t* pt;
  int64_t pt_sb;
  int32_t batch, max_pages;
};

int check_pool(const mlasd_tensor* kv, Cache* c) {
  const int64_t want[2] = {-1, MLASD_PAGE_BYTES};
  int rc = check_tensor(kv, MLASD_U8, 2, want, false);
  if (rc != MLASD_OK) return rc;
  if (kv->shape[0] < 1 || kv->stride[1] != 1 || kv->stride[0] < MLASD_PAGE_BYTES) return MLASD_ERR_SHAPE;
  if (!aligned(kv->data, 16) || kv->stride[0] % 16 != 0) return MLASD_ERR_ALIGN;
  c->kv = (const uint8_t*)kv->data;
  c->num_pages = kv->shape[0];
  c->page_stride = kv->stride[0];
  return MLASD_OK;
}

int check_page_table(const mlasd_tensor* pt, int64_t batch, Cache* c) {
  const int64_t want[2] = {batch, -1};
  int rc = check_tensor(pt, MLASD_I32, 2, want, false);
  if (rc != MLASD_OK) return rc;
  if (pt->shape[1] < 1 || pt->shape[1] > INT32_MAX || pt->stride[1] != 1) return MLASD_ERR_SHAPE;
  if (!aligned(pt->data, 4)) return MLASD_ERR_ALIGN;
  c->pt = (const int32_t*)pt->data;
  c->pt_sb = pt->stride[0];
  c->max_pages = (int32_t)pt->shape[1];
  return MLASD_OK;
}

// kv_pages, page_table, topk_idx, seq_lens of a decode-shaped call.
struct Selection {
  Cache cache;
  const int32_t* idx;
  int64_t idx_sb;
  int32_t topk;
  const int32_t* lens;
  int64_t len_s;
};

int check_selection(const mlasd_tensor* kv, const mlasd_tensor* pt, const mlasd_tensor* idx,
                    const mlasd_tensor* lens, Selection* s) {
  if (lens == nullptr || idx == nullptr || pt == nullptr || kv == nullptr) return MLASD_ERR_NULL;
  if (lens->ndim != 1 || lens->shape[0] < 0 || lens->shape[0] > INT32_MAX) return MLASD_ERR_SHAPE;
  const int64_t B = lens->shape[0];
  const int64_t wl[1] = {B};
  int rc = check_tensor(lens, MLASD_I32, 1, wl, true, false);
  if (rc != MLASD_OK) return rc;
  const int64_t wi[2] = {B, -1};
  rc = check_tensor(idx, MLASD_I32, 2, wi, true);
  if (rc != MLASD_OK) return rc;
  if (idx->shape[1] > MLASD_MAX_TOPK) return MLASD_ERR_SHAPE;
  s->cache.batch = (int32_t)B;
  s->topk = (int32_t)idx->shape[1];
  if (B == 0) return MLASD_OK;
  rc = check_pool(kv, &s->cache);
  if (rc != MLASD_OK) return rc;
  rc = check_page_table(pt, B, &s->cache);
  if (rc != MLASD_OK) return rc;
  if (!aligned(lens->data, 4) || (idx->data && !aligned(idx->data, 4))) return MLASD_ERR_ALIGN;
  s->idx = (const int32_t*)idx->data;
  s->idx_sb = idx->stride[0];
  s->lens = (const int32_t*)lens->data;
  s->len_s = lens->stride[0];
  return MLASD_OK;
}

// ---------------------------------------------------------------------------
// split scratch: one live buffer per (device, stream) plus the buffers it
// superseded, all kept until mlasd_release
// ---------------------------------------------------------------------------

struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
  std::vector<void*> retired;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

int current_device(int* dev) {
  hipError_t e = hipGetDevice(dev);
  return e == hipSuccess ? MLASD_OK : hip_fail(e);
}

// The stream's usable scratch, or (nullptr, 0).  Never allocates.
void lookup_workspace(int dev, hipStream_t stream, void** ptr, size_t* bytes) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  auto it = g_ws.find({dev, stream});
  *ptr = it == g_ws.end() ? nullptr : it->second.ptr;
  *bytes = it == g_ws.end() ? 0 : it->second.bytes;
}

int capturing(hipStream_t stream, bool* yes) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return hip_fail(e);
  *yes = cs != hipStreamCaptureStatusNone;
  return MLASD_OK;
}

int reserve_workspace(hipStream_t stream, size_t bytes) {
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != MLASD_OK) return rc;
  bool cap = false;
  rc = capturing(stream, &cap);
  if (rc != MLASD_OK) return rc;
  if (cap) return MLASD_ERR_CAPTURE;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  Workspace& w = g_ws[{dev, stream}];
  if (w.bytes >= bytes) return MLASD_OK;
  const size_t want = (bytes + (1u << 20) - 1) & ~(size_t)((1u << 20) - 1);
  void* p = nullptr;
  hipError_t e = hipMalloc(&p, want);
  if (e != hipSuccess) return hip_fail(e);
  // zeroed once, so any per-query counters kept in the scratch start at 0
  e = hipMemset(p, 0, want);
  if (e != hipSuccess) {
    (void)hipFree(p);
    return hip_fail(e);
  }
  if (w.ptr) w.retired.push_back(w.ptr);   // graphs captured earlier may still use it
  w.ptr = p;
  w.bytes = want;
  return MLASD_OK;
}

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------

// Plan: one workgroup per (query, top-k slice, head group of 32 or 64
// heads).  Without a request a query gets floor(cus / batch) workgroups, so
// one round of workgroups covers the GPU: two head groups of 32 heads when
// it gets at least two (a 32-head workgroup runs one Q K^T wave and its
// sibling reads the gathered records from L2), the rest in top-k slices of at
// least kMinAutoSlice entries (each extra slice costs an fp32 partial write
// and read, and below two tiles a workgroup's fixed start-up cost
// dominates).  A slice holds a whole number of 32-token tiles.  The split is
// then kept only if the tiles it takes off each workgroup pay for the
// combine launch and the added workgroups: measured on 256 CUs, a tile costs
// a workgroup about 0.95 us and a split about 2.5 us + 0.035 us per (query x
// slice) (split against unsplit for B = 1..64 and top-k 128..512).
constexpr int kMinAutoSlice = 64;
constexpr int64_t kTileNs = 950;             // per tile of a workgroup's slice
constexpr int64_t kSplitNs = 2500;           // a split: fixed part
constexpr int64_t kSplitNsPerSlice = 35;     //          per (query x slice)

void make_plan(int32_t batch, int32_t topk, int32_t ns_request, int32_t hg_request, int cus,
               int32_t* nsplit, int32_t* split_len, int32_t* head_groups) {
  const int tile = mlasd::kTileTokens;
  const int max_split = topk > 0 ? (topk + tile - 1) / tile : 1;
  const int per_query = batch > 0 ? cus / batch : cus;   // workgroups per query in one round
  const int hg = hg_request > 0 ? hg_request : (per_query >= 2 ? 2 : 1);
  int ns;
  if (ns_request > 0) {
    ns = ns_request;
  } else {
    ns = per_query / hg;
    const int by_len = topk > 0 ? (topk + kMinAutoSlice - 1) / kMinAutoSlice : 1;
    if (ns > by_len) ns = by_len;
  }
  if (ns > max_split) ns = max_split;
  if (ns < 1) ns = 1;
  int len = topk > 0 ? (topk + ns - 1) / ns : tile;
  len = (len + tile - 1) / tile * tile;
  ns = topk > 0 ? (topk + len - 1) / len : 1;
  if (ns_request <= 0 && ns > 1) {
    const int64_t saved = max_split - len / tile;   // tiles taken off each workgroup
    if (saved * kTileNs <= kSplitNs + kSplitNsPerSlice * (int64_t)batch * ns) {
      ns = 1;
      len = (topk + tile - 1) / tile * tile;
    }
  }
  *nsplit = ns;
  *split_len = len;
  *head_groups = hg;
}

// Bytes of split scratch for one call: fp32 partial rows, then fp32 lse values.
size_t split_scratch_bytes(int32_t batch, int32_t nsplit) {
  if (nsplit <= 1) return 0;
  const size_t n_o = (size_t)batch * nsplit * mlasd::kHeads * mlasd::kDV;
  const size_t n_l = (size_t)batch * nsplit * mlasd::kHeads;
  return (n_o + n_l) * sizeof(float);
}

bool valid_head_groups(int32_t hg) { return hg >= 0 && hg <= 2; }

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------

// Validated decode arguments.
struct DecodeCall {
  mlasd::DecodeParams p{};
  int cus = 0;
};

int prepare_decode(const mlasd_tensor* q, const mlasd_tensor* kv, const mlasd_tensor* pt,
                   const mlasd_tensor* idx, const mlasd_tensor* lens, float softmax_scale,
                   const mlasd_tensor* out, const mlasd_tensor* lse, int32_t ns_req, int32_t hg_req,
                   DecodeCall* call) {
  Selection s{};
  int rc = check_selection(kv, pt, idx, lens, &s);
  if (rc != MLASD_OK) return rc;
  if (!std::isfinite(softmax_scale)) return MLASD_ERR_VALUE;
  if (!valid_head_groups(hg_req)) return MLASD_ERR_SHAPE;
  const int64_t B = s.cache.batch;
  const int64_t wq[3] = {B, MLASD_HEADS, MLASD_D_QK};
  rc = check_tensor(q, MLASD_BF16, 3, wq, true);
  if (rc != MLASD_OK) return rc;
  const int64_t wo[3] = {B, MLASD_HEADS, MLASD_D_V};
  rc = check_tensor(out, MLASD_BF16, 3, wo, true);
  if (rc != MLASD_OK) return rc;
  const int64_t wl[2] = {B, MLASD_HEADS};
  rc = check_tensor(lse, MLASD_F32, 2, wl, true);
  if (rc != MLASD_OK) return rc;
  if (B == 0) return MLASD_OK;
  if (!aligned(q->data, 16) || !strides_multiple(q, 2, 8) || !aligned(out->data, 16) ||
      !strides_multiple(out, 2, 8) || !aligned(lse->data, 4))
    return MLASD_ERR_ALIGN;
  rc = device_cus(&call->cus);
  if (rc != MLASD_OK) return rc;

  mlasd::DecodeParams& p = call->p;
  p.q = (const uint16_t*)q->data;
  p.q_sb = q->stride[0];
  p.q_sh = q->stride[1];
  p.kv = s.cache.kv;
  p.num_pages = s.cache.num_pages;
  p.page_stride = s.cache.page_stride;
  p.page_table = s.cache.pt;
  p.pt_sb = s.cache.pt_sb;
  p.max_pages = s.cache.max_pages;
  p.topk_idx = s.idx;
  p.idx_sb = s.idx_sb;
  p.topk = s.topk;
  p.seq_lens = s.lens;
  p.len_s = s.len_s;
  p.batch = (int32_t)B;
  p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  p.out = (uint16_t*)out->data;
  p.out_sb = out->stride[0];
  p.out_sh = out->stride[1];
  p.lse = (float*)lse->data;
  p.lse_sb = lse->stride[0];
  make_plan(p.batch, p.topk, ns_req, hg_req, call->cus, &p.nsplit, &p.split_len, &p.head_groups);
  return MLASD_OK;
}

// Enqueue a validated decode with split scratch `ws` of `ws_bytes`.
int launch_decode_call(DecodeCall& call, void* ws, size_t ws_bytes, hipStream_t stream) {
  mlasd::DecodeParams& p = call.p;
  if (p.batch == 0) return MLASD_OK;
  if (p.nsplit > 1) {
    if (ws == nullptr || ws_bytes < split_scratch_bytes(p.batch, p.nsplit)) return MLASD_ERR_WORKSPACE;
    const size_t n_o = (size_t)p.batch * p.nsplit * mlasd::kHeads * mlasd::kDV;
    p.part_o = (float*)ws;
    p.part_lse = (float*)ws + n_o;
  }
  hipError_t e = mlasd::launch_decode(p, stream);
  if (e == hipSuccess && p.nsplit > 1) e = mlasd::launch_combine(p, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MLASD_OK;
}

int decode_impl(const mlasd_tensor* q, const mlasd_tensor* kv, const mlasd_tensor* pt,
                const mlasd_tensor* idx, const mlasd_tensor* lens, float scale, const mlasd_tensor* out,
                const mlasd_tensor* lse, int32_t ns_req, int32_t hg_req, hipStream_t stream) {
  DecodeCall call;
  int rc = prepare_decode(q, kv, pt, idx, lens, scale, out, lse, ns_req, hg_req, &call);
  if (rc != MLASD_OK || call.p.batch == 0) return rc;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (call.p.nsplit > 1) {
    int dev = 0;
    rc = current_device(&dev);
    if (rc != MLASD_OK) return rc;
    lookup_workspace(dev, stream, &ws, &ws_bytes);
  }
  return launch_decode_call(call, ws, ws_bytes, stream);
}

// Top-k plan: when every row can have at least kTopkMinParts compute units,
// rows of max_len >= kTopkMinParts * kTopkPartLen positions are cut into
// parts of at least kTopkPartLen positions, one workgroup each, for the
// candidate pass (a pass over a row is bound by the loads one workgroup
// keeps in flight); one workgroup per row then selects and sorts.  The
// second launch, the sampled threshold every part repeats and the join
// cost about as much as two parts save: on 256 CUs 2 parts measured slower
// than one workgroup per row at every shape tried, 4 and 8 faster.
constexpr int kTopkMaxParts = 8;
constexpr int kTopkMinParts = 4;
constexpr int kTopkPartLen = 16384;

int topk_parts(int32_t batch, int32_t max_len, int cus) {
  if (batch <= 0) return 1;
  const int parts = std::min({kTopkMaxParts, cus / batch, max_len / kTopkPartLen});
  return parts >= kTopkMinParts ? parts : 1;
}

int topk_impl(const mlasd_tensor* scores, const mlasd_tensor* seq_lens, const mlasd_tensor* topk_idx,
              int32_t parts_request, hipStream_t stream) {
  if (scores == nullptr || topk_idx == nullptr) return MLASD_ERR_NULL;
  if (scores->ndim != 2 || scores->shape[0] < 0 || scores->shape[0] > INT32_MAX || scores->shape[1] > INT32_MAX)
    return MLASD_ERR_SHAPE;
  const int64_t B = scores->shape[0];
  const int64_t wsc[2] = {B, -1};
  int rc = check_tensor(scores, MLASD_F32, 2, wsc, true);
  if (rc != MLASD_OK) return rc;
  const int64_t wl[1] = {B};
  rc = check_tensor(seq_lens, MLASD_I32, 1, wl, true, false);
  if (rc != MLASD_OK) return rc;
  if (topk_idx->ndim != 2 || topk_idx->shape[1] < 0 || topk_idx->shape[1] > MLASD_MAX_TOPK) return MLASD_ERR_SHAPE;
  const int64_t wi[2] = {B, -1};
  rc = check_tensor(topk_idx, MLASD_I32, 2, wi, true);
  if (rc != MLASD_OK) return rc;
  if (parts_request > kTopkMaxParts) return MLASD_ERR_SHAPE;
  if (B == 0 || topk_idx->shape[1] == 0) return MLASD_OK;
  if (!aligned(scores->data, 4) || !aligned(seq_lens->data, 4) || !aligned(topk_idx->data, 4)) return MLASD_ERR_ALIGN;
  int cus = 0;
  rc = device_cus(&cus);
  if (rc != MLASD_OK) return rc;
  mlasd::TopkParams p{};
  p.scores = (const float*)scores->data;
  p.sc_sb = scores->stride[0];
  p.max_len = (int32_t)scores->shape[1];
  p.seq_lens = (const int32_t*)seq_lens->data;
  p.len_s = seq_lens->stride[0];
  p.batch = (int32_t)B;
  p.topk_idx = (int32_t*)topk_idx->data;
  p.idx_sb = topk_idx->stride[0];
  p.k = (int32_t)topk_idx->shape[1];
  p.parts = parts_request > 0 ? parts_request : topk_parts(p.batch, p.max_len, cus);
  void* ws = nullptr;
  if (p.parts > 1) {
    int dev = 0;
    rc = current_device(&dev);
    if (rc != MLASD_OK) return rc;
    size_t ws_bytes = 0;
    lookup_workspace(dev, stream, &ws, &ws_bytes);
    if (ws == nullptr || ws_bytes < mlasd::topk_workspace_bytes(p.batch, p.parts)) {
      if (parts_request > 0) return MLASD_ERR_WORKSPACE;
      p.parts = 1;   // automatic plan without the stream's scratch: one workgroup per row
      ws = nullptr;
    }
  }
  hipError_t e = mlasd::launch_topk(p, ws, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MLASD_OK;
}

}  // namespace

extern "C" {

int mla_sparse_decode(const mlasd_tensor* q, const mlasd_tensor* kv_pages, const mlasd_tensor* page_table,
                      const mlasd_tensor* topk_idx, const mlasd_tensor* seq_lens, float softmax_scale,
                      const mlasd_tensor* out, const mlasd_tensor* lse, mlasd_stream_t stream) {
  return decode_impl(q, kv_pages, page_table, topk_idx, seq_lens, softmax_scale, out, lse, 0, 0,
                     (hipStream_t)stream);
}

int mla_sparse_decode_ex(const mlasd_tensor* q, const mlasd_tensor* kv_pages, const mlasd_tensor* page_table,
                         const mlasd_tensor* topk_idx, const mlasd_tensor* seq_lens, float softmax_scale,
                         const mlasd_tensor* out, const mlasd_tensor* lse, int32_t nsplit,
                         int32_t head_groups, mlasd_stream_t stream) {
  return decode_impl(q, kv_pages, page_table, topk_idx, seq_lens, softmax_scale, out, lse, nsplit,
                     head_groups, (hipStream_t)stream);
}

int mla_sparse_decode_noalloc(const mlasd_tensor* q, const mlasd_tensor* kv_pages,
                              const mlasd_tensor* page_table, const mlasd_tensor* topk_idx,
                              const mlasd_tensor* seq_lens, float softmax_scale, const mlasd_tensor* out,
                              const mlasd_tensor* lse, mlasd_stream_t stream) {
  DecodeCall call;
  int rc = prepare_decode(q, kv_pages, page_table, topk_idx, seq_lens, softmax_scale, out, lse, 0, 0, &call);
  if (rc != MLASD_OK || call.p.batch == 0) return rc;
  void* ws = nullptr;
  if (call.p.nsplit > 1) {
    int dev = 0;
    rc = current_device(&dev);
    if (rc != MLASD_OK) return rc;
    if (dev >= mlasd::kMaxDevices) return MLASD_ERR_DEVICE;
    if (split_scratch_bytes(call.p.batch, call.p.nsplit) > mlasd::kNoAllocScratchBytes) return MLASD_ERR_WORKSPACE;
    hipError_t e = mlasd::noalloc_scratch(dev, &ws);
    if (e != hipSuccess) return hip_fail(e);
  }
  return launch_decode_call(call, ws, mlasd::kNoAllocScratchBytes, (hipStream_t)stream);
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

int mla_sparse_workspace_size(int32_t batch, int32_t topk, int32_t nsplit, int32_t head_groups,
                              int32_t num_cus, size_t* bytes) {
  if (!bytes) return MLASD_ERR_NULL;
  if (batch < 0 || topk < 0 || topk > MLASD_MAX_TOPK || !valid_head_groups(head_groups))
    return MLASD_ERR_SHAPE;
  int cus = num_cus;
  if (cus <= 0) {
    int rc = device_cus(&cus);
    if (rc != MLASD_OK) return rc;
  }
  int32_t ns = 1, len = 0, hg = 1;
  make_plan(batch, topk, nsplit, head_groups, cus, &ns, &len, &hg);
  *bytes = split_scratch_bytes(batch, ns);
  return MLASD_OK;
}

int mla_sparse_gather_dequant(const mlasd_tensor* kv_pages, const mlasd_tensor* page_table,
                              const mlasd_tensor* topk_idx, const mlasd_tensor* seq_lens,
                              const mlasd_tensor* rows, const mlasd_tensor* valid, mlasd_stream_t stream) {
  Selection s{};
  int rc = check_selection(kv_pages, page_table, topk_idx, seq_lens, &s);
  if (rc != MLASD_OK) return rc;
  const int64_t B = s.cache.batch;
  const int64_t wr[3] = {B, s.topk, MLASD_D_QK};
  rc = check_tensor(rows, MLASD_F32, 3, wr, true);
  if (rc != MLASD_OK) return rc;
  const int64_t wv[2] = {B, s.topk};
  rc = check_tensor(valid, MLASD_U8, 2, wv, true);
  if (rc != MLASD_OK) return rc;
  if (B == 0 || s.topk == 0) return MLASD_OK;
  if (!aligned(rows->data, 16) || !strides_multiple(rows, 2, 4)) return MLASD_ERR_ALIGN;
  int cus = 0;
  rc = device_cus(&cus);
  if (rc != MLASD_OK) return rc;
  mlasd::GatherParams p{};
  p.kv = s.cache.kv;
  p.num_pages = s.cache.num_pages;
  p.page_stride = s.cache.page_stride;
  p.page_table = s.cache.pt;
  p.pt_sb = s.cache.pt_sb;
  p.max_pages = s.cache.max_pages;
  p.topk_idx = s.idx;
  p.idx_sb = s.idx_sb;
  p.topk = s.topk;
  p.seq_lens = s.lens;
  p.len_s = s.len_s;
  p.batch = (int32_t)B;
  p.rows = (float*)rows->data;
  p.rows_sb = rows->stride[0];
  p.rows_sj = rows->stride[1];
  p.valid = (uint8_t*)valid->data;
  p.valid_sb = valid->stride[0];
  int32_t hg_unused = 1;
  make_plan(p.batch, p.topk, 0, 0, cus, &p.nsplit, &p.split_len, &hg_unused);
  hipError_t e = mlasd::launch_gather(p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e);
  return MLASD_OK;
}

int mla_kv_append(const mlasd_tensor* latent, const mlasd_tensor* seq_ids, const mlasd_tensor* positions,
                  const mlasd_tensor* page_table, const mlasd_tensor* kv_pages, mlasd_stream_t stream) {
  if (latent == nullptr) return MLASD_ERR_NULL;
  if (latent->ndim != 2 || latent->shape[0] < 0 || latent->shape[0] > INT32_MAX) return MLASD_ERR_SHAPE;
  const int64_t n = latent->shape[0];
  const int64_t wlat[2] = {n, MLASD_D_QK};
  int rc = check_tensor(latent, MLASD_BF16, 2, wlat, true);
  if (rc != MLASD_OK) return rc;
  const int64_t wn[1] = {n};
  rc = check_tensor(seq_ids, MLASD_I32, 1, wn, true, false);
  if (rc != MLASD_OK) return rc;
  rc = check_tensor(positions, MLASD_I32, 1, wn, true, false);
  if (rc != MLASD_OK) return rc;
  if (n == 0) return MLASD_OK;
  Cache c{};
  rc = check_pool(kv_pages, &c);
  if (rc != MLASD_OK) return rc;
  if (page_table == nullptr) return MLASD_ERR_NULL;
  if (page_table->ndim != 2 || page_table->shape[0] < 1 || page_table->shape[0] > INT32_MAX)
    return MLASD_ERR_SHAPE;
  rc = check_page_table(page_table, page_table->shape[0], &c);
  if (rc != MLASD_OK) return rc;
  if (!aligned(latent->data, 16) || !strides_multiple(latent, 1, 8) || !aligned(seq_ids->data, 4) ||
      !aligned(positions->data, 4))
    return MLASD_ERR_ALIGN;
  int cus = 0;
  rc = device_cus(&cus);
  if (rc != MLASD_OK) return rc;
  mlasd::AppendParams p{};
  p.latent = (const uint16_t*)latent->data;
  p.lat_s = latent->stride[0];
  p.seq_ids = (const int32_t*)seq_ids->data;
  p.seq_s = seq_ids->stride[0];
  p.positions = (const int32_t*)positions->data;
  p.pos_s = positions->stride[0];
  p.n_tokens = (int32_t)n;
  p.page_table = c.pt;
  p.pt_sb = c.pt_sb;
  p.batch = (int32_t)page_table->shape[0];
  p.max_pages = c.max_pages;
  p.kv = (uint8_t*)c.kv;
  p.num_pages = c.num_pages;
  p.page_stride = c.page_stride;
  hipError_t e = mlasd::launch_append(p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e);
  return MLASD_OK;
}

int mla_topk_select(const mlasd_tensor* scores, const mlasd_tensor* seq_lens, const mlasd_tensor* topk_idx,
                    mlasd_stream_t stream) {
  return topk_impl(scores, seq_lens, topk_idx, 0, (hipStream_t)stream);
}

int mla_topk_select_ex(const mlasd_tensor* scores, const mlasd_tensor* seq_lens, const mlasd_tensor* topk_idx,
                       int32_t parts, mlasd_stream_t stream) {
  return topk_impl(scores, seq_lens, topk_idx, parts, (hipStream_t)stream);
}

int mla_topk_plan(int32_t batch, int32_t max_len, int32_t parts_request, int32_t num_cus, int32_t* parts,
                  size_t* bytes) {
  if (!parts || !bytes) return MLASD_ERR_NULL;
  if (batch < 0 || max_len < 0 || parts_request > kTopkMaxParts) return MLASD_ERR_SHAPE;
  int cus = num_cus;
  if (cus <= 0 && parts_request <= 0) {
    int rc = device_cus(&cus);
    if (rc != MLASD_OK) return rc;
  }
  *parts = parts_request > 0 ? parts_request : topk_parts(batch, max_len, cus);
  *bytes = mlasd::topk_workspace_bytes(batch, *parts);
  return MLASD_OK;
}

int mlasd_prepare(mlasd_stream_t stream, int32_t max_batch, int32_t max_topk) {
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
    if (split_scratch_bytes(b, ns) > need) need = split_scratch_bytes(b, ns);
  }
  if (need == 0) return MLASD_OK;
  return reserve_workspace((hipStream_t)stream, need);
}

int mlasd_reserve(mlasd_stream_t stream, size_t bytes) {
  if (bytes == 0) return MLASD_OK;
  int cus = 0;
  int rc = device_cus(&cus);
  if (rc != MLASD_OK) return rc;
  return reserve_workspace((hipStream_t)stream, bytes);
}

int mlasd_release(mlasd_stream_t stream_) {
  hipStream_t stream = (hipStream_t)stream_;
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != MLASD_OK) return rc;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  auto it = g_ws.find({dev, stream});
  if (it == g_ws.end()) return MLASD_OK;
  bool cap = false;
  rc = capturing(stream, &cap);
  if (rc != MLASD_OK) return rc;
  if (cap) return MLASD_ERR_CAPTURE;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e);
  hipError_t first = hipSuccess;
  for (void* p : it->second.retired) {
    e = hipFree(p);
    if (first == hipSuccess) first = e;
  }
  if (it->second.ptr) {
    e = hipFree(it->second.ptr);
    if (first == hipSuccess) first = e;
  }
  g_ws.erase(it);
  if (first != hipSuccess) return hip_fail(first);
  return MLASD_OK;
}

int mlasd_workspace_bytes(mlasd_stream_t stream, size_t* bytes) {
  if (bytes == nullptr) return MLASD_ERR_NULL;
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != MLASD_OK) return rc;
  void* p = nullptr;
  lookup_workspace(dev, (hipStream_t)stream, &p, bytes);
  return MLASD_OK;
}

const char* mlasd_status_string(int status) {
  switch (status) {
    case MLASD_OK: return "ok";
    case MLASD_ERR_NULL: return "null pointer argument";
    case MLASD_ERR_SHAPE: return "size, shape, stride or dtype not accepted";
    case MLASD_ERR_ALIGN: return "misaligned pointer or stride";
    case MLASD_ERR_VALUE: return "invalid scalar argument";
    case MLASD_ERR_HIP: return "HIP runtime error";
    case MLASD_ERR_DEVICE: return "current device is not gfx950";
    case MLASD_ERR_CAPTURE: return "allocating call made while the stream is capturing";
    case MLASD_ERR_WORKSPACE:
      return "split scratch for this stream is missing or too small: reserve it with mlasd_prepare";
    default: return "unknown status";
  }
}

int mlasd_last_hip_error(void) { return g_last_hip_error; }

const char* mlasd_version(void) { return "mlasd 0.2.0 (gfx950)"; }

}  // extern "C"
