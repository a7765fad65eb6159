// Internal interface between the C-ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlasd {

// Shape of the method (64 heads share one latent KV head; 448 nope + 64 rope).
constexpr int kHeads = 64;
constexpr int kDNope = 448;
constexpr int kDRope = 64;
constexpr int kDQK = 512;
constexpr int kDV = 448;
constexpr int kMaxTopk = 512;
// Paged cache layout: 256 token records of 576 B, then 256 scale records of 8 B.
constexpr int kPageTokens = 256;
constexpr int kRecordBytes = 576;
constexpr int kScaleRecordBytes = 8;
constexpr int64_t kPageBytes = 149504;
constexpr int64_t kScaleBase = 147456;

// Kernel tiling.
constexpr int kTileTokens = 32;   // tokens per LDS tile
constexpr int kThreads = 512;     // 8 waves per decode workgroup

// Strides are in elements of the tensor's own type.
struct DecodeParams {
  const uint16_t* q;          // bf16 [B, 64, 512]
  int64_t q_sb, q_sh;
  const uint8_t* kv;          // [num_pages, >= 149504]
  int64_t num_pages;
  int64_t page_stride;        // bytes between pages
  const int32_t* page_table;  // [B, max_pages]
  int64_t pt_sb;
  int32_t max_pages;
  const int32_t* topk_idx;    // [B, topk]
  int64_t idx_sb;
  int32_t topk;
  const int32_t* seq_lens;    // [B]
  int64_t len_s;
  int32_t batch;
  float scale_log2;           // softmax_scale * log2(e)
  uint16_t* out;              // bf16 [B, 64, 448]
  int64_t out_sb, out_sh;
  float* lse;                 // [B, 64]
  int64_t lse_sb;
  float* part_o;              // [B, nsplit, 64, 448] when nsplit > 1 (contiguous scratch)
  float* part_lse;            // [B, nsplit, 64]      when nsplit > 1
  int32_t nsplit;
  int32_t split_len;          // index entries per slice, multiple of kTileTokens
  int32_t head_groups;        // 1 or 2: workgroups sharing a slice's 64 heads
};

struct GatherParams {
  const uint8_t* kv;
  int64_t num_pages;
  int64_t page_stride;
  const int32_t* page_table;
  int64_t pt_sb;
  int32_t max_pages;
  const int32_t* topk_idx;
  int64_t idx_sb;
  int32_t topk;
  const int32_t* seq_lens;
  int64_t len_s;
  int32_t batch;
  float* rows;        // fp32 [B, topk, 512]
  int64_t rows_sb, rows_sj;
  uint8_t* valid;     // [B, topk]
  int64_t valid_sb;
  int32_t nsplit;
  int32_t split_len;
};

struct AppendParams {
  const uint16_t* latent;     // bf16 [n_tokens, 512]: 448 nope, 64 rope
  int64_t lat_s;
  const int32_t* seq_ids;     // [n_tokens] page-table row of each token
  int64_t seq_s;
  const int32_t* positions;   // [n_tokens] position within its sequence
  int64_t pos_s;
  int32_t n_tokens;
  const int32_t* page_table;  // [batch, max_pages]
  int64_t pt_sb;
  int32_t batch;
  int32_t max_pages;
  uint8_t* kv;                // [num_pages, >= 149504]
  int64_t num_pages;
  int64_t page_stride;
};

struct TopkParams {
  const float* scores;        // fp32 [B, max_len], innermost contiguous
  int64_t sc_sb;
  int32_t max_len;
  const int32_t* seq_lens;    // [B]
  int64_t len_s;
  int32_t batch;
  int32_t* topk_idx;          // [B, k], innermost contiguous
  int64_t idx_sb;
  int32_t k;                  // 1 .. 512
  int32_t parts;              // workgroups per long row in the candidate pass (1 .. 8)
  int32_t cap_part;           // composites per part's list (set by launch_topk)
  uint64_t* ws_list;          // [B, parts, cap_part] part lists  (parts > 1)
  uint64_t* ws_meta;          // [B, parts, 4] per part: count, t0, largest key, unused
};

// Split scratch of the entry point that allocates nothing: a static device
// array per GPU (mlasd_noalloc.hip).  noalloc_scratch returns its device
// address on device `dev`, which must be current.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(int dev, void** ptr);

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
hipError_t launch_combine(const DecodeParams& p, hipStream_t stream);
hipError_t launch_gather(const GatherParams& p, hipStream_t stream);
hipError_t launch_append(const AppendParams& p, hipStream_t stream);
// Bytes of workspace a top-k launch of `parts` parts per row needs (0 for 1).
size_t topk_workspace_bytes(int32_t batch, int32_t parts);
// ws: topk_workspace_bytes(p.batch, p.parts) bytes, 8-byte aligned (unused for parts 1).
hipError_t launch_topk(TopkParams p, void* ws, hipStream_t stream);

}  // namespace mlasd
