/*
 * mlasd.h -- sparse Multi-head Latent Attention decode over a paged FP8 KV
 * cache, for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operation (cited by page title and section of the pages it follows):
 *   For each decode query b, 64 query heads share one latent KV head
 *   ("The Turning Point", "The Reasoning Process", Step 1, and
 *   "Assumptions Made and Their Validity", Assumption 1).  A top-k index list
 *   of the query selects cached tokens; each selected token record is
 *   dequantised (fp8 e4m3 nope with UE8M0 group scales, bf16 rope), scores
 *   are taken over all 512 dims, and the kernel returns the softmax-weighted
 *   sum over the 448 nope dims plus a log-sum-exp per head ("The Moment of
 *   Validation", "Two Failures, Two Lessons"; "The Validation Gate",
 *   "Output Knowledge Created").
 *
 *   valid(b, j)  : p = topk_idx[b][j]; 0 <= p < seq_lens[b], p/256 < max_pages,
 *                  and page = page_table[b][p/256] lies in [0, num_pages).
 *   K_j[d]       : d < 448: e4m3(rec[d]) * 2^(scale[d/64] - 127);
 *                  d >= 448: bf16 rope value d-448.
 *   s_h,j        : softmax_scale * sum_{d<512} q[b][h][d] * K_j[d]
 *   lse[b][h]    : ln sum_{valid j} exp(s_h,j)       (-inf if no valid j)
 *   out[b][h][c] : sum_{valid j} exp(s_h,j - lse) * K_j[c],  c < 448
 *                  (0 if no valid j)
 *
 * Cache layout ("The Validation Gate", "The Test Design: What Gets Validated
 * and How"): uint8 [num_pages, 149504].  Page p, slot s:
 *   token record at p*149504 + s*576: 448 e4m3 bytes, 64 little-endian bf16;
 *   scale record at p*149504 + 147456 + s*8: 7 UE8M0 bytes (byte g scales
 *   nope dims [64g, 64g+64)), then one ignored pad byte.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller, contiguous,
 *     row-major, in the dtype stated.  The library never frees them.
 *   - Every call is asynchronous on `stream` (0 = the null stream): it only
 *     enqueues work and never synchronises the host.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     non-zero return nothing was enqueued (except MLASD_ERR_HIP, which
 *     reports a failed enqueue).  Data-dependent conditions (masked indices,
 *     out-of-range page ids) are not errors: such entries are skipped.
 *   - Split scratch (fp32 partial outputs when a query's top-k list is cut
 *     into slices) is owned by the library: one buffer per (device, stream),
 *     grown with hipMalloc when a call needs more and kept until the process
 *     ends.  Calls on different streams may run concurrently; calls on one
 *     stream are ordered by the stream.  Growth synchronises the stream and
 *     is refused with MLASD_ERR_CAPTURE while the stream is capturing a
 *     graph: make a first call of the largest shape before capture.
 */
#ifndef MLASD_H
#define MLASD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* mlasd_stream_t; /* same object as hipStream_t */

enum {
  MLASD_OK = 0,
  MLASD_ERR_NULL = -1,      /* a required pointer is NULL                         */
  MLASD_ERR_SHAPE = -2,     /* a size is out of range (batch<0, topk>512, ...)   */
  MLASD_ERR_ALIGN = -3,     /* a pointer is not aligned as stated                 */
  MLASD_ERR_VALUE = -4,     /* a scalar argument is invalid (non-finite scale)    */
  MLASD_ERR_HIP = -5,       /* a HIP runtime call failed (see mlasd_last_hip_error) */
  MLASD_ERR_DEVICE = -6,    /* the current device is not a gfx950 device          */
  MLASD_ERR_CAPTURE = -7    /* split scratch would have to grow during graph capture */
};

/* Fixed shape of the method. */
#define MLASD_HEADS 64
#define MLASD_D_QK 512
#define MLASD_D_V 448
#define MLASD_MAX_TOPK 512
#define MLASD_PAGE_TOKENS 256
#define MLASD_PAGE_BYTES 149504

/*
 * mla_sparse_decode -- the decode hot path.
 *
 *   q          bf16 [batch, 64, 512]; 16-byte aligned.  Dims 0..447 nope,
 *              448..511 rope ("The Turning Point", Step 1).
 *   kv_pages   uint8 [num_pages, 149504]; 16-byte aligned; num_pages >= 1.
 *   page_table int32 [batch, max_pages]; max_pages >= 1; logical page ->
 *              physical page of each sequence.
 *   topk_idx   int32 [batch, topk]; 0 <= topk <= 512; token positions in the
 *              sequence; -1 or any out-of-range value is masked.
 *   seq_lens   int32 [batch].
 *   softmax_scale  finite float multiplying every score.
 *   out        bf16 [batch, 64, 448] (written, round-to-nearest-even);
 *              8-byte aligned.
 *   lse        float32 [batch, 64] (written, natural log).
 *   stream     HIP stream to enqueue on.
 *
 * batch == 0 is a no-op.  topk == 0 writes out = 0, lse = -inf.
 * Numerics: the 448 nope dims of q and K, and the value rows, enter the
 * contractions in fp16; the 64 rope dims in bf16; sums and the softmax are
 * fp32.  Dequantised cache values are exact in fp16 while their magnitude is
 * below 65520 and they are multiples of 2^-24 (UE8M0 exponents -15..7 for
 * e4m3 bytes); q's nope values are exact in fp16 for magnitudes in
 * [2^-14, 65504] and keep every bit down to 2^-24 below that.  Larger values
 * overflow to infinity.
 * Returns MLASD_OK or a negative MLASD_ERR_* code.
 */
int mla_sparse_decode(const void* q,
                      const void* kv_pages, int64_t num_pages,
                      const int32_t* page_table, int32_t max_pages,
                      const int32_t* topk_idx, int32_t topk,
                      const int32_t* seq_lens, int32_t batch,
                      float softmax_scale,
                      void* out, float* lse,
                      mlasd_stream_t stream);

/*
 * mla_sparse_decode_ex -- mla_sparse_decode with the plan forced:
 *   nsplit       the top-k list of each query is cut into `nsplit` slices
 *                handled by separate workgroups and merged by the LSE
 *                combine ("The Turning Point", Step 5).  <= 0: automatic;
 *                larger values are clamped to ceil(topk / 32).
 *   head_groups  1: each workgroup computes all 64 heads of its slice (the
 *                pages' one-program-per-query layout, Steps 3-4); 2 or 4:
 *                that many workgroups of 32 or 16 heads share the slice's
 *                gathered records.  0: automatic for the chosen nsplit.
 *                Other values: MLASD_ERR_SHAPE.
 * Results equal mla_sparse_decode's up to floating-point rounding (the head
 * groups do not change any value; the slices change the summation order).
 * Intended for tests and benchmarks.
 */
int mla_sparse_decode_ex(const void* q,
                         const void* kv_pages, int64_t num_pages,
                         const int32_t* page_table, int32_t max_pages,
                         const int32_t* topk_idx, int32_t topk,
                         const int32_t* seq_lens, int32_t batch,
                         float softmax_scale,
                         void* out, float* lse,
                         int32_t nsplit, int32_t head_groups,
                         mlasd_stream_t stream);

/*
 * mla_sparse_plan -- the plan the library would use (host only, no device
 * work): writes the number of top-k slices per query, the number of index
 * entries per slice (a multiple of 32) and, if head_groups is not NULL, the
 * number of head groups (1, 2 or 4).  nsplit_request as in
 * mla_sparse_decode_ex.  num_cus > 0 plans for that many compute units;
 * num_cus <= 0 queries the current HIP device.
 */
int mla_sparse_plan(int32_t batch, int32_t topk, int32_t nsplit_request, int32_t num_cus,
                    int32_t* nsplit, int32_t* split_len, int32_t* head_groups);

/*
 * mla_sparse_gather_dequant -- test hook for the gather + dequant stage:
 * runs the same index resolution, page-table walk, gather and dequantisation
 * code as the decode kernel and writes what the contractions consume.
 *
 *   k_rows  bf16 [batch, topk, 512]: key row of each entry as the QK^T
 *           contraction consumes it: nope e4m3 * 2^(e-127) rounded to fp16
 *           (as in v_rows) and written widened to bf16, which is exact;
 *           rope as stored.  Zero for masked entries.
 *   v_rows  fp16 [batch, topk, 448]: the value row of each entry as the PV
 *           contraction consumes it (fp16; exact while every dequantised
 *           value is a multiple of 2^-24 of magnitude <= 65504).  Zero for
 *           masked entries.
 *   valid   uint8 [batch, topk]: 1 where the entry is valid.
 * Other arguments as in mla_sparse_decode.
 */
int mla_sparse_gather_dequant(const void* kv_pages, int64_t num_pages,
                              const int32_t* page_table, int32_t max_pages,
                              const int32_t* topk_idx, int32_t topk,
                              const int32_t* seq_lens, int32_t batch,
                              void* k_rows, void* v_rows, uint8_t* valid,
                              mlasd_stream_t stream);

/*
 * mla_kv_append -- the step before the decode: quantise token latents into
 * the paged cache ("The Turning Point", "Input Knowledge Required",
 * FP8/UE8M0 bullet; layout as above, "The Validation Gate", "The Test
 * Design").
 *
 *   latent     bf16 [n_tokens, 512]; 16-byte aligned.  Dims 0..447 nope,
 *              448..511 rope.
 *   seq_ids    int32 [n_tokens]: page-table row of each token.
 *   positions  int32 [n_tokens]: position of each token in its sequence.
 *   page_table int32 [batch, max_pages]; logical page -> physical page.
 *   kv_pages   uint8 [num_pages, 149504]; 16-byte aligned; written.
 *
 * Token i goes to page page_table[s][p / 256], slot p % 256 (s = seq_ids[i],
 * p = positions[i]).  Nope dims of group g (64 each) get scale byte
 * k + 127, k the least integer with max|x| <= 448 * 2^k clamped to
 * [-127, 127] (0 -> -127), and codes e4m3(round-to-nearest-even(x * 2^-k));
 * scale byte 7 is 0; rope values are stored as they are.  Tokens whose
 * sequence, position or page is out of range are skipped (not an error).
 * Two tokens with the same destination in one call: either may win.
 * n_tokens == 0 is a no-op.  Returns MLASD_OK or a negative MLASD_ERR_* code.
 */
int mla_kv_append(const void* latent, const int32_t* seq_ids, const int32_t* positions,
                  int32_t n_tokens, const int32_t* page_table, int32_t batch, int32_t max_pages,
                  void* kv_pages, int64_t num_pages, mlasd_stream_t stream);

/*
 * mlasd_prepare -- reserve the split scratch of `stream` (on the current
 * device) for every automatically planned mla_sparse_decode call with
 * batch <= max_batch and topk <= max_topk, so that such calls made later
 * under graph capture allocate nothing.  Everything a captured call needs
 * must exist before capture begins ("The Validation Moment", "The Weight of
 * 'CUDA Graph Capture Completed Without Errors'").  Forced plans
 * (mla_sparse_decode_ex) may need more.  Host call; may allocate and
 * synchronise the stream; refused with MLASD_ERR_CAPTURE while the stream
 * is capturing and the scratch would have to grow.  max_batch == 0 reserves
 * nothing.  Errors: MLASD_ERR_SHAPE (negative sizes, max_topk > 512),
 * MLASD_ERR_DEVICE, MLASD_ERR_HIP.
 */
int mlasd_prepare(mlasd_stream_t stream, int32_t max_batch, int32_t max_topk);

/*
 * mlasd_release -- synchronise `stream` and free its split scratch on the
 * current device (a no-op if it has none).  Refused with MLASD_ERR_CAPTURE
 * while the stream is capturing.  A later call reserves scratch again.
 * Graphs captured while the freed scratch was in use must not be replayed
 * afterwards.
 */
int mlasd_release(mlasd_stream_t stream);

/* Bytes of split scratch currently held for `stream` on the current device. */
int mlasd_workspace_bytes(mlasd_stream_t stream, size_t* bytes);

/* Static text for a status code. */
const char* mlasd_status_string(int status);

/* The last HIP error code seen by this thread (0 if none). */
int mlasd_last_hip_error(void);

/* Library version string. */
const char* mlasd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLASD_H */
