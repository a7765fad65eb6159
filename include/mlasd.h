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
 * and How"): a page is 149504 bytes.  Page p, slot s:
 *   token record at s*576: 448 e4m3 bytes, then 64 little-endian bf16;
 *   scale record at 147456 + s*8: 7 UE8M0 bytes (byte g scales nope dims
 *   [64g, 64g+64)), then one ignored pad byte.
 * Pages may sit at any row stride of at least 149504 bytes (a multiple of
 * 16), e.g. a view of a wider pool -- the pages' own harness passes such a
 * strided view ("The Validation Gate", "The Thinking Process").
 *
 * Conventions for every entry point:
 *   - Tensors are passed as mlasd_tensor descriptors: a DEVICE pointer owned
 *     by the caller, a dtype, a shape and strides in elements.  Each entry
 *     point states the dtype, shape and stride rules it accepts; the
 *     innermost dimension is always contiguous (stride 1).  The library never
 *     frees or keeps caller memory.
 *   - Every call is asynchronous on `stream` (NULL = the null stream): it
 *     only enqueues work.  No compute entry point allocates device memory or
 *     synchronises the host; only mlasd_prepare / mlasd_reserve allocate and
 *     only mlasd_release frees.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     non-zero return nothing was enqueued (except MLASD_ERR_HIP, which
 *     reports a failed enqueue).  Data-dependent conditions (masked indices,
 *     out-of-range page ids) are not errors: such entries are skipped.
 *   - Output tensors must not overlap each other or any input.
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
  MLASD_ERR_NULL = -1,      /* a required pointer is NULL                          */
  MLASD_ERR_SHAPE = -2,     /* a size, shape, stride or dtype is not accepted     */
  MLASD_ERR_ALIGN = -3,     /* a pointer or stride breaks the stated alignment    */
  MLASD_ERR_VALUE = -4,     /* a scalar argument is invalid (non-finite scale)     */
  MLASD_ERR_HIP = -5,       /* a HIP runtime call failed (see mlasd_last_hip_error) */
  MLASD_ERR_DEVICE = -6,    /* the current device is not a gfx950 device           */
  MLASD_ERR_CAPTURE = -7,   /* an allocating call was made while capturing         */
  MLASD_ERR_WORKSPACE = -8  /* the call's plan needs more split scratch than was
                               reserved for the stream (mlasd_prepare / reserve) */
};

/* Element types of mlasd_tensor. */
enum { MLASD_U8 = 1, MLASD_I32 = 2, MLASD_BF16 = 3, MLASD_F32 = 4 };

/* A strided view of device memory.  Element (i0, i1, ...) lives at
 * data + sum_k i_k * stride[k] elements.  Only the first ndim entries of
 * shape and stride are read. */
typedef struct mlasd_tensor {
  void* data;
  int32_t dtype;       /* MLASD_U8, MLASD_I32, MLASD_BF16 or MLASD_F32 */
  int32_t ndim;        /* 1..4 */
  int64_t shape[4];
  int64_t stride[4];   /* in elements, >= 0 */
} mlasd_tensor;

/* Fixed shape of the method. */
#define MLASD_HEADS 64
#define MLASD_D_QK 512
#define MLASD_D_V 448
#define MLASD_MAX_TOPK 512
#define MLASD_PAGE_TOKENS 256
#define MLASD_PAGE_BYTES 149504

/*
 * mla_sparse_decode -- the decode hot path (the step of "The Turning
 * Point", "The Reasoning Process", Steps 1-5, with the outputs of "The
 * Moment of Validation", "Two Failures, Two Lessons").
 *
 *   q          BF16 [B, 64, 512]; dims 0..447 nope, 448..511 rope ("The
 *              Turning Point", Step 1).  data 16-byte aligned, stride[0] and
 *              stride[1] multiples of 8.
 *   kv_pages   U8 [num_pages, 149504], num_pages >= 1; stride[0] >= 149504
 *              and a multiple of 16; data 16-byte aligned.
 *   page_table I32 [B, max_pages], max_pages >= 1: logical page -> physical
 *              page of each query's sequence.  Any stride[0].
 *   topk_idx   I32 [B, topk], 0 <= topk <= 512: token positions; -1 or any
 *              out-of-range value is masked.  Any stride[0].
 *   seq_lens   I32 [B].  Any stride.
 *   softmax_scale  finite float multiplying every score.
 *   out        BF16 [B, 64, 448] (written, round-to-nearest-even); data
 *              16-byte aligned, stride[0] and stride[1] multiples of 8.
 *   lse        F32 [B, 64] (written, natural log).  Any stride[0].
 *   stream     HIP stream to enqueue on.
 *
 * B == 0 is a no-op.  topk == 0 writes out = 0, lse = -inf.
 * The automatic plan cuts a query's top-k list into slices only when the
 * batch leaves compute units idle and the tiles it takes off each
 * workgroup outweigh the cost of the LSE combine.  Then the fp32 partial
 * results live in the split scratch reserved for `stream` by
 * mlasd_prepare (or mlasd_reserve); if that scratch is missing or too small
 * the call returns MLASD_ERR_WORKSPACE and enqueues nothing.  It never
 * allocates, frees or synchronises, so it may be captured into a graph.
 * Numerics: the 448 nope dims of q and K, and the value rows, enter the
 * contractions in fp16; the 64 rope dims in bf16; sums and the softmax are
 * fp32.  Cache values stay exact over the UE8M0 range: a token whose 7
 * group scales all lie in bytes 112..134 is held in fp16 as stored; any
 * other token is held as e4m3 * 2^(k_g - r) with one power of two r per
 * token (exact whenever its groups span at most 22 binades), which the
 * score and P V take back in fp32.  Each head's q is scaled by a power of
 * two that puts its largest nope value in [2^15, 2^16), so q is exact down
 * to 2^29 below that value; the softmax scale takes the power back.
 * Returns MLASD_OK or a negative MLASD_ERR_* code.
 */
int mla_sparse_decode(const mlasd_tensor* q, const mlasd_tensor* kv_pages,
                      const mlasd_tensor* page_table, const mlasd_tensor* topk_idx,
                      const mlasd_tensor* seq_lens, float softmax_scale,
                      const mlasd_tensor* out, const mlasd_tensor* lse,
                      mlasd_stream_t stream);

/*
 * mla_sparse_decode_ex -- mla_sparse_decode with the plan forced:
 *   nsplit       the top-k list of each query is cut into `nsplit` slices
 *                handled by separate workgroups and merged by the LSE
 *                combine ("The Turning Point", Step 5).  <= 0: automatic;
 *                larger values are clamped to ceil(topk / 32).
 *   head_groups  1: each workgroup computes all 64 heads of its slice (the
 *                pages' one-program-per-query layout, Steps 3-4); 2: two
 *                workgroups of 32 heads share the slice's gathered records.
 *                0: automatic for the chosen nsplit.  Other values:
 *                MLASD_ERR_SHAPE.
 * Results equal mla_sparse_decode's up to floating-point rounding: the
 * slices change the summation order of the softmax-weighted sum, and with 2
 * head groups each score is summed over the 512 dims in two parts (dims
 * 0..191 with the rope dims, and 192..447) that are then added, where 1
 * head group sums it in one pass.  The 64-head and 32-head results
 * therefore differ in the last bits; neither is the more exact.
 * Split plans need scratch as mla_sparse_decode does; mla_sparse_workspace_size
 * gives the bytes for mlasd_reserve.  Intended for tests and benchmarks.
 */
int mla_sparse_decode_ex(const mlasd_tensor* q, const mlasd_tensor* kv_pages,
                         const mlasd_tensor* page_table, const mlasd_tensor* topk_idx,
                         const mlasd_tensor* seq_lens, float softmax_scale,
                         const mlasd_tensor* out, const mlasd_tensor* lse,
                         int32_t nsplit, int32_t head_groups, mlasd_stream_t stream);

/*
 * mla_sparse_decode_noalloc -- mla_sparse_decode for callers that cannot
 * allocate device memory at all: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, plan and
 * results as mla_sparse_decode (bit for bit).  It needs no mlasd_prepare:
 * split partials go to a static device array of 16 MiB per GPU, held by
 * the library until the process ends; a call whose plan needs more
 * (B * nsplit * 64 * 449 * 4 bytes > 16 MiB; no automatic plan on 256 CUs
 * does: at most 128 slices, 14.7 MB) returns MLASD_ERR_WORKSPACE and
 * enqueues nothing.  It calls no hipMalloc, hipFree or other allocating
 * routine.  Every call on one GPU shares that GPU's array: calls that may
 * overlap in time on one GPU (different streams without ordering, or
 * replays of graphs containing this call) race on it and must be ordered
 * by the caller.  The array keeps the last call's partials; nothing in it
 * needs to start at zero.
 */
int mla_sparse_decode_noalloc(const mlasd_tensor* q, const mlasd_tensor* kv_pages,
                              const mlasd_tensor* page_table, const mlasd_tensor* topk_idx,
                              const mlasd_tensor* seq_lens, float softmax_scale,
                              const mlasd_tensor* out, const mlasd_tensor* lse,
                              mlasd_stream_t stream);

/*
 * mla_sparse_plan -- the plan the library would use (host only, no device
 * work): writes the number of top-k slices per query, the number of index
 * entries per slice (a multiple of 32) and, if head_groups is not NULL, the
 * number of head groups (1 or 2).  nsplit_request as in
 * mla_sparse_decode_ex.  num_cus > 0 plans for that many compute units;
 * num_cus <= 0 queries the current HIP device.
 */
int mla_sparse_plan(int32_t batch, int32_t topk, int32_t nsplit_request, int32_t num_cus,
                    int32_t* nsplit, int32_t* split_len, int32_t* head_groups);

/*
 * mla_sparse_workspace_size -- bytes of split scratch a decode of this shape
 * needs (host only): 0 when the plan does not split.  nsplit and
 * head_groups as in mla_sparse_decode_ex (0 = automatic); num_cus as in
 * mla_sparse_plan.
 */
int mla_sparse_workspace_size(int32_t batch, int32_t topk, int32_t nsplit, int32_t head_groups,
                              int32_t num_cus, size_t* bytes);

/*
 * mla_sparse_gather_dequant -- test hook for the gather + dequant stage:
 * runs the decode kernel's own index resolution, page-table walk, gather and
 * dequantisation, and writes each entry's key row as the contractions
 * consume it (its first 448 values are also the value row).
 *
 *   rows   F32 [B, topk, 512], innermost contiguous, data 16-byte aligned,
 *          stride[0] and stride[1] multiples of 4: nope dims are the
 *          dequantised values e4m3 * 2^(e-127) exactly as the kernel holds
 *          them (widened to fp32, which is exact), rope dims the stored bf16
 *          values.  Zero for masked entries.
 *   valid  U8 [B, topk]: 1 where the entry is valid.  Any stride[0].
 * Other arguments as in mla_sparse_decode.
 */
int mla_sparse_gather_dequant(const mlasd_tensor* kv_pages, const mlasd_tensor* page_table,
                              const mlasd_tensor* topk_idx, const mlasd_tensor* seq_lens,
                              const mlasd_tensor* rows, const mlasd_tensor* valid,
                              mlasd_stream_t stream);

/*
 * mla_kv_append -- the step before the decode: quantise token latents into
 * the paged cache ("The Turning Point", "Input Knowledge Required",
 * FP8/UE8M0 bullet; layout as above, "The Validation Gate", "The Test
 * Design").
 *
 *   latent     BF16 [N, 512]; dims 0..447 nope, 448..511 rope.  data
 *              16-byte aligned, stride[0] a multiple of 8.
 *   seq_ids    I32 [N]: page-table row of each token.  Any stride.
 *   positions  I32 [N]: position of each token in its sequence.  Any stride.
 *   page_table I32 [B, max_pages], B >= 1, max_pages >= 1.  Any stride[0].
 *   kv_pages   U8 [num_pages, 149504] as for the decode; written.
 *
 * Token i goes to page page_table[s][p / 256], slot p % 256 (s = seq_ids[i],
 * p = positions[i]).  Nope dims of group g (64 each) get scale byte
 * k + 127, k the least integer with max|x| <= 448 * 2^k clamped to
 * [-127, 127] (0 -> -127), and codes e4m3(round-to-nearest-even(x * 2^-k));
 * scale byte 7 is 0; rope values are stored as they are.  Tokens whose
 * sequence, position or page is out of range are skipped (not an error).
 * Tokens of one call must have distinct destinations: two tokens with the
 * same destination leave an undefined record there (their byte stores may
 * interleave).  N == 0 is a no-op.  Returns MLASD_OK or a negative
 * MLASD_ERR_* code.
 */
int mla_kv_append(const mlasd_tensor* latent, const mlasd_tensor* seq_ids,
                  const mlasd_tensor* positions, const mlasd_tensor* page_table,
                  const mlasd_tensor* kv_pages, mlasd_stream_t stream);

/*
 * mla_topk_select -- the other step before the decode: each query's top-k
 * index list from its indexer scores (the indexer scores every position of
 * the context in fp32: "The Turning Point", "The Strategic Context: Why
 * This Message Exists", item 3).
 *
 *   scores    F32 [B, max_len], innermost contiguous: one score per position.
 *   seq_lens  I32 [B]: positions 0 .. L-1, L = min(max(seq_len, 0), max_len),
 *             are the candidates.  Any stride.
 *   topk_idx  I32 [B, k], 0 <= k <= 512, innermost contiguous (written): the
 *             first min(k, L) candidates in rank order -- higher score
 *             first, equal scores lower position first, a NaN score ranking
 *             as -inf, -0.0 equal to +0.0 -- then -1.
 *   stream    HIP stream to enqueue on.
 * B == 0 or k == 0 is a no-op.  Allocates nothing and never synchronises.
 * Plan: when max_len is at least 65,536 and the batch leaves at least 4
 * compute units per row (mla_topk_plan), the candidate pass over each long
 * row is cut into 4 to 8 parts of one workgroup each, whose candidate lists
 * go to the split scratch reserved for `stream` (mlasd_reserve with
 * mla_topk_plan's bytes); a second launch selects and sorts each row.
 * Without enough scratch the call runs one workgroup per row instead.  Both
 * give the same result, bit for bit.
 * Returns MLASD_OK or a negative MLASD_ERR_* code.
 */
int mla_topk_select(const mlasd_tensor* scores, const mlasd_tensor* seq_lens, const mlasd_tensor* topk_idx,
                    mlasd_stream_t stream);

/*
 * mla_topk_select_ex -- mla_topk_select with the parts per row forced:
 * parts <= 0 as mla_topk_select; 1 one workgroup per row; 2..8 that many
 * parts for rows longer than max(k, 4096) positions (shorter rows are
 * selected whole), needing mla_topk_plan's bytes of the stream's split
 * scratch (MLASD_ERR_WORKSPACE without them, nothing enqueued).  parts > 8:
 * MLASD_ERR_SHAPE.  Same results as mla_topk_select.  Intended for tests
 * and benchmarks.
 */
int mla_topk_select_ex(const mlasd_tensor* scores, const mlasd_tensor* seq_lens, const mlasd_tensor* topk_idx,
                       int32_t parts, mlasd_stream_t stream);

/*
 * mla_topk_plan -- the parts per row mla_topk_select would use for B rows of
 * max_len scores (host only; parts_request as in mla_topk_select_ex), and
 * the bytes of split scratch that plan needs (0 for one part).  num_cus > 0
 * plans for that many compute units; num_cus <= 0 queries the current HIP
 * device (only when parts_request <= 0).  Errors: MLASD_ERR_NULL,
 * MLASD_ERR_SHAPE (negative sizes, parts_request > 8), MLASD_ERR_DEVICE.
 */
int mla_topk_plan(int32_t batch, int32_t max_len, int32_t parts_request, int32_t num_cus, int32_t* parts,
                  size_t* bytes);

/*
 * mlasd_prepare -- reserve the split scratch of `stream` (on the current
 * device) for every automatically planned mla_sparse_decode call with
 * batch <= max_batch and topk <= max_topk.  Everything a captured call needs
 * must exist before capture begins ("The Validation Moment", "The Weight of
 * 'CUDA Graph Capture Completed Without Errors'").  Host call; may allocate
 * (hipMalloc) and zero the new scratch; refused with MLASD_ERR_CAPTURE
 * while the stream is capturing.  Scratch only grows: when it must, the new
 * buffer replaces the old one for later calls, and the old one stays
 * allocated until mlasd_release, so graphs captured earlier stay valid.
 * max_batch == 0 reserves nothing.  Errors: MLASD_ERR_SHAPE (negative sizes,
 * max_topk > 512), MLASD_ERR_DEVICE, MLASD_ERR_HIP.
 */
int mlasd_prepare(mlasd_stream_t stream, int32_t max_batch, int32_t max_topk);

/* mlasd_reserve -- as mlasd_prepare, for at least `bytes` of split scratch
 * (e.g. mla_sparse_workspace_size of a forced plan, or mla_topk_plan's
 * bytes; the top-k selection and the decode share the stream's scratch). */
int mlasd_reserve(mlasd_stream_t stream, size_t bytes);

/*
 * mlasd_release -- synchronise `stream` and free all of its split scratch
 * on the current device, superseded buffers included (a no-op if it has
 * none).  Refused with MLASD_ERR_CAPTURE while the stream is capturing.
 * Graphs captured while any of that scratch was in use must not be replayed
 * afterwards.
 *
 * Sharing: the scratch belongs to (device, stream).  Calls enqueued on one
 * stream are ordered; a graph captured on stream S uses S's scratch
 * wherever it is replayed, so its replays must be ordered with other work
 * that uses S's scratch (eager calls on S, other graphs captured on S).
 */
int mlasd_release(mlasd_stream_t stream);

/* Bytes of split scratch currently usable by calls on `stream` (current device). */
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
