/*
 * qsaidx.h -- paged MQA-logits scoring and per-row top-k for a sparse-attention
 * (QSA-style) indexer, on AMD Instinct MI355X (gfx950).
 *
 * The library computes, for every query row r with H index heads of dimension
 * D, and every compressed key column c of the row's request:
 *
 *     logit[r, c] = sum_h w[r, h] * ReLU( q[r, h, :] . k[c, :] )      c <  ctx[r]
 *     logit[r, c] = -inf                                             ctx[r] <= c < width
 *
 * The ReLU is applied per head, before the heads are summed (ROCm/ATOM PR #2651,
 * "Changes"); zero-padded heads therefore add exactly 0 (sglang PR #48649,
 * "Accuracy Tests").  w is an f32 weight per (row, head), or 1 when absent
 * (ROCm/aiter PR #4221, "Motivation" and "Technical details").  For fp8 keys with
 * a per-key f32 scale s[c], k[c, :] is the dequantised key fp8(k8[c, :]) * s[c]
 * (same page).  Key column c of request b lives in pool block
 * block_table[b, c / B] at slot c % B (same page, block-flat commit; sglang
 * PR #48649 test body).  Columns past a row's visible count are -inf (ROCm/aiter
 * PR #4221, test gate: the -inf mask is compared exactly).
 *
 * qsa_topk then selects, per row, the k columns of [0, ctx[r]) with the largest
 * logits (vLLM PR #62589, "Details": top-k reads only [0, visible); sglang
 * PR #48649: rows that fit in k keep everything).
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is DEVICE memory owned by the caller, unless stated.
 *    The library allocates nothing, keeps no pointer after returning, and has no
 *    global state other than a thread-local error message.
 *  - Compute calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  They never synchronise the device or read device memory on the
 *    host, so they may be captured into a HIP graph.
 *  - Only host-visible scalars are validated; a failed validation returns a
 *    status with no launch.  Device values are preconditions, listed per call.
 *  - No call aborts or throws.  qsa_last_error() describes the last non-OK
 *    status of the calling thread.
 */
#ifndef QSAIDX_H
#define QSAIDX_H

#include <stdint.h>

#ifndef QSA_API
#define QSA_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qsa_status {
    QSA_OK = 0,
    QSA_E_INVALID = 1,     /* null pointer, negative or inconsistent size          */
    QSA_E_DTYPE = 2,       /* unknown dtype, or q and k dtypes differ               */
    QSA_E_UNSUPPORTED = 3, /* valid request outside the compiled set (see below)    */
    QSA_E_RANGE = 4,       /* a size or offset exceeds what the kernels address     */
    QSA_E_ALIGN = 5,       /* pointer or stride misaligned                          */
    QSA_E_HIP = 6          /* the HIP runtime rejected the launch                  */
} qsa_status;

typedef enum qsa_dtype {
    QSA_BF16 = 0,          /* bfloat16 q and keys                                   */
    QSA_FP8_E4M3FN = 1,    /* OCP fp8 E4M3 ("fn": no infinities, max 448) q and keys */
    QSA_FP16 = 2           /* IEEE binary16 q and keys (vLLM #62589, "Details": the  */
                           /* dot runs in fp16 for fp16 inputs, fp32 accumulation)   */
} qsa_dtype;

typedef enum qsa_kv_layout {
    /* kcache is [num_blocks][block_size][head_dim] elements; for fp8 an optional
     * separate kscale [num_blocks][block_size] f32.                             */
    QSA_KV_PAGED = 0,
    /* fp8 only, block-flat co-packed (ROCm/aiter PR #4221, block-flat commit):
     * each block is block_size*head_dim key bytes (key of slot s at byte
     * s*head_dim) followed by block_size little-endian f32 scales (slot s at
     * byte block_size*head_dim + 4*s); block stride block_size*(head_dim+4).  */
    QSA_KV_COPACKED = 1,
    /* fp8 only, co-packed with the keys preshuffled in 16x16-byte tiles
     * (ROCm/aiter PR #4221, preshuffle commit and the commit that unifies both
     * layouts as one coordinate space with two stride vectors): the scale tail
     * is as in QSA_KV_COPACKED; in the key section, byte d of slot s sits at
     * (s/16)*16*head_dim + (d/16)*256 + (s%16)*16 + d%16 (each group of 16
     * slots is stored as head_dim/16 chunks of 16 slots x 16 bytes).
     * block_size must be a multiple of 16.                                     */
    QSA_KV_COPACKED_SHUFFLED = 2
} qsa_kv_layout;

typedef struct qsa_logits_shape {
    int32_t num_rows;    /* R query rows                                           */
    int32_t num_heads;   /* H index heads per row, zero-padded heads included      */
    int32_t head_dim;    /* D                                                      */
    int32_t block_size;  /* B key COLUMNS per pool block                           */
    int32_t num_reqs;    /* rows of block_table                                    */
    int32_t max_blocks;  /* columns of block_table                                 */
    int32_t width;       /* W logits written per row                               */
    int32_t q_dtype;     /* qsa_dtype                                              */
    int32_t k_dtype;     /* qsa_dtype; must equal q_dtype                          */
    int32_t kv_layout;   /* qsa_kv_layout                                          */
    int64_t num_blocks;  /* blocks in the key pool                                 */
    int64_t out_stride;  /* floats between consecutive rows of out, >= width       */
} qsa_logits_shape;

/*
 * qsa_paged_logits -- the masked logits [R][W] (formula at the top of this file).
 *
 *   q           [R][H][D] elements of q_dtype, row-major; rows of one request may
 *               sit anywhere, but request-major order lets rows share key reads.
 *   w           [R][H] f32, or NULL for w = 1.
 *   kcache      key pool in kv_layout (see qsa_kv_layout).
 *   kscale      QSA_KV_PAGED + fp8: [num_blocks][B] f32 or NULL (scale 1).
 *               Must be NULL for bf16, fp16 and the co-packed layouts.
 *   block_table [num_reqs][max_blocks] int32 pool block indices.
 *   ctx_lens    [R] int32 visible columns per row.
 *   row_to_req  [R] int32 row -> block_table row.
 *   out         [R][out_stride] f32; columns [0, W) of every row are written,
 *               columns [W, out_stride) are not touched.
 *
 * Visible count: ctx_eff[r] = clamp(ctx_lens[r], 0, min(W, max_blocks*B)).
 * Device preconditions: 0 <= row_to_req[r] < num_reqs; the first
 * ceil(ctx_eff/B) table entries of each row's request index blocks of the pool;
 * fp8 scales are >= 0 (the scale is applied after the ReLU, which equals
 * applying it to the key only for non-negative scales).  Out-of-range indices are
 * never dereferenced: a row_to_req value outside [0, num_reqs) makes that row's
 * visible columns NaN, and a table entry outside [0, num_blocks) makes the
 * columns it would feed NaN (with B a multiple of 16: the 16 columns of every
 * 16-column tile it feeds).
 *
 * Compiled set (else QSA_E_UNSUPPORTED): D in {64, 128}; H in {1,2,4,8,16,32,64};
 * B in [1, 1024] (B = 1: one key per table entry, the per-token layout of
 * ROCm/aiter PR #4221 before its KVBlockSize >= 1 commit; B not a multiple of 16
 * takes a per-column gather); bf16 + PAGED, fp16 + PAGED, fp8 + PAGED,
 * fp8 + COPACKED, fp8 + COPACKED_SHUFFLED (B a multiple of 16).
 * Alignment (else QSA_E_ALIGN): q, kcache, out 16-byte aligned; out_stride % 4 == 0.
 * Range (else QSA_E_RANGE): W <= 1<<24; R*out_stride*4 and num_blocks*block
 * bytes below 2^62.
 */
QSA_API qsa_status qsa_paged_logits(const void *q, const float *w, const void *kcache,
                            const float *kscale, const int32_t *block_table,
                            const int32_t *ctx_lens, const int32_t *row_to_req, float *out,
                            const qsa_logits_shape *shape, void *stream);

/* qsa_paged_logits, with the kernel timed: start_event / stop_event (hipEvent_t
 * created by the caller, or NULL) are recorded by the dispatch itself at the
 * kernel's start and end, so hipEventElapsedTime gives the kernel's duration
 * without marker-packet overhead.  For measurement tools; otherwise identical.
 * When the call launches nothing (R = 0 or W = 0) the events are not touched. */
QSA_API qsa_status qsa_paged_logits_timed(const void *q, const float *w, const void *kcache,
                                          const float *kscale, const int32_t *block_table,
                                          const int32_t *ctx_lens, const int32_t *row_to_req,
                                          float *out, const qsa_logits_shape *shape, void *stream,
                                          void *start_event, void *stop_event);

/* Validation of qsa_paged_logits' host-visible arguments only: no HIP call, no
 * launch.  Returns what qsa_paged_logits would return before launching. */
QSA_API qsa_status qsa_paged_logits_check(const void *q, const float *w, const void *kcache,
                                  const float *kscale, const int32_t *block_table,
                                  const int32_t *ctx_lens, const int32_t *row_to_req,
                                  const float *out, const qsa_logits_shape *shape);

/*
 * qsa_topk -- per row r, the k columns of its candidate range with the largest
 * logits; equal logits (+0 and -0 are equal) are broken toward the lower
 * column.  Rows with n_r <= k keep their whole range.
 *
 * Candidate range (vLLM PR #62589, "Details": top-k reads only the visible
 * columns; sglang PR #48649, "Accuracy Tests": the top-k takes per-row starts
 * and context lengths, and rows that fit in k keep everything):
 *   s_r = clamp(row_starts[r], 0, width)  (0 when row_starts is NULL),
 *   n_r = clamp(ctx_lens[r], 0, width - s_r),
 * the columns [s_r, s_r + n_r) of row r.  An index is reported as the offset
 * of its column from s_r, in [0, n_r): a row's result does not depend on where
 * its range sits in the buffer.
 *
 *   logits     [num_rows][logits_stride] f32 (the buffer holds num_rows *
 *              logits_stride floats); only the candidate range decides the
 *              result (reads are widened to whole 16-byte groups inside the
 *              row's stride).
 *   ctx_lens   [num_rows] int32: candidate count per row.
 *   row_starts [num_rows] int32, or NULL: first candidate column per row.
 *              Starts that are multiples of 4 take the same paths as no
 *              starts; other starts are exact but use the slower full-row
 *              selection for rows longer than k.
 *   idx_out    [num_rows][k] int32: the selected offsets in ascending order,
 *              then -1 in slots [min(k, n_r), k).  The order is part of this
 *              implementation, not of the selection's definition (a set).
 *
 * Device precondition: no NaN inside a candidate range (a NaN ranks by its bit
 * pattern: above +inf when its sign is clear, below -inf when set).
 *
 *   workspace  device scratch owned by the caller, or NULL.  With NULL every
 *              row is selected by one workgroup.  Otherwise it must hold at
 *              least qsa_topk_workspace_bytes(num_rows, width, k) bytes (else
 *              QSA_E_INVALID) at a 16-byte aligned address (else QSA_E_ALIGN).
 *              When that size is non-zero (at most 128 rows, width > 4096,
 *              and fewer than 48 rows or width > 32768), each row is shared
 *              by several workgroups in two kernels that pass counts and
 *              candidates through the workspace.  Its contents need
 *              no initialisation and are not kept between calls; calls that
 *              share a workspace must be ordered (same stream).  The selection
 *              does not depend on which path runs.
 *
 * Compiled set (else QSA_E_UNSUPPORTED): 1 <= k <= 2048; width <= 69632.
 * Alignment (else QSA_E_ALIGN): logits 16-byte aligned, logits_stride % 4 == 0.
 */
QSA_API qsa_status qsa_topk(const float *logits, int64_t logits_stride, const int32_t *ctx_lens,
                            const int32_t *row_starts, int32_t num_rows, int32_t width, int32_t k,
                            int32_t *idx_out, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * qsa_paged_logits_topk -- qsa_paged_logits, then qsa_topk on the logits it wrote
 * (row stride shape->out_stride, candidates [0, clamp(ctx_lens[r], 0, width)),
 * no row starts), in one call: the logits in `out` and the indices in idx_out
 * are exactly those of the two calls.  The pages time the whole selection, not
 * the scoring alone (vLLM PR #62589, "Performance": score + top-k, CUDA events
 * around both); here, for shapes that the per-tile scorer takes with 4 or fewer
 * heads (decode batches), its epilogue also writes each row's 16 largest scores
 * of every 64-column chunk into the workspace, and one selection kernel works
 * from those lists (a quarter of the row) instead of a sampling kernel and a
 * resolve kernel over the whole row.  Other shapes run the scoring kernel and
 * the plain selection.
 *
 *   q .. shape   as qsa_paged_logits (out is both its output and the
 *                selection's input).
 *   k, idx_out   as qsa_topk ([num_rows][k] int32, ascending, -1 padded).
 *   workspace    device scratch owned by the caller of at least
 *                qsa_paged_logits_topk_workspace_bytes(shape, k) bytes, 16-byte
 *                aligned (else QSA_E_INVALID / QSA_E_ALIGN), or NULL: no fusion
 *                and one workgroup per row for the selection (the results do
 *                not change).  No initialisation needed, nothing kept between
 *                calls; calls sharing a workspace must be ordered.
 *
 * Errors: those of qsa_paged_logits and of qsa_topk.  Device preconditions: both
 * calls'.  Asynchronous on `stream`; graph-capturable.
 */
QSA_API qsa_status qsa_paged_logits_topk(const void *q, const float *w, const void *kcache, const float *kscale,
                                         const int32_t *block_table, const int32_t *ctx_lens,
                                         const int32_t *row_to_req, float *out, const qsa_logits_shape *shape,
                                         int32_t k, int32_t *idx_out, void *workspace, int64_t workspace_bytes,
                                         void *stream);

/* Bytes of workspace qsa_paged_logits_topk uses for this shape (0 when none);
 * host-only, no HIP call. */
QSA_API int64_t qsa_paged_logits_topk_workspace_bytes(const qsa_logits_shape *shape, int32_t k);

/* qsa_paged_logits_topk with dispatch-recorded events (as qsa_paged_logits_timed):
 * start_event at the scoring kernel's start, mid_event at its end, stop_event at
 * the end of the selection.  Events may be NULL. */
QSA_API qsa_status qsa_paged_logits_topk_timed(const void *q, const float *w, const void *kcache,
                                               const float *kscale, const int32_t *block_table,
                                               const int32_t *ctx_lens, const int32_t *row_to_req, float *out,
                                               const qsa_logits_shape *shape, int32_t k, int32_t *idx_out,
                                               void *workspace, int64_t workspace_bytes, void *stream,
                                               void *start_event, void *mid_event, void *stop_event);

/*
 * qsa_topk_noalloc -- qsa_topk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same selection as qsa_topk with a workspace of
 * qsa_topk_workspace_bytes(num_rows, width, k) bytes, but the workspace is a
 * fixed 9 MiB device array held by the library (one per GPU, until the process
 * ends), so the call allocates nothing.  Every supported shape fits (the
 * largest needs 8,652,800 bytes); a shape that would not returns QSA_E_RANGE.
 * The array is that of the calling thread's current device, which must be the
 * device of `stream`.  Calls on one GPU share the array: calls that overlap
 * (concurrent streams, several threads) race; order them on one stream.
 * Arguments and other errors as qsa_topk.
 */
QSA_API qsa_status qsa_topk_noalloc(const float *logits, int64_t logits_stride, const int32_t *ctx_lens,
                                    const int32_t *row_starts, int32_t num_rows, int32_t width, int32_t k,
                                    int32_t *idx_out, void *stream);

/* Bytes of workspace qsa_topk uses for this shape; 0 when every row is selected
 * by one workgroup whatever the workspace.  Host-only, no HIP call; k does not
 * change the size in this version of the library. */
QSA_API int64_t qsa_topk_workspace_bytes(int32_t num_rows, int32_t width, int32_t k);

/* qsa_topk with its kernels timed by dispatch-recorded events (as
 * qsa_paged_logits_timed): start_event at the start of the first kernel,
 * stop_event at the end of the last. */
QSA_API qsa_status qsa_topk_timed(const float *logits, int64_t logits_stride, const int32_t *ctx_lens,
                                  const int32_t *row_starts, int32_t num_rows, int32_t width, int32_t k,
                                  int32_t *idx_out, void *workspace, int64_t workspace_bytes, void *stream,
                                  void *start_event, void *stop_event);

/* Validation of qsa_topk's host-visible arguments only: no HIP call, no launch. */
QSA_API qsa_status qsa_topk_check(const float *logits, int64_t logits_stride, const int32_t *ctx_lens,
                                  const int32_t *row_starts, int32_t num_rows, int32_t width, int32_t k,
                                  const int32_t *idx_out, const void *workspace, int64_t workspace_bytes);

/*
 * qsa_expand -- the step after the selection: each selected compressed column
 * becomes the key tokens it stands for.  The pages time a full selection as
 * "score + top-k + expand" with a compression ratio of 4 (vLLM PR #62589,
 * "Performance" and the MI355X comment) without defining the step; this is the
 * plain reading: compressed column c covers tokens [c * ratio, c * ratio + ratio).
 *
 *   idx         [num_rows][k] int32 selected columns (qsa_topk's output; -1 is
 *               padding).
 *   token_lens  [num_rows] int32 tokens per row, or NULL for no bound.
 *   tokens_out  [num_rows][k * ratio] int32: slot p * ratio + j holds
 *               idx[r][p] * ratio + j when idx[r][p] >= 0 and that token is below
 *               token_lens[r] (and fits in int32), else -1.  Ascending columns
 *               give ascending tokens.
 *
 * Errors: QSA_E_INVALID for null pointers with num_rows > 0, num_rows < 0,
 * k < 1 or ratio < 1; QSA_E_RANGE when k * ratio > 2^24.
 */
QSA_API qsa_status qsa_expand(const int32_t *idx, int32_t num_rows, int32_t k, int32_t ratio,
                              const int32_t *token_lens, int32_t *tokens_out, void *stream);

/* Message for the calling thread's last non-OK status ("" if none). Owned by the
 * library; valid until the thread's next call. */
QSA_API const char *qsa_last_error(void);

/* Library version string, e.g. "qsaidx 0.1.0 gfx950". */
QSA_API const char *qsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSAIDX_H */
