// C-ABI entry points of libqsaidx: argument validation, variant choice and
// launches.  Validation reads host scalars only; nothing here synchronises the
// device or reads device memory, so every call can be graph-captured
// (vLLM PR #62589, Dispatch: host values only, no device sync).
#include <stdarg.h>
#include <stdio.h>

#include "qsa_internal.h"
#include "qsaidx.h"

namespace {

thread_local char g_err[512] = "";

qsa_status fail(qsa_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

qsa_status ok() {
    g_err[0] = '\0';
    return QSA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxBytes = (int64_t)1 << 62;

qsa_status check_logits(const void *q, const float *w, const void *kcache, const float *kscale,
                        const int32_t *block_table, const int32_t *ctx_lens,
                        const int32_t *row_to_req, const float *out, const qsa_logits_shape *s) {
    (void)w;
    if (!s) return fail(QSA_E_INVALID, "shape is NULL");
    if (s->num_rows < 0) return fail(QSA_E_INVALID, "num_rows = %d < 0", s->num_rows);
    if (s->width < 0) return fail(QSA_E_INVALID, "width = %d < 0", s->width);
    if (s->num_heads < 1 || s->head_dim < 1 || s->block_size < 1 || s->num_reqs < 1 ||
        s->max_blocks < 1 || s->num_blocks < 1)
        return fail(QSA_E_INVALID,
                    "num_heads, head_dim, block_size, num_reqs, max_blocks and num_blocks must be >= 1");
    if (s->out_stride < s->width)
        return fail(QSA_E_INVALID, "out_stride = %lld < width = %d", (long long)s->out_stride, s->width);
    const bool empty = s->num_rows == 0 || s->width == 0;
    if (!empty && (!q || !kcache || !block_table || !ctx_lens || !row_to_req || !out))
        return fail(QSA_E_INVALID, "q, kcache, block_table, ctx_lens, row_to_req and out must be non-NULL");
    auto known = [](int32_t d) { return d == QSA_BF16 || d == QSA_FP8_E4M3FN || d == QSA_FP16; };
    if (!known(s->q_dtype) || !known(s->k_dtype))
        return fail(QSA_E_DTYPE, "unknown dtype (q %d, k %d)", s->q_dtype, s->k_dtype);
    if (s->q_dtype != s->k_dtype)
        return fail(QSA_E_DTYPE, "q and k dtypes differ (q %d, k %d)", s->q_dtype, s->k_dtype);
    if (s->kv_layout != QSA_KV_PAGED && s->kv_layout != QSA_KV_COPACKED && s->kv_layout != QSA_KV_COPACKED_SHUFFLED)
        return fail(QSA_E_INVALID, "unknown kv_layout %d", s->kv_layout);
    const bool copacked = s->kv_layout != QSA_KV_PAGED;
    if (copacked && s->k_dtype != QSA_FP8_E4M3FN)
        return fail(QSA_E_UNSUPPORTED, "the co-packed layouts hold fp8 keys only");
    if (s->kv_layout == QSA_KV_COPACKED_SHUFFLED && s->block_size % 16 != 0)
        return fail(QSA_E_UNSUPPORTED, "the preshuffled layout needs block_size %% 16 == 0 (got %d)", s->block_size);
    if (kscale && (s->k_dtype != QSA_FP8_E4M3FN || s->kv_layout != QSA_KV_PAGED))
        return fail(QSA_E_INVALID, "kscale applies to fp8 keys in the paged layout only");
    if (s->head_dim != 128 && s->head_dim != 64)
        return fail(QSA_E_UNSUPPORTED, "head_dim = %d (built: 64, 128)", s->head_dim);
    const int H = s->num_heads;
    if (H > 64 || (H & (H - 1)) != 0)
        return fail(QSA_E_UNSUPPORTED, "num_heads = %d (built: 1, 2, 4, 8, 16, 32, 64)", H);
    if (s->block_size > 1024)
        return fail(QSA_E_UNSUPPORTED, "block_size = %d (built: 1 to 1024)", s->block_size);
    if (s->width > (1 << 24)) return fail(QSA_E_RANGE, "width = %d > 2^24", s->width);
    if ((int64_t)s->num_rows * s->out_stride > kMaxBytes / 4)
        return fail(QSA_E_RANGE, "num_rows * out_stride too large");
    const int64_t elt = s->k_dtype == QSA_FP8_E4M3FN ? 1 : 2;
    const int64_t block_bytes = (int64_t)s->block_size * s->head_dim * elt +
                                (copacked ? 4 * (int64_t)s->block_size : 0);
    if (s->num_blocks > kMaxBytes / block_bytes) return fail(QSA_E_RANGE, "key pool too large");
    if ((int64_t)s->num_reqs * s->max_blocks > ((int64_t)1 << 40))
        return fail(QSA_E_RANGE, "block table too large");
    if (!empty && (!aligned16(q) || !aligned16(kcache) || !aligned16(out)))
        return fail(QSA_E_ALIGN, "q, kcache and out must be 16-byte aligned");
    if (!empty && s->out_stride % 4 != 0) return fail(QSA_E_ALIGN, "out_stride must be a multiple of 4");
    return ok();
}

// row_starts needs no host check: NULL means every start is 0, and any device
// value is clamped to [0, width] by the kernels.
qsa_status check_topk(const float *logits, int64_t stride, const int32_t *ctx_lens, int32_t num_rows,
                      int32_t width, int32_t k, const int32_t *idx_out, const void *workspace,
                      int64_t workspace_bytes) {
    if (num_rows < 0) return fail(QSA_E_INVALID, "num_rows = %d < 0", num_rows);
    if (width < 0) return fail(QSA_E_INVALID, "width = %d < 0", width);
    if (k < 1) return fail(QSA_E_INVALID, "k = %d < 1", k);
    if (stride < width) return fail(QSA_E_INVALID, "logits_stride = %lld < width = %d", (long long)stride, width);
    if (num_rows > 0 && (!logits || !ctx_lens || !idx_out))
        return fail(QSA_E_INVALID, "logits, ctx_lens and idx_out must be non-NULL");
    if (k > 2048) return fail(QSA_E_UNSUPPORTED, "k = %d (built: 1..2048)", k);
    if (qsa::topk_groups_for_width(width) == 0)
        return fail(QSA_E_UNSUPPORTED, "width = %d (built: up to 69632)", width);
    if ((int64_t)num_rows * stride > kMaxBytes / 4) return fail(QSA_E_RANGE, "num_rows * logits_stride too large");
    if (num_rows > 0 && !aligned16(logits)) return fail(QSA_E_ALIGN, "logits must be 16-byte aligned");
    if (num_rows > 0 && stride % 4 != 0) return fail(QSA_E_ALIGN, "logits_stride must be a multiple of 4");
    if (workspace) {
        const int64_t need = qsa::topk_workspace_bytes(num_rows, width);
        if (workspace_bytes < need)
            return fail(QSA_E_INVALID, "workspace_bytes = %lld < %lld", (long long)workspace_bytes, (long long)need);
        if (need > 0 && !aligned16(workspace)) return fail(QSA_E_ALIGN, "workspace must be 16-byte aligned");
    }
    return ok();
}

// The fused call writes chunk candidates from the scoring epilogue when the
// per-tile kernel scores the shape with 4 or fewer heads (one score per lane
// and 16-column tile, 64-column chunks); every other shape runs the scoring
// kernel and then the plain selection.
bool fused_candidates(const qsa::LogitsPlan &p, const qsa_logits_shape *s) {
    return !p.prefill && !p.mtp && p.iters == 0 && s->num_heads <= 4 && p.tiles_per_prog == 4;
}

int64_t fused_workspace_bytes(const qsa_logits_shape *s) {
    if (s->num_rows <= 0 || s->width <= 0) return 0;
    const qsa::LogitsPlan p = qsa::plan_logits(s->k_dtype, s->kv_layout, s->head_dim, s->num_heads, s->num_rows,
                                               s->num_reqs, s->width, s->block_size, s->out_stride);
    if (fused_candidates(p, s)) return (int64_t)s->num_rows * ((s->width + 63) / 64) * 128;
    return qsa::topk_workspace_bytes(s->num_rows, s->width);
}

}  // namespace

extern "C" {

qsa_status qsa_paged_logits_check(const void *q, const float *w, const void *kcache, const float *kscale,
                                  const int32_t *block_table, const int32_t *ctx_lens,
                                  const int32_t *row_to_req, const float *out, const qsa_logits_shape *shape) {
    return check_logits(q, w, kcache, kscale, block_table, ctx_lens, row_to_req, out, shape);
}

qsa_status qsa_paged_logits(const void *q, const float *w, const void *kcache, const float *kscale,
                            const int32_t *block_table, const int32_t *ctx_lens, const int32_t *row_to_req,
                            float *out, const qsa_logits_shape *s, void *stream) {
    return qsa_paged_logits_timed(q, w, kcache, kscale, block_table, ctx_lens, row_to_req, out, s, stream,
                                  nullptr, nullptr);
}

}  // extern "C"

namespace {

// The launch description of a checked qsa_paged_logits call.
qsa::LogitsArgs logits_args(const void *q, const float *w, const void *kcache, const float *kscale,
                            const int32_t *block_table, const int32_t *ctx_lens, const int32_t *row_to_req,
                            float *out, const qsa_logits_shape *s, const qsa::LogitsPlan &plan) {
    const bool fp8 = s->k_dtype == QSA_FP8_E4M3FN;
    const int64_t elt = fp8 ? 1 : 2;
    qsa::LogitsArgs a = {};
    a.q = q;
    a.w = w;
    a.kcache = static_cast<const uint8_t *>(kcache);
    a.kscale = kscale;
    a.block_table = block_table;
    a.ctx_lens = ctx_lens;
    a.row_to_req = row_to_req;
    a.out = out;
    a.num_rows = s->num_rows;
    a.num_heads = s->num_heads;
    a.block_size = s->block_size;
    a.num_reqs = s->num_reqs;
    a.max_blocks = s->max_blocks;
    a.width = s->width;
    const int64_t table_cols = (int64_t)s->max_blocks * s->block_size;
    a.cap = (int32_t)(table_cols < s->width ? table_cols : s->width);
    a.num_row_tiles = plan.mtp ? plan.row_tiles : (s->num_rows + plan.rows_per_tile - 1) / plan.rows_per_tile;
    a.mtp_aligned = plan.mtp && plan.mtp_aligned;
    const int chunk_cols = 16 * plan.tiles_per_prog;
    a.num_chunks = (s->width + chunk_cols - 1) / chunk_cols;
    a.dtype = s->k_dtype;
    a.layout = s->kv_layout;
    a.num_blocks = s->num_blocks;
    a.out_stride = s->out_stride;
    a.key_stride = s->head_dim * elt;
    a.head_dim = s->head_dim;
    a.block_bytes = (int64_t)s->block_size * a.key_stride + (s->kv_layout != QSA_KV_PAGED ? 4 * s->block_size : 0);
    a.scale_offset = (int64_t)s->block_size * a.key_stride;
    a.iters = plan.iters;
    a.cand = nullptr;
    return a;
}

qsa::LogitsPlan plan_of(const qsa_logits_shape *s) {
    // the kernels' dtype codes are the qsa_dtype values
    static_assert(QSA_BF16 == qsa::kBF16 && QSA_FP8_E4M3FN == qsa::kFP8 && QSA_FP16 == qsa::kFP16, "dtype codes");
    return qsa::plan_logits(s->k_dtype, s->kv_layout, s->head_dim, s->num_heads, s->num_rows, s->num_reqs, s->width,
                            s->block_size, s->out_stride);
}

}  // namespace

extern "C" {

qsa_status qsa_paged_logits_timed(const void *q, const float *w, const void *kcache, const float *kscale,
                                  const int32_t *block_table, const int32_t *ctx_lens,
                                  const int32_t *row_to_req, float *out, const qsa_logits_shape *s,
                                  void *stream, void *start_event, void *stop_event) {
    qsa_status st = check_logits(q, w, kcache, kscale, block_table, ctx_lens, row_to_req, out, s);
    if (st != QSA_OK) return st;
    if (s->num_rows == 0 || s->width == 0) return ok();
    const qsa::LogitsPlan plan = plan_of(s);
    qsa::LogitsArgs a = logits_args(q, w, kcache, kscale, block_table, ctx_lens, row_to_req, out, s, plan);
    if ((int64_t)a.num_row_tiles * a.num_chunks > 0x7FFFFFFF)
        return fail(QSA_E_RANGE, "grid too large (%d row tiles x %d chunks)", a.num_row_tiles, a.num_chunks);
    hipError_t e = qsa::launch_paged_logits(a, plan, static_cast<hipStream_t>(stream),
                                            static_cast<hipEvent_t>(start_event),
                                            static_cast<hipEvent_t>(stop_event));
    if (e != hipSuccess) return fail(QSA_E_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

int64_t qsa_paged_logits_topk_workspace_bytes(const qsa_logits_shape *shape, int32_t k) {
    (void)k;
    if (!shape) return 0;
    return fused_workspace_bytes(shape);
}

qsa_status qsa_paged_logits_topk_timed(const void *q, const float *w, const void *kcache, const float *kscale,
                                       const int32_t *block_table, const int32_t *ctx_lens,
                                       const int32_t *row_to_req, float *out, const qsa_logits_shape *s,
                                       int32_t k, int32_t *idx_out, void *workspace, int64_t workspace_bytes,
                                       void *stream, void *start_event, void *mid_event, void *stop_event) {
    qsa_status st = check_logits(q, w, kcache, kscale, block_table, ctx_lens, row_to_req, out, s);
    if (st != QSA_OK) return st;
    st = check_topk(out, s->out_stride, ctx_lens, s->num_rows, s->width, k, idx_out, nullptr, 0);
    if (st != QSA_OK) return st;
    const int64_t need = fused_workspace_bytes(s);
    if (workspace) {
        if (workspace_bytes < need)
            return fail(QSA_E_INVALID, "workspace_bytes = %lld < %lld", (long long)workspace_bytes, (long long)need);
        if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
            return fail(QSA_E_ALIGN, "workspace must be 16-byte aligned");
    }
    if (s->num_rows == 0) return ok();
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const qsa::LogitsPlan plan = plan_of(s);
    qsa::LogitsArgs a = logits_args(q, w, kcache, kscale, block_table, ctx_lens, row_to_req, out, s, plan);
    if ((int64_t)a.num_row_tiles * a.num_chunks > 0x7FFFFFFF)
        return fail(QSA_E_RANGE, "grid too large (%d row tiles x %d chunks)", a.num_row_tiles, a.num_chunks);
    const bool fused = workspace && s->width > 0 && fused_candidates(plan, s);
    if (fused) a.cand = static_cast<uint32_t *>(workspace);
    hipError_t e = hipSuccess;
    if (s->width > 0)
        e = qsa::launch_paged_logits(a, plan, hs, static_cast<hipEvent_t>(start_event),
                                     static_cast<hipEvent_t>(mid_event));
    if (e != hipSuccess) return fail(QSA_E_HIP, "launch failed: %s", hipGetErrorString(e));
    qsa::TopkArgs t = {};
    t.logits = out;
    t.stride = s->out_stride;
    t.ctx_lens = ctx_lens;
    t.row_starts = nullptr;
    t.num_rows = s->num_rows;
    t.width = s->width;
    t.k = k;
    t.idx_out = idx_out;
    t.slices = 1;
    t.slice_len = s->width;
    if (fused) {
        t.cand = a.cand;
        t.cand_chunks = a.num_chunks;
        t.cap = a.cap;
        e = qsa::launch_topk_cand(t, hs, nullptr, static_cast<hipEvent_t>(stop_event));
    } else {
        if (workspace) {
            const qsa::TopkPlan p = qsa::plan_topk(s->num_rows, s->width);
            if (p.slices > 1) {
                t.workspace = static_cast<uint8_t *>(workspace);
                t.slices = p.slices;
                t.slice_len = p.slice_len;
                t.groups = p.groups;
                t.cand_shift = p.cand_shift;
            }
        }
        e = qsa::launch_topk(t, hs, nullptr, static_cast<hipEvent_t>(stop_event));
    }
    if (e != hipSuccess) return fail(QSA_E_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

qsa_status qsa_paged_logits_topk(const void *q, const float *w, const void *kcache, const float *kscale,
                                 const int32_t *block_table, const int32_t *ctx_lens, const int32_t *row_to_req,
                                 float *out, const qsa_logits_shape *shape, int32_t k, int32_t *idx_out,
                                 void *workspace, int64_t workspace_bytes, void *stream) {
    return qsa_paged_logits_topk_timed(q, w, kcache, kscale, block_table, ctx_lens, row_to_req, out, shape, k,
                                       idx_out, workspace, workspace_bytes, stream, nullptr, nullptr, nullptr);
}

int64_t qsa_topk_workspace_bytes(int32_t num_rows, int32_t width, int32_t k) {
    (void)k;
    if (num_rows < 0 || width < 0) return 0;
    return qsa::topk_workspace_bytes(num_rows, width);
}

qsa_status qsa_topk_check(const float *logits, int64_t logits_stride, const int32_t *ctx_lens,
                          const int32_t *row_starts, int32_t num_rows, int32_t width, int32_t k,
                          const int32_t *idx_out, const void *workspace, int64_t workspace_bytes) {
    (void)row_starts;
    return check_topk(logits, logits_stride, ctx_lens, num_rows, width, k, idx_out, workspace, workspace_bytes);
}

qsa_status qsa_topk(const float *logits, int64_t logits_stride, const int32_t *ctx_lens, const int32_t *row_starts,
                    int32_t num_rows, int32_t width, int32_t k, int32_t *idx_out, void *workspace,
                    int64_t workspace_bytes, void *stream) {
    return qsa_topk_timed(logits, logits_stride, ctx_lens, row_starts, num_rows, width, k, idx_out, workspace,
                          workspace_bytes, stream, nullptr, nullptr);
}

qsa_status qsa_topk_timed(const float *logits, int64_t logits_stride, const int32_t *ctx_lens,
                          const int32_t *row_starts, int32_t num_rows, int32_t width, int32_t k, int32_t *idx_out,
                          void *workspace, int64_t workspace_bytes, void *stream, void *start_event,
                          void *stop_event) {
    qsa_status st = check_topk(logits, logits_stride, ctx_lens, num_rows, width, k, idx_out, workspace,
                               workspace_bytes);
    if (st != QSA_OK) return st;
    if (num_rows == 0) return ok();
    qsa::TopkArgs a = {};
    a.logits = logits;
    a.stride = logits_stride;
    a.ctx_lens = ctx_lens;
    a.row_starts = row_starts;
    a.num_rows = num_rows;
    a.width = width;
    a.k = k;
    a.idx_out = idx_out;
    a.slices = 1;
    a.slice_len = width;
    if (workspace) {
        const qsa::TopkPlan p = qsa::plan_topk(num_rows, width);
        if (p.slices > 1) {
            a.workspace = static_cast<uint8_t *>(workspace);
            a.slices = p.slices;
            a.slice_len = p.slice_len;
            a.groups = p.groups;
            a.cand_shift = p.cand_shift;
        }
    }
    hipError_t e = qsa::launch_topk(a, static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(start_event),
                                    static_cast<hipEvent_t>(stop_event));
    if (e != hipSuccess) return fail(QSA_E_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

qsa_status qsa_topk_noalloc(const float *logits, int64_t logits_stride, const int32_t *ctx_lens,
                            const int32_t *row_starts, int32_t num_rows, int32_t width, int32_t k,
                            int32_t *idx_out, void *stream) {
    qsa_status st = check_topk(logits, logits_stride, ctx_lens, num_rows, width, k, idx_out, nullptr, 0);
    if (st != QSA_OK) return st;
    if (num_rows == 0) return ok();
    const int64_t need = qsa::topk_workspace_bytes(num_rows, width);
    if (need > qsa::kTopkScratchBytes)
        return fail(QSA_E_RANGE, "the selection needs %lld bytes of scratch; the library holds %lld",
                    (long long)need, (long long)qsa::kTopkScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        hipError_t e = qsa::topk_scratch(&ws);
        if (e != hipSuccess) return fail(QSA_E_HIP, "scratch lookup failed: %s", hipGetErrorString(e));
    }
    return qsa_topk_timed(logits, logits_stride, ctx_lens, row_starts, num_rows, width, k, idx_out, ws, need,
                          stream, nullptr, nullptr);
}

qsa_status qsa_expand(const int32_t *idx, int32_t num_rows, int32_t k, int32_t ratio, const int32_t *token_lens,
                      int32_t *tokens_out, void *stream) {
    if (num_rows < 0) return fail(QSA_E_INVALID, "num_rows = %d < 0", num_rows);
    if (k < 1) return fail(QSA_E_INVALID, "k = %d < 1", k);
    if (ratio < 1) return fail(QSA_E_INVALID, "ratio = %d < 1", ratio);
    if ((int64_t)k * ratio > ((int64_t)1 << 24))
        return fail(QSA_E_RANGE, "k * ratio = %lld > 2^24", (long long)k * ratio);
    if (num_rows == 0) return ok();
    if (!idx || !tokens_out) return fail(QSA_E_INVALID, "idx and tokens_out must be non-NULL");
    qsa::ExpandArgs a = {idx, token_lens, tokens_out, num_rows, k, ratio};
    hipError_t e = qsa::launch_expand(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(QSA_E_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

const char *qsa_last_error(void) { return g_err; }

const char *qsa_version(void) { return "qsaidx 0.1.0 gfx950"; }

}  // extern "C"
