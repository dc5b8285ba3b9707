/*
 * CPU oracle for paged MQA-logits scoring and per-row top-k.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the GPU path computes.  Only the test-suite, the smoke
 * check and the benchmark's CPU-baseline leg load it; the product path never
 * does.  It shares no source, header or helper with the HIP library.
 *
 * Arithmetic is float64 (inputs are bf16 / fp16 / fp8 / f32, all exact in float64),
 * loops run in the order the definition is written, and the file is compiled
 * with -O2 -ffp-contract=off and without -ffast-math.  OpenMP only splits rows
 * across threads; each output is computed by one thread in a fixed order.
 *
 * Sources (pages on the subject):
 *  - ROCm/ATOM PR #2651, "Changes": a row's heads are scored against a key
 *    column, ReLU is applied per head, then the heads are summed.
 *  - sglang PR #48649, "Accuracy Tests": zero-padded heads add 0 after the ReLU.
 *  - ROCm/aiter PR #4221, "Motivation" and "Technical details": fp8 e4m3 q and
 *    keys, per-key f32 scale, f32 weights w[row, head], output f32; the
 *    block-flat co-packed block (KVB key rows, then KVB f32 scales) and the
 *    block-table gather kv_indices[b, col // KVB], slot col % KVB (the commit
 *    that extends the fp8 paged kernel to any block size); the -inf mask is
 *    compared exactly by its test gate.
 *  - vLLM PR #62589, "Overview"/"Details": columns past a row's visible count
 *    are masked; "Validation": top-k reads only [0, visible), compared as sets;
 *    "Details": fp16 q and keys are scored as fp16 (dtype code 2 here).
 *
 * Pins (tests/test_oracle_pins.py) tie every function here to something other
 * than itself: library fp8/bf16/fp16 conversions, one-hot closed forms, GEMV special
 * cases, invariants (zero heads, permutation, scale powers of two), and brute
 * force over all subsets for the selection.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORA_OK 0
#define ORA_E_ARG (-1)
#define ORA_E_NAN (-2)
#define ORA_E_TABLE (-3)

/* bfloat16 is the top half of an IEEE binary32; widening is exact. */
double ora_bf16_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * IEEE 754 binary16: 1 sign bit, 5 exponent bits with bias 15, 10 mantissa
 * bits; exponent field 0 encodes subnormals m/1024 * 2^-14; exponent field 31
 * is infinity (m = 0) or NaN.  Every binary16 value is exact in float64.
 */
double ora_fp16_to_double(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1F;
    int m = bits & 0x3FF;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m / 1024.0, -14);
    else
        v = ldexp(1.0 + (double)m / 1024.0, e - 15);
    return sign ? -v : v;
}

/* element `at` of a bf16 (dtype 0) or fp16 (dtype 2) array, as float64 */
static double half_elem(const void *p, int dtype, int64_t at)
{
    uint16_t b = ((const uint16_t *)p)[at];
    return dtype == 0 ? ora_bf16_to_double(b) : ora_fp16_to_double(b);
}

/*
 * OCP 8-bit floating point, E4M3 "fn" variant (the fp8 e4m3 of ROCm/aiter
 * PR #4221 on gfx950): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent field 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN;
 * there are no infinities, so S.1111.110 = 448 is the largest magnitude.
 */
double ora_e4m3fn_to_double(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* fetch key column `col` of request `req` through the block table, dequantised
 * to float64 (ROCm/aiter PR #4221 KVBlockSize commit; sglang PR #48649 test
 * body: page_table rows index a [pages, page_size, 1, D] cache). */
static int fetch_key(double *kd, int dtype, int layout, const void *kcache, const float *kscale,
                     const int32_t *block_table, int max_blocks, int64_t num_blocks,
                     int block_size, int head_dim, int req, int col)
{
    int32_t blk = block_table[(int64_t)req * max_blocks + col / block_size];
    int slot = col % block_size;
    if (blk < 0 || (int64_t)blk >= num_blocks)
        return ORA_E_TABLE;
    if (dtype == 0 || dtype == 2) {
        int64_t base = ((int64_t)blk * block_size + slot) * head_dim;
        for (int d = 0; d < head_dim; ++d)
            kd[d] = half_elem(kcache, dtype, base + d);
        return ORA_OK;
    }
    const uint8_t *k;
    double s = 1.0;
    if (layout == 0) {
        k = (const uint8_t *)kcache + ((int64_t)blk * block_size + slot) * head_dim;
        if (kscale)
            s = (double)kscale[(int64_t)blk * block_size + slot];
    } else {
        /* co-packed block: block_size keys of head_dim bytes, then block_size
         * little-endian f32 scales */
        const uint8_t *base = (const uint8_t *)kcache +
                              (int64_t)blk * block_size * (head_dim + 4);
        float sf;
        memcpy(&sf, base + (int64_t)block_size * head_dim + 4 * slot, sizeof sf);
        s = (double)sf;
        if (layout == 2) {
            /* preshuffled keys (ROCm/aiter PR #4221, preshuffle commit): each
             * group of 16 slots is head_dim/16 chunks of 16 slots x 16 bytes */
            const uint8_t *g = base + (int64_t)(slot / 16) * 16 * head_dim;
            for (int d = 0; d < head_dim; ++d)
                kd[d] = ora_e4m3fn_to_double(g[(d / 16) * 256 + (slot % 16) * 16 + d % 16]) * s;
            return ORA_OK;
        }
        k = base + (int64_t)slot * head_dim;
    }
    /* dequantise, then dot: k_f[d] = fp8(k[d]) * scale */
    for (int d = 0; d < head_dim; ++d)
        kd[d] = ora_e4m3fn_to_double(k[d]) * s;
    return ORA_OK;
}

/*
 * logit[row, col] = sum_h w[row, h] * ReLU( sum_d q[row, h, d] * k[col, d] )
 * for col < ctx_eff[row]; -inf for ctx_eff[row] <= col < width.
 * ctx_eff = clamp(ctx[row], 0, min(width, max_blocks * block_size)).
 * w == NULL means every weight is 1.
 *
 * `rows` selects which rows to compute (NULL: all); out is [n_rows][width].
 */
int ora_paged_logits(const void *q, int dtype, const float *w, const void *kcache, int layout,
                     const float *kscale, const int32_t *block_table, const int32_t *ctx_lens,
                     const int32_t *row_to_req, int num_rows, int num_heads, int head_dim,
                     int block_size, int num_reqs, int max_blocks, int64_t num_blocks,
                     int width, const int32_t *rows, int n_rows, double *out, int n_threads)
{
    if (!q || !kcache || !block_table || !ctx_lens || !row_to_req || !out)
        return ORA_E_ARG;
    if (num_rows < 0 || num_heads < 1 || head_dim < 1 || block_size < 1 || num_reqs < 1 ||
        max_blocks < 1 || num_blocks < 1 || width < 0 || n_rows < 0)
        return ORA_E_ARG;
    if (dtype != 0 && dtype != 1 && dtype != 2)
        return ORA_E_ARG;
    if (dtype != 1 && layout != 0)
        return ORA_E_ARG;
    if (layout < 0 || layout > 2 || (layout == 2 && (block_size % 16 != 0 || head_dim % 16 != 0)))
        return ORA_E_ARG;
    if (!rows)
        n_rows = num_rows;
    int64_t cap = (int64_t)max_blocks * block_size;
    if (cap > width)
        cap = width;
    int status = ORA_OK;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int i = 0; i < n_rows; ++i) {
        int row = rows ? rows[i] : i;
        double *o = out + (int64_t)i * width;
        if (row < 0 || row >= num_rows) {
            status = ORA_E_ARG;
            continue;
        }
        int req = row_to_req[row];
        if (req < 0 || req >= num_reqs) {
            status = ORA_E_ARG;
            continue;
        }
        int64_t ctx = ctx_lens[row];
        if (ctx < 0)
            ctx = 0;
        if (ctx > cap)
            ctx = cap;
        double *qd = (double *)malloc(sizeof(double) * (size_t)num_heads * head_dim);
        double *kd = (double *)malloc(sizeof(double) * (size_t)head_dim);
        if (!qd || !kd) {
            free(qd);
            free(kd);
            status = ORA_E_ARG;
            continue;
        }
        for (int h = 0; h < num_heads; ++h)
            for (int d = 0; d < head_dim; ++d) {
                int64_t at = ((int64_t)row * num_heads + h) * head_dim + d;
                qd[h * head_dim + d] = dtype == 1 ? ora_e4m3fn_to_double(((const uint8_t *)q)[at])
                                                  : half_elem(q, dtype, at);
            }
        for (int64_t col = 0; col < ctx; ++col) {
            if (fetch_key(kd, dtype, layout, kcache, kscale, block_table, max_blocks, num_blocks,
                          block_size, head_dim, req, (int)col) != ORA_OK) {
                status = ORA_E_TABLE;
                o[col] = NAN;
                continue;
            }
            double acc = 0.0;
            for (int h = 0; h < num_heads; ++h) {
                double dot = 0.0;
                for (int d = 0; d < head_dim; ++d)
                    dot += qd[h * head_dim + d] * kd[d];
                double relu = dot > 0.0 ? dot : 0.0;
                double wh = w ? (double)w[(int64_t)row * num_heads + h] : 1.0;
                acc += wh * relu;
            }
            o[col] = acc;
        }
        for (int64_t col = ctx; col < width; ++col)
            o[col] = -INFINITY;
        free(qd);
        free(kd);
    }
    return status;
}

/* ------------------------------------------------------------------------ */
/* per-row top-k                                                              */
/* ------------------------------------------------------------------------ */

typedef struct {
    float v;
    int32_t i;
} ora_cand;

/* larger value first; equal values (+0 and -0 are equal) by lower column */
static int cand_cmp(const void *pa, const void *pb)
{
    const ora_cand *a = (const ora_cand *)pa, *b = (const ora_cand *)pb;
    if (a->v > b->v)
        return -1;
    if (a->v < b->v)
        return 1;
    return (a->i > b->i) - (a->i < b->i);
}

/*
 * Per row: candidates are the n columns from the row's start s, with
 * s = clamp(row_starts[row], 0, width) (0 without starts) and
 * n = clamp(ctx[row], 0, width - s); the min(k, n) with the largest logits are
 * kept, among equal logits the lower column.  Each is reported as its offset
 * from s (sglang PR #48649 test body: the top-k takes per-row starts and
 * context lengths).  Slots past min(k, n) hold -1.  Emitted in (value desc,
 * column asc) order; the contract is the set (vLLM PR #62589, Validation:
 * compared as sets; the same test body: entries < 0 are padding).
 * Returns ORA_E_NAN when a NaN lies inside a candidate range: a precondition
 * violation.
 */
int ora_topk(const float *logits, int64_t stride, const int32_t *ctx_lens, const int32_t *row_starts,
             int num_rows, int width, int k, int32_t *idx_out, int n_threads)
{
    if (!logits || !ctx_lens || !idx_out || num_rows < 0 || width < 0 || k < 1 ||
        stride < width)
        return ORA_E_ARG;
    int status = ORA_OK;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int row = 0; row < num_rows; ++row) {
        int64_t s = row_starts ? row_starts[row] : 0;
        if (s < 0)
            s = 0;
        if (s > width)
            s = width;
        int64_t n = ctx_lens[row];
        if (n < 0)
            n = 0;
        if (n > width - s)
            n = width - s;
        int32_t *o = idx_out + (int64_t)row * k;
        ora_cand *c = (ora_cand *)malloc(sizeof(ora_cand) * (size_t)(n > 0 ? n : 1));
        if (!c) {
            status = ORA_E_ARG;
            continue;
        }
        const float *x = logits + (int64_t)row * stride + s;
        int bad = 0;
        for (int64_t j = 0; j < n; ++j) {
            c[j].v = x[j];
            c[j].i = (int32_t)j;
            if (isnan(x[j]))
                bad = 1;
        }
        if (bad) {
            status = ORA_E_NAN;
            for (int j = 0; j < k; ++j)
                o[j] = -1;
            free(c);
            continue;
        }
        qsort(c, (size_t)n, sizeof(ora_cand), cand_cmp);
        int64_t take = n < k ? n : k;
        for (int64_t j = 0; j < take; ++j)
            o[j] = c[j].i;
        for (int64_t j = take; j < k; ++j)
            o[j] = -1;
        free(c);
    }
    return status;
}

/*
 * Expand: the tokens of each selected compressed column.  The pages time the
 * full selection as score + top-k + expand with compression ratio 4 (vLLM
 * PR #62589, Performance table heading and the MI355X comment) but do not
 * define the step; the reading taken: column c stands for the `ratio` tokens
 * c * ratio + j, j = 0 .. ratio - 1.  out[row][p * ratio + j] is that token for
 * the p-th selected column when the column is not padding (>= 0) and the token
 * lies below the row's token count (no bound without token_lens) and fits in
 * int32; -1 otherwise.
 */
int ora_expand(const int32_t *idx, int num_rows, int k, int ratio, const int32_t *token_lens,
               int32_t *out)
{
    if (!idx || !out || num_rows < 0 || k < 1 || ratio < 1)
        return ORA_E_ARG;
    for (int row = 0; row < num_rows; ++row) {
        for (int p = 0; p < k; ++p) {
            int32_t c = idx[(int64_t)row * k + p];
            for (int j = 0; j < ratio; ++j) {
                int64_t tok = (int64_t)c * ratio + j;
                int keep = c >= 0 && tok <= INT32_MAX &&
                           (!token_lens || tok < (int64_t)token_lens[row]);
                out[((int64_t)row * k + p) * ratio + j] = keep ? (int32_t)tok : -1;
            }
        }
    }
    return ORA_OK;
}

int ora_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
