// Paged MQA-logits scoring, fp8 with 16+ heads: one wave scores a long column
// range.

#include "logits_frag.h"

namespace qsa {
namespace {

// Looped variant for fp8 with 16+ heads: the MFMA work per key column is large
// (H x RT rows), so the per-program set-up (row info, resident Q and weights)
// and per-tile address work would otherwise dominate the instruction stream.
// One program scores a long column range: `iters` groups of TPI key tiles, the
// next group's keys in flight while the current group is scored (two register
// buffers), the scores collected in LDS and every global store issued at the
// end -- loads and stores share one memory counter on gfx9, so a store inside
// the loop would hold up the next wait on keys.
// ONE_BLOCK: block_size is a multiple of the group's 16 TPI columns, so every
// group lies in one pool block (group starts are multiples of 16 TPI): one
// table entry and one base address per group, the tiles at fixed offsets.
template <int H, int MT, int TPI, bool HAS_W, bool HAS_SCALE, bool ONE_BLOCK>
__global__ __launch_bounds__(64) void looped_logits_kernel(LogitsArgs a) {
    typedef Frag<kFP8> F;
    constexpr int M = 16 * MT;
    constexpr int RT = M / H;
    static_assert(H >= 16 && RT >= 1 && RT <= 4, "looped variant: H >= 16, at most 4 rows");
    constexpr int kMaxCols = 16 * TPI * 32;  // columns per program at most (iters <= 32)
    __shared__ float obuf[RT][kMaxCols];

    const int l = lane_id();
    const int g = l >> 4;
    const int tile = blockIdx.x / a.num_chunks;
    const int chunk = blockIdx.x - tile * a.num_chunks;
    const int row0 = tile * RT;
    const int ncols = 16 * TPI * a.iters;
    const int c0 = chunk * ncols;

    int ctx_r[RT], req_r[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int row = min(row0 + r, a.num_rows - 1);
        ctx_r[r] = a.ctx_lens[row];
        req_r[r] = a.row_to_req[row];
    }
    uint32_t todo = 0u;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const bool valid = row0 + r < a.num_rows;
        ctx_r[r] = valid ? min(max(ctx_r[r], 0), a.cap) : 0;
        req_r[r] = valid ? req_r[r] : -1;
        todo |= (valid ? 1u : 0u) << r;
    }
    typename F::T qa[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + (l & 15);
        const int row = row0 + m / H, h = m % H;
        const uint8_t *qrow = reinterpret_cast<const uint8_t *>(a.q) + ((int64_t)row * H + h) * F::kRowBytes;
        qa[mt] = (row < a.num_rows) ? F::load(qrow + F::lane_bytes(l), 0) : F::zero();
    }
    float wv[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * mt + 4 * g + i;
            const int row = row0 + m / H, h = m % H;
            wv[mt][i] = (HAS_W && row < a.num_rows) ? a.w[(int64_t)row * H + h] : 1.0f;
        }

    const float neg_inf = -__builtin_inff();
    const float qnan = __builtin_nanf("");
    while (todo) {
        const int r0 = __builtin_ctz(todo);
        int req = 0;
#pragma unroll
        for (int r = 0; r < RT; ++r) req = (r == r0) ? req_r[r] : req;
        uint32_t set = 0u;
        int vis = 0;
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            if (((todo >> r) & 1u) && req_r[r] == req) {
                set |= 1u << r;
                vis = max(vis, ctx_r[r]);
            }
        }
        todo &= ~set;
        const bool req_ok = req >= 0 && req < a.num_reqs;
        const int32_t *bt = a.block_table + (req_ok ? (int64_t)req * a.max_blocks : 0);

        if (c0 < vis) {
            // Three-stage pipeline over groups of TPI key tiles: block-table
            // entries (scalar loads) two groups ahead, keys and scales one
            // group ahead, scoring of the current group.  A tile past the
            // visible range or with an out-of-range table entry loads from
            // block 0 and is not scored.
            // the table stage and the key stage each walk the columns with a cursor
            ColCursor tab(c0, a.block_size), key(c0, a.block_size);
            auto fetch_table = [&](int (&blk)[TPI]) {
                if (ONE_BLOCK) {
                    blk[0] = req_ok ? bt[min(tab.q, a.max_blocks - 1)] : -1;
                    // next group: the same block or the next one
                    tab.r += 16 * TPI;
                    const bool wrap = tab.r >= a.block_size;
                    tab.r = wrap ? 0 : tab.r;
                    tab.q = wrap ? tab.q + 1 : tab.q;
                } else {
#pragma unroll
                    for (int t = 0; t < TPI; ++t) {
                        blk[t] = req_ok ? bt[min(tab.q, a.max_blocks - 1)] : -1;
                        tab.step(a.block_size);
                    }
                }
            };
            auto load_group = [&](int cg, const int (&blk)[TPI], typename F::T (&b)[TPI], float (&sc)[TPI],
                                  bool (&ok)[TPI]) {
                if (ONE_BLOCK) {
                    const bool bok = (blk[0] >= 0) & ((int64_t)blk[0] < a.num_blocks);
                    const int64_t bbase = bok ? (int64_t)blk[0] * a.block_bytes : 0;
                    const int slot0 = bok ? key.r : 0;
                    key.r += 16 * TPI;
                    const bool wrap = key.r >= a.block_size;
                    key.r = wrap ? 0 : key.r;
                    const uint8_t *kg = a.kcache + bbase + (int64_t)slot0 * F::kRowBytes;  // first 16-token group
                    const float *sb = HAS_SCALE ? (a.layout != 0 ? reinterpret_cast<const float *>(a.kcache + bbase + a.scale_offset)
                                                                 : a.kscale + (bok ? (int64_t)blk[0] * a.block_size : 0))
                                                 + slot0 + (l & 15)
                                                : nullptr;
#pragma unroll
                    for (int t = 0; t < TPI; ++t) {
                        ok[t] = bok & (cg + 16 * t < vis);
                        b[t] = load_key_frag_fp8(kg + 16 * t * F::kRowBytes, l, a.layout == 2);
                        sc[t] = HAS_SCALE ? sb[16 * t] : 1.0f;
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < TPI; ++t) {
                        const int col0 = cg + 16 * t;
                        ok[t] = (col0 < vis) & (blk[t] >= 0) & ((int64_t)blk[t] < a.num_blocks);
                        const int64_t bbase = ok[t] ? (int64_t)blk[t] * a.block_bytes : 0;
                        const int tslot = ok[t] ? key.r : 0;
                        key.step(a.block_size);
                        b[t] = load_key_frag_fp8(a.kcache + bbase + (int64_t)tslot * a.key_stride, l, a.layout == 2);
                        sc[t] = 1.0f;
                        if (HAS_SCALE) {
                            if (a.layout != 0)
                                sc[t] = reinterpret_cast<const float *>(a.kcache + bbase + a.scale_offset)[tslot + (l & 15)];
                            else
                                sc[t] = a.kscale[(ok[t] ? (int64_t)blk[t] * a.block_size : 0) + tslot + (l & 15)];
                        }
                    }
                }
            };
            // scores of one group into obuf
            auto score_group = [&](int cg, const typename F::T (&b)[TPI], const float (&sc)[TPI],
                                   const bool (&ok)[TPI]) {
                // every MFMA of the group first, into its own accumulator, so the
                // matrix unit streams while the reductions wait for results
                f32x4 acc[TPI][MT];
#pragma unroll
                for (int t = 0; t < TPI; ++t)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = F::mma(qa[mt], b[t], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int t = 0; t < TPI; ++t) {
                    float val[RT];
#pragma unroll
                    for (int j = 0; j < RT; ++j) val[j] = 0.0f;
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        float c = 0.0f;
#pragma unroll
                        for (int i = 0; i < 4; ++i) c += wv[mt][i] * relu(acc[t][mt][i]);
                        val[(16 * mt) / H] += c;  // every slot of tile mt is in row 16mt/H
                    }
#pragma unroll
                    for (int j = 0; j < RT; ++j) {
                        val[j] = xor32_sum(xor16_sum(val[j]));
                        // every lane group holds the sums: all write (no branch
                        // splitting the group's schedule), equal values per address
                        obuf[j][cg - c0 + 16 * t + (l & 15)] = ok[t] ? val[j] * sc[t] : qnan;
                    }
                }
            };
            constexpr int GC = 16 * TPI;  // columns per group
            int tA[TPI], tB[TPI];
            typename F::T bA[TPI], bB[TPI];
            float sA[TPI], sB[TPI];
            bool oA[TPI], oB[TPI];
            fetch_table(tA);
            fetch_table(tB);
            load_group(c0, tA, bA, sA, oA);
#pragma unroll 1
            for (int it = 0; it < a.iters; it += 2) {  // iters is even
                const int cg = c0 + GC * it;
                load_group(cg + GC, tB, bB, sB, oB);  // (past the end: block 0, discarded)
                fetch_table(tA);
                score_group(cg, bA, sA, oA);
                load_group(cg + 2 * GC, tA, bA, sA, oA);
                fetch_table(tB);
                score_group(cg + GC, bB, sB, oB);
            }
        }

        // every store of the request's rows, from LDS (or -inf past the
        // visible range): lane l writes 4 consecutive columns per step
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            if (!((set >> j) & 1u)) continue;
            float *orow = a.out + (int64_t)(row0 + j) * a.out_stride;
            const int ctx = ctx_r[j];
            for (int cc = 4 * l; cc < ncols; cc += 256) {
                const int col = c0 + cc;
                if (col >= a.width) break;
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = (col + e < ctx && c0 < vis) ? obuf[j][cc + e] : neg_inf;
                if (col + 3 < a.width) {
                    *reinterpret_cast<f32x4 *>(orow + col) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < a.width) orow[col + e] = v[e];
                }
            }
        }
    }
}

template <int H, int MT, int TPI, bool HAS_W, bool HAS_SCALE>
static void launch_looped_b(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    dim3 grid((unsigned)a.num_row_tiles * (unsigned)a.num_chunks), block(64);
    if (a.block_size % (16 * TPI) == 0)
        hipExtLaunchKernelGGL((looped_logits_kernel<H, MT, TPI, HAS_W, HAS_SCALE, true>), grid, block, 0, s, e0, e1, 0, a);
    else
        hipExtLaunchKernelGGL((looped_logits_kernel<H, MT, TPI, HAS_W, HAS_SCALE, false>), grid, block, 0, s, e0, e1, 0, a);
}

template <int H, int MT, int TPI>
hipError_t launch_looped(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const bool has_w = a.w != nullptr;
    const bool has_s = a.layout != 0 || a.kscale != nullptr;
    if (has_w && has_s)
        launch_looped_b<H, MT, TPI, true, true>(a, s, e0, e1);
    else if (has_w)
        launch_looped_b<H, MT, TPI, true, false>(a, s, e0, e1);
    else if (has_s)
        launch_looped_b<H, MT, TPI, false, true>(a, s, e0, e1);
    else
        launch_looped_b<H, MT, TPI, false, false>(a, s, e0, e1);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_looped_fp8(const LogitsArgs &a, int rows_per_tile, hipStream_t s, hipEvent_t e0,
                             hipEvent_t e1) {
    switch (a.num_heads * 4 + rows_per_tile) {
        case 16 * 4 + 1: return launch_looped<16, 1, 4>(a, s, e0, e1);
        case 16 * 4 + 4: return launch_looped<16, 4, 4>(a, s, e0, e1);
        case 32 * 4 + 1: return launch_looped<32, 2, 4>(a, s, e0, e1);
        case 64 * 4 + 1: return launch_looped<64, 4, 4>(a, s, e0, e1);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qsa
