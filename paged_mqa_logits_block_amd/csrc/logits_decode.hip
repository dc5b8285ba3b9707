// Paged MQA-logits scoring on gfx950: stacked-M MFMA kernel.
//
// Method (ROCm/ATOM PR #2651, "Changes"): the rows x heads that share a
// request's keys form the M operand of one matrix multiply, so a key tile is
// read from HBM once per request instead of once per row; the per-head ReLU is
// applied to the accumulator before the heads are summed back out of M.  Key
// columns are gathered through the block table (ROCm/aiter PR #4221, block-flat
// commit: block kv_indices[b, col // KVB], slot col % KVB).  Programs whose
// column chunk lies past every row's visible count only write -inf (vLLM
// PR #62589, "Overview" and "Details"; sglang PR #48649, "Modifications").
//
// Layout of the work:
//  * one program = one wave64 = (row tile, column chunk); a row tile is RT rows
//    whose RT*H (row, head) pairs fill MT stacked 16-row MFMA tiles;
//  * a column chunk is TPW tiles of 16 key columns; with B % 16 == 0 a tile
//    never straddles a pool block and costs one table lookup (a scalar load);
//    other block sizes take the per-column gather (GATHER below);
//  * the key tile is loaded straight from the pool into the MFMA B operand:
//    lane l reads key column (l % 16), 16 contiguous bytes per K step (bf16,
//    fp16), so each load instruction moves 16 rows x 64 contiguous bytes, or
//    32 bytes in one K step (fp8: contiguous, or two 16-byte pieces of a
//    preshuffled 16-key group);
//  * inputs: bf16, fp16 or fp8 q and keys (DT), head dim 128 or 64 (D);
//  * Q (the A operand) stays in registers for the whole program;
//  * accumulator lane l holds M rows 4*(l/16)..+3 of column l % 16; with
//    m = row*H + head, the head sum is in-lane for H <= 4, plus one or two
//    cross-lane steps for H >= 8.
#include "logits_frag.h"

namespace qsa {
namespace {

// ---- the selection's first pass, in the epilogue -------------------------
//
// With CAND the kernel also writes, for every stored row and 64-column chunk,
// the chunk's 32 largest scores as packed keys: the top 26 bits of the score's
// order key (a float order with -0 = +0) over 63 - (column in the chunk).  The
// packed order is (truncated score desc, column asc), every key of a row is
// distinct, and the resolve step of the selection works on these lists (half
// the row) instead of the row.  Columns that are not candidates (past the
// row's visible count) get key 0, below every packed key.

__device__ __forceinline__ void cas_desc(uint32_t &a, uint32_t &b) {
    const uint32_t hi = max(a, b), lo = min(a, b);
    a = hi;
    b = lo;
}

// k[s] against the partner lane's k[REV ? 3 - s : s]; upper lanes keep the
// larger of each pair, the others the smaller
template <int CTRL, bool REV>
__device__ __forceinline__ void half_clean(uint32_t (&k)[4], bool upper) {
    uint32_t p[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) p[s] = dpp_u32<CTRL>(k[REV ? 3 - s : s]);
#pragma unroll
    for (int s = 0; s < 4; ++s) k[s] = upper ? max(k[s], p[s]) : min(k[s], p[s]);
}

// a bitonic run of 4 in one lane, sorted descending
__device__ __forceinline__ void sort_bitonic4(uint32_t (&k)[4]) {
    cas_desc(k[0], k[2]);
    cas_desc(k[1], k[3]);
    cas_desc(k[0], k[1]);
    cas_desc(k[2], k[3]);
}

// The 32 largest of the 64 keys a 16-lane row holds, 4 per lane (every lane
// of the wave runs it; each row works on its own keys), by bitonic merging:
// each lane sorts its 4; lane pairs merge into sorted runs of 8, lane quads
// into sorted runs of 16 and 8-lane halves into sorted runs of 32; lanes 0..7
// keep the larger 32 of the two halves' (against lanes 15..8).  On return lanes
// 0..7 of every row hold its 32 largest keys, in no particular order.
// i = lane & 15.
__device__ __forceinline__ void top32_of_64(uint32_t (&k)[4], int i) {
    cas_desc(k[0], k[1]);
    cas_desc(k[2], k[3]);
    cas_desc(k[0], k[2]);
    cas_desc(k[1], k[3]);
    cas_desc(k[1], k[2]);
    half_clean<kDppXor1, true>(k, (i & 1) == 0);
    sort_bitonic4(k);
    half_clean<kDppXor3, true>(k, (i & 2) == 0);
    half_clean<kDppXor1, false>(k, (i & 1) == 0);
    sort_bitonic4(k);
    half_clean<kDppHalfMirror, true>(k, (i & 4) == 0);
    half_clean<kDppXor2, false>(k, (i & 2) == 0);
    half_clean<kDppXor1, false>(k, (i & 1) == 0);
    sort_bitonic4(k);
    uint32_t p[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) p[s] = dpp_u32<kDppMirror>(k[3 - s]);
#pragma unroll
    for (int s = 0; s < 4; ++s) k[s] = max(k[s], p[s]);
}

// H heads, MT stacked 16-row tiles, TPW 16-column tiles per program.
// GATHER: the block size is not a multiple of 16 (down to one key per block),
// so a 16-column tile may straddle blocks: every lane reads the table entry of
// its own column (which is also the accumulator column it holds) and gathers
// its key slice from that block.
// D: head dim, 128 or 64 (a template argument, so that D = 128 carries no
// run-time test in the hot loop).
// CAND: also write the chunk candidates of the selection (4 or fewer heads, 64-column chunks).
template <int DT, int H, int MT, int TPW, bool HAS_W, bool HAS_SCALE, bool GATHER, int D, bool CAND>
__global__ __launch_bounds__(64) void paged_logits_kernel(LogitsArgs a) {
    typedef Frag<DT> F;
    constexpr int M = 16 * MT;
    static_assert(M % H == 0, "a row's heads must fit in the stacked tiles");
    constexpr int RT = M / H;  // rows per tile
    static_assert(RT >= 1 && RT <= 16, "row info is held by lanes 0..15");
    // After the head reduction a lane stores NR rows: for H <= 4 the 4/H rows
    // whose heads sit in its own 4 accumulator slots; for H >= 8 one row per
    // stacked tile group (the lane group that owns it stores it).
    constexpr int NR = (H <= 4) ? 4 / H : RT;
    // With 8+ heads the scores leave through LDS: written in accumulator
    // order, read back as VEC consecutive columns of one row per lane, so the
    // wave stores each row's CW columns with whole-lane vector stores (one
    // instruction per 64 * VEC floats) instead of one 4-byte store per lane
    // of one lane group and tile.  With 4 or fewer heads every lane already
    // holds a score per tile, 16 lanes write 64 contiguous bytes of a row per
    // instruction, and these direct stores measured faster on MI355X than
    // both the LDS round trip (16.1-16.6 vs 15.0 us on the 36-row decode
    // batch; it also gives each one-wave workgroup an LDS allocation) and a
    // quad transpose to 16-byte stores whose adjacent lanes write different
    // 64-byte segments (about 25 us).
    constexpr bool LDS_STORE = H >= 8;
    static_assert(!CAND || (H <= 4 && TPW == 4), "candidates: one score per lane and tile, 64-column chunks");
    constexpr int CW = TPW * 16;        // columns per program
    constexpr int PER = RT * CW / 64;   // floats per lane after the transpose
    constexpr int VEC = PER >= 4 ? 4 : PER;
    static_assert(!LDS_STORE || (PER >= 1 && PER % VEC == 0 && CW % VEC == 0), "whole vectors per lane");

    const int l = lane_id();
    const int g = l >> 4;  // lane group
    // head dim D = 128, or 64: the bf16/fp16 K steps past D/32, and the fp8
    // lanes of lane groups past D/32, hold zeros (the fp8 MFMA's K is 128)
    static_assert(D == 128 || D == 64, "head dim");
    constexpr int dk = D >> 5;
    constexpr int kRow = D * (DT == kFP8 ? 1 : 2);  // bytes of a q or key row
    auto frag_on = [&](int s) { return DT == kFP8 ? (dk == 4 || g < dk) : s < dk; };
    const int tile = blockIdx.x / a.num_chunks;
    const int chunk = blockIdx.x - tile * a.num_chunks;
    const int row0 = tile * RT;
    const int c0 = chunk * TPW * 16;

    // per-row info of the tile, wave-uniform: every load issued before any use
    // (indices clamped in bounds, padding rows masked afterwards)
    int ctx_r[RT], req_r[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int row = min(row0 + r, a.num_rows - 1);
        ctx_r[r] = a.ctx_lens[row];
        req_r[r] = a.row_to_req[row];
    }
    // The table entries of the chunk for a guessed request, loaded in the same
    // round trip as the row info: request-major rows, the same count per
    // request (every decode batch here) make the guess exact; a wrong guess
    // only costs a second round of table loads below.
    // Only for 4 or fewer heads: with more, most programs of the long mixed
    // single-row batch lie past their row's context and the guessed loads
    // are wasted there.
    constexpr bool GUESS = H <= 4 && !GATHER;
    const int guess = GUESS ? min((int)(((int64_t)row0 * a.num_reqs) / a.num_rows), a.num_reqs - 1) : -1;
    int gblk[TPW];
    if constexpr (GUESS) {
        const int32_t *gbt = a.block_table + (int64_t)guess * a.max_blocks;
        ColCursor cur(c0, a.block_size);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            gblk[t] = gbt[min(cur.q, a.max_blocks - 1)];
            cur.step(a.block_size);
        }
    }
    uint32_t todo = 0u;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const bool valid = row0 + r < a.num_rows;
        ctx_r[r] = valid ? min(max(ctx_r[r], 0), a.cap) : 0;
        req_r[r] = valid ? req_r[r] : -1;
        todo |= (valid ? 1u : 0u) << r;
    }

    // resident Q: the A operand of every stacked tile and K step;
    // stacked row m = 16*mt + (l % 16) is (tile row m / H, head m % H)
    typename F::T qa[MT][F::kSteps];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + (l & 15);
        const int row = row0 + m / H, h = m % H;
        const uint8_t *qrow = reinterpret_cast<const uint8_t *>(a.q) +
                              ((int64_t)row * H + h) * kRow + F::lane_bytes(l);
#pragma unroll
        for (int s = 0; s < F::kSteps; ++s)
            qa[mt][s] = (row < a.num_rows && frag_on(s)) ? F::load(qrow, s) : F::zero();
    }

    // weights of the accumulator slots this lane holds: slot (mt, i) is stacked
    // row m = 16*mt + 4*g + i
    float wv[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * mt + 4 * g + i;
            const int row = row0 + m / H, h = m % H;
            wv[mt][i] = (HAS_W && row < a.num_rows) ? a.w[(int64_t)row * H + h] : 1.0f;
        }

    // tile row of the j-th row this lane stores, and whether this lane stores it
    int st_rr[NR];
    bool st_lane[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        if (H <= 4) {
            st_rr[j] = (4 * g + j * H) / H;
            st_lane[j] = true;
        } else {
            // row j occupies stacked rows j*H .. j*H+H-1, i.e. lane groups
            // (j*H/4) % 4 .. ; the lowest of them stores it
            st_rr[j] = j;
            st_lane[j] = (H >= 16) ? (g == 0) : (g == (j * H / 4) % 4);
        }
    }

    const float neg_inf = -__builtin_inff();
    const float qnan = __builtin_nanf("");

    while (todo) {
        // the rows of one request: the lowest pending row's request
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
        // a row_to_req value outside the table is never dereferenced: its rows
        // read no keys and their visible columns are written as NaN
        const bool req_ok = req >= 0 && req < a.num_reqs;
        const int32_t *bt = a.block_table + (req_ok ? (int64_t)req * a.max_blocks : 0);

        // per stored row: its visible count
        int st_ctx[NR];
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            int c = 0;
#pragma unroll
            for (int r = 0; r < RT; ++r) c = (st_rr[j] == r) ? ctx_r[r] : c;
            st_ctx[j] = c;
        }

        // Keys of the chunk: all table entries, then all key tiles, issued
        // before the first is used.  A tile that is past the visible range or
        // whose table entry is out of range loads block 0 (always in the pool)
        // and its scores are discarded.  A chunk entirely past the visible
        // range loads nothing.
        const bool any_live = c0 < vis;
        typename F::T b[TPW][F::kSteps];
        float kscale[TPW];
        bool ok[TPW];
        if (any_live && GATHER) {
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int c = c0 + 16 * t + (l & 15);  // this lane's column
                const int qb = c / a.block_size;
                const int blk = req_ok ? bt[min(qb, a.max_blocks - 1)] : -1;
                // the tile is live as a whole (columns past a row's count are
                // masked at the store); a column whose entry is out of range
                // reads block 0 and is scored NaN
                ok[t] = c0 + 16 * t < vis && blk >= 0 && (int64_t)blk < a.num_blocks;
                const int64_t bbase = ok[t] ? (int64_t)blk * a.block_bytes : 0;
                const int slot = ok[t] ? c - qb * a.block_size : 0;
                const uint8_t *kp = a.kcache + bbase + (int64_t)slot * a.key_stride + F::lane_bytes(l);
#pragma unroll
                for (int s = 0; s < F::kSteps; ++s) b[t][s] = frag_on(s) ? F::load(kp, s) : F::zero();
                kscale[t] = 1.0f;
                if (HAS_SCALE) {
                    if (a.layout != 0)
                        kscale[t] = reinterpret_cast<const float *>(a.kcache + bbase + a.scale_offset)[slot];
                    else
                        kscale[t] = a.kscale[(ok[t] ? (int64_t)blk * a.block_size : 0) + slot];
                }
            }
        } else if (any_live) {
            int blk[TPW], slot0[TPW];
            ColCursor cur(c0, a.block_size);
            if (GUESS && req == guess) {
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    blk[t] = gblk[t];
                    slot0[t] = cur.r;
                    cur.step(a.block_size);
                }
            } else {
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    blk[t] = req_ok ? bt[min(cur.q, a.max_blocks - 1)] : -1;
                    slot0[t] = cur.r;
                    cur.step(a.block_size);
                }
            }
            // per lane: key column l % 16 of the tile, its slice of the row
            const int lane_key = (l & 15) * (int)a.key_stride + F::lane_bytes(l);
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int col0 = c0 + 16 * t;
                ok[t] = col0 < vis && blk[t] >= 0 && (int64_t)blk[t] < a.num_blocks;
                // wave-uniform tile base (block 0 when the tile is not scored)
                const int64_t bbase = ok[t] ? (int64_t)blk[t] * a.block_bytes : 0;
                const int tslot = ok[t] ? slot0[t] : 0;
                const uint8_t *kt = a.kcache + bbase + (int64_t)tslot * a.key_stride;
                if constexpr (DT == kFP8) {
                    // one K step; slot0 is a multiple of 16: kt is a 16-token group
                    b[t][0] = frag_on(0) ? load_key_frag_fp8(kt, l, a.layout == 2, kRow) : F::zero();
                } else {
#pragma unroll
                    for (int s = 0; s < F::kSteps; ++s) b[t][s] = frag_on(s) ? F::load(kt + lane_key, s) : F::zero();
                }
                kscale[t] = 1.0f;
                if (HAS_SCALE) {
                    if (a.layout != 0)
                        kscale[t] = reinterpret_cast<const float *>(a.kcache + bbase + a.scale_offset)[tslot + (l & 15)];
                    else
                        kscale[t] = a.kscale[(ok[t] ? (int64_t)blk[t] * a.block_size : 0) + tslot + (l & 15)];
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                ok[t] = false;
                kscale[t] = 1.0f;
#pragma unroll
                for (int s = 0; s < F::kSteps; ++s) b[t][s] = F::zero();
            }
        }

        // Scores of every tile first, stores after: on gfx9 the memory counter
        // that orders a wait on loaded data also covers earlier stores, so a
        // store between two tiles would hold the next tile until it lands.
        float val[TPW][NR];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            f32x4 acc[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int s = 0; s < F::kSteps; ++s)
                    if (DT == kFP8 || s < dk) acc[mt] = F::mma(qa[mt][s], b[t][s], acc[mt]);

            // head reduction: per stored row, sum of w * ReLU over its heads
            if (H <= 4) {
#pragma unroll
                for (int j = 0; j < NR; ++j) {
                    float v = 0.0f;
#pragma unroll
                    for (int i = j * H; i < j * H + H; ++i) v += wv[0][i] * relu(acc[0][i]);
                    val[t][j] = v;
                }
            } else {
#pragma unroll
                for (int j = 0; j < NR; ++j) val[t][j] = 0.0f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    // all 4 slots of tile mt belong to tile row (16*mt + 4*g) / H
                    // (16*mt / H for H >= 16: known at compile time)
                    const int rr = H >= 16 ? (16 * mt) / H : (16 * mt + 4 * g) / H;
                    float c = 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) c += wv[mt][i] * relu(acc[mt][i]);
#pragma unroll
                    for (int j = 0; j < NR; ++j)
                        if (j == rr) val[t][j] += c;
                }
#pragma unroll
                for (int j = 0; j < NR; ++j) {
                    if (H >= 8) val[t][j] = xor16_sum(val[t][j]);
                    if (H >= 16) val[t][j] = xor32_sum(val[t][j]);
                }
            }
        }

        if constexpr (LDS_STORE) {
            __shared__ __align__(16) float tbuf[RT * CW];
            // mask into LDS: slot (tile row, column - c0)
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int col0 = c0 + 16 * t;
                const bool live = col0 < vis;
                const int cc = 16 * t + (l & 15);  // column - c0
#pragma unroll
                for (int j = 0; j < NR; ++j) {
                    if (st_lane[j]) {
                        const float v = live ? (ok[t] ? val[t][j] * kscale[t] : qnan) : neg_inf;
                        tbuf[st_rr[j] * CW + cc] = c0 + cc < st_ctx[j] ? v : neg_inf;
                    }
                }
            }
            __syncthreads();
            // store: lane l takes VEC consecutive columns of one row per step
#pragma unroll
            for (int k = 0; k < PER / VEC; ++k) {
                const int f = (k * 64 + l) * VEC;
                const int r = f / CW, cc = f % CW;
                if ((set >> r) & 1u) {
                    float *dst = a.out + (int64_t)(row0 + r) * a.out_stride + c0 + cc;
                    const float *src = tbuf + f;
                    if (c0 + cc + VEC <= a.width) {
                        if constexpr (VEC == 4)
                            *reinterpret_cast<f32x4 *>(dst) = *reinterpret_cast<const f32x4 *>(src);
                        else if constexpr (VEC == 2)
                            *reinterpret_cast<float2 *>(dst) = *reinterpret_cast<const float2 *>(src);
                        else
                            dst[0] = src[0];
                    } else {
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            if (c0 + cc + e < a.width) dst[e] = src[e];
                    }
                }
            }
            __syncthreads();  // tbuf is rewritten by the next request's rows
        } else {
            // mask and store: lane writes column col0 + l%16 of each row it stores
            float *orow[NR];
#pragma unroll
            for (int j = 0; j < NR; ++j) orow[j] = a.out + (int64_t)(row0 + st_rr[j]) * a.out_stride + c0;
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int col0 = c0 + 16 * t;
                const bool live = col0 < vis;
                const int cc = 16 * t + (l & 15);  // column - c0
#pragma unroll
                for (int j = 0; j < NR; ++j) {
                    if (st_lane[j] && ((set >> st_rr[j]) & 1u) && c0 + cc < a.width) {
                        const float v = live ? (ok[t] ? val[t][j] * kscale[t] : qnan) : neg_inf;
                        orow[j][cc] = c0 + cc < st_ctx[j] ? v : neg_inf;
                    }
                }
            }
            if constexpr (CAND) {
                // the chunk's 32 largest stored scores of each row, as packed keys
                const int i = l & 15;
#pragma unroll
                for (int j = 0; j < NR; ++j) {
                    uint32_t key[4];
#pragma unroll
                    for (int t = 0; t < TPW; ++t) {
                        const int cc = 16 * t + i;
                        // a candidate column is visible, hence live: the stored value
                        const float v = ok[t] ? val[t][j] * kscale[t] : qnan;
                        key[t] = c0 + cc < st_ctx[j] ? ((order_key(v) & ~63u) | (uint32_t)(63 - cc)) : 0u;
                    }
                    top32_of_64(key, i);
                    if (i < 8 && ((set >> st_rr[j]) & 1u) && c0 < st_ctx[j]) {
                        uint32_t *dst = a.cand + ((int64_t)(row0 + st_rr[j]) * a.num_chunks + chunk) * 32 + 4 * i;
                        *reinterpret_cast<uint4 *>(dst) = make_uint4(key[0], key[1], key[2], key[3]);
                    }
                }
            }
        }
    }
}

template <int DT, int H, int MT, int TPW, bool GATHER, int D, bool CAND>
hipError_t launch_hgc(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    dim3 grid((unsigned)a.num_row_tiles * (unsigned)a.num_chunks), block(64);
    const bool has_w = a.w != nullptr;
    const bool has_s = DT == kFP8 && (a.layout != 0 || a.kscale != nullptr);
    if (has_w && has_s)
        hipExtLaunchKernelGGL((paged_logits_kernel<DT, H, MT, TPW, true, true, GATHER, D, CAND>), grid, block, 0, s, e0, e1, 0, a);
    else if (has_w)
        hipExtLaunchKernelGGL((paged_logits_kernel<DT, H, MT, TPW, true, false, GATHER, D, CAND>), grid, block, 0, s, e0, e1, 0, a);
    else if (has_s)
        hipExtLaunchKernelGGL((paged_logits_kernel<DT, H, MT, TPW, false, true, GATHER, D, CAND>), grid, block, 0, s, e0, e1, 0, a);
    else
        hipExtLaunchKernelGGL((paged_logits_kernel<DT, H, MT, TPW, false, false, GATHER, D, CAND>), grid, block, 0, s, e0, e1, 0, a);
    return hipGetLastError();
}

template <int DT, int H, int MT, int TPW, bool GATHER, int D>
hipError_t launch_hg(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if constexpr (H <= 4 && TPW == 4) {
        if (a.cand) return launch_hgc<DT, H, MT, TPW, GATHER, D, true>(a, s, e0, e1);
    }
    if (a.cand) return hipErrorInvalidValue;  // the planner never asks for this
    return launch_hgc<DT, H, MT, TPW, GATHER, D, false>(a, s, e0, e1);
}

template <int DT, int H, int MT, int TPW>
hipError_t launch_h(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if (a.head_dim == 64)
        return a.block_size % 16 == 0 ? launch_hg<DT, H, MT, TPW, false, 64>(a, s, e0, e1)
                                      : launch_hg<DT, H, MT, TPW, true, 64>(a, s, e0, e1);
    return a.block_size % 16 == 0 ? launch_hg<DT, H, MT, TPW, false, 128>(a, s, e0, e1)
                                  : launch_hg<DT, H, MT, TPW, true, 128>(a, s, e0, e1);
}

// (stacked tiles, tiles per program) by head count, as plan_logits chooses them
template <int DT>
hipError_t launch_heads(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    switch (a.num_heads) {
        case 1: return launch_h<DT, 1, 1, 4>(a, s, e0, e1);
        case 2: return launch_h<DT, 2, 1, 4>(a, s, e0, e1);
        case 4: return launch_h<DT, 4, 1, 4>(a, s, e0, e1);
        case 8: return launch_h<DT, 8, 1, 8>(a, s, e0, e1);
        case 16: return launch_h<DT, 16, 1, 8>(a, s, e0, e1);
        case 32: return launch_h<DT, 32, 2, 8>(a, s, e0, e1);
        case 64: return launch_h<DT, 64, 4, 8>(a, s, e0, e1);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    switch (a.dtype) {
        case kBF16: return launch_heads<kBF16>(a, s, e0, e1);
        case kFP8: return launch_heads<kFP8>(a, s, e0, e1);
        case kFP16: return launch_heads<kFP16>(a, s, e0, e1);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qsa
