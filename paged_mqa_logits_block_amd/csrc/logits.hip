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
//  * a column chunk is TPW tiles of 16 key columns; B % 16 == 0 so a tile never
//    straddles a pool block and costs one table lookup (a scalar load);
//  * the key tile is loaded straight from the pool into the MFMA B operand:
//    lane l reads key column (l % 16), 16 contiguous bytes per K step, so each
//    load instruction moves 16 rows x 64 contiguous bytes;
//  * Q (the A operand) stays in registers for the whole program;
//  * accumulator lane l holds M rows 4*(l/16)..+3 of column l % 16; with
//    m = row*H + head, the head sum is in-lane for H <= 4, plus one or two
//    cross-lane steps for H >= 8.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kD = 128;

// Column -> (block index, slot) walked in steps of one 16-column tile: one
// division per program instead of a division and a remainder per tile (a
// runtime divisor costs dozens of scalar instructions).  Needs B >= 16.
struct ColCursor {
    int q, r;  // block index and slot of the current column
    __device__ __forceinline__ ColCursor(int col, int bs) : q(col / bs), r(col - (col / bs) * bs) {}
    __device__ __forceinline__ void step(int bs) {
        r += 16;
        const bool wrap = r >= bs;
        r = wrap ? r - bs : r;
        q = wrap ? q + 1 : q;
    }
};

template <bool FP8>
struct Frag;

// bf16: v_mfma_f32_16x16x32_bf16, four K steps of 32 over D = 128.
template <>
struct Frag<false> {
    static constexpr int kSteps = 4;
    typedef bf16x8 T;
    // byte offset of lane l's slice inside a 16-element row of D (K step 0)
    __device__ static int lane_bytes(int l) { return (l >> 4) * 16; }
    // the slice for K step s at p (p includes the lane's offset)
    __device__ static T load(const uint8_t *p, int s) { return *reinterpret_cast<const T *>(p + s * 64); }
    __device__ static T zero() {
        T z;
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
        return z;
    }
    __device__ static f32x4 mma(T a, T b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static constexpr int kRowBytes = kD * 2;
};

// fp8 e4m3fn: v_mfma_scale_f32_16x16x128_f8f6f4 with unit (E8M0 127) scales,
// one K step covers D = 128.
template <>
struct Frag<true> {
    static constexpr int kSteps = 1;
    typedef i32x8 T;
    __device__ static int lane_bytes(int l) { return (l >> 4) * 32; }
    __device__ static T load(const uint8_t *p, int s) {
        (void)s;
        return *reinterpret_cast<const T *>(p);  // 32 bytes, 32-byte aligned
    }
    __device__ static T zero() {
        T z;
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = 0;
        return z;
    }
    __device__ static f32x4 mma(T a, T b, f32x4 c) {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
    }
    static constexpr int kRowBytes = kD;
};

// H heads, MT stacked 16-row tiles, TPW 16-column tiles per program.
template <bool FP8, int H, int MT, int TPW, bool HAS_W, bool HAS_SCALE>
__global__ __launch_bounds__(64) void paged_logits_kernel(LogitsArgs a) {
    typedef Frag<FP8> F;
    constexpr int M = 16 * MT;
    static_assert(M % H == 0, "a row's heads must fit in the stacked tiles");
    constexpr int RT = M / H;  // rows per tile
    static_assert(RT >= 1 && RT <= 16, "row info is held by lanes 0..15");
    // After the head reduction a lane stores NR rows: for H <= 4 the 4/H rows
    // whose heads sit in its own 4 accumulator slots; for H >= 8 one row per
    // stacked tile group (the lane group that owns it stores it).
    constexpr int NR = (H <= 4) ? 4 / H : RT;

    const int l = lane_id();
    const int g = l >> 4;  // lane group
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
                              ((int64_t)row * H + h) * F::kRowBytes + F::lane_bytes(l);
#pragma unroll
        for (int s = 0; s < F::kSteps; ++s)
            qa[mt][s] = (row < a.num_rows) ? F::load(qrow, s) : F::zero();
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

        // per stored row: its visible count, and whether this request owns it
        int st_ctx[NR];
        bool st_on[NR];
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            int c = 0;
#pragma unroll
            for (int r = 0; r < RT; ++r) c = (st_rr[j] == r) ? ctx_r[r] : c;
            st_ctx[j] = c;
            st_on[j] = st_lane[j] && ((set >> st_rr[j]) & 1u);
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
        if (any_live) {
            int blk[TPW], slot0[TPW];
            ColCursor cur(c0, a.block_size);
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                blk[t] = req_ok ? bt[min(cur.q, a.max_blocks - 1)] : -1;
                slot0[t] = cur.r;
                cur.step(a.block_size);
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
#pragma unroll
                for (int s = 0; s < F::kSteps; ++s) b[t][s] = F::load(kt + lane_key, s);
                kscale[t] = 1.0f;
                if (HAS_SCALE) {
                    if (a.layout == 1)
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
                for (int s = 0; s < F::kSteps; ++s) acc[mt] = F::mma(qa[mt][s], b[t][s], acc[mt]);

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
                if (st_on[j] && c0 + cc < a.width) {
                    const float v = live ? (ok[t] ? val[t][j] * kscale[t] : qnan) : neg_inf;
                    orow[j][cc] = c0 + cc < st_ctx[j] ? v : neg_inf;
                }
            }
        }
    }
}

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
    typedef Frag<true> F;
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
            const int lane_key = (l & 15) * (int)a.key_stride + F::lane_bytes(l);
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
                    const uint8_t *kb = a.kcache + bbase + (int64_t)slot0 * F::kRowBytes + lane_key;
                    const float *sb = HAS_SCALE ? (a.layout == 1 ? reinterpret_cast<const float *>(a.kcache + bbase + a.scale_offset)
                                                                 : a.kscale + (bok ? (int64_t)blk[0] * a.block_size : 0))
                                                 + slot0 + (l & 15)
                                                : nullptr;
#pragma unroll
                    for (int t = 0; t < TPI; ++t) {
                        ok[t] = bok & (cg + 16 * t < vis);
                        b[t] = F::load(kb + 16 * t * F::kRowBytes, 0);
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
                        b[t] = F::load(a.kcache + bbase + (int64_t)tslot * a.key_stride + lane_key, 0);
                        sc[t] = 1.0f;
                        if (HAS_SCALE) {
                            if (a.layout == 1)
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
    const bool has_s = a.layout == 1 || a.kscale != nullptr;
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

// fp8 with 32 or 64 heads and requests of 4 rows (the MTP verify shape): one
// workgroup of 4 waves per (4-row tile, column chunk), one row -- all its heads,
// Q resident -- per wave.  The 4 rows of a request read the same keys, so every
// 64-column run of keys and scales (one pool block; the plan requires blocks of
// a multiple of 64 columns) is fetched once per workgroup, 32 contiguous bytes
// per thread, D runs ahead into a ring of registers, and staged in LDS with
// each key padded to 144 bytes (conflict-free fragment reads).  Scores are
// collected in LDS and stored after the loop, so the loop issues no stores and
// the waits on the key fetches stay exact (loads and stores share one counter
// on gfx9).  A tile whose rows belong to several requests walks them one at a
// time; the waves whose row is not in the current request skip the scoring.
constexpr int kMtpRun = kMtpRunCols;          // columns per run
constexpr int kMtpKeyLds = 144;               // padded key in LDS (bytes)
constexpr int kMtpDepth = 4;                  // runs in flight
constexpr int kMtpMaxRuns = kMtpMaxRunsPerGroup;  // runs per workgroup at most

template <int H, bool HAS_W, bool HAS_SCALE>
__global__ __launch_bounds__(256, 4) void mtp_fp8_kernel(LogitsArgs a) {
    typedef Frag<true> F;
    constexpr int MT = H / 16;
    constexpr int D = kMtpDepth;
    static_assert(D % 2 == 0, "the LDS buffer parity follows the ring slot");
    __shared__ __align__(16) uint8_t kbuf[2][kMtpRun * kMtpKeyLds];
    __shared__ float sbuf[2][kMtpRun];
    __shared__ int okbuf[2];
    __shared__ float obuf[4][kMtpRun * kMtpMaxRuns];

    const int t = threadIdx.x;
    const int l = lane_id();
    const int g = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave = row of the tile
    const int tile = blockIdx.x / a.num_chunks;
    const int chunk = blockIdx.x - tile * a.num_chunks;
    const int ncols = kMtpRun * a.iters;
    const int c0 = chunk * ncols;
    const int row = tile * 4 + w;

    // the tile's rows: visible counts and requests (every wave reads all 4)
    int ctx_r[4], req_r[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int rr = min(tile * 4 + r, a.num_rows - 1);
        const bool valid = tile * 4 + r < a.num_rows;
        ctx_r[r] = valid ? min(max(a.ctx_lens[rr], 0), a.cap) : 0;
        req_r[r] = valid ? a.row_to_req[rr] : -1;
    }
    int my_ctx = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) my_ctx = (r == w) ? ctx_r[r] : my_ctx;

    // resident Q of this wave's row (stacked row m = 16 mt + l % 16 is head m)
    typename F::T qa[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const uint8_t *qrow = reinterpret_cast<const uint8_t *>(a.q) +
                              ((int64_t)min(row, a.num_rows - 1) * H + 16 * mt + (l & 15)) * F::kRowBytes;
        qa[mt] = F::load(qrow + F::lane_bytes(l), 0);
    }
    // weights of the accumulator slots: slot (mt, i) is head 16 mt + 4 g + i
    float wv[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            wv[mt][i] = HAS_W ? a.w[(int64_t)min(row, a.num_rows - 1) * H + 16 * mt + 4 * g + i] : 1.0f;

    const float neg_inf = -__builtin_inff();
    const float qnan = __builtin_nanf("");
    // fetch: thread t holds bytes 32 t .. 32 t + 31 of the run's 8 KB of keys
    // (key t / 4, bytes 32 (t % 4) ..); threads 0..63 also the run's scales
    const int lane_key_lds = (t >> 2) * kMtpKeyLds + 32 * (t & 3);
    const int frag = (l & 15) * kMtpKeyLds + F::lane_bytes(l);

    uint32_t todo = 0u;  // tile rows not yet handled
#pragma unroll
    for (int r = 0; r < 4; ++r) todo |= (tile * 4 + r < a.num_rows ? 1u : 0u) << r;
    while (todo) {
        const int r0 = __builtin_ctz(todo);
        int req = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) req = (r == r0) ? req_r[r] : req;
        uint32_t set = 0u;
        int vis = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool in = (((todo >> r) & 1u) != 0u) & (req_r[r] == req);
            set |= (in ? 1u : 0u) << r;
            vis = in ? max(vis, ctx_r[r]) : vis;
        }
        todo &= ~set;
        const bool mine = ((set >> w) & 1u) != 0u;
        const int nruns = vis > c0 ? min(a.iters, (vis - c0 + kMtpRun - 1) / kMtpRun) : 0;
        if (nruns > 0) {
            const bool req_ok = (req >= 0) & (req < a.num_reqs);
            // the table is read-only here: reading it through the constant
            // address space keeps its loads scalar
            const __attribute__((address_space(4))) int32_t *bt =
                (const __attribute__((address_space(4))) int32_t *)a.block_table +
                (req_ok ? (int64_t)req * a.max_blocks : 0);
            int tq = c0 / a.block_size, tr = c0 - tq * a.block_size;  // run cursor
            int cl = c0;
            // runs the ring fetches past this workgroup's last one read block 0
            // (cached), not the next chunk's keys
            const int cend = min(vis, c0 + kMtpRun * nruns);
            auto fetch = [&](i32x8 &kr, float &sr) -> bool {
                const int blk = req_ok ? bt[min(tq, a.max_blocks - 1)] : -1;
                const bool ok = (cl < cend) & (blk >= 0) & ((int64_t)blk < a.num_blocks);
                const int64_t bbase = ok ? (int64_t)blk * a.block_bytes : 0;
                const int slot = ok ? tr : 0;
                kr = *reinterpret_cast<const i32x8 *>(a.kcache + bbase + (int64_t)slot * F::kRowBytes + 32 * t);
                sr = 1.0f;
                if (HAS_SCALE && t < kMtpRun) {
                    if (a.layout == 1)
                        sr = reinterpret_cast<const float *>(a.kcache + bbase + a.scale_offset)[slot + t];
                    else
                        sr = a.kscale[(ok ? (int64_t)blk * a.block_size : 0) + slot + t];
                }
                cl += kMtpRun;
                tr += kMtpRun;
                const bool wrap = tr >= a.block_size;
                tr = wrap ? 0 : tr;
                tq = wrap ? tq + 1 : tq;
                return ok;
            };
            auto put = [&](int buf, const i32x8 &kr, float sr, bool ok) {
                *reinterpret_cast<i32x8 *>(kbuf[buf] + lane_key_lds) = kr;
                if (t < kMtpRun) sbuf[buf][t] = sr;
                if (t == 0) okbuf[buf] = ok;
            };
            // scores of run j (in LDS buffer buf) into obuf
            auto score = [&](int j, int buf) {
                // lane 16 g + i: this lane group's heads summed for column
                // 16 tt + i of each tile tt
                float part[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const typename F::T b =
                        *reinterpret_cast<const typename F::T *>(kbuf[buf] + tt * 16 * kMtpKeyLds + frag);
                    // the tile's MFMAs first, into separate accumulators (one
                    // reused accumulator would serialise each MFMA behind the
                    // head sums of the one before)
                    f32x4 acc[MT];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[mt] = F::mma(qa[mt], b, f32x4{0.f, 0.f, 0.f, 0.f});
                    float v = 0.0f;
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) v += wv[mt][i] * relu(acc[mt][i]);
                    part[tt] = v;
                }
                // sum over the 4 lane groups, scattered so that lane l ends
                // with column l: exchanging the halves (tiles 0/2 and 1/3)
                // leaves tiles 0, 1 summed over groups {g, g^2} in the lower
                // half and tiles 2, 3 in the upper; exchanging odd and even
                // 16-lane rows then leaves tile g in group g
                const auto x02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]),
                                                                  false, false);
                const auto x13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]),
                                                                  false, false);
                const float r0 = __uint_as_float(x02[0]) + __uint_as_float(x02[1]);
                const float r1 = __uint_as_float(x13[0]) + __uint_as_float(x13[1]);
                const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(r0), __float_as_uint(r1), false, false);
                const float val = __uint_as_float(y[0]) + __uint_as_float(y[1]);
                const bool ok = __builtin_amdgcn_readfirstlane(okbuf[buf]) != 0;
                const float sc = HAS_SCALE ? sbuf[buf][l] : 1.0f;
                obuf[w][kMtpRun * j + l] = ok ? val * sc : qnan;
            };

            i32x8 kring[D];
            float sring[D];
            bool okr[D];
#pragma unroll
            for (int k = 0; k < D; ++k) okr[k] = fetch(kring[k], sring[k]);  // runs 0 .. D-1
            put(0, kring[0], sring[0], okr[0]);
            __syncthreads();
            // run j (slot k = j mod D, LDS buffer j mod 2): fetch run j + D into
            // slot k, score run j, run j + 1 to the other buffer, barrier
#pragma unroll 1
            for (int j0 = 0; j0 < nruns; j0 += D) {
#pragma unroll
                for (int k = 0; k < D; ++k) {
                    okr[k] = fetch(kring[k], sring[k]);
                    if (mine & (j0 + k < nruns)) score(j0 + k, k & 1);
                    put((k + 1) & 1, kring[(k + 1) % D], sring[(k + 1) % D], okr[(k + 1) % D]);
                    __syncthreads();
                }
            }
        }
        // this wave's row, if it belongs to the request: every column of the
        // chunk from obuf (or -inf past the visible range)
        if (mine) {
            float *orow = a.out + (int64_t)row * a.out_stride;
            for (int cc = 4 * l; cc < ncols; cc += 256) {
                const int col = c0 + cc;
                if (col >= a.width) break;
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = (col + e < my_ctx && cc + e < kMtpRun * nruns) ? obuf[w][cc + e] : neg_inf;
                if (col + 3 < a.width) {
                    *reinterpret_cast<f32x4 *>(orow + col) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < a.width) orow[col + e] = v[e];
                }
            }
        }
        __syncthreads();  // obuf and the LDS runs are reused by the next request
    }
}

template <int H>
static hipError_t launch_mtp(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    dim3 grid((unsigned)a.num_row_tiles * (unsigned)a.num_chunks), block(256);
    const bool has_w = a.w != nullptr;
    const bool has_s = a.layout == 1 || a.kscale != nullptr;
    if (has_w && has_s)
        hipExtLaunchKernelGGL((mtp_fp8_kernel<H, true, true>), grid, block, 0, s, e0, e1, 0, a);
    else if (has_w)
        hipExtLaunchKernelGGL((mtp_fp8_kernel<H, true, false>), grid, block, 0, s, e0, e1, 0, a);
    else if (has_s)
        hipExtLaunchKernelGGL((mtp_fp8_kernel<H, false, true>), grid, block, 0, s, e0, e1, 0, a);
    else
        hipExtLaunchKernelGGL((mtp_fp8_kernel<H, false, false>), grid, block, 0, s, e0, e1, 0, a);
    return hipGetLastError();
}

// Prefill variant (bf16, 4 heads, one request holding many rows): every row
// tile reads the whole key range of the request, so rows are stacked wide and
// keys streamed through the 32x32x16 bf16 MFMA (twice the rate of the
// 16x16x32 form on gfx950).
//
// A workgroup has NW consumer waves, 16 rows each, and one producer wave.  It
// walks its column range 32 columns (one 8 KB run of keys inside one pool
// block) per step.  The producer fetches runs D steps ahead into a ring of its
// own registers with contiguous 16-byte loads -- the fetch competes with the
// output stream for HBM and its latency is long -- and writes each run to LDS
// one step ahead of use, every key padded to 272 bytes so that the consumers
// read their MFMA fragments without bank conflicts.  (Fragment loads straight
// from global memory would touch a different cache line in every lane.)  LDS
// holds two runs, one barrier per step.  The consumers issue no global loads
// in the loop, so their stores never wait behind a key fetch (loads and
// stores share one counter on gfx9).  Steps past the workgroup's visible
// range only store -inf.
//
// Each consumer holds its 16 rows as 64 stacked (row, head) pairs in two
// 32-row M tiles with Q resident.  The 32x32 accumulator gives lane l the 4
// heads of rows 2q + l/32 (q = 0..3) of each M tile for column l % 32, so the
// head sum is in-lane.  K step s of the MFMA takes elements 16 s + 8 (l / 32)
// + 0..7 of the head dimension on both operands.  Scores leave through buffer
// stores, one descriptor per pair of output rows: a lane whose store must not
// happen (outside the chunk, past the width) gets an offset beyond the
// descriptor's range and the hardware drops it.
typedef __bf16 pf_bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t pf_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPfKeyLds = 272;               // padded key in LDS (bytes)
constexpr int kPfRunLds = 32 * kPfKeyLds;    // one 32-key run
constexpr int kPfDepth = 4;                  // runs in flight per workgroup
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9 buffer descriptor word 3 (32-bit data)
constexpr int kDropOffset = (int)0x80000000u;  // beyond any descriptor range used here

template <bool HAS_W, int NW>
__global__ __launch_bounds__(64 * (NW + 1), 3) void prefill_logits_kernel(LogitsArgs a) {
    constexpr int H = 4;
    constexpr int D = kPfDepth;
    constexpr int LPL = 8192 / (16 * 64);  // 16-byte loads per producer lane per run
    __shared__ __align__(16) uint8_t kbuf[2][kPfRunLds];
    __shared__ int okbuf[2];
    __shared__ __align__(16) float wsm[HAS_W ? NW : 1][16][4];  // weights of each consumer's rows

    const int l = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index (uniform)
    const int rb = blockIdx.x / a.num_chunks;
    const int chunk = blockIdx.x - rb * a.num_chunks;
    const int c0 = chunk * 32 * a.iters;
    if (c0 >= a.width) return;  // the whole workgroup
    const int nsteps = min(a.iters, (a.width - c0 + 31) / 32);
    // visible range of the workgroup: how far key runs are fetched and scored
    int vis_wg = 0;
    for (int r = l; r < 16 * NW; r += 64) {
        const int row = min(rb * 16 * NW + r, a.num_rows - 1);
        vis_wg = max(vis_wg, min(max(a.ctx_lens[row], 0), a.cap));
    }
    vis_wg = readlane(wave_max_i(vis_wg), 0);
    const int nA = vis_wg > c0 ? min(nsteps, (vis_wg - c0 + 31) / 32) : 0;  // scored steps
    const int nR = (nA + D - 1) / D * D;  // steps of the loop (whole rounds of D)

    if (w == NW) {  // producer
        if (nA == 0) return;
        // the table is read-only here: reading it through the constant address
        // space keeps its loads scalar
        const __attribute__((address_space(4))) int32_t *bt =
            (const __attribute__((address_space(4))) int32_t *)a.block_table;
        // table cursor of the run fetched next (block_size is a multiple of 32,
        // so a run lies in one pool block), and the entry of the run after it
        int tq = c0 / a.block_size, tr = c0 - tq * a.block_size;
        int ent = bt[min(tq, a.max_blocks - 1)];
        int ent_next = bt[min(tq + (tr + 32 >= a.block_size ? 1 : 0), a.max_blocks - 1)];
        int cl = c0;  // first column of the run fetched next
        // fetch the next run (past the visible range: the first run of block
        // 0, always in the pool, never scored); lane l holds bytes 16 (l + 64 i)
        auto fetch = [&](pf_u32x4 (&r)[LPL]) -> bool {
            const bool ok = cl < vis_wg && ent >= 0 && (int64_t)ent < a.num_blocks;
            const uint8_t *kt = a.kcache + (ok ? (int64_t)ent * a.block_bytes + (int64_t)tr * a.key_stride : 0);
#pragma unroll
            for (int i = 0; i < LPL; ++i) r[i] = *reinterpret_cast<const pf_u32x4 *>(kt + 16 * (l + 64 * i));
            cl += 32;
            tr += 32;
            const bool wrap = tr >= a.block_size;
            tr = wrap ? tr - a.block_size : tr;
            tq = wrap ? tq + 1 : tq;
            ent = ent_next;
            ent_next = bt[min(tq + (tr + 32 >= a.block_size ? 1 : 0), a.max_blocks - 1)];
            return ok;
        };
        // byte e of the run (key e / 256, byte e % 256) goes to key slot e / 256
        auto put = [&](int buf, const pf_u32x4 (&r)[LPL], bool ok) {
#pragma unroll
            for (int i = 0; i < LPL; ++i) {
                const int e = 16 * (l + 64 * i);
                *reinterpret_cast<pf_u32x4 *>(kbuf[buf] + (e >> 8) * kPfKeyLds + (e & 255)) = r[i];
            }
            if (l == 0) okbuf[buf] = ok;
        };
        pf_u32x4 ring[D][LPL];
        bool okr[D];
#pragma unroll
        for (int k = 0; k < D; ++k) okr[k] = fetch(ring[k]);  // runs 0 .. D-1
        put(0, ring[0], okr[0]);
        __syncthreads();
        // step st (slot k = st mod D): fetch run st + D into slot k (run st
        // left it one step ago), run st + 1 to LDS, barrier
#pragma unroll 1
        for (int st = 0; st < nR; st += D) {
#pragma unroll
            for (int k = 0; k < D; ++k) {
                okr[k] = fetch(ring[k]);
                put((k + 1) & 1, ring[(k + 1) % D], okr[(k + 1) % D]);
                __syncthreads();
            }
        }
        return;
    }

    // consumers
    const int gk = l >> 5;  // lane half
    // The wave's 16 rows.  Past the last row (a ragged row count; the plan
    // guarantees at least 16 rows) the wave shifts back to end at the last
    // row: it recomputes rows of the wave before and rewrites the same values.
    const int row0 = min(rb * 16 * NW + w * 16, a.num_rows - 16);
    // Row info, lane j < 16: row row0 + j.  There is one request; a row whose
    // row_to_req names anything else reads no keys and its visible columns
    // are written as NaN.
    int ctx_l, rok_l;
    {
        const int row = row0 + (l & 15);
        ctx_l = min(max(a.ctx_lens[row], 0), a.cap);
        rok_l = a.row_to_req[row] == 0;
    }
    // resident Q: A operand of M tile mt, K step s: stacked pair 32 mt + l%32
    pf_bf16x8 qa[2][8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int m = 32 * mt + (l & 31);
        const __bf16 *qr = reinterpret_cast<const __bf16 *>(a.q) + ((int64_t)(row0 + m / H) * H + m % H) * kD + 8 * gk;
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) qa[mt][s2] = *reinterpret_cast<const pf_bf16x8 *>(qr + 16 * s2);
    }
    // Weights of the wave's rows, kept in LDS (registers are the limit here)
    // and read back per row in the epilogue: lane l stores row l / 4, head l % 4.
    if (HAS_W) wsm[w][l >> 2][l & 3] = a.w[(int64_t)(row0 + (l >> 2)) * H + (l & 3)];
    // Accumulator slot 4q + h of M tile mt holds head h of wave row
    // 8 mt + 2 q + gk for column l % 32: its visible count and request check;
    // the descriptor of output rows 8 mt + 2 q and the next.
    int ctx_q[2][4];
    bool rok_q[2][4];
    __amdgpu_buffer_rsrc_t orsrc[2][4];
    const int rec = (int)(2 * a.out_stride * 4);  // bytes of two output rows
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int j = 8 * mt + 2 * q;
            ctx_q[mt][q] = gk ? readlane(ctx_l, j + 1) : readlane(ctx_l, j);
            rok_q[mt][q] = (gk ? readlane(rok_l, j + 1) : readlane(rok_l, j)) != 0;
            orsrc[mt][q] = __builtin_amdgcn_make_buffer_rsrc(a.out + (int64_t)(row0 + j) * a.out_stride, (short)0,
                                                             rec, kRawBufferWord3);
        }
    const int lane_row_off = gk * (int)a.out_stride;
    // byte offset of this lane's score for step st at column col
    auto out_off = [&](int st, int col) -> int {
        const bool live = (st < nsteps) & (col < a.width);
        return live ? 4 * (lane_row_off + col) : kDropOffset;
    };
    auto store8 = [&](int off, const float (&val)[2][4]) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val[mt][q]), orsrc[mt][q], off, 0, 0);
    };
    const float neg_inf = -__builtin_inff();
    const float qnan = __builtin_nanf("");

    // head sums, masks and stores of M tile mt for step st (its scores in acc)
    auto epilogue = [&](int mt, int st, const f32x16 &acc, bool ok) {
        const int col = c0 + 32 * st + (l & 31);
        const bool live = (st >= 0) & (st < nsteps) & (col < a.width);
        const int off = live ? 4 * (lane_row_off + col) : kDropOffset;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float v = 0.0f;
            if (HAS_W) {
                typedef float f32x4_t __attribute__((ext_vector_type(4)));
                const f32x4_t wq = *reinterpret_cast<const f32x4_t *>(&wsm[w][8 * mt + 2 * q + gk][0]);
#pragma unroll
                for (int h = 0; h < 4; ++h) v += wq[h] * relu(acc[4 * q + h]);
            } else {
#pragma unroll
                for (int h = 0; h < 4; ++h) v += relu(acc[4 * q + h]);
            }
            const float x = (ok & rok_q[mt][q]) ? v : qnan;
            const float y = col < ctx_q[mt][q] ? x : neg_inf;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), orsrc[mt][q], off, 0, 0);
        }
    };

    if (nA > 0) {
        __syncthreads();  // run 0 in kbuf[0]
        // Step st, two stages per M tile: MFMAs of tile 0 for run st beside
        // the epilogue of tile 1 for run st - 1, then MFMAs of tile 1 beside
        // the epilogue of tile 0 for run st; barrier.  The epilogue of tile 1
        // for the last run follows the loop (step -1's is dropped).
        f32x16 acc0, acc1 = f32x16{};
        bool ok_prev = false;
#pragma unroll 1
        for (int st = 0; st < nR; st += 2) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const uint8_t *kf = kbuf[k] + (l & 31) * kPfKeyLds + 16 * gk;
                pf_bf16x8 b[8];
#pragma unroll
                for (int s2 = 0; s2 < 8; ++s2) b[s2] = *reinterpret_cast<const pf_bf16x8 *>(kf + 32 * s2);
                const bool ok = __builtin_amdgcn_readfirstlane(okbuf[k]) != 0;
                acc0 = f32x16{};
#pragma unroll
                for (int s2 = 0; s2 < 8; ++s2)
                    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s2], b[s2], acc0, 0, 0, 0);
                epilogue(1, st + k - 1, acc1, ok_prev);
                acc1 = f32x16{};
#pragma unroll
                for (int s2 = 0; s2 < 8; ++s2)
                    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s2], b[s2], acc1, 0, 0, 0);
                epilogue(0, st + k, acc0, ok);
                ok_prev = ok;
                __syncthreads();
            }
        }
        epilogue(1, nR - 1, acc1, ok_prev);
    }
    // steps past the loop
    float ninf8[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) ninf8[mt][q] = neg_inf;
#pragma unroll 1
    for (int st = nR; st < nsteps; ++st) store8(out_off(st, c0 + 32 * st + (l & 31)), ninf8);
}

template <bool HAS_W_, int NW>
static hipError_t launch_prefill_w(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    dim3 grid((unsigned)a.num_row_tiles * (unsigned)a.num_chunks), block(64 * (NW + 1));
    hipExtLaunchKernelGGL((prefill_logits_kernel<HAS_W_, NW>), grid, block, 0, s, e0, e1, 0, a);
    return hipGetLastError();
}

template <bool FP8, int H, int MT, int TPW>
hipError_t launch_h(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    dim3 grid((unsigned)a.num_row_tiles * (unsigned)a.num_chunks), block(64);
    const bool has_w = a.w != nullptr;
    const bool has_s = FP8 && (a.layout == 1 || a.kscale != nullptr);
    if (has_w && has_s)
        hipExtLaunchKernelGGL((paged_logits_kernel<FP8, H, MT, TPW, true, true>), grid, block, 0, s, e0, e1, 0, a);
    else if (has_w)
        hipExtLaunchKernelGGL((paged_logits_kernel<FP8, H, MT, TPW, true, false>), grid, block, 0, s, e0, e1, 0, a);
    else if (has_s)
        hipExtLaunchKernelGGL((paged_logits_kernel<FP8, H, MT, TPW, false, true>), grid, block, 0, s, e0, e1, 0, a);
    else
        hipExtLaunchKernelGGL((paged_logits_kernel<FP8, H, MT, TPW, false, false>), grid, block, 0, s, e0, e1, 0, a);
    return hipGetLastError();
}

template <bool FP8>
hipError_t launch_dtype(const LogitsArgs &a, const LogitsPlan &p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    // (heads, stacked tiles, tiles per program) as chosen by plan_logits
    if constexpr (!FP8) {
        if (p.prefill)
            return a.w ? launch_prefill_w<true, kPrefillWaves>(a, s, e0, e1)
                       : launch_prefill_w<false, kPrefillWaves>(a, s, e0, e1);
    }
    if constexpr (FP8) {
        if (p.mtp) return a.num_heads == 64 ? launch_mtp<64>(a, s, e0, e1) : launch_mtp<32>(a, s, e0, e1);
        if (p.iters > 0) {  // looped variant (plan_logits: fp8, 16+ heads)
            switch (a.num_heads * 4 + p.rows_per_tile) {
                case 16 * 4 + 1: return launch_looped<16, 1, 4>(a, s, e0, e1);
                case 16 * 4 + 4: return launch_looped<16, 4, 4>(a, s, e0, e1);
                case 32 * 4 + 1: return launch_looped<32, 2, 4>(a, s, e0, e1);
                case 64 * 4 + 1: return launch_looped<64, 4, 4>(a, s, e0, e1);
                default: return hipErrorInvalidValue;
            }
        }
    }
    switch (a.num_heads) {
        case 1: return launch_h<FP8, 1, 1, 4>(a, s, e0, e1);
        case 2: return launch_h<FP8, 2, 1, 4>(a, s, e0, e1);
        case 4: return launch_h<FP8, 4, 1, 4>(a, s, e0, e1);
        case 8: return launch_h<FP8, 8, 1, 8>(a, s, e0, e1);
        case 16: return launch_h<FP8, 16, 1, 8>(a, s, e0, e1);
        case 32: return launch_h<FP8, 32, 2, 8>(a, s, e0, e1);
        case 64: return launch_h<FP8, 64, 4, 8>(a, s, e0, e1);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

LogitsPlan plan_logits(int dtype, int num_heads, int num_rows, int num_reqs, int width, int block_size,
                       int64_t out_stride) {
    LogitsPlan p;
    p.iters = 0;
    p.prefill = false;
    p.mtp = false;
    // fp8, 32 or 64 heads, 4 rows per request on average (MTP verify), pool
    // blocks of a multiple of 64 columns: 4-row workgroups sharing each key
    // run; chunks sized for about four workgroups per CU
    if (dtype == 1 && (num_heads == 32 || num_heads == 64) && num_reqs > 0 && num_rows == 4 * num_reqs &&
        block_size % kMtpRunCols == 0) {
        p.mtp = true;
        p.rows_per_tile = 4;
        p.m_tiles = num_heads / 16;
        const int row_tiles = num_rows / 4;
        const int runs = (width + kMtpRunCols - 1) / kMtpRunCols;
        int per = 1;
        while (per < kMtpMaxRunsPerGroup && (int64_t)row_tiles * ((runs + per - 1) / per) > 1024) per *= 2;
        p.iters = per;
        p.tiles_per_prog = per * kMtpRunCols / 16;
        return p;
    }
    // bf16, 4 heads, a single request holding all rows (a prefill chunk), pool
    // blocks of a multiple of 32 columns: the prefill variant, 64 rows per
    // workgroup, columns split so that about two workgroups run per CU
    if (dtype == 0 && num_heads == 4 && num_reqs == 1 && num_rows >= 256 && block_size % 32 == 0 &&
        out_stride < ((int64_t)1 << 27)) {
        p.prefill = true;
        p.rows_per_tile = 16 * kPrefillWaves;
        p.m_tiles = 1;
        // column splits: enough workgroups for every CU's resident slots
        const int row_tiles = (num_rows + p.rows_per_tile - 1) / p.rows_per_tile;
        const int steps = (width + 31) / 32;
        const int target = 256 * kPrefillGroupsPerCU;
        const int splits = max(1, min(steps, (target + row_tiles - 1) / row_tiles));
        p.iters = (steps + splits - 1) / splits;
        p.tiles_per_prog = 2 * p.iters;  // in 16-column tiles
        return p;
    }
    p.m_tiles = num_heads > 16 ? num_heads / 16 : 1;
    p.rows_per_tile = 16 * p.m_tiles / num_heads;
    // 16-column tiles per program: 4 for the few-head decode shapes (a sweep on
    // MI355X found 1..8 within 4% there), 8 where each program's rows read more
    // key bytes per column (long single-row and many-head fp8 shapes gained
    // 3..15%)
    p.tiles_per_prog = num_heads <= 4 ? 4 : 8;
    // fp8 with 16+ heads: the looped variant, 4 key tiles per group and as many
    // groups per program as leave about four programs per SIMD; with 16 heads
    // and several rows per request (MTP verify rows) 4 rows share a program
    if (dtype == 1 && num_heads >= 16) {
        const int rows_per_req = num_reqs > 0 ? num_rows / num_reqs : 1;
        if (num_heads == 16 && rows_per_req >= 4) {
            p.rows_per_tile = 4;
            p.m_tiles = 4;
        }
        const int tpi = 4;
        const int row_tiles = (num_rows + p.rows_per_tile - 1) / p.rows_per_tile;
        const int col_tiles = (width + 15) / 16;
        int iters = 32;
        while (iters > 2 && (int64_t)row_tiles * ((col_tiles + tpi * iters - 1) / (tpi * iters)) < 4096) iters /= 2;
        p.iters = iters;
        p.tiles_per_prog = tpi * iters;
    }
    return p;
}

hipError_t launch_paged_logits(const LogitsArgs &a, const LogitsPlan &p, hipStream_t s, hipEvent_t e0,
                               hipEvent_t e1) {
    if (a.num_row_tiles == 0 || a.num_chunks == 0) return hipSuccess;
    return a.dtype == 0 ? launch_dtype<false>(a, p, s, e0, e1) : launch_dtype<true>(a, p, s, e0, e1);
}

}  // namespace qsa
