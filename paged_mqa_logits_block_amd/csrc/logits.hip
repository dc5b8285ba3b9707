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

template <bool FP8>
struct Frag;

// bf16: v_mfma_f32_16x16x32_bf16, four K steps of 32 over D = 128.
template <>
struct Frag<false> {
    static constexpr int kSteps = 4;
    typedef bf16x8 T;
    // lane's slice of one 16-element row of D for K step s
    __device__ static T load(const uint8_t *row_bytes, int l, int s) {
        return *reinterpret_cast<const T *>(row_bytes + s * 64 + (l >> 4) * 16);
    }
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
    __device__ static T load(const uint8_t *row_bytes, int l, int s) {
        (void)s;
        const i32x4 *p = reinterpret_cast<const i32x4 *>(row_bytes + (l >> 4) * 32);
        i32x4 lo = p[0], hi = p[1];
        T r;
        r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
        r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
        return r;
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
                              ((int64_t)row * H + h) * F::kRowBytes;
#pragma unroll
        for (int s = 0; s < F::kSteps; ++s)
            qa[mt][s] = (row < a.num_rows) ? F::load(qrow, l, s) : F::zero();
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
            int blk[TPW];
#pragma unroll
            for (int t = 0; t < TPW; ++t)
                blk[t] = req_ok ? bt[min((c0 + 16 * t) / a.block_size, a.max_blocks - 1)] : -1;
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int col0 = c0 + 16 * t;
                ok[t] = col0 < vis && blk[t] >= 0 && (int64_t)blk[t] < a.num_blocks;
                const int slot = (col0 % a.block_size) + (l & 15);
                const int64_t boff = ok[t] ? (int64_t)blk[t] * a.block_bytes : 0;
                const uint8_t *kb = a.kcache + boff;
                const uint8_t *krow = kb + (int64_t)(ok[t] ? slot : (l & 15)) * a.key_stride;
#pragma unroll
                for (int s = 0; s < F::kSteps; ++s) b[t][s] = F::load(krow, l, s);
                kscale[t] = 1.0f;
                if (HAS_SCALE) {
                    if (a.layout == 1)
                        kscale[t] = *reinterpret_cast<const float *>(kb + a.scale_offset + 4 * (ok[t] ? slot : 0));
                    else
                        kscale[t] = a.kscale[ok[t] ? (int64_t)blk[t] * a.block_size + slot : 0];
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
                    for (int i = j * H; i < j * H + H; ++i) v += wv[0][i] * fmaxf(acc[0][i], 0.0f);
                    val[t][j] = v;
                }
            } else {
#pragma unroll
                for (int j = 0; j < NR; ++j) val[t][j] = 0.0f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    // all 4 slots of tile mt belong to tile row (16*mt + 4*g) / H
                    const int rr = (16 * mt + 4 * g) / H;
                    float c = 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) c += wv[mt][i] * fmaxf(acc[mt][i], 0.0f);
#pragma unroll
                    for (int j = 0; j < NR; ++j)
                        if (j == rr) val[t][j] += c;
                }
#pragma unroll
                for (int j = 0; j < NR; ++j) {
                    if (H >= 8) val[t][j] += xor_lane_f(val[t][j], 16);
                    if (H >= 16) val[t][j] += xor_lane_f(val[t][j], 32);
                }
            }
        }

        // mask and store: lane writes column col0 + l%16 of each row it stores
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int col0 = c0 + 16 * t;
            const bool live = col0 < vis;
            const int col = col0 + (l & 15);
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                if (st_on[j] && col < a.width) {
                    const float v = live ? (ok[t] ? val[t][j] * kscale[t] : qnan) : neg_inf;
                    a.out[(int64_t)(row0 + st_rr[j]) * a.out_stride + col] = col < st_ctx[j] ? v : neg_inf;
                }
            }
        }
    }
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
    // chunk width per program (tiles of 16 columns) follows plan_logits
    (void)p;
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

LogitsPlan plan_logits(int dtype, int num_heads, int num_rows, int width) {
    (void)dtype;
    (void)num_rows;
    (void)width;
    LogitsPlan p;
    p.m_tiles = num_heads > 16 ? num_heads / 16 : 1;
    p.rows_per_tile = 16 * p.m_tiles / num_heads;
    // 16-column tiles per program: 4 for the few-head decode shapes (a sweep on
    // MI355X found 1..8 within 4% there), 8 where each program's rows read more
    // key bytes per column (long single-row and many-head fp8 shapes gained
    // 3..15%)
    p.tiles_per_prog = num_heads <= 4 ? 4 : 8;
    return p;
}

hipError_t launch_paged_logits(const LogitsArgs &a, const LogitsPlan &p, hipStream_t s, hipEvent_t e0,
                               hipEvent_t e1) {
    if (a.num_row_tiles == 0 || a.num_chunks == 0) return hipSuccess;
    return a.dtype == 0 ? launch_dtype<false>(a, p, s, e0, e1) : launch_dtype<true>(a, p, s, e0, e1);
}

}  // namespace qsa
