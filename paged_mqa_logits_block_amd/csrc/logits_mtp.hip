// Paged MQA-logits scoring, fp8 with 32/64 heads and 4-row requests.

#include "logits_frag.h"

namespace qsa {
namespace {

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
//
// Tiles: 4 consecutive rows each, or, when the planner asks for it (at most
// kMtpAlignedMaxRows rows), tiles that follow the requests: a segment (a
// maximal run of consecutive rows of one request) is cut into tiles of 4 rows
// from its first row, and tiles are numbered in row order.  Every workgroup
// finds the tile starts itself (thread t stands for row t: a max-scan of the
// segments' first rows, then a count of the starts before it), so a ragged
// number of rows per request (1..8 verify rows) costs one key pass per tile
// instead of one per request that a tile touches.  The grid holds as many tiles
// as rows grouped by request can need; when the rows come in another order and
// make more tiles than that, every workgroup takes the plain 4-row tile instead
// (the grid always holds those), so every row is covered whatever the order.
constexpr int kMtpRun = kMtpRunCols;          // columns per run
constexpr int kMtpKeyLds = 144;               // padded key in LDS (bytes)
constexpr int kMtpDepth = 4;                  // runs in flight
constexpr int kMtpMaxRuns = kMtpMaxRunsPerGroup;  // runs per workgroup at most

// GATHER: the pool block holds fewer than a run's 64 columns, or runs straddle
// blocks (any block size not a multiple of 64, down to one key per block).
// The table entry of every column of the chunk is staged in LDS once per
// request (one round of loads before the ring starts), and each thread fetches
// its key slice and, for every fourth thread, its key's scale from the block
// of its own column; validity is kept per column.  Reading the entries from
// LDS keeps them off the vector-memory counter that orders the key ring.
template <int H, bool HAS_W, bool HAS_SCALE, bool GATHER>
__global__ __launch_bounds__(256, 4) void mtp_fp8_kernel(LogitsArgs a) {
    typedef Frag<kFP8> F;
    constexpr int MT = H / 16;
    constexpr int D = GATHER ? 2 : kMtpDepth;  // ring depth (gather: fewer registers free for the per-thread addresses)
    static_assert(D % 2 == 0, "the LDS buffer parity follows the ring slot");
    __shared__ __align__(16) uint8_t kbuf[2][kMtpRun * kMtpKeyLds];
    __shared__ float sbuf[2][kMtpRun];
    __shared__ int okbuf[2][GATHER ? kMtpRun : 1];  // per run, or per column (GATHER)
    __shared__ float obuf[4][kMtpRun * kMtpMaxRuns];
    __shared__ int tcol[GATHER ? kMtpRun * kMtpMaxRuns : 1];  // GATHER: table entry per chunk column

    const int t = threadIdx.x;
    const int l = lane_id();
    const int g = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave = row of the tile
    const int chunk = blockIdx.x % a.num_chunks;
    const int ncols = kMtpRun * a.iters;
    const int c0 = chunk * ncols;

    // the tile's first row and its row count
    const int tile = blockIdx.x / a.num_chunks;
    int trow0 = tile * 4, tn = min(4, a.num_rows - trow0);
    if (a.mtp_aligned) {
        __shared__ int tmax[4], tcnt[4], tsel[2];
        const bool in = t < a.num_rows;
        const int rq = in ? a.row_to_req[t] : 0;
        const int rp = (in && t > 0) ? a.row_to_req[t - 1] : rq;
        const bool first = in && (t == 0 || rq != rp);
        int ss = wave_scan_dpp(first ? t : 0, 0, OpMaxI());  // first row of t's segment (within the wave)
        if (l == 63) tmax[w] = ss;
        __syncthreads();
        for (int u = 0; u < w; ++u) ss = max(ss, tmax[u]);
        const bool st = in && ((t - ss) & 3) == 0;
        const uint64_t b = ballot(st);
        if (l == 0) tcnt[w] = __popcll(b);
        __syncthreads();
        const int ntiles = tcnt[0] + tcnt[1] + tcnt[2] + tcnt[3];
        // more tiles than the grid holds (rows not grouped by request): plain
        // tiles of 4 rows, which cover every row in any order
        if (ntiles <= a.num_row_tiles) {
            if (tile >= ntiles) return;
            int off = 0;
            for (int u = 0; u < w; ++u) off += tcnt[u];
            const int k = st ? off + mask_prefix(b) : -1;  // number of the tile starting at row t
            if (k == tile) tsel[0] = t;
            if (k == tile + 1) tsel[1] = t;
            __syncthreads();
            trow0 = tsel[0];
            tn = (tile + 1 < ntiles ? tsel[1] : a.num_rows) - trow0;
        }
    }
    if (tn <= 0) return;
    const int row = trow0 + w;

    // the tile's rows: visible counts and requests (every wave reads all 4)
    int ctx_r[4], req_r[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int rr = min(trow0 + r, a.num_rows - 1);
        const bool valid = r < tn;
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

    uint32_t todo = (1u << tn) - 1u;  // tile rows not yet handled
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
            if constexpr (GATHER) {
                const int32_t *btv = a.block_table + (req_ok ? (int64_t)req * a.max_blocks : 0);
                for (int i = t; i < cend - c0; i += 256)
                    tcol[i] = req_ok ? btv[min((c0 + i) / a.block_size, a.max_blocks - 1)] : -1;
                __syncthreads();
            }
            // GATHER: thread t's column of the run and the block it lives in
            auto fetch_gather = [&](i32x8 &kr, float &sr) -> bool {
                const int col = cl + (t >> 2);
                const int blk = col < cend ? tcol[col - c0] : -1;
                const bool ok = (col < cend) & (blk >= 0) & ((int64_t)blk < a.num_blocks);
                const int64_t bbase = ok ? (int64_t)blk * a.block_bytes : 0;
                const int slot = ok ? col - (col / a.block_size) * a.block_size : 0;
                // block-flat keys only: the planner sends preshuffled keys here
                // only with blocks of whole 64-column runs (no gather)
                kr = *reinterpret_cast<const i32x8 *>(a.kcache + bbase + (int64_t)slot * F::kRowBytes + 32 * (t & 3));
                sr = 1.0f;
                if (HAS_SCALE && (t & 3) == 0) {
                    if (a.layout != 0)
                        sr = reinterpret_cast<const float *>(a.kcache + bbase + a.scale_offset)[slot];
                    else
                        sr = a.kscale[(ok ? (int64_t)blk * a.block_size : 0) + slot];
                }
                cl += kMtpRun;
                return ok;
            };
            auto fetch = [&](i32x8 &kr, float &sr) -> bool {
                if constexpr (GATHER) return fetch_gather(kr, sr);
                const int blk = req_ok ? bt[min(tq, a.max_blocks - 1)] : -1;
                const bool ok = (cl < cend) & (blk >= 0) & ((int64_t)blk < a.num_blocks);
                const int64_t bbase = ok ? (int64_t)blk * a.block_bytes : 0;
                const int slot = ok ? tr : 0;
                kr = *reinterpret_cast<const i32x8 *>(a.kcache + bbase + (int64_t)slot * F::kRowBytes + 32 * t);
                sr = 1.0f;
                if (HAS_SCALE && t < kMtpRun) {
                    if (a.layout != 0)
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
                if (!GATHER && a.layout == 2) {
                    // a run's 8 KB are 4 preshuffled 16-token groups: thread t
                    // holds 16 bytes (chunk k) of tokens i and i + 1 of group gq
                    const int gq = t >> 6, k = (t & 63) >> 3, i = 2 * (t & 7);
                    uint8_t *d = kbuf[buf] + (16 * gq + i) * kMtpKeyLds + 16 * k;
                    *reinterpret_cast<i32x4 *>(d) = i32x4{kr[0], kr[1], kr[2], kr[3]};
                    *reinterpret_cast<i32x4 *>(d + kMtpKeyLds) = i32x4{kr[4], kr[5], kr[6], kr[7]};
                } else {
                    *reinterpret_cast<i32x8 *>(kbuf[buf] + lane_key_lds) = kr;
                }
                if constexpr (GATHER) {
                    if ((t & 3) == 0) {  // column t / 4 of the run
                        sbuf[buf][t >> 2] = sr;
                        okbuf[buf][t >> 2] = ok;
                    }
                } else {
                    if (t < kMtpRun) sbuf[buf][t] = sr;
                    if (t == 0) okbuf[buf][0] = ok;
                }
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
                const bool ok = GATHER ? okbuf[buf][l] != 0 : __builtin_amdgcn_readfirstlane(okbuf[buf][0]) != 0;
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

template <int H, bool G>
static hipError_t launch_mtp_g(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    dim3 grid((unsigned)a.num_row_tiles * (unsigned)a.num_chunks), block(256);
    const bool has_w = a.w != nullptr;
    const bool has_s = a.layout != 0 || a.kscale != nullptr;
    if (has_w && has_s)
        hipExtLaunchKernelGGL((mtp_fp8_kernel<H, true, true, G>), grid, block, 0, s, e0, e1, 0, a);
    else if (has_w)
        hipExtLaunchKernelGGL((mtp_fp8_kernel<H, true, false, G>), grid, block, 0, s, e0, e1, 0, a);
    else if (has_s)
        hipExtLaunchKernelGGL((mtp_fp8_kernel<H, false, true, G>), grid, block, 0, s, e0, e1, 0, a);
    else
        hipExtLaunchKernelGGL((mtp_fp8_kernel<H, false, false, G>), grid, block, 0, s, e0, e1, 0, a);
    return hipGetLastError();
}

}  // namespace

template <int H>
static hipError_t launch_mtp(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    return a.block_size % kMtpRun == 0 ? launch_mtp_g<H, false>(a, s, e0, e1) : launch_mtp_g<H, true>(a, s, e0, e1);
}

hipError_t launch_mtp_fp8(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    return a.num_heads == 64 ? launch_mtp<64>(a, s, e0, e1) : launch_mtp<32>(a, s, e0, e1);
}

}  // namespace qsa
