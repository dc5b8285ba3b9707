// Paged MQA-logits scoring, prefill shape (bf16 or fp16, 4 heads, one request, many rows).

#include "logits_frag.h"

namespace qsa {
namespace {

// Prefill variant (bf16, 4 heads, one request holding many rows): every row
// tile reads the whole key range of the request, so rows are stacked wide and
// keys streamed through the 32x32x16 bf16 MFMA (twice the rate of the
// 16x16x32 form on gfx950).
//
// A workgroup has NW consumer waves, 16 rows each, and one producer wave.  It
// walks its column range 32 columns (one 8 KB run of keys inside one pool
// block) per step.  The producer fetches runs D steps ahead into a ring of its
// own registers with contiguous 16-byte loads -- the fetch competes with the
// output stream for HBM and its latency is long -- and writes them to LDS one
// phase of 8 steps ahead of use, every key padded to 272 bytes so that the
// consumers read their MFMA fragments without bank conflicts.  (Fragment loads
// straight from global memory would touch a different cache line in every
// lane.)  LDS holds two phases of runs, with one barrier per phase: between
// barriers the consumer waves drift apart, so that one wave's LDS reads and
// stores overlap another's MFMAs instead of every wave waiting on the same
// pipe at once (one barrier per step was 11% slower, one per 4 steps 1.5%).
// The consumers issue no global loads in the loop, so their stores never wait
// behind a key fetch (loads and stores share one counter on gfx9).  Steps past
// the workgroup's visible range only store -inf.
//
// Each consumer holds its 16 rows as 64 stacked (row, head) pairs in two
// 32-row M tiles with Q resident.  The 32x32 accumulator gives lane l the 4
// heads of rows 2q + l/32 (q = 0..3) of each M tile for column l % 32, so the
// head sum is in-lane.  K step s of the MFMA takes elements 16 s + 8 (l / 32)
// + 0..7 of the head dimension on both operands.  Scores leave through buffer
// stores, one descriptor per pair of output rows: a lane whose store must not
// happen (outside the chunk, past the width) gets an offset beyond the
// descriptor's range and the hardware drops it.
typedef float f32x16 __attribute__((ext_vector_type(16)));

// element type and 32x32x16 MFMA per input dtype (bf16 or fp16)
template <int DT>
struct PfType;
template <>
struct PfType<kBF16> {
    typedef __bf16 E;
    typedef __bf16 V __attribute__((ext_vector_type(8)));
    __device__ static f32x16 mma(V a, V b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }
};
template <>
struct PfType<kFP16> {
    typedef _Float16 E;
    typedef _Float16 V __attribute__((ext_vector_type(8)));
    __device__ static f32x16 mma(V a, V b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }
};
typedef uint32_t pf_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPfKeyLds = 272;               // padded key in LDS (bytes)
constexpr int kPfRunLds = 32 * kPfKeyLds;    // one 32-key run
constexpr int kPfDepth = 4;                  // runs in flight per workgroup
constexpr int kPfEarly = 4;                  // next-step key fragments read before the epilogue
constexpr int kPfPhase = 8;                  // steps between barriers (LDS holds two phases of runs)
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9 buffer descriptor word 3 (32-bit data)
constexpr int kDropOffset = (int)0x80000000u;  // beyond any descriptor range used here

template <int DT, bool HAS_W, int NW>
__global__ __launch_bounds__(64 * (NW + 1), 3) void prefill_logits_kernel(LogitsArgs a) {
    constexpr int H = 4;
    constexpr int D = kPfDepth;
    constexpr int LPL = 8192 / (16 * 64);  // 16-byte loads per producer lane per run
    constexpr int S = kPfPhase;
    static_assert(S % D == 0, "a phase is whole rounds of the ring");
    __shared__ __align__(16) uint8_t kbuf[2 * S][kPfRunLds];
    __shared__ int okbuf[2 * S];
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
    const int nR = (nA + kPfPhase - 1) / kPfPhase * kPfPhase;  // steps of the loop (whole phases)

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
        // each run put to LDS makes room in the ring for the run D later
#pragma unroll 1
        for (int kk = 0; kk < S; kk += D) {
#pragma unroll
            for (int k = 0; k < D; ++k) {
                put(kk + k, ring[k], okr[k]);  // runs 0 .. S-1 to the first half
                okr[k] = fetch(ring[k]);
            }
        }
        __syncthreads();
        // phase ph (runs S ph .. S ph + S-1 being scored from LDS half ph & 1):
        // the next phase's runs to the other half, barrier
#pragma unroll 1
        for (int st = 0; st < nR; st += S) {
            const int half = ((st / S) + 1) & 1;
#pragma unroll 1
            for (int kk = 0; kk < S; kk += D) {
#pragma unroll
                for (int k = 0; k < D; ++k) {
                    put(S * half + kk + k, ring[k], okr[k]);
                    okr[k] = fetch(ring[k]);
                }
            }
            __syncthreads();
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
    typedef PfType<DT> P;
    typedef typename P::V pf_v8;
    pf_v8 qa[2][8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int m = 32 * mt + (l & 31);
        const typename P::E *qr = reinterpret_cast<const typename P::E *>(a.q) + ((int64_t)(row0 + m / H) * H + m % H) * kD + 8 * gk;
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) qa[mt][s2] = *reinterpret_cast<const pf_v8 *>(qr + 16 * s2);
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
                // an opaque zero keeps these reads in the loop: hoisted out of
                // it, the weights take 32 registers and the loop spills
                int z = 0;
                asm volatile("" : "+v"(z));
                const f32x4_t wq = *reinterpret_cast<const f32x4_t *>(&wsm[w][8 * mt + 2 * q + gk + z][0]);
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
        __syncthreads();  // runs 0 .. S-1 in the first half
        // Step st, two stages per M tile: MFMAs of tile 0 for run st beside
        // the epilogue of tile 1 for run st - 1, then MFMAs of tile 1 beside
        // the epilogue of tile 0 for run st; a barrier after every S steps.
        // The epilogue of tile 1 for the last run follows the loop (step -1's
        // is dropped).
        // The next step's key fragments are read into b as tile 1's MFMAs
        // release it (the first kPfEarly before tile 0's epilogue, the rest
        // after it, within the register budget), so their LDS latency passes
        // under the rest of the step (the last step of a phase re-reads its
        // own run: the next phase's first run is read after the barrier).
        f32x16 acc0, acc1 = f32x16{};
        bool ok_prev = false;
        const int lane_off = (l & 31) * kPfKeyLds + 16 * gk;
#pragma unroll 1
        for (int st = 0; st < nR; st += S) {
            const int half = (st / S) & 1;
            pf_v8 b[8];
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2)
                b[s2] = *reinterpret_cast<const pf_v8 *>(kbuf[S * half] + lane_off + 32 * s2);
#pragma unroll 1
            for (int k = 0; k < S; ++k) {
                const uint8_t *kn = kbuf[S * half + min(k + 1, S - 1)] + lane_off;
                const bool ok = __builtin_amdgcn_readfirstlane(okbuf[S * half + k]) != 0;
                acc0 = f32x16{};
#pragma unroll
                for (int s2 = 0; s2 < 8; ++s2)
                    acc0 = P::mma(qa[0][s2], b[s2], acc0);
                epilogue(1, st + k - 1, acc1, ok_prev);
                acc1 = f32x16{};
#pragma unroll
                for (int s2 = 0; s2 < 8; ++s2) {
                    acc1 = P::mma(qa[1][s2], b[s2], acc1);
                    if (s2 < kPfEarly) b[s2] = *reinterpret_cast<const pf_v8 *>(kn + 32 * s2);
                }
                epilogue(0, st + k, acc0, ok);
#pragma unroll
                for (int s2 = kPfEarly; s2 < 8; ++s2) b[s2] = *reinterpret_cast<const pf_v8 *>(kn + 32 * s2);
                ok_prev = ok;
            }
            __syncthreads();
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

template <int DT, bool HAS_W_, int NW>
static hipError_t launch_prefill_w(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    dim3 grid((unsigned)a.num_row_tiles * (unsigned)a.num_chunks), block(64 * (NW + 1));
    hipExtLaunchKernelGGL((prefill_logits_kernel<DT, HAS_W_, NW>), grid, block, 0, s, e0, e1, 0, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if (a.dtype == kFP16)
        return a.w ? launch_prefill_w<kFP16, true, kPrefillWaves>(a, s, e0, e1)
                   : launch_prefill_w<kFP16, false, kPrefillWaves>(a, s, e0, e1);
    return a.w ? launch_prefill_w<kBF16, true, kPrefillWaves>(a, s, e0, e1)
               : launch_prefill_w<kBF16, false, kPrefillWaves>(a, s, e0, e1);
}

}  // namespace qsa
