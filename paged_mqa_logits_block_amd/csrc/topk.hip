// Per-row top-k selection on gfx950.
//
// Selects, per row, the k columns of [0, n) with the largest logits, ties to
// the lower column (+0 and -0 equal), and writes them in ascending column order
// followed by -1 padding.  With row starts, a row's candidates are the n
// columns from its start s, and the indices written are offsets from s (the
// sglang PR #48649 test body passes per-row starts to its top-k).  Rows with n <= k keep all of [0, n) (sglang
// PR #48649, Accuracy Tests: rows that fit in k need no selection); nothing past n
// is used (vLLM PR #62589, Details and Validation).
//
// A row is selected by one workgroup of 1024 threads (16 waves); many-row calls
// loop each workgroup over rows (topk_rows_kernel), few-row calls may share a
// row among several workgroups (the split selection further down).  The
// selection is reduced to finding the k-th element in (value desc, column asc)
// order, a pair (T, Ct): column c is kept iff key(c) > T, or key(c) == T and
// c <= Ct, where key is the order-preserving u32 image of the float.
//
// Rows of up to 32768 columns are held in registers (8 float4 per thread); a
// finite row is selected from there with float compares (select_fast), any
// other is staged once in LDS as keys (128 KB).  Longer rows are re-read from
// memory (L2) on every pass.  The steps:
//
//  1. Finite min and max of the row (while staging; DPP wave reductions).
//  2. A 2048-bucket histogram, buckets linear in value between min and max
//     (bucket 0 = largest).  The map is monotone, so the bucket b* holding the
//     k-th largest value is found by one scan: buckets < b* are kept outright,
//     buckets > b* dropped.  Linear-in-value buckets spread a dense cluster of
//     logits over many bins, so LDS atomics rarely collide (radix digits of the
//     float bits would pile a whole octave into a few bins).
//  3. The members of b* (normally a few dozen) go to an LDS list as (key,
//     column) pairs.  Up to 64 of them: one wave ranks each pair against all
//     others by (key desc, column asc), and the pair of rank need-1 is (T, Ct) --
//     no barrier.  Larger lists: radix select (11, 11, 10 bits) for T, then the
//     tie column from column-order ranks of the keys equal to T.  A bucket too
//     large for the list runs the same radix passes over the row.
//  4. The kept set, ranked in column order and written.  Per thread and float4
//     group, the kept count is packed three groups to a word; DPP wave scans of
//     the packed words give every lane its offset inside the wave, and one scan
//     of per-(group, wave) totals gives each wave's offset.
#include <mutex>

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kStage = 32768;    // longest row staged in LDS
constexpr int kMaxWidth = 69632;
constexpr int kCand = 2048;      // (key, column) list of the crossing bucket
constexpr int kRankAll = 24;     // fused resolve: member lists this short are ranked by every wave
constexpr int kChunk = 8;        // float4 groups ranked per compaction round
constexpr int kStageGroups = kStage / 4 / kThreads;
constexpr int kMaxGroups = (kMaxWidth + 4 * kThreads - 1) / (4 * kThreads);

struct Shared {
    uint32_t keys[kStage];  // staged row (order keys), column order
    uint32_t hist[kBins];
    uint32_t cand_key[kCand];
    int cand_col[kCand];
    int grp[kChunk * kWaves];  // per (group, wave) kept counts -> offsets
    uint32_t red_max[kWaves];
    uint32_t red_min[kWaves];
    uint32_t red_nf[kWaves];
    int wave_tot[kWaves];
    int cross_bin;
    int cross_above;
    int cross_cnt;
    int ncand;
    int tie_col;
    uint32_t thr_key;
    int ntie;      // fused selection: the tie group's count
    // register path: the previous row's kept columns (n <= kStage < 65536),
    // written out after the next row's first barrier, and the kept counts of
    // each (group slice, wave)
    uint16_t kept16[kCand];
    alignas(16) uint32_t ktot[kStageGroups * kWaves];
    // split selection (resolve kernel)
    int split_above;   // columns of the row above the window
    int split_before;  // columns kept before this slice, known before the resolve
    int split_over;    // a slice recorded more members than it has slots
    int split_n;       // window members of the row
    int kept_before;   // kept crossing-bucket members before this slice
};

__device__ __forceinline__ float key_value(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ f32x4 load4(const float *src, int i) {
    return *reinterpret_cast<const f32x4 *>(src + 4 * i);
}

// A row as the kernels see it.  A row whose candidates start at column s is
// read from its 16-byte aligned base s & ~3: the `dead` = s & 3 columns in
// front of the start are part of the view but never candidates, n counts them
// too (dead + the visible count), and every index written is a view column
// minus dead.  Without row starts dead is 0 and the view is the row itself.
struct RowView {
    const float *src;
    int n;     // columns of the view: dead + visible
    int dead;  // leading columns before the row's start (0..3)
    int vis;   // visible columns from the start
};

__device__ __forceinline__ RowView row_view(const TopkArgs &a, int r, int ctx, int start) {
    const int s = a.row_starts ? min(max(start, 0), a.width) : 0;
    const int vis = min(max(ctx, 0), a.width - s);
    const int base = s & ~3;
    return RowView{a.logits + (int64_t)r * a.stride + base, vis + (s - base), s - base, vis};
}

__device__ __forceinline__ RowView row_view(const TopkArgs &a, int r) {
    return row_view(a, r, a.ctx_lens[r], a.row_starts ? a.row_starts[r] : 0);
}

// The dead columns of group i (only group 0 has any) read as the NaN whose
// order key is 0: below every value, never above or inside a float threshold,
// and a non-finite value that keeps the row off the register path.
__device__ __forceinline__ f32x4 kill_dead(f32x4 x, int i, int dead) {
    if (dead && i == 0) {
#pragma unroll
        for (int e = 0; e < 3; ++e)
            if (e < dead) x[e] = __uint_as_float(0xFFFFFFFFu);
    }
    return x;
}

template <class Sh>
__device__ __forceinline__ void clear_hist(Sh &sh) {
    for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[i] = 0;
}

// Exclusive scan of hist in bin order; finds the bin where the running count
// first reaches `need` (1 <= need <= total).  Result lands in sh.cross_*.
// All threads; ends with a barrier.
template <class Sh>
__device__ __forceinline__ void find_crossing(Sh &sh, int need) {
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int h0 = (int)sh.hist[2 * t], h1 = (int)sh.hist[2 * t + 1];
    const int s = h0 + h1;
    const int incl = wave_incl_sum(s);
    if ((t & 63) == 63) sh.wave_tot[w] = incl;
    __syncthreads();
    int base = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) base += (i < w) ? sh.wave_tot[i] : 0;
    const int excl = base + incl - s;
    if (excl < need && excl + h0 >= need) {
        sh.cross_bin = 2 * t;
        sh.cross_above = excl;
        sh.cross_cnt = h0;
    } else if (excl + h0 < need && excl + s >= need) {
        sh.cross_bin = 2 * t + 1;
        sh.cross_above = excl + h0;
        sh.cross_cnt = h1;
    }
    __syncthreads();
}

// find_crossing with one barrier, its result in every thread's registers: each
// wave finds, from the waves' totals, the wave whose bins hold the crossing and
// scans that wave's 128 bins itself.  All threads, fully active.
struct Crossing {
    int bin, above, cnt;
};
__device__ __forceinline__ Crossing find_crossing_w(Shared &sh, int need) {
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int l = t & 63;
    const int h0 = (int)sh.hist[2 * t], h1 = (int)sh.hist[2 * t + 1];
    const int incl = wave_incl_sum(h0 + h1);
    if (l == 63) sh.wave_tot[w] = incl;
    __syncthreads();
    const int wt = l < kWaves ? sh.wave_tot[l] : 0;
    const int winc = row16_scan_dpp(wt, 0, OpAdd());  // lanes 0..15: the waves' running totals
    const int cw = __builtin_ctzll(ballot(l < kWaves && winc >= need) | (1ull << (kWaves - 1)));
    const int before = readlane(winc - wt, cw);
    const int b = 2 * (64 * cw + l);
    const int g0 = (int)sh.hist[b], g1 = (int)sh.hist[b + 1];
    const int ginc = wave_incl_sum(g0 + g1);
    const int excl = before + ginc - g0 - g1;
    const bool c0 = excl < need && excl + g0 >= need;
    const bool c1 = excl + g0 < need && excl + g0 + g1 >= need;
    const int cl = __builtin_ctzll(ballot(c0 | c1) | (1ull << 63));
    const bool second = readlane(c1 ? 1 : 0, cl) != 0;
    Crossing r;
    r.bin = 2 * (64 * cw + cl) + (second ? 1 : 0);
    r.above = readlane(second ? excl + g0 : excl, cl);
    r.cnt = readlane(second ? g1 : g0, cl);
    return r;
}

// Value buckets: bucket 0 holds the largest values.  A finite value goes to
// 1 + floor((vmax - v) * scale), clamped to [1, kBins-2].  +inf and NaN with the
// sign clear go to bucket 0, -inf and NaN with the sign set to kBins-1.
// Monotone non-increasing in the value; equal keys share a bucket.
template <bool ALL_FINITE>
struct Bucketer {
    float vmax, scale;
    __device__ __forceinline__ int of_value(float v) const {
        const float d = (vmax - v) * scale;
        return 1 + (d < (float)(kBins - 3) ? (int)d : (kBins - 3));
    }
    __device__ __forceinline__ int operator()(uint32_t kx) const {
        if (!ALL_FINITE) {
            if (kx >= 0xFF800000u) return 0;
            if (kx <= 0x007FFFFFu) return kBins - 1;
        }
        return of_value(key_value(kx));
    }
};

// Keys of a row staged in LDS (column order).
struct StagedKeys {
    const uint32_t *keys;
    int n;
    // keys of this thread's float4 group j (columns 4*(t + 1024*j) ..)
    __device__ __forceinline__ uint4 group(int j) const {
        const int i = threadIdx.x + kThreads * j;
        return (4 * i < n) ? reinterpret_cast<const uint4 *>(keys)[i] : make_uint4(0u, 0u, 0u, 0u);
    }
};

// Keys of a row re-read from memory on every pass.
struct StreamKeys {
    const float *src;
    int n;
    int dead;
    __device__ __forceinline__ uint4 group(int j) const {
        const int i = threadIdx.x + kThreads * j;
        if (4 * i >= n) return make_uint4(0u, 0u, 0u, 0u);
        const f32x4 x = kill_dead(load4(src, i), i, dead);
        return make_uint4(order_key(x[0]), order_key(x[1]), order_key(x[2]), order_key(x[3]));
    }
};

// f(col, key) for every column of the row, over thread-strided float4 groups
template <int G, class Keys, class F>
__device__ __forceinline__ void for_each_key(const Keys &src, int n, F f) {
#pragma unroll 1
    for (int c = 0; c < G; c += kChunk) {
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            if (c + j < G) {
                const uint4 k4 = src.group(c + j);
                const uint32_t kk[4] = {k4.x, k4.y, k4.z, k4.w};
                const int c0 = 4 * (threadIdx.x + kThreads * (c + j));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c0 + e < n) f(c0 + e, kk[e]);
            }
        }
    }
}

// Column-order ranks of flagged elements in one chunk of kChunk float4 groups.
// Flag bit 4*j + e marks element e of this thread's group j of the chunk.
// Returns in off[j] the number of flagged elements of the chunk that precede
// this thread's group j (the caller adds its own earlier flags in the group) and
// the chunk's total.  All threads, fully active; ends with a barrier.
__device__ __forceinline__ int chunk_ranks(Shared &sh, uint32_t flag, int (&off)[kChunk]) {
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int l = t & 63;
    int cnt[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) cnt[j] = __popc((flag >> (4 * j)) & 0xFu);
    // three groups per word, 10 bits each (a wave's count per group <= 256)
    const int w0 = cnt[0] | (cnt[1] << 10) | (cnt[2] << 20);
    const int w1 = cnt[3] | (cnt[4] << 10) | (cnt[5] << 20);
    const int w2 = cnt[6] | (cnt[7] << 10);
    const int s0 = wave_incl_sum(w0), s1 = wave_incl_sum(w1), s2 = wave_incl_sum(w2);
    const int e0 = s0 - w0, e1 = s1 - w1, e2 = s2 - w2;  // exclusive, per field
    const int t0 = readlane(s0, 63), t1 = readlane(s1, 63), t2 = readlane(s2, 63);
    const int lane_excl[kChunk] = {e0 & 0x3FF, (e0 >> 10) & 0x3FF, (e0 >> 20) & 0x3FF,
                                   e1 & 0x3FF, (e1 >> 10) & 0x3FF, (e1 >> 20) & 0x3FF,
                                   e2 & 0x3FF, (e2 >> 10) & 0x3FF};
    const int wave_cnt[kChunk] = {t0 & 0x3FF, (t0 >> 10) & 0x3FF, (t0 >> 20) & 0x3FF,
                                  t1 & 0x3FF, (t1 >> 10) & 0x3FF, (t1 >> 20) & 0x3FF,
                                  t2 & 0x3FF, (t2 >> 10) & 0x3FF};
    if (l < kChunk) {
        int v = 0;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) v = (l == j) ? wave_cnt[j] : v;
        sh.grp[l * kWaves + w] = v;  // group-major: column order is (group, wave)
    }
    __syncthreads();
    if (w == 0) {  // exclusive scan over (group, wave), two entries per lane
        const int a = sh.grp[2 * l], b = sh.grp[2 * l + 1];
        const int incl = wave_incl_sum(a + b);
        sh.grp[2 * l] = incl - a - b;
        sh.grp[2 * l + 1] = incl - b;
        if (l == 63) sh.wave_tot[0] = incl;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kChunk; ++j) off[j] = sh.grp[j * kWaves + w] + lane_excl[j];
    const int total = sh.wave_tot[0];
    __syncthreads();  // grp and wave_tot are reused by the next call
    return total;
}

// Radix select over keys produced by `each` (each(f) calls f(key) for every
// member of the set), 11, 11 and 10 bits, largest digit first.  In: 1 <= need
// <= size of the set.  Out: T, the need-th largest key of the set; need becomes
// the number of keys equal to T that are kept, cnt the number equal to T.
template <class Each>
__device__ __forceinline__ void radix_select(Shared &sh, Each each, uint32_t &T, int &need, int &cnt) {
    uint32_t P = 0, M = 0;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shf = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
        __syncthreads();  // the previous crossing has been read by all threads
        clear_hist(sh);
        __syncthreads();
        each([&](uint32_t kx) {
            if ((kx & M) == P) atomicAdd(&sh.hist[dmask - ((kx >> shf) & dmask)], 1u);
        });
        __syncthreads();
        find_crossing(sh, need);
        P |= (dmask - (uint32_t)sh.cross_bin) << shf;
        M |= dmask << shf;
        need -= sh.cross_above;
        cnt = sh.cross_cnt;
    }
    T = P;
}

// Column of the need-th key equal to T in column order (1 <= need <= count).
template <int G, class Keys>
__device__ __forceinline__ int tie_column(Shared &sh, const Keys &src, int n, uint32_t T, int need) {
    const int t = threadIdx.x;
    int carry = 0;
#pragma unroll 1
    for (int c = 0; c < G; c += kChunk) {
        uint32_t eq = 0u;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const uint4 k4 = src.group(c + j);
            const uint32_t kk[4] = {k4.x, k4.y, k4.z, k4.w};
            const int c0 = 4 * (t + kThreads * (c + j));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (c0 + e < n && kk[e] == T) eq |= 1u << (4 * j + e);
        }
        int off[kChunk];
        const int tot = chunk_ranks(sh, eq, off);
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            int r = carry + off[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if ((eq >> (4 * j + e)) & 1u) {
                    if (r == need - 1) sh.tie_col = 4 * (t + kThreads * (c + j)) + e;
                    ++r;
                }
            }
        }
        carry += tot;
    }
    __syncthreads();
    return sh.tie_col;
}

// Steps 3 and 4 on a row whose bucket histogram is in sh.hist.  G = float4
// groups per thread covering the row.
template <int G, class Keys, class Bk>
__device__ __forceinline__ void select_row(Shared &sh, const Keys &src, int n, int k, const Bk &bucket,
                                           int32_t *out, int dead = 0) {
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int l = t & 63;
    find_crossing(sh, k);
    const int bstar = sh.cross_bin;
    int need = k - sh.cross_above;
    int cnt = sh.cross_cnt;

    // ---- 3. the k-th pair (T, Ct) inside bucket b* -----------------------
    uint32_t T;
    int tie_col;
    if (cnt <= kCand) {
        if (t == 0) sh.ncand = 0;
        __syncthreads();
#pragma unroll 1
        for (int c = 0; c < G; c += kChunk) {
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                const int i = t + kThreads * (c + j);
                if (c + j < G && 4 * i < n) {
                    const uint4 k4 = src.group(c + j);
                    const uint32_t kk[4] = {k4.x, k4.y, k4.z, k4.w};
                    bool hit[4];
                    bool any = false;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        hit[e] = (4 * i + e < n) && bucket(kk[e]) == bstar;
                        any |= hit[e];
                    }
                    if (ballot(any)) {  // rare: a wave holds a member of b*
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint64_t m = ballot(hit[e]);
                            if (m) {
                                const int lead = __builtin_ctzll(m);
                                int base = 0;
                                if (l == lead) base = atomicAdd(&sh.ncand, __popcll(m));
                                base = readlane(base, lead);
                                const int at = base + mask_prefix(m);
                                if (hit[e] && at < kCand) {
                                    sh.cand_key[at] = kk[e];
                                    sh.cand_col[at] = 4 * i + e;
                                }
                            }
                        }
                    }
                }
            }
        }
        __syncthreads();
        const int nc = sh.ncand;  // == cnt
        if (nc <= 64) {
            // rank every pair against all others by (key desc, column asc)
            if (w == 0) {
                const uint32_t mk = l < nc ? sh.cand_key[l] : 0u;
                const int mc = l < nc ? sh.cand_col[l] : 0x7FFFFFFF;
                int rank = 0;
                for (int j = 0; j < nc; ++j) {
                    const uint32_t kj = (uint32_t)readlane((int)mk, j);
                    const int cj = readlane(mc, j);
                    rank += (kj > mk || (kj == mk && cj < mc)) ? 1 : 0;
                }
                if (l < nc && rank == need - 1) {
                    sh.thr_key = mk;
                    sh.tie_col = mc;
                }
            }
            __syncthreads();
            T = sh.thr_key;
            tie_col = sh.tie_col;
        } else {
            radix_select(sh, [&](auto f) {
                for (int j = t; j < nc; j += kThreads) f(sh.cand_key[j]);
            }, T, need, cnt);
            tie_col = cnt > need ? tie_column<G>(sh, src, n, T, need) : 0x7FFFFFFF;
        }
    } else {
        radix_select(sh, [&](auto f) {
            for_each_key<G>(src, n, [&](int, uint32_t kx) {
                if (bucket(kx) == bstar) f(kx);
            });
        }, T, need, cnt);
        tie_col = cnt > need ? tie_column<G>(sh, src, n, T, need) : 0x7FFFFFFF;
    }
    // Every key above T is kept and every key below dropped; of the keys equal
    // to T, those at columns <= tie_col are kept.

    // ---- 4. the kept set, ranked in column order, written -----------------
    int carry = 0;
#pragma unroll 1
    for (int c = 0; c < G; c += kChunk) {
        uint32_t sel = 0u;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const uint4 k4 = src.group(c + j);
            const uint32_t kk[4] = {k4.x, k4.y, k4.z, k4.w};
            const int c0 = 4 * (t + kThreads * (c + j));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int col = c0 + e;
                const bool keep = col < n && (kk[e] > T || (kk[e] == T && col <= tie_col));
                sel |= (keep ? 1u : 0u) << (4 * j + e);
            }
        }
        int off[kChunk];
        const int tot = chunk_ranks(sh, sel, off);
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            int p = carry + off[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if ((sel >> (4 * j + e)) & 1u) {
                    if (p < k) out[p] = 4 * (t + kThreads * (c + j)) + e - dead;
                    ++p;
                }
            }
        }
        carry += tot;
    }
}

// Finite min / max (as order keys) and whether any visible value is not finite,
// across the block.  All threads; ends with a barrier; also clears the
// histogram.
struct RowRange {
    float vmax, scale;
    bool all_finite;
};

// Each wave's finite min / max (as order keys) and non-finite flag, reduced
// across the wave and written to LDS for range_read.
template <class Sh>
__device__ __forceinline__ void range_publish(Sh &sh, uint32_t kmax, uint32_t kmin, uint32_t nonfinite, int t) {
    const int w = t >> 6;
    kmax = wave_total_umax(kmax);
    const uint32_t nkmin = wave_total_umax(~kmin);
    nonfinite = wave_total_umax(nonfinite);
    if ((t & 63) == 0) {
        sh.red_max[w] = kmax;
        sh.red_min[w] = nkmin;
        sh.red_nf[w] = nonfinite;
    }
}

// The block's range from the waves' published partials (after a barrier).
template <class Sh>
__device__ __forceinline__ RowRange range_read(Sh &sh) {
    // lane i < kWaves takes wave i's partials (all lanes active); the lane
    // index is made here: one kept live across the row loop was spilled
    int li;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(li));
    static_assert(kWaves == 16, "one 16-lane row holds the waves' partials");
    const uint32_t a = row16_total_umax(li < kWaves ? sh.red_max[li] : 0u);
    const uint32_t b = row16_total_umax(li < kWaves ? sh.red_min[li] : 0u);
    const uint32_t c = row16_total_umax(li < kWaves ? sh.red_nf[li] : 0u);
    // with no finite value at all, a = 0 and ~b = ~0: the map is never used
    const float vmax = key_value(a), vmin = key_value(~b);
    const float span = vmax - vmin;
    // a span narrower than about 6e-36 makes the scale (and the register path's
    // offset vmax * scale) overflow; then one bucket holds the whole row, which
    // keeps every later step exact
    const float scale = (float)(kBins - 3) / span;
    const bool usable = a != 0u && span > 0.0f && __builtin_isfinite(span) && __builtin_isfinite(scale) &&
                        __builtin_isfinite(vmax * scale);
    return RowRange{vmax, usable ? scale : 0.0f, c == 0u};
}

template <class Sh>
__device__ __forceinline__ RowRange row_range(Sh &sh, uint32_t kmax, uint32_t kmin, uint32_t nonfinite,
                                              int t = (int)threadIdx.x) {
    range_publish(sh, kmax, kmin, nonfinite, t);
    clear_hist(sh);
    __syncthreads();
    return range_read(sh);
}

// running finite range and non-finite flag over one visible value
__device__ __forceinline__ void track(float x, bool valid, uint32_t &kmax, uint32_t &kmin, uint32_t &nf) {
    const uint32_t kx = order_key(x);
    const bool fin = __builtin_isfinite(x);
    kmax = (valid && fin) ? max(kmax, kx) : kmax;
    kmin = (valid && fin) ? min(kmin, kx) : kmin;
    nf |= (valid && !fin) ? 1u : 0u;
}

// The whole selection of one row with n > k columns, by one workgroup.  STAGE:
// rows of up to kStage columns are staged in LDS; without it (a lighter body
// for a rare path) every row is re-read from memory on each pass.
// Steps 1-4 on a row of k < n <= kStage columns whose float4 groups are in
// registers (x[j] = group t + kThreads*j; groups at or past (n+3)/4, and
// columns past n, hold anything): keys staged to LDS, then the selection.
__device__ __forceinline__ void select_staged(Shared &sh, const f32x4 (&x)[kStageGroups], int n, int k,
                                              int32_t *out, int dead = 0) {
    const int t = threadIdx.x;
    const int n4 = (n + 3) >> 2;
    uint32_t kmax = 0u, kmin = 0xFFFFFFFFu, nonfinite = 0u;
    {
#pragma unroll
        for (int j = 0; j < kStageGroups; ++j) {
            const int i = t + kThreads * j;
            if (i < n4) {
                uint4 k4;
                k4.x = order_key(x[j][0]);
                k4.y = order_key(x[j][1]);
                k4.z = order_key(x[j][2]);
                k4.w = order_key(x[j][3]);
                reinterpret_cast<uint4 *>(sh.keys)[i] = k4;
#pragma unroll
                for (int e = 0; e < 4; ++e) track(x[j][e], 4 * i + e < n, kmax, kmin, nonfinite);
            }
        }
        const RowRange rr = row_range(sh, kmax, kmin, nonfinite);
        const StagedKeys sk{sh.keys, n};
        // ---- 2. bucket histogram ------------------------------------------
        if (rr.all_finite) {
            const Bucketer<true> bucket{rr.vmax, rr.scale};
#pragma unroll
            for (int j = 0; j < kStageGroups; ++j) {
                const int i = t + kThreads * j;
                if (i < n4) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * i + e < n) atomicAdd(&sh.hist[bucket.of_value(x[j][e])], 1u);
                }
            }
            __syncthreads();
            select_row<kStageGroups>(sh, sk, n, k, bucket, out, dead);
        } else {
            const Bucketer<false> bucket{rr.vmax, rr.scale};
            for_each_key<kStageGroups>(sk, n, [&](int, uint32_t kx) { atomicAdd(&sh.hist[bucket(kx)], 1u); });
            __syncthreads();
            select_row<kStageGroups>(sh, sk, n, k, bucket, out, dead);
        }
    }
}

template <bool STAGE = true>
__device__ __forceinline__ void select_full_row(Shared &sh, const float *src, int n, int k, int32_t *out,
                                                int dead = 0) {
    const int t = threadIdx.x;
    const int n4 = (n + 3) >> 2;
    uint32_t kmax = 0u, kmin = 0xFFFFFFFFu, nonfinite = 0u;
    if (STAGE && n <= kStage) {
        // ---- 1. stage the row: all loads in flight, then keys to LDS ------
        f32x4 x[kStageGroups];
#pragma unroll
        for (int j = 0; j < kStageGroups; ++j) {
            const int i = t + kThreads * j;
            x[j] = (i < n4) ? kill_dead(load4(src, i), i, dead) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        select_staged(sh, x, n, k, out, dead);
    } else {
        const StreamKeys sk{src, n, dead};
#pragma unroll 1
        for (int i0 = t; i0 < n4; i0 += 4 * kThreads) {  // four float4 loads in flight
            f32x4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * kThreads;
                x[u] = (i < n4) ? kill_dead(load4(src, i), i, dead) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) track(x[u][e], 4 * (i0 + u * kThreads) + e < n, kmax, kmin, nonfinite);
        }
        const RowRange rr = row_range(sh, kmax, kmin, nonfinite);
        const Bucketer<false> bucket{rr.vmax, rr.scale};
        for_each_key<kMaxGroups>(sk, n, [&](int, uint32_t kx) { atomicAdd(&sh.hist[bucket(kx)], 1u); });
        __syncthreads();
        select_row<kMaxGroups>(sh, sk, n, k, bucket, out, dead);
    }
}

// ---- register-resident selection of a finite row ---------------------------
//
// The same selection as select_staged for the common case -- every visible
// value finite and at most kCand values in the crossing bucket -- with the
// row kept in registers and compared as floats, so that each pass
// costs a few vector operations per element:
//  * range: NaN-propagating max3/min3 (a NaN or an infinity sends the row to
//    select_staged);
//  * buckets: 1 + floor(vmax*s - v*s) with one fma, clamped to [1, kBins-2],
//    i.e. monotone non-increasing in v.  The fma's result f can fall below 0
//    (vmax*s is rounded, and once vmax/span exceeds about 16K that rounding
//    exceeds 1), hence the lower clamp.  Bucket b holds exactly the f in [b-1, b), the first bucket
//    everything below 1 and the last everything from kBins-3 up, so the
//    crossing bucket's members are found by two compares on f;
//  * the kept set: v >= T as floats (for finite values the float order with
//    +0 == -0 is the key order) when every key equal to T is kept; when the
//    column order drops some, v > T or (v == T and column <= Ct), with Ct the
//    k-th pair's column (from the one-wave ranking of a short member list, or
//    a radix select over the tied members' columns).
// The kept columns are ranked in column order into LDS and written with
// contiguous stores.  Returns false, having written nothing, in any other case.

__device__ __forceinline__ int fast_bucket(float v, float s, float off) {
    return 1 + max(min((int)__builtin_fmaf(v, -s, off), kBins - 3), 0);
}

// The bucket map of the workgroup's previous row (its own range, handed on
// when it completed this path): the next row's histogram is taken with it in
// the same pass as that row's range, which saves the range's barrier.  The map
// is monotone whatever row it came from, and the end buckets are open-ended,
// so the crossing and its members stay exact; only a crossing bucket too
// crowded for the member list sends the row to a histogram over its own range.
struct FastMap {
    float sc, off;
    bool valid;
};

// Writes the k column indices of the workgroup's previous register-path row
// (left in sh.kept16) to `out`.
__device__ __forceinline__ void flush_kept(const Shared &sh, int k, int32_t *out) {
    for (int p = threadIdx.x; p < k; p += kThreads) out[p] = (int32_t)sh.kept16[p];
}

// `issue` is called once, by every thread, just before the row's first
// barrier: the caller issues its next row's prefetch there, when the waves
// that finish their histogram early would otherwise wait.
template <class Issue>
__device__ __forceinline__ bool select_fast(Shared &sh, f32x4 (&x)[kStageGroups], int n, int k, int32_t *out,
                                            int32_t *&pend, FastMap &map, Issue &&issue) {
    int t = threadIdx.x;
    // opaque to the optimiser: column indices derived from t are recomputed
    // per row rather than kept live (in registers the row needs) across rows
    asm volatile("" : "+v"(t));
    const int w = t >> 6;
    const int l = t & 63;
    const int n4 = (n + 3) >> 2;
    // columns past n (in the last group, and in the copies of it that threads
    // past the row loaded) take the value of the group's first column, which
    // is visible: the range is unchanged, and every count below tests the
    // column
    const int tail = n - 4 * (n4 - 1);  // visible columns of the last group, 1..4
    // first thread of this wave, as a scalar: whether a wave's group j reaches
    // past n is uniform, so waves whose columns are all visible skip the fixes
    const int wt0 = __builtin_amdgcn_readfirstlane(t & ~63);
    const FastMap pm = map;
    map.valid = false;
    // the histogram of the row's visible columns over a map (counts of the
    // last group's columns past n are 0)
    auto histogram = [&](float hs, float hoff) {
#pragma unroll
        for (int j = 0; j < kStageGroups; ++j) {
            const int i = t + kThreads * j;
            if (4 * i + 4 <= n) {
#pragma unroll
                for (int e = 0; e < 4; ++e) atomicAdd(&sh.hist[fast_bucket(x[j][e], hs, hoff)], 1u);
            } else if (i < n4) {
#pragma unroll
                for (int e = 0; e < 4; ++e) atomicAdd(&sh.hist[fast_bucket(x[j][e], hs, hoff)], e < tail ? 1u : 0u);
            }
        }
    };
    float mx = x[0][0], mn = x[0][0];
#pragma unroll
    for (int j = 0; j < kStageGroups; ++j) {
        const int i = t + kThreads * j;
        if (4 * (wt0 + 63 + kThreads * j) + 4 > n && i >= n4 - 1) {
#pragma unroll
            for (int e = 1; e < 4; ++e) x[j][e] = e < tail ? x[j][e] : x[j][0];
        }
        mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(x[j][0], x[j][1]));
        mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(x[j][2], x[j][3]));
        mn = __builtin_elementwise_minimum(mn, __builtin_elementwise_minimum(x[j][0], x[j][1]));
        mn = __builtin_elementwise_minimum(mn, __builtin_elementwise_minimum(x[j][2], x[j][3]));
    }
    const bool fin = __builtin_isfinite(mx) && __builtin_isfinite(mn);
    float sc = pm.sc, off = pm.off;
    RowRange rr;
    Crossing cr;
    if (pm.valid) {
        // the previous row's map, before the range's barrier (the histogram
        // was left cleared); a non-finite value's bucket is clamped, and the
        // row then leaves this path
        histogram(sc, off);
        range_publish(sh, fin ? order_key(mx) : 0u, fin ? order_key(mn) : 0xFFFFFFFFu, fin ? 0u : 1u, t);
        if (t == 0) sh.ncand = 0;  // the member count below (its barriers order it)
        issue();
        __syncthreads();
        if (pend) {  // the previous row's kept list (ordered by the barrier)
            flush_kept(sh, k, pend);
            pend = nullptr;
        }
        rr = range_read(sh);
        if (!rr.all_finite) {
            __syncthreads();
            return false;
        }
        cr = find_crossing_w(sh, k);
    }
    if (!pm.valid || cr.cnt > kCand) {  // the row's own map
        if (pm.valid) {
            __syncthreads();  // every wave is done reading the histogram
            clear_hist(sh);
            __syncthreads();
        } else {
            issue();
            rr = row_range(sh, fin ? order_key(mx) : 0u, fin ? order_key(mn) : 0xFFFFFFFFu, fin ? 0u : 1u, t);
            if (pend) {
                flush_kept(sh, k, pend);
                pend = nullptr;
            }
            if (!rr.all_finite) {
                __syncthreads();
                return false;
            }
        }
        sc = rr.scale;
        off = rr.vmax * rr.scale;
        histogram(sc, off);
        if (t == 0) sh.ncand = 0;  // the member count below (its barriers order it)
        __syncthreads();
        cr = find_crossing_w(sh, k);
    }
    const int bstar = cr.bin;
    int need = k - cr.above;
    int cnt = cr.cnt;
    if (cnt > kCand) {
        __syncthreads();
        return false;
    }

    // ---- the members of the crossing bucket, as (key, column) ------------
    // fast_bucket(v) == bstar exactly when the fma's f lies in [f_lo, f_hi)
    const float f_lo = bstar <= 1 ? -__builtin_inff() : (float)(bstar - 1);
    const float f_hi = bstar >= kBins - 2 ? __builtin_inff() : (float)bstar;
#pragma unroll
    for (int j = 0; j < kStageGroups; ++j) {
        const int i = t + kThreads * j;
        bool hit[4];
        bool any = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float f = __builtin_fmaf(x[j][e], -sc, off);
            hit[e] = (4 * i + e < n) & (f >= f_lo) & (f < f_hi);
            any |= hit[e];
        }
        if (ballot(any)) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint64_t m = ballot(hit[e]);
                if (m) {
                    const int lead = __builtin_ctzll(m);
                    int base = 0;
                    if (l == lead) base = atomicAdd(&sh.ncand, __popcll(m));
                    base = readlane(base, lead);
                    const int at = base + mask_prefix(m);
                    if (hit[e]) {  // at < cnt <= kCand
                        sh.cand_key[at] = order_key(x[j][e]);
                        sh.cand_col[at] = 4 * i + e;
                    }
                }
            }
        }
    }
    __syncthreads();
    const int nc = sh.ncand;  // == cnt: the same test as the histogram's
    if (nc != cnt) {  // never expected; uniform (read after the barrier)
        __syncthreads();
        return false;
    }

    // ---- the k-th pair (T, Ct) -------------------------------------------
    // (one wave ranks a short list and hands the result on through LDS: 16
    // waves ranking it each for itself, without the barrier, were slower once
    // the kept set needed fewer barriers)
    uint32_t T;
    // a tie at T that the column order cuts: the values equal to T are kept
    // at columns <= Ct only, else Ct = INT_MAX
    int Ct = 0x7FFFFFFF;
    if (nc <= 64) {
        if (w == 0) {
            const uint32_t mk = l < nc ? sh.cand_key[l] : 0u;
            const int mc = l < nc ? sh.cand_col[l] : 0x7FFFFFFF;
            int rank = 0;
            for (int j = 0; j < nc; ++j) {
                const uint32_t kj = (uint32_t)readlane((int)mk, j);
                const int cj = readlane(mc, j);
                rank += (kj > mk || (kj == mk && cj < mc)) ? 1 : 0;
            }
            const bool is_kth = l < nc && rank == need - 1;
            if (is_kth) sh.thr_key = mk;
            // a key equal to the k-th at a later column would be dropped
            const int kl = __builtin_ctzll(ballot(is_kth) | (1ull << 63));  // defined for an empty mask
            const uint32_t tk = (uint32_t)readlane((int)mk, kl);
            const int tc = readlane(mc, kl);
            const bool cut = ballot(l < nc && mk == tk && mc > tc) != 0ull;
            if (l == 0) sh.tie_col = cut ? tc : 0x7FFFFFFF;
        }
        __syncthreads();
        T = sh.thr_key;
        Ct = __builtin_amdgcn_readfirstlane(sh.tie_col);
    } else {
        radix_select(sh, [&](auto f) {
            for (int j = t; j < nc; j += kThreads) f(sh.cand_key[j]);
        }, T, need, cnt);
        if (cnt > need) {
            // the column order decides among the cnt members equal to T: Ct is
            // the need-th smallest of their columns (columns < 65536, so the
            // need-th largest of 0xFFFF - column; columns are distinct)
            uint32_t cm;
            int need2 = need, cnt2 = 0;
            radix_select(sh, [&](auto f) {
                for (int j = t; j < nc; j += kThreads)
                    if (sh.cand_key[j] == T) f(0xFFFFu - (uint32_t)sh.cand_col[j]);
            }, cm, need2, cnt2);
            Ct = __builtin_amdgcn_readfirstlane(0xFFFF - (int)cm);
        }
    }
    const float Tf = key_value(T);

    // ---- the kept set in column order -----------------------------------
    // Slice j of wave w (its lanes' group j) is the 256 columns from
    // 4096 j + 256 w, so the column order of the slices is (j, w).  The wave
    // turns its 8 x 64 flag nibbles around through its own 512 bytes of the
    // histogram's words (last read before the members' barrier; no other wave
    // touches them): lane l then holds the 32 consecutive columns from
    // 4096 (l / 8) + 256 w + 32 (l % 8) as one flag byte per float4 group.  A
    // scan over each 8-lane segment ranks them inside the slice, and one scan
    // of the 128 slice totals in (j, w) order, after one barrier, places the
    // slices.  Each wave then clears its part of the histogram for the next row.
    uint8_t *wf = reinterpret_cast<uint8_t *>(sh.hist) + 512 * w;
    static_assert(kStageGroups * kThreads <= (int)sizeof(uint32_t) * kBins, "a byte per group fits the histogram");
    if (Ct == 0x7FFFFFFF) {
#pragma unroll
        for (int j = 0; j < kStageGroups; ++j) {
            uint32_t nib = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) nib |= (((x[j][e] >= Tf) & (4 * (t + kThreads * j) + e < n)) ? 1u : 0u) << e;
            wf[64 * j + l] = (uint8_t)nib;
        }
    } else {  // (Ct < n)
        // column tests of their own: shared with the branch above, the
        // compiler hoists them out of both into scalar masks that spill
        int tc = t;
        asm volatile("" : "+v"(tc));
#pragma unroll
        for (int j = 0; j < kStageGroups; ++j) {
            uint32_t nib = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int col = 4 * (tc + kThreads * j) + e;
                nib |= (((x[j][e] > Tf) & (col < n)) | ((x[j][e] == Tf) & (col <= Ct)) ? 1u : 0u) << e;
            }
            wf[64 * j + l] = (uint8_t)nib;
        }
    }
    const uint2 fw = reinterpret_cast<const uint2 *>(wf)[l];  // lanes 8 (l % 8) .. +7 of slice l / 8
    {
        uint32_t z;  // made here: a zero pair kept live across the row loop was spilled
        asm volatile("v_mov_b32 %0, 0" : "=v"(z));
        reinterpret_cast<uint2 *>(wf)[l] = make_uint2(z, z);
    }
    const int mine = __popc(fw.x) + __popc(fw.y);
    int seg = mine;  // inclusive scan over the lane's 8-lane segment
    {
        const int s1 = __builtin_amdgcn_update_dpp(0, seg, kDppRowShr1, 0xF, 0xF, false);
        seg += (l & 7) >= 1 ? s1 : 0;
        const int s2 = __builtin_amdgcn_update_dpp(0, seg, kDppRowShr2, 0xF, 0xF, false);
        seg += (l & 7) >= 2 ? s2 : 0;
        const int s4 = __builtin_amdgcn_update_dpp(0, seg, kDppRowShr4, 0xF, 0xF, false);
        seg += (l & 7) >= 4 ? s4 : 0;
    }
    if ((l & 7) == 7) sh.ktot[kWaves * (l >> 3) + w] = (uint32_t)seg;
    __syncthreads();
    int p;
    {
        const uint2 tt2 = reinterpret_cast<const uint2 *>(sh.ktot)[l];  // slices 2l, 2l + 1 in (j, w) order
        const int a0 = (int)tt2.x, a1 = (int)tt2.y;
        const int incl = wave_incl_sum(a0 + a1);
        const int before = (w & 1) ? incl - a1 : incl - a0 - a1;  // kept before slice 2l + (w & 1)
        p = shfl_i(before, (kWaves * (l >> 3) + w) >> 1) + seg - mine;
    }
    uint16_t *kept = sh.kept16;
    const int c0 = 4096 * (l >> 3) + 256 * w + 32 * (l & 7);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t word = h ? fw.y : fw.x;  // bit 8b + e: column c0 + 16h + 4b + e
        while (word) {
            const int b = __builtin_ctz(word);
            word &= word - 1u;
            if (p < k) kept[p] = (uint16_t)(c0 + 16 * h + 4 * (b >> 3) + (b & 7));
            ++p;
        }
    }
    // this row's own map for the next row
    map.sc = rr.scale;
    map.off = rr.vmax * rr.scale;
    map.valid = rr.scale > 0.0f;
    // the k columns stay in sh.kept16 until the next row's first barrier (or
    // the caller's), when their stores no longer hold up a wait on the
    // caller's prefetch
    pend = out;
    return true;
}

// Rows of a many-row call, round robin over a grid of workgroups that each take
// at most kRowsPerGroup rows.  The next row that takes the register path is
// copied into LDS (the staging area of the full selection, unused by
// select_fast) by direct global-to-LDS loads while the current row is
// selected, so its HBM reads overlap the selection and hold no registers.
// These loads are issued from inline assembly: the compiler then neither
// knows of them nor orders the selection's own LDS accesses behind them (it
// would, for the builtin form, wait for every one before any LDS access); the
// wait for them is explicit.  They are issued just before a row's first
// barrier, when early waves would wait anyway (issued at the top of the row,
// all 16 waves queued their copies at once and the last waves stalled).  A
// row's output indices stay in LDS until the next row's first barrier and are
// stored then: stores and loads retire in order on one counter, so the next
// wait on a prefetch also waits for stores issued before it, which by then
// have long completed.  Rows the register path does not take (longer than
// kStage, or refused by select_fast) are marked and selected after the loop by
// the staged or streaming selection.
constexpr int kRowsPerGroup = 2048;

// 16 bytes per lane from global memory to LDS at lds_wave + 16 * lane (lds_wave
// wave-uniform).  Leaves the load outstanding on the vector memory counter.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_wave) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(lds_wave)
        : "memory");
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// STARTS: the call has row starts.  Rows whose start is a multiple of 4 take
// the same path as without them, from the shifted row; any other start (its
// view has dead columns) is set aside for the full selection.
template <bool STARTS>
__global__ __launch_bounds__(kThreads) void topk_rows_kernel(TopkArgs a) {
    __shared__ Shared sh;
    __shared__ uint32_t later[kRowsPerGroup / 32];
    const int t = threadIdx.x;
    const int k = a.k;
    const int stride = (int)gridDim.x;
    f32x4 *pref = reinterpret_cast<f32x4 *>(sh.keys);  // the next row, group i at pref[i]
    // read-only: through the constant address space its loads stay scalar
    const __attribute__((address_space(4))) int32_t *ctx =
        (const __attribute__((address_space(4))) int32_t *)a.ctx_lens;
    const __attribute__((address_space(4))) int32_t *starts =
        (const __attribute__((address_space(4))) int32_t *)a.row_starts;
    auto start_of = [&](int r) { return STARTS ? min(max(starts[r], 0), a.width) : 0; };
    auto visible = [&](int r, int s) { return min(max(ctx[r], 0), a.width - s); };
    auto fast_row = [&](int nn, int s) { return k < nn && nn <= kStage && (s & 3) == 0; };
    // every load at an in-row group (clamped)
    auto prefetch = [&](int r, int nn, int s) {
        int tt = t;
        asm volatile("" : "+v"(tt));  // addresses recomputed per row, not kept live across rows
        const f32x4 *src = reinterpret_cast<const f32x4 *>(a.logits + (int64_t)r * a.stride + s);
        const int last = ((nn + 3) >> 2) - 1;
        const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)(uint32_t)(uintptr_t)(pref + (tt & ~63)));
#pragma unroll
        for (int j = 0; j < kStageGroups; ++j)
            dma16(src + min(tt + kThreads * j, last), lds + 16u * kThreads * j);
    };
    for (int i = t; i < kRowsPerGroup / 32; i += kThreads) later[i] = 0u;
    bool any_later = false;  // uniform
    int rows_taken = 0;
    int row = blockIdx.x;
    int st = start_of(row);
    int n = visible(row, st);
    if (fast_row(n, st)) prefetch(row, n, st);
    f32x4 x[kStageGroups];
    int32_t *pend = nullptr;  // the previous row's output, its columns still in LDS
    FastMap fmap{0.0f, 0.0f, false};  // the register path's map for its next row
#pragma unroll 1
    for (int m = 0;; ++m) {
        const int nxt = row + stride;
        const bool more = nxt < a.num_rows;
        const int nst = more ? start_of(nxt) : 0;
        const int nn = more ? visible(nxt, nst) : 0;
        const bool fast = fast_row(n, st);
        // Every thread reads back only the slots its own lane copied, so the
        // copy needs no barrier: the wave's wait covers its own copies, and the
        // reads complete before the next copy into the same slots is issued.
        if (fast) {
            wait_dma();
            int tt = t;
            asm volatile("" : "+v"(tt));
#pragma unroll
            for (int j = 0; j < kStageGroups; ++j) x[j] = pref[tt + kThreads * j];
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        auto issue_next = [&]() {
            if (more && fast_row(nn, nst)) prefetch(nxt, nn, nst);
        };
        // (a row that takes the register path issues it before its first
        // barrier; any other row here)
        if (!fast) issue_next();
        int32_t *out = a.idx_out + (int64_t)row * k;
        // The previous row's kept list is written out after the first barrier
        // of select_fast, or here for a row that does not take it.
        if (pend && !fast) {
            __syncthreads();
            flush_kept(sh, k, pend);
            pend = nullptr;
        }
        if (n <= k) {
            for (int j = t; j < k; j += kThreads) out[j] = j < n ? j : -1;
        } else if (fast && select_fast(sh, x, n, k, out, pend, fmap, issue_next)) {
        } else {
            if (t == 0) later[m >> 5] |= 1u << (m & 31);
            any_later = true;
        }
        rows_taken = m + 1;
        if (!more) break;
        row = nxt;
        n = nn;
        st = nst;
    }
    if (pend) {
        __syncthreads();
        flush_kept(sh, k, pend);
    }
    if (!any_later) return;
    __syncthreads();
#pragma unroll 1
    for (int wd = 0; wd < (rows_taken + 31) >> 5; ++wd) {
        uint32_t bits = later[wd];
        while (bits) {
            const int m = 32 * wd + __builtin_ctz(bits);
            bits &= bits - 1u;
            const int r = (int)blockIdx.x + m * stride;
            const RowView v = row_view(a, r);
            select_full_row<false>(sh, v.src, v.n, k, a.idx_out + (int64_t)r * k, v.dead);
            __syncthreads();
        }
    }
}

// ---- split selection: several workgroups per row ----------------------------
//
// With few rows (decode), one workgroup per row leaves most CUs idle and runs
// every pass over its row on one CU.  The row is cut into `slices` contiguous
// slices, one workgroup each; thread t of a slice owns G consecutive float4
// (columns lo + 4Gt ..), so that column order is thread order.  Two kernels:
//
//  window:  every workgroup of a row draws the same sample of the row (128 runs
//           of 16 columns spread evenly; the whole row when shorter than 2048),
//           buckets it linearly between its finite min and max, and takes the
//           buckets holding the sample ranks k*m/n -/+ (4 sigma + 8) of a
//           binomial count: their edges give thresholds a > b.  Columns >= a
//           are "above", columns in [b, a) are the window's members.  It counts
//           its slice's columns above, and records each member (key, column,
//           member bucket) plus the slice's histogram over kMBins member
//           buckets, a map linear over the window that every workgroup of the
//           row shares.
//  resolve: every workgroup of the row loads the row's counts, histograms and
//           members and its own slice in one round of loads, finds the member
//           bucket of the (k - above)-th largest, takes (T, Ct) among that
//           bucket's members exactly, and writes the kept columns of its slice
//           at the offset counted from the earlier slices (above + members in
//           higher buckets + kept members of the crossing bucket).
//
// Every workgroup of a row takes the same decisions from the same data, so no
// workgroup waits for another.  A window that misses the k-th value, or a slice
// with more members than slots, sends the row down the one-workgroup selection
// (in the resolve kernel's first slice): the sample decides speed, never the
// result.  Loads are unconditional at clamped in-row addresses, so a wait for
// one load never waits for later ones, and the tests are branch-free.

constexpr int kSample = 2048;         // sampled columns per row
constexpr int kSampleRuns = kSample / 16;
constexpr int kMBins = 256;           // member buckets
constexpr int kSliceGroups = 8;       // float4 per thread at most: slices <= 32768 columns
constexpr int kSlotLoads = 8;         // member slots a resolve thread loads
constexpr int kHistLoads = 5;         // histogram words a resolve thread loads (17 slices)
constexpr int kSplitCUs = 256;        // workgroups that fill the chip once
constexpr int kSplitMaxRows = kSplitCUs / 2;
// From this many rows, rows that fit the register path (width <= kStage) take
// one workgroup each: 64 rows of 32,768 columns in 13.4 us against 14.3 us
// split; 36 rows of 29,408 columns 13.2 against 13.4 us
constexpr int kRowsMinRows = 48;
constexpr int kRowsGrid = 256;         // one workgroup per CU (LDS)

struct WindowShared {
    alignas(16) uint32_t hist[kBins];
    uint32_t mhist[kMBins];
    uint32_t red_max[kWaves];
    uint32_t red_min[kWaves];
    int u_top;
    int u_bot;
    int nmem;
    int nabove;
};

// Buckets linear in the value, bucket 1 holding vmax and above, bucket
// top + 1 holding vmax - top/scale and below (infinities clamp to the ends, NaN
// goes to bucket 1).  Monotone non-increasing in the value.
struct RangeBucketer {
    float vmax, scale, top;
    __device__ __forceinline__ int operator()(float v) const {
        return 1 + (int)fminf(fmaxf((vmax - v) * scale, 0.0f), top);
    }
};

// Range map over [key_value(kmin), key_value(kmax)] with nb buckets (1 .. nb-2);
// a degenerate range maps everything to bucket 1.
__device__ __forceinline__ RangeBucketer make_range(float vmax, float vmin, int nb) {
    const float span = vmax - vmin;
    const float scale = (float)(nb - 3) / span;
    const bool usable = span > 0.0f && __builtin_isfinite(span) && __builtin_isfinite(scale);
    return RangeBucketer{vmax, usable ? scale : 0.0f, (float)(nb - 3)};
}

// unsigned max over the kWaves per-wave partials (one LDS read per wave)
__device__ __forceinline__ uint32_t partials_umax(const uint32_t *red) {
    const int l = lane_id();
    return row16_total_umax(l < kWaves ? red[l] : 0u);
}

// Bin of hist (64 * 4 * Q bins, in order) where the running count first
// reaches `need` (1 <= need <= total), and the count before that bin.  One full
// wave: 4Q bins per lane, then the owning lane's bins one per lane.
template <int Q>
__device__ __forceinline__ void wave_crossing(const uint32_t *hist, int need, int &bin, int &before) {
    constexpr int P = 4 * Q;  // bins per lane
    const int l = lane_id();
    const uint4 *h4 = reinterpret_cast<const uint4 *>(hist) + Q * l;
    int s = 0;
#pragma unroll
    for (int i = 0; i < Q; ++i) {
        const uint4 v = h4[i];
        s += (int)(v.x + v.y + v.z + v.w);
    }
    const int incl = wave_incl_sum(s);
    const uint64_t mo = ballot(incl >= need);  // never empty for need <= total
    const int owner = mo ? __builtin_ctzll(mo) : 63;
    const int base = readlane(incl - s, owner);
    const int c = l < P ? (int)hist[P * owner + l] : 0;
    const int ci = wave_incl_sum(c);
    const uint64_t ms = ballot(base + ci >= need);
    const int sub = ms ? min(__builtin_ctzll(ms), P - 1) : P - 1;
    bin = P * owner + sub;
    before = base + readlane(ci - c, sub);
}

struct SplitWorkspace {
    int2 *meta;      // [rows * slices]: (columns above the window, window members)
    uint32_t *hist;  // [rows * slices][kMBins]: members per member bucket
    uint2 *slot;     // [rows * slices][cand_cap]: (key, column | member bucket << 17)
};

__host__ __device__ __forceinline__ int64_t split_meta_bytes(int rows, int slices) {
    return ((int64_t)rows * slices * 8 + 255) & ~(int64_t)255;
}

__device__ __forceinline__ SplitWorkspace split_ws(const TopkArgs &a) {
    const int64_t rs = (int64_t)a.num_rows * a.slices;
    SplitWorkspace w;
    w.meta = reinterpret_cast<int2 *>(a.workspace);
    w.hist = reinterpret_cast<uint32_t *>(a.workspace + split_meta_bytes(a.num_rows, a.slices));
    w.slot = reinterpret_cast<uint2 *>(reinterpret_cast<uint8_t *>(w.hist) + rs * kMBins * 4);
    return w;
}

// value of register slot b (float4 b >> 2, element b & 3) of x: static selects
template <int G>
__device__ __forceinline__ float pick(const f32x4 (&x)[G], int b) {
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < 4 * G; ++q) v = (q == b) ? x[q >> 2][q & 3] : v;
    return v;
}

template <int G>
__global__ __launch_bounds__(kThreads) void topk_window_kernel(TopkArgs a) {
    __shared__ WindowShared sh;
    const int row = blockIdx.x / a.slices;
    const int s = blockIdx.x - row * a.slices;
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int l = t & 63;
    const RowView view = row_view(a, row);
    const int n = view.n;
    const int k = a.k;
    const int lo = s * a.slice_len;
    if (view.vis <= k || lo >= n) return;
    const int hi = min(n, lo + a.slice_len);
    const int n4 = (n + 3) >> 2;
    const float *src = view.src;

    // the sample first (it is used first), then this thread's float4 of the slice
    const int m = n >= kSample ? kSample : n;
    const int ts = t & (kSample / 4 - 1);
    int sc;
    if (n >= kSample) {
        const int run = ts >> 2;
        const int center = (int)(((int64_t)(2 * run + 1) * n) / (2 * kSampleRuns));
        sc = (min(max(center - 8, 0), n - 16) & ~3) + 4 * (ts & 3);
    } else {
        sc = 4 * ts;
    }
    const f32x4 y = kill_dead(load4(src, min(sc >> 2, n4 - 1)), min(sc >> 2, n4 - 1), view.dead);
    if (t >= kSample / 4) sc = n;  // one sample per column: the first 512 threads
    const int c0 = lo + 4 * G * t;   // this thread's first column
    f32x4 x[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const int i = min((c0 >> 2) + j, n4 - 1);
        x[j] = kill_dead(load4(src, i), i, view.dead);
    }

    clear_hist(sh);
    if (t < kMBins) sh.mhist[t] = 0u;
    if (t == 0) {
        sh.nmem = 0;
        sh.nabove = 0;
    }
    // finite range of the sample
    uint32_t kmax = 0u, kmin = 0xFFFFFFFFu, nonfinite = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) track(y[e], sc + e < n, kmax, kmin, nonfinite);
    kmax = wave_total_umax(kmax);
    const uint32_t nkmin = wave_total_umax(~kmin);
    if (l == 0) {
        sh.red_max[w] = kmax;
        sh.red_min[w] = nkmin;
    }
    __syncthreads();
    const uint32_t gmax = partials_umax(sh.red_max);
    const uint32_t gmin = ~partials_umax(sh.red_min);
    const bool have = gmax != 0u;  // some finite sample
    const float smax = key_value(gmax), smin = key_value(gmin);
    const RangeBucketer sb = have ? make_range(smax, smin, kBins) : RangeBucketer{0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (sc + e < n) atomicAdd(&sh.hist[sb(y[e])], 1u);
    __syncthreads();
    if (w == 0) {  // sample buckets of the ranks around the k-th largest
        const float p = (float)k / (float)n;
        const float mean = p * (float)m;
        const float dev = 4.0f * sqrtf((float)m * p * (1.0f - p)) + 8.0f;
        const int top_rank = (int)floorf(mean - dev);
        const int bot_rank = (int)ceilf(mean + dev);
        int u_top = 0, u_bot = kBins - 1, before;
        if (top_rank >= 1) wave_crossing<kBins / 256>(sh.hist, top_rank, u_top, before);
        if (bot_rank <= m) wave_crossing<kBins / 256>(sh.hist, bot_rank, u_bot, before);
        if (l == 0) {
            sh.u_top = u_top;
            sh.u_bot = u_bot;
        }
    }
    __syncthreads();
    // thresholds at the bucket edges (any values give the right result)
    const int u_top = sh.u_top, u_bot = sh.u_bot;
    const bool sampled = sb.scale > 0.0f;
    const float a_val = (u_top <= 1 || !sampled) ? __builtin_inff() : sb.vmax - (float)(u_top - 1) / sb.scale;
    const float b_val = (u_bot >= kBins - 2 || !sampled) ? -__builtin_inff() : sb.vmax - (float)u_bot / sb.scale;
    // member buckets: linear over the window, or over the sampled range where
    // the window is open
    const float mtop = __builtin_isfinite(a_val) ? a_val : smax;
    const float mlow = __builtin_isfinite(b_val) ? b_val : smin;
    const RangeBucketer mbk = have ? make_range(mtop, mlow, kMBins) : RangeBucketer{0.0f, 0.0f, 0.0f};

    // the slice: columns above, member bits (bit 4j + e)
    int above = 0;
    uint32_t mbits = 0u;
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v = x[j][e];
            const bool valid = c0 + 4 * j + e < hi;
            const bool ge_a = v >= a_val;
            above += __popcll(ballot(valid & ge_a));
            mbits |= (uint32_t)(valid & (v >= b_val) & !ge_a) << (4 * j + e);
        }
    }
    const int nmem = __popc(mbits);
    const int mincl = wave_incl_sum(nmem);
    int wbase = 0;
    if (l == 63 && mincl > 0) wbase = atomicAdd(&sh.nmem, mincl);
    wbase = readlane(wbase, 63);
    if (l == 0 && above) atomicAdd(&sh.nabove, above);
    const SplitWorkspace ws = split_ws(a);
    const int64_t rs = (int64_t)row * a.slices + s;
    uint2 *slot = ws.slot + (rs << a.cand_shift);
    const int cap = 1 << a.cand_shift;
    int at = wbase + mincl - nmem;
    while (mbits) {  // ~ a few percent of the columns: per-lane loop
        const int b = __builtin_ctz(mbits);
        mbits &= mbits - 1u;
        const float v = pick<G>(x, b);
        const int mb = mbk(v);
        if (at < cap) slot[at] = make_uint2(order_key(v), (uint32_t)(c0 + b) | ((uint32_t)mb << 17));
        atomicAdd(&sh.mhist[mb], 1u);
        ++at;
    }
    __syncthreads();
    if (t < kMBins) ws.hist[rs * kMBins + t] = sh.mhist[t];
    if (t == 0) ws.meta[rs] = make_int2(sh.nabove, sh.nmem);
}

template <int G>
__global__ __launch_bounds__(kThreads) void topk_resolve_kernel(TopkArgs a) {
    __shared__ Shared sh;
    const int row = blockIdx.x / a.slices;
    const int s = blockIdx.x - row * a.slices;
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int l = t & 63;
    const RowView view = row_view(a, row);
    const int n = view.n;
    const int k = a.k;
    int32_t *out = a.idx_out + (int64_t)row * k;
    const float *src = view.src;
    if (view.vis <= k) {
        if (s == 0)
            for (int j = t; j < k; j += kThreads) out[j] = j < view.vis ? j : -1;
        return;
    }
    const int lo = s * a.slice_len;
    if (lo >= n) return;
    const int hi = min(n, lo + a.slice_len);
    const int ns = (n + a.slice_len - 1) / a.slice_len;  // slices of this row (<= 64)
    const int n4 = (n + 3) >> 2;

    // one round of loads: this thread's slice float4, the row's counts,
    // histograms and member slots (unconditional, clamped)
    const int c0 = lo + 4 * G * t;
    f32x4 x[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const int i = min((c0 >> 2) + j, n4 - 1);
        x[j] = kill_dead(load4(src, i), i, view.dead);
    }
    const SplitWorkspace ws = split_ws(a);
    const int64_t rs0 = (int64_t)row * a.slices;
    const int2 mt = ws.meta[rs0 + min(l, ns - 1)];
    const int nh = ns * kMBins;
    uint32_t hv[kHistLoads];
#pragma unroll
    for (int u = 0; u < kHistLoads; ++u) hv[u] = ws.hist[rs0 * kMBins + min(t + kThreads * u, nh - 1)];
    const int nslots = ns << a.cand_shift;
    uint2 sv[kSlotLoads];
#pragma unroll
    for (int u = 0; u < kSlotLoads; ++u) sv[u] = ws.slot[(rs0 << a.cand_shift) + min(t + kThreads * u, nslots - 1)];

    // row totals; histograms into LDS (per slice, and summed over slices)
    uint32_t *hs = sh.keys;  // [ns][kMBins]
    uint32_t *tot = sh.hist; // [kMBins]
    if (t < kMBins) tot[t] = 0u;
    if (t == 0) sh.ncand = 0;
    if (w == 0) {
        const int ab = l < ns ? mt.x : 0;
        const int nm = l < ns ? mt.y : 0;
        const int ai = wave_incl_sum(ab);
        const uint64_t over = ballot(nm > (1 << a.cand_shift));
        if (l < ns) sh.grp[l] = nm;  // members of slice l
        if (l == s) sh.split_before = ai - ab;
        if (l == 63) {
            sh.split_above = ai;
            sh.split_over = over != 0;
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kHistLoads; ++u) {
        const int f = t + kThreads * u;
        if (f < nh) {
            hs[f] = hv[u];
            if (hv[u]) atomicAdd(&tot[f & (kMBins - 1)], hv[u]);
        }
    }
    __syncthreads();
    const int need = k - sh.split_above;
    if (w == 0) {  // crossing bucket; members above it in earlier slices
        int nall = 0;
        {
            const uint4 v = reinterpret_cast<const uint4 *>(tot)[l];
            nall = wave_total_sum((int)(v.x + v.y + v.z + v.w));
        }
        int bin = 0, before = 0;
        if (need >= 1 && need <= nall) wave_crossing<1>(tot, need, bin, before);
        int below = 0;  // members of slices < s in buckets < bin
        for (int j = 0; j < s; ++j) {
            const uint4 v = reinterpret_cast<const uint4 *>(hs + j * kMBins)[l];
            const int b0 = 4 * l;
            below += (b0 < bin ? (int)v.x : 0) + (b0 + 1 < bin ? (int)v.y : 0) +
                     (b0 + 2 < bin ? (int)v.z : 0) + (b0 + 3 < bin ? (int)v.w : 0);
        }
        below = wave_total_sum(below);
        if (l == 0) {
            sh.split_n = nall;
            sh.cross_bin = bin;
            sh.cross_above = before;
            sh.cross_cnt = (int)tot[bin];
            sh.split_before += below;
            sh.kept_before = 0;
        }
    }
    __syncthreads();
    const int N = sh.split_n;
    const int cnt = sh.cross_cnt;
    if (sh.split_over || need < 1 || need > N || cnt > kCand) {
        if (s == 0) select_full_row<false>(sh, src, n, k, out, view.dead);
        return;
    }
    const int bstar = sh.cross_bin;
    const int need2 = need - sh.cross_above;

    // members of the crossing bucket -> (key, column) list
#pragma unroll
    for (int u = 0; u < kSlotLoads; ++u) {
        const int f = t + kThreads * u;
        const int j = f >> a.cand_shift;
        const bool hit = f < nslots && (f & ((1 << a.cand_shift) - 1)) < sh.grp[min(j, ns - 1)] &&
                         (int)(sv[u].y >> 17) == bstar;
        const uint64_t mk = ballot(hit);
        if (mk) {
            const int lead = __builtin_ctzll(mk);
            int base = 0;
            if (l == lead) base = atomicAdd(&sh.ncand, __popcll(mk));
            base = readlane(base, lead);
            if (hit) {
                const int at = base + mask_prefix(mk);
                sh.cand_key[at] = sv[u].x;
                sh.cand_col[at] = (int)(sv[u].y & 0x1FFFFu);
            }
        }
    }
    __syncthreads();

    // the k-th pair (T, Ct) inside the crossing bucket
    uint32_t T;
    int Ct;
    if (cnt <= 64) {
        if (w == 0) {
            const uint32_t mk = l < cnt ? sh.cand_key[l] : 0u;
            const int mc = l < cnt ? sh.cand_col[l] : 0x7FFFFFFF;
            int rank = 0;
            for (int j = 0; j < cnt; ++j) {
                const uint32_t kj = (uint32_t)readlane((int)mk, j);
                const int cj = readlane(mc, j);
                rank += (kj > mk || (kj == mk && cj < mc)) ? 1 : 0;
            }
            if (l < cnt && rank == need2 - 1) {
                sh.thr_key = mk;
                sh.tie_col = mc;
            }
            // kept members of the crossing bucket in earlier slices
            const bool kept_early = l < cnt && mc < lo && rank <= need2 - 1;
            const int kb = __popcll(ballot(kept_early));
            if (l == 0) sh.kept_before = kb;
        }
        __syncthreads();
        T = sh.thr_key;
        Ct = sh.tie_col;
    } else {
        int need3 = need2, cnt3 = 0;
        radix_select(sh, [&](auto f) {
            for (int j = t; j < cnt; j += kThreads) f(sh.cand_key[j]);
        }, T, need3, cnt3);
        if (cnt3 > need3) {  // split the keys equal to T: need3-th lowest column
            uint32_t nc_key;
            int need4 = need3, cnt4 = 0;
            radix_select(sh, [&](auto f) {
                for (int j = t; j < cnt; j += kThreads)
                    if (sh.cand_key[j] == T) f(~(uint32_t)sh.cand_col[j]);
            }, nc_key, need4, cnt4);
            Ct = (int)~nc_key;
        } else {
            Ct = 0x7FFFFFFF;
        }
        int kb = 0;
        for (int j = t; j < cnt; j += kThreads) {
            const uint32_t key = sh.cand_key[j];
            const int col = sh.cand_col[j];
            kb += (col < lo && (key > T || (key == T && col <= Ct))) ? 1 : 0;
        }
        kb = wave_total_sum(kb);
        if (l == 0 && kb) atomicAdd(&sh.kept_before, kb);
    }
    const float tv = key_value(T);

    // this slice's kept columns: thread order is column order
    uint32_t sel = 0u;
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int col = c0 + 4 * j + e;
            const float v = x[j][e];
            sel |= (uint32_t)((col < hi) & ((v > tv) | ((v == tv) & (col <= Ct)))) << (4 * j + e);
        }
    const int mine = __popc(sel);
    const int incl = wave_incl_sum(mine);
    if (l == 63) sh.wave_tot[w] = incl;
    __syncthreads();
    const int wt = l < kWaves ? sh.wave_tot[l] : 0;
    const int wincl = row16_scan_dpp(wt, 0, OpAdd());  // lanes 0..15: the waves' running totals
    int p = sh.split_before + sh.kept_before + readlane(wincl - wt, w) + incl - mine;
    while (sel) {
        const int b = __builtin_ctz(sel);
        sel &= sel - 1u;
        if (p < k) out[p] = c0 + b - view.dead;
        ++p;
    }
}

// ---- fused selection: the resolve from the scoring kernel's candidates -----
//
// The per-tile scoring kernel has written, for every row and 64-column chunk,
// the chunk's 32 largest scores as packed keys (the score's order key with its
// low 6 bits replaced by 63 - the column in the chunk: the order (truncated
// score desc, column asc), distinct within a row).  One workgroup per row,
// thread t holding the list of chunk t (and t + 1024) in registers:
//
//  1. the lists' range and count (a list covers every column of a chunk with
//     at most 32 visible ones);
//  2. a bucket histogram over the truncated scores, the crossing bucket, and
//     among its members the k-th largest packed key P;
//  3. keys whose truncated score is above P's are kept; those equal to it (P,
//     and rarely columns within 64 ulp of it) are ranked on their exact logits
//     (value desc, column asc) for the remaining places.  A full chunk whose
//     32nd key has P's truncated score or more might hold unlisted columns of
//     the selection: then, as for a non-finite candidate, fewer listed keys than
//     k, a crowded bucket or tie group, or a row whose visible count exceeds
//     what the scoring wrote candidates for, the row takes the full selection
//     from its logits, so the result is always the unique one;
//  4. the kept columns, marked in a bitmask of the row, are written in order.
constexpr int kCandChunk = 64;                 // columns per candidate list
constexpr int kCandList = 32;                  // keys per list
constexpr int kCandTies = 64;                  // tie group ranked by one wave
static_assert(kMaxWidth % kCandChunk == 0, "whole chunks");
static_assert(kMaxWidth / 32 <= kStage, "the bitmask fits the staging area");

// KPT keys per thread: thread t holds keys [KPT t, KPT t + KPT) of the row's
// concatenated lists (16: half a list, while the row has at most 512 chunks).
// The per-key passes run only in waves that hold keys of the row.
template <int KPT>
__device__ __forceinline__ bool select_from_lists(Shared &sh, const TopkArgs &a, int row, int n, int32_t *out,
                                                  const float *src) {
    static_assert(kCandList % KPT == 0 || KPT % kCandList == 0, "whole lists or whole parts of one");
    static_assert(KPT % 4 == 0, "whole 16-byte loads");
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int l = t & 63;
    const int k = a.k;
    const int nch = (n + kCandChunk - 1) / kCandChunk;
    const int nkeys = nch * kCandList;
    const int nw = (n + 31) >> 5;
    uint32_t *bits = sh.keys;  // [nw] kept columns
    const bool wave_has = w * 64 * KPT < nkeys;  // uniform: this wave holds keys of the row
    const int s0 = KPT * t;                     // first key slot of this thread
    auto col_of = [](int slot, uint32_t kk) { return (slot / kCandList) * kCandChunk + 63 - (int)(kk & 63u); };

    // ---- 1. keys, range, count -----------------------------------------------
    uint32_t key[KPT];
    uint32_t kmax = 0u, kmin = 0xFFFFFFFFu, nf = 0u;
    int nvalid = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = 0u;
    if (wave_has) {
        const uint4 *lp = reinterpret_cast<const uint4 *>(a.cand + (int64_t)row * a.cand_chunks * kCandList) +
                          (s0 < nkeys ? s0 / 4 : 0);
#pragma unroll
        for (int q = 0; q < KPT / 4; ++q) {
            const uint4 v = s0 + 4 * q < nkeys ? lp[q] : make_uint4(0u, 0u, 0u, 0u);
            key[4 * q] = v.x;
            key[4 * q + 1] = v.y;
            key[4 * q + 2] = v.z;
            key[4 * q + 3] = v.w;
        }
        // Only the row's last chunk has columns past n (its list then holds
        // keys 0 or columns past n): the keys of the other chunks are all valid.
        if (s0 + KPT > (nch - 1) * kCandList) {
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                const uint32_t kk = key[j];
                const bool valid = s0 + j < nkeys && kk != 0u && col_of(s0 + j, kk) < n;
                key[j] = valid ? kk : 0u;
                nvalid += valid ? 1 : 0;
                kmax = valid ? max(kmax, kk) : kmax;
                kmin = valid ? min(kmin, kk) : kmin;
            }
        } else {
            nvalid = KPT;
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                kmax = max(kmax, key[j]);
                kmin = min(kmin, key[j]);
            }
        }
        // a key at or above +inf's (or at or below -inf's) holds a non-finite score
        nf = (nvalid > 0 && (kmax >= 0xFF800000u || kmin <= 0x007FFFFFu)) ? 1u : 0u;
        kmax = nf ? 0u : kmax;
        kmin = nf ? 0xFFFFFFFFu : kmin;
    }
    for (int i = t; i < nw; i += kThreads) bits[i] = 0u;
    {
        const int c = wave_total_sum(nvalid);
        if (l == 0) sh.grp[w] = c;
    }
    if (t == 0) {
        sh.ncand = 0;
        sh.split_over = 0;
        sh.ntie = 0;
    }
    const RowRange rr = row_range(sh, kmax, kmin, nf, t);  // clears the histogram; barrier
    int total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) total += sh.grp[i];
    if (!rr.all_finite || total < k) return false;
    const float sc = rr.scale, off = rr.vmax * rr.scale;

    // ---- 2. histogram, crossing bucket, the k-th key ------------------------
    // (buckets kept in registers for up to 16 keys, recomputed above that)
    constexpr bool kKeepBuckets = KPT <= 16;
    int bk[kKeepBuckets ? KPT : 1];
    // the map reads a packed key as a float (its column bits move it by less
    // than 64 ulp): monotone in the packed order, which is all it needs; keys
    // below the range's low end (by those bits) clamp to the last bucket
    auto bucket_of = [&](int j) {
        if constexpr (kKeepBuckets) return bk[j];
        else return fast_bucket(key_value(key[j]), sc, off);
    };
    if (wave_has) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int b = fast_bucket(key_value(key[j]), sc, off);
            if constexpr (kKeepBuckets) bk[j] = b;
            if (key[j]) atomicAdd(&sh.hist[b], 1u);
        }
    }
    __syncthreads();
    const Crossing cr = find_crossing_w(sh, k);
    const int bstar = cr.bin;
    int need = k - cr.above;
    int cnt = cr.cnt;
    if (cnt > kCand) return false;
    if (wave_has) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const bool hit = key[j] != 0u && bucket_of(j) == bstar;
            const uint64_t m = ballot(hit);
            if (m) {
                const int lead = __builtin_ctzll(m);
                int base = 0;
                if (l == lead) base = atomicAdd(&sh.ncand, __popcll(m));
                base = readlane(base, lead);
                if (hit) sh.cand_key[base + mask_prefix(m)] = key[j];
            }
        }
    }
    __syncthreads();
    uint32_t P;
    const int nc = sh.ncand;  // == cnt
    if (nc <= kRankAll) {  // keys are distinct: rank by key alone, every wave for itself
        const uint32_t mk = l < nc ? sh.cand_key[l] : 0u;
        int rank = 0;
        for (int j = 0; j < nc; ++j) rank += ((uint32_t)readlane((int)mk, j) > mk) ? 1 : 0;
        P = (uint32_t)readlane((int)mk, __builtin_ctzll(ballot(l < nc && rank == need - 1) | (1ull << 63)));
    } else if (nc <= 64) {
        if (w == 0) {
            const uint32_t mk = l < nc ? sh.cand_key[l] : 0u;
            int rank = 0;
            for (int j = 0; j < nc; ++j) rank += ((uint32_t)readlane((int)mk, j) > mk) ? 1 : 0;
            if (l < nc && rank == need - 1) sh.thr_key = mk;
        }
        __syncthreads();
        P = sh.thr_key;
    } else {
        radix_select(sh, [&](auto f) {
            for (int j = t; j < nc; j += kThreads) f(sh.cand_key[j]);
        }, P, need, cnt);
    }

    // ---- 3. kept keys, the tie group, lists that might miss columns ---------
    const uint32_t tstar = P >> 6;
    int above = 0;
    bool sat = false;
    if (wave_has) {
        // smallest key of each list (or of this thread's part of its list)
        constexpr int kParts = KPT < kCandList ? 1 : KPT / kCandList;
        constexpr int kPartKeys = KPT < kCandList ? KPT : kCandList;
        uint32_t lmin[kParts];
#pragma unroll
        for (int q = 0; q < kParts; ++q) lmin[q] = 0xFFFFFFFFu;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const uint32_t kk = key[j];
            lmin[j / kPartKeys] = min(lmin[j / kPartKeys], kk);
            const uint32_t tk = kk >> 6;
            if (kk != 0u && tk >= tstar) {
                const int col = col_of(s0 + j, kk);
                if (tk > tstar) {
                    atomicOr(&bits[col >> 5], 1u << (col & 31));
                    ++above;
                } else {
                    const int at = atomicAdd(&sh.ntie, 1);
                    if (at < kCandTies) sh.cand_col[at] = col;
                }
            }
        }
        // the 32nd key of each list: the smaller of its parts' minima
        if constexpr (KPT < kCandList) {
#pragma unroll
            for (int m = 1; m < kCandList / KPT; m <<= 1) lmin[0] = min(lmin[0], (uint32_t)xor_lane_i((int)lmin[0], m));
        }
#pragma unroll
        for (int q = 0; q < kParts; ++q) {
            const int s = s0 + q * kPartKeys;
            const int c = s / kCandList;
            sat |= s < nkeys && n - kCandChunk * c > kCandList && (lmin[q] >> 6) >= tstar;
        }
    }
    {
        const int c = wave_total_sum(above);
        const bool any_sat = ballot(sat) != 0ull;
        if (l == 0) {
            sh.grp[w] = c;
            if (any_sat) sh.split_over = 1;
        }
    }
    __syncthreads();
    int nabove = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) nabove += sh.grp[i];
    const int nt = sh.ntie;
    const int need_t = k - nabove;
    if (sh.split_over || nt > kCandTies || need_t < 1 || need_t > nt) return false;
    if (w == 0) {
        if (nt == 1) {  // P alone: it takes the last place
            if (l == 0) {
                const int mc = sh.cand_col[0];
                atomicOr(&bits[mc >> 5], 1u << (mc & 31));
            }
        } else {  // rank the tie group on the exact logits: (value desc, column asc)
            const int mc = l < nt ? sh.cand_col[l] : 0x7FFFFFFF;
            const uint32_t mk = l < nt ? order_key(src[mc]) : 0u;
            int rank = 0;
            for (int j = 0; j < nt; ++j) {
                const uint32_t kj = (uint32_t)readlane((int)mk, j);
                const int cj = readlane(mc, j);
                rank += (kj > mk || (kj == mk && cj < mc)) ? 1 : 0;
            }
            if (l < nt && rank < need_t) atomicOr(&bits[mc >> 5], 1u << (mc & 31));
        }
    }
    __syncthreads();

    // ---- 4. the kept columns in order ----------------------------------------
    const int per = (nw + kThreads - 1) / kThreads;
    const int w0 = t * per;
    int mine = 0;
    for (int u = 0; u < per; ++u)
        if (w0 + u < nw) mine += __popc(bits[w0 + u]);
    const int incl = wave_incl_sum(mine);
    if (l == 63) sh.wave_tot[w] = incl;
    __syncthreads();
    const int wt = l < kWaves ? sh.wave_tot[l] : 0;
    const int wincl = row16_scan_dpp(wt, 0, OpAdd());  // lanes 0..15: the waves' running totals
    int p = readlane(wincl - wt, w) + incl - mine;
    for (int u = 0; u < per; ++u) {
        if (w0 + u >= nw) break;
        uint32_t word = bits[w0 + u];
        while (word) {
            const int b = __builtin_ctz(word);
            word &= word - 1u;
            if (p < k) out[p] = 32 * (w0 + u) + b;
            ++p;
        }
    }
    return true;
}

// The full selection of one row, kept out of line: the fallback of the
// selection from lists, called from one place so that the kernel's own code
// stays small (each CU runs it once, from a cold instruction cache).
__device__ __attribute__((noinline)) void select_full_row_cold(Shared &sh, const float *src, int n, int k,
                                                                int32_t *out) {
    select_full_row<true>(sh, src, n, k, out);
}

template <int KPT>
__global__ __launch_bounds__(kThreads) void topk_cand_kernel(TopkArgs a) {
    __shared__ Shared sh;
    const int row = blockIdx.x;
    const int t = threadIdx.x;
    const int k = a.k;
    const int n = min(max(a.ctx_lens[row], 0), a.width);
    int32_t *out = a.idx_out + (int64_t)row * k;
    const float *src = a.logits + (int64_t)row * a.stride;
    if (n <= k) {
        for (int j = t; j < k; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    // past the table the logits are -inf and there are no candidates
    if (n <= a.cap && select_from_lists<KPT>(sh, a, row, n, out, src)) return;
    __syncthreads();
    select_full_row_cold(sh, src, n, k, out);
}

}  // namespace

int topk_groups_for_width(int width) { return width <= kMaxWidth ? 1 : 0; }

TopkPlan plan_topk(int num_rows, int width) {
    TopkPlan p{1, width, 0, 0};
    if (num_rows <= 0 || num_rows > kSplitMaxRows || width <= 4 * kThreads) return p;
    if (num_rows >= kRowsMinRows && width <= kStage) return p;
    const int by_len = (width + 4 * kThreads - 1) / (4 * kThreads);  // slices of >= 4096 columns
    const int min_sl = (width + 4 * kThreads * kSliceGroups - 1) / (4 * kThreads * kSliceGroups);
    int sl = kSplitCUs / num_rows;  // one round of workgroups
    sl = sl < by_len ? sl : by_len;
    sl = sl > min_sl ? sl : min_sl;
    if (sl < 2) return p;
    int len = (width + sl - 1) / sl;
    len = (len + 3) & ~3;
    p.slices = (width + len - 1) / len;
    p.slice_len = len;
    p.groups = (len + 4 * kThreads - 1) / (4 * kThreads);
    // member slots per slice: a power of two >= 1/12 of the slice, all of a
    // row's slots loadable by one resolve workgroup in one round
    int shift = 8;
    while ((1 << shift) < len / 12) ++shift;
    while (shift > 6 && ((int64_t)p.slices << shift) > (int64_t)kSlotLoads * kThreads) --shift;
    p.cand_shift = shift;
    return p;
}

int64_t topk_workspace_bytes(int num_rows, int width) {
    const TopkPlan p = plan_topk(num_rows, width);
    if (p.slices < 2) return 0;
    const int64_t rs = (int64_t)num_rows * p.slices;
    return split_meta_bytes(num_rows, p.slices) + rs * kMBins * 4 + (rs << p.cand_shift) * 8;
}

// ---- library-held scratch for callers that cannot allocate ------------------
//
// The split selection's workspace, as a fixed device array of the library: one
// copy per GPU, at its own address, held until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is only a handle);
// it passes the device address hipGetSymbolAddress gives for the current
// device, looked up once per device.  The split workspace needs no
// initialisation (every count, histogram and used member slot is written by
// the window kernel before the resolve kernel reads it), so nothing is
// cleared.  Calls that overlap on one GPU share the array and race.
static __device__ __align__(256) uint8_t scratch[kTopkScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t topk_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

template <int G>
static void launch_split(const TopkArgs &a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    const unsigned g = (unsigned)a.num_rows * (unsigned)a.slices;
    hipExtLaunchKernelGGL(topk_window_kernel<G>, dim3(g), dim3(kThreads), 0, s, start, nullptr, 0, a);
    hipExtLaunchKernelGGL(topk_resolve_kernel<G>, dim3(g), dim3(kThreads), 0, s, nullptr, stop, 0, a);
}

hipError_t launch_topk_cand(const TopkArgs &a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    if (a.num_rows == 0) return hipSuccess;
    // keys per thread: 16 (half a list) for rows of up to 512 chunks (32,768
    // columns), 32 up to 1,024 chunks, else 64
    const int64_t keys = (int64_t)a.cand_chunks * kCandList;
    if (keys <= 16 * kThreads)
        hipExtLaunchKernelGGL(topk_cand_kernel<16>, dim3((unsigned)a.num_rows), dim3(kThreads), 0, s, start, stop, 0, a);
    else if (keys <= 32 * kThreads)
        hipExtLaunchKernelGGL(topk_cand_kernel<32>, dim3((unsigned)a.num_rows), dim3(kThreads), 0, s, start, stop, 0, a);
    else
        hipExtLaunchKernelGGL(topk_cand_kernel<64>, dim3((unsigned)a.num_rows), dim3(kThreads), 0, s, start, stop, 0, a);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    if (a.num_rows == 0) return hipSuccess;
    if (a.slices > 1) {
        switch (a.groups) {
            case 1: launch_split<1>(a, s, start, stop); break;
            case 2: launch_split<2>(a, s, start, stop); break;
            case 3: launch_split<3>(a, s, start, stop); break;
            case 4: launch_split<4>(a, s, start, stop); break;
            case 5: launch_split<5>(a, s, start, stop); break;
            case 6: launch_split<6>(a, s, start, stop); break;
            case 7: launch_split<7>(a, s, start, stop); break;
            case 8: launch_split<8>(a, s, start, stop); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        // one workgroup per CU, more when a workgroup would take over kRowsPerGroup rows
        unsigned g = (unsigned)(a.num_rows < kRowsGrid ? a.num_rows : kRowsGrid);
        g = g > (unsigned)((a.num_rows + kRowsPerGroup - 1) / kRowsPerGroup) ? g : (unsigned)((a.num_rows + kRowsPerGroup - 1) / kRowsPerGroup);
        if (a.row_starts)
            hipExtLaunchKernelGGL(topk_rows_kernel<true>, dim3(g), dim3(kThreads), 0, s, start, stop, 0, a);
        else
            hipExtLaunchKernelGGL(topk_rows_kernel<false>, dim3(g), dim3(kThreads), 0, s, start, stop, 0, a);
    }
    return hipGetLastError();
}

}  // namespace qsa
