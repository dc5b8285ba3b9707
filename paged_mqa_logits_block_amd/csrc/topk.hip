// Per-row top-k selection on gfx950.
//
// Selects, per row, the k columns of [0, n) with the largest logits, ties to
// the lower column (+0 and -0 equal), and writes them in ascending column order
// followed by -1 padding.  Rows with n <= k keep all of [0, n) (sglang
// PR #48649, Accuracy Tests: "decode skips rows that fit topk"); nothing past n
// is used (vLLM PR #62589, Details and Validation).
//
// One workgroup of 1024 threads (16 waves) per row.  The selection is reduced to
// finding the k-th element in (value desc, column asc) order, a pair (T, Ct):
// column c is kept iff key(c) > T, or key(c) == T and c <= Ct, where key is the
// order-preserving u32 image of the float.
//
// Rows of up to 32768 columns are staged once in LDS as keys (128 KB; every
// global load of the row is in flight before the first is used); longer rows
// are re-read from memory (L2) on every pass.
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
};

__device__ __forceinline__ float key_value(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ f32x4 load4(const float *src, int i) {
    return *reinterpret_cast<const f32x4 *>(src + 4 * i);
}

__device__ __forceinline__ void clear_hist(Shared &sh) {
    for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[i] = 0;
}

// Exclusive scan of hist in bin order; finds the bin where the running count
// first reaches `need` (1 <= need <= total).  Result lands in sh.cross_*.
// All threads; ends with a barrier.
__device__ __forceinline__ void find_crossing(Shared &sh, int need) {
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
    __device__ __forceinline__ uint4 group(int j) const {
        const int i = threadIdx.x + kThreads * j;
        if (4 * i >= n) return make_uint4(0u, 0u, 0u, 0u);
        const f32x4 x = load4(src, i);
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
                                           int32_t *out) {
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
                    if (p < k) out[p] = 4 * (t + kThreads * (c + j)) + e;
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

__device__ __forceinline__ RowRange row_range(Shared &sh, uint32_t kmax, uint32_t kmin, uint32_t nonfinite) {
    const int w = threadIdx.x >> 6;
    kmax = wave_total_umax(kmax);
    const uint32_t nkmin = wave_total_umax(~kmin);
    nonfinite = wave_total_umax(nonfinite);
    if ((threadIdx.x & 63) == 0) {
        sh.red_max[w] = kmax;
        sh.red_min[w] = nkmin;
        sh.red_nf[w] = nonfinite;
    }
    clear_hist(sh);
    __syncthreads();
    uint32_t a = 0, b = 0, c = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        a = max(a, sh.red_max[i]);
        b = max(b, sh.red_min[i]);
        c = max(c, sh.red_nf[i]);
    }
    // with no finite value at all, a = 0 and ~b = ~0: the map is never used
    const float vmax = key_value(a), vmin = key_value(~b);
    const float span = vmax - vmin;
    const bool usable = a != 0u && span > 0.0f && __builtin_isfinite(span);
    return RowRange{vmax, usable ? (float)(kBins - 3) / span : 0.0f, c == 0u};
}

// running finite range and non-finite flag over one visible value
__device__ __forceinline__ void track(float x, bool valid, uint32_t &kmax, uint32_t &kmin, uint32_t &nf) {
    const uint32_t kx = order_key(x);
    const bool fin = __builtin_isfinite(x);
    kmax = (valid && fin) ? max(kmax, kx) : kmax;
    kmin = (valid && fin) ? min(kmin, kx) : kmin;
    nf |= (valid && !fin) ? 1u : 0u;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
    __shared__ Shared sh;
    const int row = blockIdx.x;
    const int t = threadIdx.x;
    const int n = min(max(a.ctx_lens[row], 0), a.width);
    const int k = a.k;
    int32_t *out = a.idx_out + (int64_t)row * k;

    if (n <= k) {  // the whole visible range is the selection
        for (int j = t; j < k; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }

    const float *src = a.logits + (int64_t)row * a.stride;
    const int n4 = (n + 3) >> 2;
    uint32_t kmax = 0u, kmin = 0xFFFFFFFFu, nonfinite = 0u;

    if (n <= kStage) {
        // ---- 1. stage the row: all loads in flight, then keys to LDS ------
        f32x4 x[kStageGroups];
#pragma unroll
        for (int j = 0; j < kStageGroups; ++j) {
            const int i = t + kThreads * j;
            x[j] = (i < n4) ? load4(src, i) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
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
            select_row<kStageGroups>(sh, sk, n, k, bucket, out);
        } else {
            const Bucketer<false> bucket{rr.vmax, rr.scale};
            for_each_key<kStageGroups>(sk, n, [&](int, uint32_t kx) { atomicAdd(&sh.hist[bucket(kx)], 1u); });
            __syncthreads();
            select_row<kStageGroups>(sh, sk, n, k, bucket, out);
        }
    } else {
        const StreamKeys sk{src, n};
#pragma unroll 1
        for (int i0 = t; i0 < n4; i0 += 4 * kThreads) {  // four float4 loads in flight
            f32x4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * kThreads;
                x[u] = (i < n4) ? load4(src, i) : f32x4{0.f, 0.f, 0.f, 0.f};
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
        select_row<kMaxGroups>(sh, sk, n, k, bucket, out);
    }
}

}  // namespace

int topk_groups_for_width(int width) { return width <= kMaxWidth ? 1 : 0; }

hipError_t launch_topk(const TopkArgs &a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    if (a.num_rows == 0) return hipSuccess;
    hipExtLaunchKernelGGL(topk_kernel, dim3((unsigned)a.num_rows), dim3(kThreads), 0, s, start, stop, 0, a);
    return hipGetLastError();
}

}  // namespace qsa
