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
// global load of the row is issued before the first is consumed) and every
// later pass reads LDS.  Longer rows are re-read from memory (L2) per pass.
//
//  1. The row's finite min and max (while staging).
//  2. A 2048-bucket histogram, buckets linear in value between min and max
//     (bucket 0 = largest).  The map is monotone, so the bucket b* holding the
//     k-th largest value is found by one scan: buckets < b* are kept outright,
//     buckets > b* dropped.  Linear-in-value buckets spread a dense cluster of
//     logits over many bins, so the LDS atomics rarely collide (radix digits of
//     the float bits would pile a whole octave into a few bins).
//  3. Inside b*: radix passes (11, 11, 10 bits of the key, largest first) over
//     the bucket's members, stopping as soon as the crossing digit bin is taken
//     whole.  Normally b* holds a few dozen values.
//  4. Only when several keys equal T and not all of them fit: Ct is the column
//     of the need-th such key in column order.
//  5. The kept set, ranked in column order and written.  Ranks come from wave
//     ballots over the thread-strided layout (conflict-free LDS reads) and one
//     scan of per-(group, wave) counts.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kStage = 32768;    // longest row staged in LDS
constexpr int kMaxWidth = 69632;
constexpr int kCand = 4096;      // candidate list (keys of the crossing bucket)
constexpr int kStageGroups = kStage / 4 / kThreads;  // float4 groups per thread
constexpr int kMaxGroups = (kMaxWidth + 4 * kThreads - 1) / (4 * kThreads);

struct Shared {
    uint32_t keys[kStage];  // staged row (order keys), column order
    uint32_t hist[kBins];
    uint32_t cand[kCand];   // keys of the crossing bucket
    int ncand;
    float red_max[kWaves];
    float red_min[kWaves];
    int wave_tot[kWaves];
    int cnt[kWaves * 8];  // per (group, wave) counts of one chunk, group-major
    int chunk_total;
    int cross_bin;
    int cross_above;
    int cross_cnt;
    int tie_col;
};

// Exclusive scan of hist in bin order; finds the bin where the running count
// first reaches `need` (1 <= need <= total).  Result lands in sh.cross_*.
// All threads; ends with a barrier.
__device__ __forceinline__ void find_crossing(Shared &sh, int need) {
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int h0 = (int)sh.hist[2 * t], h1 = (int)sh.hist[2 * t + 1];
    const int s = h0 + h1;
    const int incl = wave_incl_scan_i(s);
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

__device__ void clear_hist(Shared &sh) {
    for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[i] = 0;
}

__device__ __forceinline__ float key_value(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// Value buckets: bucket 0 holds the largest values.  For a row of finite
// values, bucket = 1 + floor((vmax - v) * scale) clamped to [1, kBins-2].  With
// non-finite values present, +inf and NaN with the sign clear go to bucket 0 and
// -inf and NaN with the sign set to kBins-1.  Monotone non-increasing in the
// value; equal keys share a bucket.
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

__device__ __forceinline__ f32x4 load4(const float *src, int i) {
    return *reinterpret_cast<const f32x4 *>(src + 4 * i);
}

// Keys of a row staged in LDS (column order).
struct StagedKeys {
    const uint32_t *keys;
    int n;
    // f(col, key) for every column of the row, thread-strided float4 groups
    template <class F>
    __device__ __forceinline__ void each(F f) const {
        const int n4 = (n + 3) >> 2;
        for (int i = threadIdx.x; i < n4; i += kThreads) {
            const uint4 k4 = reinterpret_cast<const uint4 *>(keys)[i];
            const uint32_t kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * i + e < n) f(4 * i + e, kk[e]);
        }
    }
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
    template <class F>
    __device__ __forceinline__ void each(F f) const {
        const int n4 = (n + 3) >> 2;
        // four float4 loads in flight per thread
        for (int i0 = threadIdx.x; i0 < n4; i0 += 4 * kThreads) {
            f32x4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * kThreads;
                x[u] = (i < n4) ? load4(src, i) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * kThreads;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * i + e < n) f(4 * i + e, order_key(x[u][e]));
            }
        }
    }
    __device__ __forceinline__ uint4 group(int j) const {
        const int i = threadIdx.x + kThreads * j;
        if (4 * i >= n) return make_uint4(0u, 0u, 0u, 0u);
        const f32x4 x = load4(src, i);
        return make_uint4(order_key(x[0]), order_key(x[1]), order_key(x[2]), order_key(x[3]));
    }
};

// Column-order ranks over thread-strided float4 groups, for one chunk of
// kChunk groups (4096*kChunk consecutive columns).  Flag bit 4*j + e marks
// element e of this thread's group j of the chunk.  On return base[j] counts the
// chunk's flagged columns before this thread's group j (the caller adds its own
// earlier flags of the group); the result is the chunk's total.  Wave ballots
// give the order inside a wave; per-(group, wave) totals, scanned once, give
// each wave's offset.  All threads; ends with a barrier.
constexpr int kChunk = 8;

__device__ __forceinline__ int strided_bases(Shared &sh, uint32_t flag, int (&base)[kChunk]) {
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int l = t & 63;
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
        int before = 0, tot = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint64_t m = ballot((flag >> (4 * j + e)) & 1u);
            before += mask_prefix(m);
            tot += __popcll(m);
        }
        base[j] = before;
        if (l == 0) sh.cnt[j * kWaves + w] = tot;
    }
    __syncthreads();
    if (w == 0) {  // exclusive scan of cnt[0 .. kChunk*kWaves), two entries per lane
        constexpr int PER = kChunk * kWaves / 64;
        int v[PER];
        int s = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            v[i] = sh.cnt[l * PER + i];
            s += v[i];
        }
        const int incl = wave_incl_scan_i(s);
        int run = incl - s;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            sh.cnt[l * PER + i] = run;
            run += v[i];
        }
        if (l == 63) sh.chunk_total = incl;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kChunk; ++j) base[j] += sh.cnt[j * kWaves + w];
    const int total = sh.chunk_total;
    __syncthreads();  // cnt and chunk_total are reused by the next call
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

// Steps 2..5 on a row whose range is known and whose bucket histogram is in
// sh.hist.  G = float4 groups per thread covering the row.
template <int G, class Keys, class Bk>
__device__ __forceinline__ void select_row(Shared &sh, const Keys &src, int n, int k, const Bk &bucket,
                                           int32_t *out) {
    const int t = threadIdx.x;
    const int l = t & 63;
    find_crossing(sh, k);
    const int bstar = sh.cross_bin;
    int need = k - sh.cross_above;
    int cnt = sh.cross_cnt;

    // ---- 3. the exact k-th key T, from the members of bucket b* ----------
    uint32_t T;
    if (cnt <= kCand) {
        if (t == 0) sh.ncand = 0;
        __syncthreads();
        src.each([&](int, uint32_t kx) {
            const bool c = bucket(kx) == bstar;
            const uint64_t m = ballot(c);
            if (m) {
                int base = 0;
                if (l == __builtin_ctzll(m)) base = atomicAdd(&sh.ncand, __popcll(m));
                base = readlane(base, __builtin_ctzll(m));
                if (c) sh.cand[base + mask_prefix(m)] = kx;
            }
        });
        __syncthreads();
        const int nc = sh.ncand;
        radix_select(sh, [&](auto f) {
            for (int j = t; j < nc; j += kThreads) f(sh.cand[j]);
        }, T, need, cnt);
    } else {
        radix_select(sh, [&](auto f) {
            src.each([&](int, uint32_t kx) {
                if (bucket(kx) == bstar) f(kx);
            });
        }, T, need, cnt);
    }
    // Every key above T is kept, every key below dropped; of the cnt keys equal
    // to T the need lowest columns are kept.

    int base[kChunk];
    int tie_col = 0x7FFFFFFF;

    // ---- 4. ties at T: the need lowest columns win ------------------------
    if (cnt > need) {
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
            const int tot = strided_bases(sh, eq, base);
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                int r = carry + base[j];
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
        tie_col = sh.tie_col;
    }

    // ---- 5. the kept set, ranked in column order, written -----------------
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
                if (keep) sel |= 1u << (4 * j + e);
            }
        }
        const int tot = strided_bases(sh, sel, base);
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            int p = carry + base[j];
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

// Finite min / max and the count of non-finite values across the block (all
// threads; ends with a barrier; also clears the histogram).
struct RowRange {
    float vmax, scale;
    bool all_finite;
};

__device__ __forceinline__ RowRange row_range(Shared &sh, float vmax, float vmin, int nonfinite) {
    const int w = threadIdx.x >> 6;
    vmax = wave_max_f(vmax);
    vmin = wave_min_f(vmin);
    nonfinite = wave_max_i(nonfinite);
    if ((threadIdx.x & 63) == 0) {
        sh.red_max[w] = vmax;
        sh.red_min[w] = vmin;
        sh.wave_tot[w] = nonfinite;
    }
    clear_hist(sh);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        vmax = fmaxf(vmax, sh.red_max[i]);
        vmin = fminf(vmin, sh.red_min[i]);
        nonfinite = max(nonfinite, sh.wave_tot[i]);
    }
    const float span = vmax - vmin;
    return RowRange{vmax, (span > 0.0f && __builtin_isfinite(span)) ? (float)(kBins - 3) / span : 0.0f,
                    nonfinite == 0};
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
    float vmax = -__builtin_huge_valf(), vmin = __builtin_huge_valf();
    int nonfinite = 0;

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
                for (int e = 0; e < 4; ++e)
                    if (4 * i + e < n) {
                        if (__builtin_isfinite(x[j][e])) {
                            vmax = fmaxf(vmax, x[j][e]);
                            vmin = fminf(vmin, x[j][e]);
                        } else {
                            nonfinite = 1;
                        }
                    }
            }
        }
        const RowRange rr = row_range(sh, vmax, vmin, nonfinite);
        const StagedKeys sk{sh.keys, n};
        // ---- 2. bucket histogram ------------------------------------------
        if (rr.all_finite) {
            const Bucketer<true> bucket{rr.vmax, rr.scale};
            sk.each([&](int, uint32_t kx) { atomicAdd(&sh.hist[bucket(kx)], 1u); });
            __syncthreads();
            select_row<kStageGroups>(sh, sk, n, k, bucket, out);
        } else {
            const Bucketer<false> bucket{rr.vmax, rr.scale};
            sk.each([&](int, uint32_t kx) { atomicAdd(&sh.hist[bucket(kx)], 1u); });
            __syncthreads();
            select_row<kStageGroups>(sh, sk, n, k, bucket, out);
        }
    } else {
        const StreamKeys sk{src, n};
        sk.each([&](int, uint32_t kx) {
            const float v = key_value(kx);
            if (__builtin_isfinite(v)) {
                vmax = fmaxf(vmax, v);
                vmin = fminf(vmin, v);
            } else {
                nonfinite = 1;
            }
        });
        const RowRange rr = row_range(sh, vmax, vmin, nonfinite);
        const Bucketer<false> bucket{rr.vmax, rr.scale};
        sk.each([&](int, uint32_t kx) { atomicAdd(&sh.hist[bucket(kx)], 1u); });
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
