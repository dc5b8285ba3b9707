// Per-row top-k selection on gfx950.
//
// Selects, per row, the k columns of [0, n) with the largest logits, ties to
// the lower column (+0 and -0 equal), and writes them in ascending column order
// followed by -1 padding.  Rows with n <= k keep all of [0, n) (sglang
// PR #48649, Accuracy Tests: "decode skips rows that fit topk"); nothing past n
// is used (vLLM PR #62589, Details and Validation).
//
// One workgroup of 1024 threads (16 waves) per row.  The selection is reduced to
// finding the k-th element in (value desc, column asc) order, which is a pair
// (T, Ct): element c is kept iff key(c) > T, or key(c) == T and c <= Ct, where
// key is the order-preserving u32 image of the float.  Steps, each a coalesced
// re-read of the row (which stays in L2 between steps):
//
//  1. The row's finite min and max.
//  2. A 2048-bucket histogram, buckets linear in value between min and max
//     (bucket 0 = largest).  The map is monotone, so the bucket b* holding the
//     k-th largest value is found by one scan: buckets < b* are kept outright,
//     buckets > b* dropped.  Linear-in-value buckets spread a dense cluster of
//     logits over many bins, so the LDS atomics rarely collide (radix digits of
//     the float bits would pile a whole octave into a few bins).
//  3. The candidates of b* (normally a few dozen) are appended to an LDS list
//     and radix-selected there (11, 11, 10 bits of the key, stopping as soon as
//     the crossing digit bin is taken whole).  If b* is too large for the list,
//     the same radix passes run over re-reads of the row instead.
//  4. Only when several keys equal T and not all of them fit: Ct is the column
//     of the need-th such key, found from per-thread 32-column bit words and a
//     block scan of their popcounts.
//  5. The kept set as 32-column bit words (thread t owns consecutive words), one
//     block scan of popcounts, and each thread writes its columns in order.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kCap = 16384;     // LDS candidate list (64 KB)
constexpr int kMaxWidth = 69632;

struct Shared {
    uint32_t hist[kBins];
    uint32_t cand_key[kCap];
    float red_max[kWaves];
    float red_min[kWaves];
    int wave_tot[kWaves];
    int cross_bin;
    int cross_above;
    int cross_cnt;
    int ncand;
    int tie_col;
};

// Exclusive scan of hist in bin order; finds the bin where the running count
// first reaches `need` (1 <= need <= total).  Result lands in sh.cross_*.
// All threads; ends with a barrier.
__device__ void find_crossing(Shared &sh, int need) {
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

// Block-wide exclusive scan of one int per thread (thread order); also returns
// the total.  All threads; ends with a barrier.
__device__ int block_excl_scan(Shared &sh, int v, int &total) {
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int incl = wave_incl_scan_i(v);
    __syncthreads();  // wave_tot may still be read by a previous caller
    if ((t & 63) == 63) sh.wave_tot[w] = incl;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int x = sh.wave_tot[i];
        base += (i < w) ? x : 0;
        tot += x;
    }
    total = tot;
    return base + incl - v;
}

__device__ __forceinline__ float key_value(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

struct Bucketer {
    float vmax, scale;
    // 0: +inf and NaN with the sign clear; 1 .. kBins-2: finite values, linear
    // in (vmax - v); kBins-1: -inf and NaN with the sign set.  Monotone
    // non-increasing in the value; equal keys share a bucket.
    __device__ __forceinline__ int operator()(uint32_t kx) const {
        if (kx >= 0xFF800000u) return 0;
        if (kx <= 0x007FFFFFu) return kBins - 1;
        const float d = (vmax - key_value(kx)) * scale;
        return 1 + (d < (float)(kBins - 3) ? (int)d : (kBins - 3));
    }
};

// the float4 group starting at column 4*i of the row (columns >= n are masked
// by the callers; the group itself lies inside the row's stride)
__device__ __forceinline__ f32x4 load4(const float *src, int i) {
    return *reinterpret_cast<const f32x4 *>(src + 4 * i);
}

// Radix passes (11, 11, 10 bits, largest digit first) over the keys produced by
// `each` (called as each(f) with f(key) for every candidate).  In: need <= cnt.
// Out: T (the resolved prefix, low bits 0), need and cnt for keys with that
// prefix.  Stops once the crossing bin is taken whole (cnt == need).
template <class Each>
__device__ void radix_passes(Shared &sh, Each each, uint32_t &T, int &need, int &cnt) {
    uint32_t P = 0, M = 0;
#pragma unroll 1
    for (int pass = 0; pass < 3 && cnt > need; ++pass) {
        const int shf = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
        __syncthreads();  // previous crossing fully read
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

__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
    __shared__ Shared sh;
    const int row = blockIdx.x;
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int l = t & 63;
    const int n = min(max(a.ctx_lens[row], 0), a.width);
    const int k = a.k;
    int32_t *out = a.idx_out + (int64_t)row * k;

    if (n <= k) {  // the whole visible range is the selection
        for (int j = t; j < k; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }

    const float *src = a.logits + (int64_t)row * a.stride;
    const int n4 = (n + 3) >> 2;

    // ---- 1. finite range ---------------------------------------------------
    float vmax = -__builtin_huge_valf(), vmin = __builtin_huge_valf();
    for (int i = t; i < n4; i += kThreads) {
        const f32x4 x = load4(src, i);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * i + e < n && __builtin_isfinite(x[e])) {
                vmax = fmaxf(vmax, x[e]);
                vmin = fminf(vmin, x[e]);
            }
    }
    vmax = wave_max_f(vmax);
    vmin = wave_min_f(vmin);
    if (l == 0) {
        sh.red_max[w] = vmax;
        sh.red_min[w] = vmin;
    }
    clear_hist(sh);
    if (t == 0) sh.ncand = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        vmax = fmaxf(vmax, sh.red_max[i]);
        vmin = fminf(vmin, sh.red_min[i]);
    }
    const float span = vmax - vmin;
    const Bucketer bucket{vmax, (span > 0.0f && __builtin_isfinite(span)) ? (float)(kBins - 3) / span : 0.0f};

    // ---- 2. bucket histogram -----------------------------------------------
    for (int i = t; i < n4; i += kThreads) {
        const f32x4 x = load4(src, i);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * i + e < n) atomicAdd(&sh.hist[bucket(order_key(x[e]))], 1u);
    }
    __syncthreads();
    find_crossing(sh, k);
    const int bstar = sh.cross_bin;
    int need = k - sh.cross_above;
    int cnt = sh.cross_cnt;
    uint32_t T = 0;          // with the whole bucket taken every key passes key >= 0
    int tie_col = 0x7FFFFFFF;

    // ---- 3. resolve inside bucket b* ---------------------------------------
    if (cnt > need) {
        if (cnt <= kCap) {
            for (int i = t; i < n4; i += kThreads) {
                const f32x4 x = load4(src, i);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t kx = order_key(x[e]);
                    const bool c = (4 * i + e < n) && bucket(kx) == bstar;
                    const uint64_t m = ballot(c);
                    if (m) {
                        int base = 0;
                        if (l == 0) base = atomicAdd(&sh.ncand, __popcll(m));
                        base = readlane(base, 0);
                        if (c) sh.cand_key[base + mask_prefix(m)] = kx;
                    }
                }
            }
            __syncthreads();
            const int nc = sh.ncand;
            radix_passes(sh, [&](auto f) {
                for (int j = t; j < nc; j += kThreads) f(sh.cand_key[j]);
            }, T, need, cnt);
        } else {
            radix_passes(sh, [&](auto f) {
                for (int i = t; i < n4; i += kThreads) {
                    const f32x4 x = load4(src, i);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t kx = order_key(x[e]);
                        if (4 * i + e < n && bucket(kx) == bstar) f(kx);
                    }
                }
            }, T, need, cnt);
        }
    }

    // per-thread ownership of consecutive 32-column words, for steps 4 and 5
    const int nw = (n + 31) >> 5;
    const int wpt = (nw + kThreads - 1) / kThreads;  // <= 3 for n <= kMaxWidth
    const int w0 = t * wpt;

    // ---- 4. ties at T: the need lowest columns win --------------------------
    if (cnt > need) {
        uint32_t eq[3] = {0u, 0u, 0u};
        int mine = 0;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int wd = w0 + j;
            if (j < wpt && wd < nw) {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int i = 8 * wd + q;  // float4 group
                    if (4 * i < n) {
                        const f32x4 x = load4(src, i);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t kx = order_key(x[e]);
                            if (4 * i + e < n && kx == T && bucket(kx) == bstar) eq[j] |= 1u << (4 * q + e);
                        }
                    }
                }
                mine += __popc(eq[j]);
            }
        }
        int total;
        const int before = block_excl_scan(sh, mine, total);
        if (before < need && before + mine >= need) {
            int r = need - before;  // 1-based rank inside this thread's words
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                uint32_t m = eq[j];
                const int c = __popc(m);
                if (r > 0 && r <= c) {
                    for (int z = 1; z < r; ++z) m &= m - 1;
                    sh.tie_col = 32 * (w0 + j) + __builtin_ctz(m);
                }
                r -= c;
            }
        }
        __syncthreads();
        tie_col = sh.tie_col;
    }

    // ---- 5. kept set as bit words, scan, write ------------------------------
    uint32_t selw[3] = {0u, 0u, 0u};
    int mine = 0;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int wd = w0 + j;
        if (j < wpt && wd < nw) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int i = 8 * wd + q;
                if (4 * i < n) {
                    const f32x4 x = load4(src, i);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int col = 4 * i + e;
                        const uint32_t kx = order_key(x[e]);
                        const int b = bucket(kx);
                        const bool keep = col < n &&
                                          (b < bstar || (b == bstar && (kx > T || (kx == T && col <= tie_col))));
                        if (keep) selw[j] |= 1u << (4 * q + e);
                    }
                }
            }
            mine += __popc(selw[j]);
        }
    }
    int total;
    int p = block_excl_scan(sh, mine, total);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        uint32_t m = selw[j];
        while (m) {
            const int bit = __builtin_ctz(m);
            m &= m - 1;
            if (p < k) out[p] = 32 * (w0 + j) + bit;
            ++p;
        }
    }
}

}  // namespace

int topk_groups_for_width(int width) { return width <= kMaxWidth ? 1 : 0; }

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
    if (a.num_rows == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.num_rows), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace qsa
