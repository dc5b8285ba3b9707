// Device-side helpers shared by the gfx950 kernels of libqsaidx.
//
// Wave64 primitives (ballot, lane masks, readlane), the MFMA vector types and
// the order-preserving float key used by the selection kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() {
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0));
}

// number of set bits of `mask` below the calling lane
__device__ __forceinline__ int mask_prefix(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

__device__ __forceinline__ uint64_t ballot(bool p) {
    return __builtin_amdgcn_ballot_w64(p);
}

__device__ __forceinline__ int readlane(int v, int lane) {
    return __builtin_amdgcn_readlane(v, lane);
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// value of `v` held by lane (lane_id ^ m); m < 64
__device__ __forceinline__ float xor_lane_f(float v, int m) {
    int src = (lane_id() ^ m) << 2;
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(v)));
}

__device__ __forceinline__ int xor_lane_i(int v, int m) {
    int src = (lane_id() ^ m) << 2;
    return __builtin_amdgcn_ds_bpermute(src, v);
}

// value of `v` held by lane `src` (any lane)
__device__ __forceinline__ int shfl_i(int v, int src) {
    return __builtin_amdgcn_ds_bpermute(src << 2, v);
}

__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) v = max(v, xor_lane_i(v, m));
    return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) v += xor_lane_i(v, m);
    return v;
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) v = fmaxf(v, xor_lane_f(v, m));
    return v;
}

__device__ __forceinline__ float wave_min_f(float v) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) v = fminf(v, xor_lane_f(v, m));
    return v;
}

// inclusive prefix sum across the wave
__device__ __forceinline__ int wave_incl_scan_i(int v) {
    const int l = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int u = shfl_i(v, l >= d ? l - d : l);
        if (l >= d) v += u;
    }
    return v;
}

// DPP (data-parallel primitive) controls, GFX9 encoding
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// Inclusive scan across the wave with DPP moves (no LDS traffic): row_shr 1, 2,
// 4, 8 scan each 16-lane row, row_bcast:15 / row_bcast:31 carry row totals into
// the following rows.  Lanes without a source take `identity`.  All 64 lanes
// must be active.
template <class Op>
__device__ __forceinline__ int wave_scan_dpp(int v, int identity, Op op) {
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowShr1, 0xF, 0xF, false));
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowShr2, 0xF, 0xF, false));
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowShr4, 0xF, 0xF, false));
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowShr8, 0xF, 0xF, false));
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowBcast15, 0xA, 0xF, false));
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowBcast31, 0xC, 0xF, false));
    return v;
}

struct OpAdd {
    __device__ __forceinline__ int operator()(int a, int b) const { return a + b; }
};
struct OpMaxI {
    __device__ __forceinline__ int operator()(int a, int b) const { return max(a, b); }
};
struct OpMaxU {
    __device__ __forceinline__ int operator()(int a, int b) const {
        return (int)max((uint32_t)a, (uint32_t)b);
    }
};

// inclusive prefix sum across the (fully active) wave
__device__ __forceinline__ int wave_incl_sum(int v) { return wave_scan_dpp(v, 0, OpAdd()); }

// The same inside each 16-lane row only (row_shr 1, 2, 4, 8): lanes 0..15 hold
// the scan of lanes 0..15.  All 64 lanes must be active.
template <class Op>
__device__ __forceinline__ int row16_scan_dpp(int v, int identity, Op op) {
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowShr1, 0xF, 0xF, false));
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowShr2, 0xF, 0xF, false));
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowShr4, 0xF, 0xF, false));
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowShr8, 0xF, 0xF, false));
    return v;
}

// wave-uniform sum / unsigned max (result read from the last lane)
__device__ __forceinline__ int wave_total_sum(int v) { return readlane(wave_incl_sum(v), 63); }
__device__ __forceinline__ uint32_t wave_total_umax(uint32_t v) {
    return (uint32_t)readlane(wave_scan_dpp((int)v, 0, OpMaxU()), 63);
}
// unsigned max of lanes 0..15 (all lanes active)
__device__ __forceinline__ uint32_t row16_total_umax(uint32_t v) {
    return (uint32_t)readlane(row16_scan_dpp((int)v, 0, OpMaxU()), 15);
}

// v + (v of lane l ^ 16) and v + (v of lane l ^ 32), each with one gfx950
// lane-swap instruction and an add, no LDS round trip.  permlane16_swap(a, b)
// exchanges the odd 16-lane rows of a with the even rows of b, and
// permlane32_swap(a, b) the upper half of a with the lower half of b; with
// a = b = v the two results hold, in every lane, v and its partner's v.
__device__ __forceinline__ float xor16_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max(x, 0) for finite x in one instruction: v_med3_f32(x, 0, FLT_MAX).
// fmaxf(x, 0) costs two (a NaN-quieting canonicalize of x first, as the
// compiler cannot see that an MFMA result is never a signalling NaN), and a
// +inf upper bound lets the compiler turn med3 back into that fmaxf.  Scores
// are finite (bounded products of finite bf16 / fp8 inputs).
__device__ __forceinline__ float relu(float x) {
    return __builtin_amdgcn_fmed3f(x, 0.0f, 3.402823466e+38f);
}

// DPP lane patterns inside each 16-lane row: quad_perm [1,0,3,2] (lane ^ 1),
// [2,3,0,1] (lane ^ 2), [3,2,1,0] (lane ^ 3), row_half_mirror (lane ^ 7) and
// row_mirror (lane ^ 15)
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppXor3 = 0x1B, kDppHalfMirror = 0x141, kDppMirror = 0x140;

// value of `v` in the lane given by the DPP pattern (all lanes active)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

// f32 bits -> u32 whose unsigned order is the float order; -0 is folded onto +0
// so that the two zeros compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    u = (u == 0x80000000u) ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace qsa
