// Pieces shared by the scoring kernels: the head dimension, the column cursor
// over pool blocks, the MFMA fragment types per input dtype, and the
// launchers each kernel file provides to the planner in logits.hip.
#pragma once

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

template <int DT>
struct Frag;

// bf16: v_mfma_f32_16x16x32_bf16, four K steps of 32 over D = 128.
template <>
struct Frag<kBF16> {
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
struct Frag<kFP8> {
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

// fp16: v_mfma_f32_16x16x32_f16, four K steps of 32 over D = 128 (the same
// operand layout as bf16).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
template <>
struct Frag<kFP16> {
    static constexpr int kSteps = 4;
    typedef f16x8 T;
    __device__ static int lane_bytes(int l) { return (l >> 4) * 16; }
    __device__ static T load(const uint8_t *p, int s) { return *reinterpret_cast<const T *>(p + s * 64); }
    __device__ static T zero() {
        T z;
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = (_Float16)0.0f;
        return z;
    }
    __device__ static f32x4 mma(T a, T b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static constexpr int kRowBytes = kD * 2;
};

// fp8 key fragment of lane l for the MFMA B operand: head-dim bytes 32 (l / 16)
// .. +31 of token l % 16 of the 16-token group at `group`.  Block-flat keys
// (layouts 0 and 1) are 128 contiguous bytes per token; the preshuffled
// co-packed layout (2) stores a 16-token group as 8 chunks of 16 tokens x 16
// bytes (byte d of token i at (d / 16) * 256 + i * 16 + d % 16), so the 32
// bytes are two 16-byte pieces 256 bytes apart (for any D: a group is 16 D
// bytes, and a lane's pieces sit at the same offsets inside it).
// row_bytes = D (128, or 64 with the caller zeroing lanes 32..63).
__device__ __forceinline__ i32x8 load_key_frag_fp8(const uint8_t *group, int l, bool shuffled, int row_bytes = kD) {
    if (shuffled) {
        const uint8_t *p = group + (l & 15) * 16 + (l >> 4) * 512;
        const i32x4 lo = *reinterpret_cast<const i32x4 *>(p);
        const i32x4 hi = *reinterpret_cast<const i32x4 *>(p + 256);
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    return *reinterpret_cast<const i32x8 *>(group + (l & 15) * row_bytes + (l >> 4) * 32);
}

}  // namespace

// One launcher per kernel file; each returns the launch status.
// per-tile kernel (bf16, fp8 or fp16; 1..64 heads): logits_decode.hip
hipError_t launch_decode(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
// looped fp8 kernel (16+ heads, rows_per_tile from the plan): logits_looped.hip
hipError_t launch_looped_fp8(const LogitsArgs &a, int rows_per_tile, hipStream_t s, hipEvent_t e0,
                             hipEvent_t e1);
// 4-row fp8 kernel (32/64 heads): logits_mtp.hip
hipError_t launch_mtp_fp8(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
// prefill kernel (bf16 or fp16, 4 heads, one request): logits_prefill.hip
hipError_t launch_prefill(const LogitsArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1);

}  // namespace qsa
