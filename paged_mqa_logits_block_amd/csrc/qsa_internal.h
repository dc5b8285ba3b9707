// Host/device interface between the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// input dtype codes, equal to the qsa_dtype values: bf16, fp8 e4m3fn, fp16
constexpr int kBF16 = 0, kFP8 = 1, kFP16 = 2;

// Launch description of one qsa_paged_logits call, fully resolved on the host.
struct LogitsArgs {
    const void *q;
    const float *w;
    const uint8_t *kcache;
    const float *kscale;
    const int32_t *block_table;
    const int32_t *ctx_lens;
    const int32_t *row_to_req;
    float *out;
    int32_t num_rows;
    int32_t num_heads;
    int32_t block_size;
    int32_t num_reqs;
    int32_t max_blocks;
    int32_t width;
    int32_t cap;            // min(width, max_blocks * block_size)
    int32_t num_row_tiles;  // ceil(num_rows / rows per tile)
    int32_t num_chunks;     // column chunks per row tile
    int32_t dtype;          // kBF16, kFP8 or kFP16
    int32_t layout;         // 0 paged, 1 co-packed, 2 co-packed preshuffled
    int32_t head_dim;       // D: 128, or 64 (per-tile kernel only)
    int64_t num_blocks;
    int64_t out_stride;
    int64_t block_bytes;    // stride between pool blocks
    int64_t key_stride;     // bytes between keys inside a block
    int64_t scale_offset;   // co-packed: byte offset of the scales inside a block
    int32_t iters;          // looped variant: key-tile groups per program
    int32_t pad2_;
    int32_t mtp_aligned;    // 4-row fp8 variant: tiles follow the requests (see logits_mtp.hip)
    int32_t pad3_;
    uint32_t *cand;         // or null: the per-tile kernel also writes each row's chunk candidates
                            // ([rows][num_chunks][32] packed keys) for the fused selection
};

// Variant chosen for a call: rows per tile and column tiles per program.
struct LogitsPlan {
    int rows_per_tile;
    int tiles_per_prog;  // 16-column tiles per program
    int m_tiles;         // 16-row MFMA tiles stacked per program
    int iters;           // > 0: looped variant with this many key-tile groups
                         // (prefill variant: 32-column steps per program)
    bool prefill;        // prefill variant (bf16, 4 heads, one request)
    bool mtp;            // 4-row fp8 variant (32/64 heads; iters = 64-column runs per program)
    bool mtp_aligned;    // its tiles follow the requests (row tiles: an upper bound of their count)
    int row_tiles;       // row tiles of the grid
};

// 4-row fp8 variant: columns per key run, runs per program at most, and the
// most rows for which its tiles follow the requests (each workgroup finds its
// tile by scanning row_to_req)
constexpr int kMtpRunCols = 64;
constexpr int kMtpMaxRunsPerGroup = 16;
constexpr int kMtpAlignedMaxRows = 256;

// consumer waves per workgroup of the prefill variant (16 rows each; one
// producer wave besides), and how many of its workgroups one CU holds at once
// (VGPR-bound: 3 waves per SIMD)
constexpr int kPrefillWaves = 8;
constexpr int kPrefillGroupsPerCU = 12 / (kPrefillWaves + 1);

LogitsPlan plan_logits(int dtype, int layout, int head_dim, int num_heads, int num_rows, int num_reqs,
                       int width, int block_size, int64_t out_stride);
// start / stop (may be null) are recorded by the dispatch packet itself at the
// kernel's start and end.
hipError_t launch_paged_logits(const LogitsArgs &a, const LogitsPlan &p, hipStream_t s,
                               hipEvent_t start, hipEvent_t stop);

struct TopkArgs {
    const float *logits;
    int64_t stride;
    const int32_t *ctx_lens;
    const int32_t *row_starts;  // first candidate column per row, or null (0)
    int32_t num_rows;
    int32_t width;
    int32_t k;
    int32_t *idx_out;
    uint8_t *workspace;  // split selection only
    int32_t slices;      // workgroups per row (1: one workgroup per row)
    int32_t slice_len;   // columns per slice, a multiple of 4
    int32_t groups;      // consecutive float4 per thread covering a slice
    int32_t cand_shift;  // log2 of the member slots per slice
    // fused selection: the scoring kernel's chunk candidates ([rows][cand_chunks][32]
    // packed keys) and the visible limit of that scoring (min(width, table columns))
    const uint32_t *cand;
    int32_t cand_chunks;
    int32_t cap;
};

// How a top-k call is spread: one workgroup per row, or `slices` workgroups
// per row (few rows) passing counts and members through a workspace.
struct TopkPlan {
    int slices;
    int slice_len;
    int groups;
    int cand_shift;
};

int topk_groups_for_width(int width);  // 1 if the width is supported, else 0
TopkPlan plan_topk(int num_rows, int width);
int64_t topk_workspace_bytes(int num_rows, int width);  // 0: no workspace used
// Bytes of the library-held split-selection scratch per GPU: the largest
// workspace any supported shape uses (8,652,800 bytes, at 128 rows x 49,169
// columns), rounded up to 9 MiB.
constexpr int64_t kTopkScratchBytes = (int64_t)9 << 20;
// Device address of that scratch on the calling thread's current device
// (looked up on the first call per device).
hipError_t topk_scratch(void **ptr);
hipError_t launch_topk(const TopkArgs &a, hipStream_t s, hipEvent_t start, hipEvent_t stop);
// The fused selection's resolve: one workgroup per row, from a.cand.
hipError_t launch_topk_cand(const TopkArgs &a, hipStream_t s, hipEvent_t start, hipEvent_t stop);

// Selected compressed columns -> tokens (qsa_expand).
struct ExpandArgs {
    const int32_t *idx;         // [num_rows][k]
    const int32_t *token_lens;  // [num_rows] or null
    int32_t *tokens_out;        // [num_rows][k * ratio]
    int32_t num_rows;
    int32_t k;
    int32_t ratio;
};

hipError_t launch_expand(const ExpandArgs &a, hipStream_t s);

}  // namespace qsa
