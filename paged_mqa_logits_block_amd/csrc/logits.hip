// Paged MQA-logits scoring: the planner (variant and launch shape from host
// values only) and the dispatch to the kernel files.

#include "logits_frag.h"

namespace qsa {


LogitsPlan plan_logits(int dtype, int layout, int head_dim, int num_heads, int num_rows, int num_reqs,
                       int width, int block_size, int64_t out_stride) {
    LogitsPlan p;
    p.iters = 0;
    p.prefill = false;
    p.mtp = false;
    p.mtp_aligned = false;
    // the looped, 4-row and prefill kernels are built for D = 128; other head
    // dims take the per-tile kernel
    const bool d128 = head_dim == 128;
    // fp8, 32 or 64 heads, 2 or more rows per request on average (MTP verify,
    // ragged included): 4-row workgroups sharing each key run (a tile whose
    // rows belong to several requests walks them one at a time; any block
    // size for block-flat keys, whole 64-column runs per block for preshuffled
    // ones); chunks sized for about four workgroups per CU
    if (d128 && dtype == kFP8 && (num_heads == 32 || num_heads == 64) && num_reqs > 0 && num_rows >= 2 * num_reqs &&
        (layout != 2 || block_size % kMtpRunCols == 0)) {
        p.mtp = true;
        p.rows_per_tile = 4;
        p.m_tiles = num_heads / 16;
        // Tiles of up to 4 consecutive rows of one request when the rows per
        // request may differ (R != 4 * reqs, at most kMtpAlignedMaxRows rows):
        // a request's rows are cut into tiles of 4 from its first row, so a
        // tile never walks two requests.  Rows grouped by request make at most
        // sum ceil(n_i / 4) <= (R + 3 min(reqs, R)) / 4 tiles; the kernel takes
        // plain tiles when the rows make more (grouped otherwise).  R = 4 * reqs
        // is taken as 4 rows per request, where plain tiles are the same.
        p.mtp_aligned = num_rows <= kMtpAlignedMaxRows && num_rows != 4 * num_reqs;
        const int row_tiles =
            p.mtp_aligned ? min(num_rows, (num_rows + 3 * min(num_reqs, num_rows)) / 4) : (num_rows + 3) / 4;
        p.row_tiles = row_tiles;
        const int runs = (width + kMtpRunCols - 1) / kMtpRunCols;
        int per = 1;
        while (per < kMtpMaxRunsPerGroup && (int64_t)row_tiles * ((runs + per - 1) / per) > 1024) per *= 2;
        p.iters = per;
        p.tiles_per_prog = per * kMtpRunCols / 16;
        return p;
    }
    // bf16 or fp16, 4 heads, a single request holding all rows (a prefill chunk), pool
    // blocks of a multiple of 32 columns: the prefill variant, 64 rows per
    // workgroup, columns split so that about two workgroups run per CU
    if (d128 && (dtype == kBF16 || dtype == kFP16) && num_heads == 4 && num_reqs == 1 && num_rows >= 256 &&
        block_size % 32 == 0 &&
        out_stride < ((int64_t)1 << 27)) {
        p.prefill = true;
        p.rows_per_tile = 16 * kPrefillWaves;
        p.m_tiles = 1;
        // column splits: enough workgroups for every CU's resident slots
        const int row_tiles = (num_rows + p.rows_per_tile - 1) / p.rows_per_tile;
        const int steps = (width + 31) / 32;
        const int target = 256 * kPrefillGroupsPerCU;
        const int splits = max(1, min(steps, (target + row_tiles - 1) / row_tiles));
        p.iters = (steps + splits - 1) / splits;
        p.tiles_per_prog = 2 * p.iters;  // in 16-column tiles
        return p;
    }
    p.m_tiles = num_heads > 16 ? num_heads / 16 : 1;
    p.rows_per_tile = 16 * p.m_tiles / num_heads;
    // 16-column tiles per program: 4 for the few-head decode shapes (a sweep on
    // MI355X found 1..8 within 4% there), 8 where each program's rows read more
    // key bytes per column (long single-row and many-head fp8 shapes gained
    // 3..15%)
    p.tiles_per_prog = num_heads <= 4 ? 4 : 8;
    // fp8 with 16+ heads and blocks of a multiple of 16 columns: the looped
    // variant, 4 key tiles per group and as many
    // groups per program as leave about four programs per SIMD; with 16 heads
    // and several rows per request (MTP verify rows) 4 rows share a program
    if (d128 && dtype == kFP8 && num_heads >= 16 && block_size % 16 == 0) {
        const int rows_per_req = num_reqs > 0 ? num_rows / num_reqs : 1;
        if (num_heads == 16 && rows_per_req >= 4) {
            p.rows_per_tile = 4;
            p.m_tiles = 4;
        }
        const int tpi = 4;
        const int row_tiles = (num_rows + p.rows_per_tile - 1) / p.rows_per_tile;
        const int col_tiles = (width + 15) / 16;
        int iters = 32;
        while (iters > 2 && (int64_t)row_tiles * ((col_tiles + tpi * iters - 1) / (tpi * iters)) < 4096) iters /= 2;
        p.iters = iters;
        p.tiles_per_prog = tpi * iters;
    }
    return p;
}

hipError_t launch_paged_logits(const LogitsArgs &a, const LogitsPlan &p, hipStream_t s, hipEvent_t e0,
                               hipEvent_t e1) {
    if (a.num_row_tiles == 0 || a.num_chunks == 0) return hipSuccess;
    if (a.dtype != kFP8 && p.prefill) return launch_prefill(a, s, e0, e1);
    if (a.dtype == kFP8 && p.mtp) return launch_mtp_fp8(a, s, e0, e1);
    if (a.dtype == kFP8 && p.iters > 0) return launch_looped_fp8(a, p.rows_per_tile, s, e0, e1);
    return launch_decode(a, s, e0, e1);
}

}  // namespace qsa
