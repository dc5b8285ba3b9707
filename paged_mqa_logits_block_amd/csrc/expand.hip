// Expand: selected compressed columns -> the key tokens each one stands for.
//
// The pages time a full selection as score + top-k + expand, with a
// compression ratio of 4 (vLLM PR #62589, "Performance" and the MI355X
// comment); compressed column c covers tokens [c * ratio, c * ratio + ratio).
// One thread per output slot: consecutive threads write consecutive slots, and
// the `ratio` threads of one selected column read the same index (one cache
// line serves a wave).

#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kExpandThreads = 256;

__global__ __launch_bounds__(kExpandThreads) void expand_kernel(ExpandArgs a) {
    const int64_t per_row = (int64_t)a.k * a.ratio;
    const int64_t total = (int64_t)a.num_rows * per_row;
    for (int64_t o = (int64_t)blockIdx.x * kExpandThreads + threadIdx.x; o < total;
         o += (int64_t)gridDim.x * kExpandThreads) {
        const int64_t r = o / per_row;
        const int64_t in_row = o - r * per_row;
        const int64_t p = in_row / a.ratio;
        const int j = (int)(in_row - p * a.ratio);
        const int32_t c = a.idx[r * a.k + p];
        const int64_t tok = (int64_t)c * a.ratio + j;
        const int64_t lim = a.token_lens ? (int64_t)a.token_lens[r] : (int64_t)0x7FFFFFFF + 1;
        a.tokens_out[o] = (c >= 0 && tok < lim && tok <= 0x7FFFFFFF) ? (int32_t)tok : -1;
    }
}

}  // namespace

hipError_t launch_expand(const ExpandArgs &a, hipStream_t s) {
    const int64_t total = (int64_t)a.num_rows * a.k * a.ratio;
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + kExpandThreads - 1) / kExpandThreads;
    if (blocks > 8192) blocks = 8192;  // grid-stride beyond that
    hipLaunchKernelGGL(expand_kernel, dim3((unsigned)blocks), dim3(kExpandThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace qsa
