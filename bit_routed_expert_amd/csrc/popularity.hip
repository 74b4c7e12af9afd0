// Expert popularity -> resident set.  The expert cache keeps the experts
// the workload picks most and adapts to use as it goes (wiselychen.com,
// technique 2 "專家快取與 CPU／GPU 分工"; wiki.nginx.tw, "Strata：把 1250 億參數的
// Qwen3.8-Flash-Next 跑在遊戲顯卡上", the dynamic expert cache item, which puts
// its hit rate near 72% against 50% for a fixed cache).  Here: running
// per-expert pick counts (the routing's counts, added call by call) and the
// n most-picked experts as a resident mask, ordered by (count desc, index
// asc) so equal counts resolve the same way every time.
#include "common.hpp"
#include "strata_moe.h"

namespace strata {

__global__ __launch_bounds__(256) void counts_accumulate_kernel(int64_t *acc, const int32_t *counts, int E) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e < E) acc[e] += counts[e];
}

// One block of 1024 threads (E <= 1024): thread e ranks expert e against
// every other from an LDS copy of the counts; wave w's ballot is the mask
// words of experts 64w .. 64w + 63.
__global__ __launch_bounds__(1024) void resident_topn_kernel(const int64_t *acc, int E, int n, uint32_t *mask) {
    __shared__ int64_t c[1024];
    const int th = threadIdx.x, lane = th & 63, w = th >> 6;
    if (th < E) c[th] = acc[th];
    __syncthreads();
    bool in = false;
    if (th < E) {
        const int64_t mine = c[th];
        int rank = 0;
        for (int j = 0; j < E; ++j) {
            const int64_t o = c[j];
            rank += (o > mine || (o == mine && j < th)) ? 1 : 0;
        }
        in = rank < n;
    }
    const uint64_t b = __ballot(in);
    if (lane == 0 && 64 * w < E) mask[2 * w] = (uint32_t)b;
    if (lane == 0 && 64 * w + 32 < E) mask[2 * w + 1] = (uint32_t)(b >> 32);
}

}  // namespace strata

using namespace strata;

extern "C" {

strata_status strata_moe_counts_accumulate(int64_t *counts_acc, const int32_t *counts, int32_t n_experts,
                                           void *stream) {
    if (!counts_acc || !counts || n_experts < 1 || n_experts > 1024) return STRATA_EINVAL;
    STRATA_LAUNCH(counts_accumulate_kernel, dim3((n_experts + 255) / 256), dim3(256), 0, (hipStream_t)stream,
                  counts_acc, counts, n_experts);
    return hip_status(hipGetLastError());
}

strata_status strata_moe_resident_topn(const int64_t *counts_acc, int32_t n_experts, int32_t n_resident,
                                       uint32_t *mask_out, void *stream) {
    if (!counts_acc || !mask_out || n_experts < 1 || n_experts > 1024 || n_resident < 0 || n_resident > n_experts)
        return STRATA_EINVAL;
    STRATA_LAUNCH(resident_topn_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, counts_acc, n_experts,
                  n_resident, mask_out);
    return hip_status(hipGetLastError());
}

}  // extern "C"
