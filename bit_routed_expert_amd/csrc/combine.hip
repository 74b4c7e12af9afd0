// Combine of one layer: out[t] = y_shared[t] + sum over r ascending of
// gate[t][r] * y_{idx[t][r]}[t] for resident experts (fixed order, no
// atomics, so repeated calls are bitwise identical), then the residual
// stream x_{l+1} = x_l + out in fp32.
//
// The shared expert is added with weight 1 and every token uses it
// (greenbean-ai, "Strata 如何讓 12GB 顯卡跑 Qwen3.8-Flash-Next？", section 一:
// 10 routed + 1 shared expert per token); experts missing from the GPU are
// left to another processor and so contribute nothing here (wiselychen.com,
// technique 2 "專家快取與 CPU／GPU 分工").
#include "common.hpp"

namespace strata {

constexpr int KMAX = 32;

template <int XBF16>
__global__ __launch_bounds__(256) void combine_kernel(LayerArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int d = a.d, k = a.k, T = a.T;
    if (gid >= (int64_t)T * d) return;
    const int t = (int)(gid / d), i = (int)(gid % d);
    const float *__restrict__ Y = a.Y;
    // all routing reads first (independent loads), then all expert rows
    int pr[KMAX];
    float gr[KMAX];
    bool on[KMAX];
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
        if (r < k) {
            const int e = a.idx[t * k + r];
            pr[r] = a.pos[t * k + r];
            gr[r] = a.gate[t * k + r];
            on[r] = !a.mask || ((a.mask[e >> 5] >> (e & 31)) & 1u);
        }
    }
    float s = Y[((int64_t)T * k + t) * d + i];
    float yv[KMAX];
#pragma unroll
    for (int r = 0; r < KMAX; ++r)
        if (r < k) yv[r] = on[r] ? Y[(int64_t)pr[r] * d + i] : 0.f;
#pragma unroll
    for (int r = 0; r < KMAX; ++r)
        if (r < k && on[r]) s = fmaf(gr[r], yv[r], s);
    a.out[gid] = s;
    if (a.x_next) {
        const float xv = XBF16 ? bf16_to_float(((const uint16_t *)a.x)[gid]) : ((const float *)a.x)[gid];
        a.x_next[gid] = xv + s;
    }
}

hipError_t launch_combine(const LayerArgs &a, hipStream_t s) {
    const int64_t n = (int64_t)a.T * a.d;
    const int blocks = (int)((n + 255) / 256);
    if (a.x_is_bf16)
        hipLaunchKernelGGL(combine_kernel<1>, dim3(blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(combine_kernel<0>, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace strata
