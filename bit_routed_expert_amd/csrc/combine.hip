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

constexpr int KB = 16;          // picks gathered per batch (top_k <= 32: at most two batches)
constexpr int CB_COLS = 1024;   // columns per block (4 per thread)

// One block per (token, 1024-column segment): the token's routing is
// block-uniform, every thread gathers 4 columns of the picked rows.
template <int XBF16>
__global__ __launch_bounds__(256) void combine_kernel(LayerArgs a) {
    const int d = a.d, k = a.k, T = a.T;
    const int segs = (d + CB_COLS - 1) / CB_COLS;
    const int t = blockIdx.x / segs;
    const int i = (blockIdx.x - t * segs) * CB_COLS + threadIdx.x * 4;
    if (i >= d) return;
    const float *__restrict__ Y = a.Y;
    const int64_t row = (int64_t)t * d + i;
    float4 s = *(const float4 *)(Y + ((int64_t)T * k + t) * d + i);
    for (int r0 = 0; r0 < k; r0 += KB) {
        int pr[KB];
        float gr[KB];
#pragma unroll
        for (int r = 0; r < KB; ++r) {
            pr[r] = -1;
            gr[r] = 0.f;
            if (r0 + r < k) {
                const int e = a.idx[t * k + r0 + r];
                if (!a.mask || ((a.mask[e >> 5] >> (e & 31)) & 1u)) {
                    pr[r] = a.pos[t * k + r0 + r];
                    gr[r] = a.gate[t * k + r0 + r];
                }
            }
        }
        float4 yv[KB];
#pragma unroll
        for (int r = 0; r < KB; ++r)
            yv[r] = pr[r] >= 0 ? *(const float4 *)(Y + (int64_t)pr[r] * d + i) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int r = 0; r < KB; ++r) {
            if (pr[r] >= 0) {
                s.x = fmaf(gr[r], yv[r].x, s.x);
                s.y = fmaf(gr[r], yv[r].y, s.y);
                s.z = fmaf(gr[r], yv[r].z, s.z);
                s.w = fmaf(gr[r], yv[r].w, s.w);
            }
        }
    }
    *(float4 *)(a.out + row) = s;
    if (a.x_next) {
        float4 xv;
        if (XBF16) {
            const uint2 q = *(const uint2 *)((const uint16_t *)a.x + row);
            xv = make_float4(__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xFFFF0000u),
                             __uint_as_float(q.y << 16), __uint_as_float(q.y & 0xFFFF0000u));
        } else {
            xv = *(const float4 *)((const float *)a.x + row);
        }
        *(float4 *)(a.x_next + row) = make_float4(xv.x + s.x, xv.y + s.y, xv.z + s.z, xv.w + s.w);
    }
}

hipError_t launch_combine(const LayerArgs &a, hipStream_t s) {
    const int blocks = a.T * ((a.d + CB_COLS - 1) / CB_COLS);
    if (a.x_is_bf16)
        STRATA_LAUNCH(combine_kernel<1>, dim3(blocks), dim3(256), 0, s, a);
    else
        STRATA_LAUNCH(combine_kernel<0>, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace strata
