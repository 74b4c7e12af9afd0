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
// block-uniform, every thread gathers 4 columns of the picked rows.  YTOK:
// Y rows in token order (pick r of token t at row t*k + r) and residency
// from rbits, so the rows load with the gates in one round trip; else the
// rows sit at the picks' slots (pos) and residency comes from the mask.
// Four consecutive values of the residual input x (bf16 or fp32) as fp32.
template <int XBF16> __device__ __forceinline__ float4 load_x4(const void *x, int64_t at) {
    if (XBF16) {
        const uint2 q = *(const uint2 *)((const uint16_t *)x + at);
        return make_float4(__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xFFFF0000u), __uint_as_float(q.y << 16),
                           __uint_as_float(q.y & 0xFFFF0000u));
    }
    return *(const float4 *)((const float *)x + at);
}

template <int XBF16, int YTOK>
__global__ __launch_bounds__(256) void combine_kernel(LayerArgs a) {
    const int d = a.d, k = a.k, T = a.T;
    const int segs = (d + CB_COLS - 1) / CB_COLS;
    const int t = blockIdx.x / segs;
    const int i = (blockIdx.x - t * segs) * CB_COLS + threadIdx.x * 4;
    if (i >= d) return;
    const float *__restrict__ Y = a.Y;
    const int64_t row = (int64_t)t * d + i;
    float4 s = *(const float4 *)(Y + ((int64_t)T * k + t) * d + i);
    // the residual input, loaded with the first reads (not after the output store)
    const float4 xv = a.x_next ? load_x4<XBF16>(a.x, row) : make_float4(0.f, 0.f, 0.f, 0.f);
    const uint32_t rb = (YTOK && a.mask) ? (uint32_t)a.rbits[t] : 0xFFFFFFFFu;
    for (int r0 = 0; r0 < k; r0 += KB) {
        int pr[KB];
        float gr[KB];
#pragma unroll
        for (int r = 0; r < KB; ++r) {
            pr[r] = -1;
            gr[r] = 0.f;
            if (r0 + r < k) {
                if (YTOK) {
                    if ((rb >> (r0 + r)) & 1u) {
                        pr[r] = t * k + r0 + r;
                        gr[r] = a.gate[t * k + r0 + r];
                    }
                } else {   // pick, slot and gate read together; the mask test picks them afterwards
                    const int e = a.idx[t * k + r0 + r], p = a.pos[t * k + r0 + r];
                    const float g = a.gate[t * k + r0 + r];
                    if (!a.mask || ((a.mask[e >> 5] >> (e & 31)) & 1u)) {
                        pr[r] = p;
                        gr[r] = g;
                    }
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
    if (a.x_next) *(float4 *)(a.x_next + row) = make_float4(xv.x + s.x, xv.y + s.y, xv.z + s.z, xv.w + s.w);
}

// out[i] += add[i], then x_next[i] = x[i] + out[i] (4 values per thread).
template <int XBF16>
__global__ __launch_bounds__(256) void add_rows_kernel(LayerArgs a, const float *add) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= (int64_t)a.T * a.d) return;
    const float4 v = *(const float4 *)(add + i);
    float4 o = *(const float4 *)(a.out + i);
    const float4 xv = a.x_next ? load_x4<XBF16>(a.x, i) : make_float4(0.f, 0.f, 0.f, 0.f);
    o = make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w);
    *(float4 *)(a.out + i) = o;
    if (a.x_next) *(float4 *)(a.x_next + i) = make_float4(xv.x + o.x, xv.y + o.y, xv.z + o.z, xv.w + o.w);
}

hipError_t launch_add_rows(const LayerArgs &a, const float *add, hipStream_t s) {
    const int64_t n4 = (int64_t)a.T * a.d / 4;
    const dim3 grid((unsigned)((n4 + 255) / 256));
    if (a.x_is_bf16)
        hipLaunchKernelGGL(add_rows_kernel<1>, grid, dim3(256), 0, s, a, add);
    else
        hipLaunchKernelGGL(add_rows_kernel<0>, grid, dim3(256), 0, s, a, add);
    return hipGetLastError();
}

hipError_t launch_combine(const LayerArgs &a, hipStream_t s) {
    const int blocks = a.T * ((a.d + CB_COLS - 1) / CB_COLS);
    if (a.ytok) {
        if (a.x_is_bf16)
            STRATA_LAUNCH((combine_kernel<1, 1>), dim3(blocks), dim3(256), 0, s, a);
        else
            STRATA_LAUNCH((combine_kernel<0, 1>), dim3(blocks), dim3(256), 0, s, a);
    } else {
        if (a.x_is_bf16)
            STRATA_LAUNCH((combine_kernel<1, 0>), dim3(blocks), dim3(256), 0, s, a);
        else
            STRATA_LAUNCH((combine_kernel<0, 0>), dim3(blocks), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace strata
