// Peak probes: a stream read from HBM and bf16 matrix-core chains (the
// achievable ceilings of the layer's decode and prefill kernels).
#include "mfma.hpp"
#include "strata_probe.h"

namespace strata {

constexpr int PROBE_UNROLL = 8;   // 16-byte loads in flight per thread

__global__ __launch_bounds__(256) void probe_read_kernel(const uint4 *__restrict__ buf, size_t n16, uint32_t *sink) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (PROBE_UNROLL - 1) * stride < n16; i += PROBE_UNROLL * stride) {
        uint4 v[PROBE_UNROLL];
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; ++u) v[u] = buf[i + u * stride];
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = buf[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, WAVE);
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

constexpr int PROBE_CHAINS = 4;

__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float *sink) {
    const int lane = threadIdx.x & 63;
    bf16x8_t a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(1e-3f * (float)((lane + j) & 7));
        b[j] = (__bf16)(1e-3f * (float)((lane * 3 + j) & 7));
    }
    f32x16_t c[PROBE_CHAINS];
#pragma unroll
    for (int q = 0; q < PROBE_CHAINS; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) c[q][v] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int q = 0; q < PROBE_CHAINS; ++q) c[q] = mfma(a, b, c[q]);
    }
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < PROBE_CHAINS; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += c[q][v];
    s = wave_sum(s);
    __shared__ float red[4];
    if (lane == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

}  // namespace strata

using namespace strata;

extern "C" {

strata_status strata_probe_hbm_read(const void *buf, size_t bytes, uint32_t *sink, int32_t blocks, void *stream) {
    if (!buf || !sink || ((uintptr_t)buf & 15u) || bytes == 0 || bytes % 16 || blocks < 1 || blocks > 65536)
        return STRATA_EINVAL;
    hipLaunchKernelGGL(probe_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4 *)buf,
                       bytes / 16, sink);
    return hip_status(hipGetLastError());
}

strata_status strata_probe_mfma_bf16(int32_t iters, float *sink, int32_t blocks, double *flops, void *stream) {
    if (!sink || !flops || iters < 1 || iters > (1 << 20) || blocks < 1 || blocks > 65536) return STRATA_EINVAL;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
    *flops = (double)blocks * 4 * iters * PROBE_CHAINS * (2.0 * 32 * 32 * 16);
    return hip_status(hipGetLastError());
}

}  // extern "C"
