// GEMM path of the expert FFNs (token counts above the decode sizes):
// the activation prep kernel and the dispatch to the instantiations in
// gemm_{gu,dn}{2,3}.hip.
#include "gemm_impl.hpp"

namespace strata {

extern template hipError_t gemm_gateup_launch<3, 1>(const LayerArgs &, int, hipStream_t);
extern template hipError_t gemm_gateup_launch<3, 2>(const LayerArgs &, int, hipStream_t);
extern template hipError_t gemm_gateup_launch<2, 1>(const LayerArgs &, int, hipStream_t);
extern template hipError_t gemm_gateup_launch<2, 2>(const LayerArgs &, int, hipStream_t);
extern template hipError_t gemm_down_launch<3>(const LayerArgs &, int, hipStream_t);
extern template hipError_t gemm_down_launch<2>(const LayerArgs &, int, hipStream_t);

// Per token: 1/rms (normalised layers), then the layer input u = x / rms as
// bf16 hi (and lo = bf16(u - hi) unless u is exactly bf16) in the permuted
// column order of the gate/up GEMM, and the sum of hi + lo over every
// 128-column step.  One block per token, 8 columns per thread.
__global__ __launch_bounds__(256) void gemm_prep_kernel(LayerArgs a) {
    __shared__ float red[4];
    const int t = blockIdx.x, th = threadIdx.x;
    const float inv = token_inv_rms(a, t, red);
    if (th == 0) a.inv_rms[t] = inv;
    if (a.route_only) return;
    const int d = a.d, ng = d / 8, nsteps = d / 128;
    const int64_t row = (int64_t)t * d, TD = (int64_t)a.T * d;
    for (int q0 = 0; q0 < ng; q0 += 256) {
        const int q = q0 + th;
        const bool valid = q < ng;
        float u[8];
        if (a.x_is_bf16) {
            const uint4 v = valid ? *(const uint4 *)((const uint16_t *)a.x + row + 8 * q) : make_uint4(0, 0, 0, 0);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u[2 * j] = __uint_as_float(w[j] << 16);
                u[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
            }
        } else {
            const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 v0 = valid ? *(const float4 *)((const float *)a.x + row + 8 * q) : z;
            const float4 v1 = valid ? *(const float4 *)((const float *)a.x + row + 8 * q + 4) : z;
            u[0] = v0.x; u[1] = v0.y; u[2] = v0.z; u[3] = v0.w;
            u[4] = v1.x; u[5] = v1.y; u[6] = v1.z; u[7] = v1.w;
        }
        uint32_t hw[4], lw[4];
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            // element j holds column 8q + [0,4,1,5,2,6,3,7][j]
            const float v0 = u[j >> 1] * inv, v1 = u[(j >> 1) + 4] * inv;
            const uint16_t h0 = f2bf(v0), h1 = f2bf(v1);
            const uint16_t l0 = f2bf(v0 - bf16_to_float(h0)), l1 = f2bf(v1 - bf16_to_float(h1));
            hw[j >> 1] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lw[j >> 1] = (uint32_t)l0 | ((uint32_t)l1 << 16);
            s += (bf16_to_float(h0) + bf16_to_float(l0)) + (bf16_to_float(h1) + bf16_to_float(l1));
        }
        const int64_t pos = row + 128 * (q >> 4) + step_pos((8 * q) & 127);
        if (valid) {
            *(uint4 *)(a.xa + pos) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            if (a.xpasses == 2) *(uint4 *)(a.xa + TD + pos) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        }
        s += lane_xor<1>(s);
        s += lane_xor<2>(s);
        s += lane_xor<4>(s);
        s += lane_xor<8>(s);
        if (valid && (q & 15) == 0) a.sx[(int64_t)t * nsteps + (q >> 4)] = s;
    }
}

bool gemm_supported(int d, int f) {
    return d % 128 == 0 && f % 128 == 0 && d <= GEMM_MAX_K && f <= GEMM_MAX_K;
}

hipError_t launch_gemm_prep(const LayerArgs &a, hipStream_t s) {
    STRATA_LAUNCH(gemm_prep_kernel, dim3(a.T), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gemm_gateup(const LayerArgs &a, int max_items, hipStream_t s) {
    if (a.bits == 3)
        return a.xpasses == 1 ? gemm_gateup_launch<3, 1>(a, max_items, s) : gemm_gateup_launch<3, 2>(a, max_items, s);
    return a.xpasses == 1 ? gemm_gateup_launch<2, 1>(a, max_items, s) : gemm_gateup_launch<2, 2>(a, max_items, s);
}

hipError_t launch_gemm_down(const LayerArgs &a, int max_items, hipStream_t s) {
    return a.bits == 3 ? gemm_down_launch<3>(a, max_items, s) : gemm_down_launch<2>(a, max_items, s);
}

}  // namespace strata
