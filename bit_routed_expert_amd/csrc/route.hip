// Routing of one MoE layer: router logits, ordered top-k with gates, the
// stable per-expert permutation, the expert work list, the miss list of
// non-resident experts, and the fixed-point digit planes of the layer input.
//
// Per-layer routing of 10 of 512 experts (plus one shared expert) per token
// is the model the pages describe (greenbean-ai, "Strata 如何讓 12GB 顯卡跑
// Qwen3.8-Flash-Next？", section 一); the GPU runs the router (same page,
// section 二).  Logits are fp32; top-k is ordered by (logit desc, index asc);
// gates are the softmax renormalised over the k picks.
#include "routing.hpp"

namespace strata {

// Every kernel here stays within the 64 KiB of LDS a block gets by default;
// a launch that would need more is refused rather than attempted.
constexpr size_t LDS_LIMIT = 64 * 1024;

// ------------------------------------------------------ input digit planes
// For token t: inverse RMS (or 1) and the digit planes of u = x * inv_rms:
// per 256-column group an exponent E with max|u| * 2^E inside the 4-digit
// range, X = rint(u * 2^E), and its balanced base-16 digits packed 8 columns
// per word (nibble n of word (unit U, plane p, i) = digit p of column 32U+8i+n).
// Runs on one block of `nth` threads (multiple of 64).
__device__ void prep_token(const LayerArgs &a, int t, float *red /*lds, >= nth/64 floats*/, float inv) {
    const int d = a.d, nth = blockDim.x, th = threadIdx.x;
    const int nchunk = d / 8;  // 8 columns per chunk
    const int Q = d / 128;
    const int G = (d + 255) / 256;
    (void)Q;
    for (int base = 0; base < nchunk; base += nth) {
        int c = base + th;
        bool valid = c < nchunk;
        float u[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            float xv = 0.f;
            if (valid) {
                size_t i = (size_t)t * d + c * 8 + n;
                xv = a.x_is_bf16 ? bf16_to_float(((const uint16_t *)a.x)[i]) : ((const float *)a.x)[i];
            }
            u[n] = xv * inv;
        }
        float m = 0.f;
#pragma unroll
        for (int n = 0; n < 8; ++n) m = fmaxf(m, fabsf(u[n]));
        // group max over the 32 chunks of a 256-column group (32 consecutive lanes)
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, WAVE));
        int E = fixed_point_exponent<XPLANES>(m);
        int X[8];
        int sx = 0;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            X[n] = (int)rintf(ldexpf(u[n], E));
            sx += X[n];
        }
        uint32_t word[XPLANES];
#pragma unroll
        for (int p = 0; p < XPLANES; ++p) word[p] = 0;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            int dg[XPLANES];
            to_digits<XPLANES>(X[n], dg);
#pragma unroll
            for (int p = 0; p < XPLANES; ++p) word[p] |= ((uint32_t)dg[p] & 15u) << (4 * n);
        }
        // digit sums per 32-column unit (4 consecutive chunks)
        sx += __shfl_xor(sx, 1, WAVE);
        sx += __shfl_xor(sx, 2, WAVE);
        if (valid) {
            int U = c / 4, i = c % 4;
            uint32_t *dst = a.xq + ((size_t)t * (d / 32) + U) * (XPLANES * 4);
#pragma unroll
            for (int p = 0; p < XPLANES; ++p) dst[p * 4 + i] = word[p];
            if (i == 0) a.xsum[(size_t)t * (d / 32) + U] = sx;
            if ((c & 31) == 0) a.xscl[(size_t)t * G + c / 32] = ldexpf(1.f, -E);
        }
    }
    (void)red;
}

// Inverse RMS of token t's row (1 when the layer input is not normalised).


// ------------------------------------------------------ decode-size route
// T <= 8.  Blocks [0, ceil(E/4)): one router row per wave, its loads issued
// before anything else, dotted with the T token rows staged in LDS; the
// unnormalised logits go to z.  Blocks past those: one per token, its
// inverse RMS and (unless routing only) its input digit planes.  The top-k
// is taken later by every consumer block from z (a few KB), so no block
// waits on another inside this kernel.
constexpr int RS_WAVES = 4;   // router rows per block
constexpr int RS_MAXJ = 8;    // float4 per lane per 2048-column chunk

template <int XBF16>
__global__ __launch_bounds__(256) void route_logits_small_kernel(LayerArgs a) {
    extern __shared__ float lds[];
    const int th = threadIdx.x, lane = th & 63, wave = th >> 6;
    const int d = a.d, T = a.T, E = a.E;
    const int nrow_blocks = (E + RS_WAVES - 1) / RS_WAVES;
    if ((int)blockIdx.x >= nrow_blocks) {
        const int t = blockIdx.x - nrow_blocks;
        const float inv = token_inv_rms(a, t, lds);
        if (th == 0) a.inv_rms[t] = inv;
        if (!a.route_only) prep_token(a, t, nullptr, inv);
        return;
    }
    const int e = blockIdx.x * RS_WAVES + wave;
    const float *wrow = a.Wr + (size_t)(e < E ? e : 0) * d;
    float *xs = lds;  // [T][d]
    for (int c0 = 0; c0 < d; c0 += 64 * 4 * RS_MAXJ) {
        float4 wv[RS_MAXJ];
#pragma unroll
        for (int j = 0; j < RS_MAXJ; ++j) {
            const int i = c0 + lane * 4 + 256 * j;
            wv[j] = (e < E && i < d) ? *(const float4 *)(wrow + i) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (c0 == 0) {
            for (int i = th; i < T * d; i += 256)
                xs[i] = XBF16 ? bf16_to_float(((const uint16_t *)a.x)[i]) : ((const float *)a.x)[i];
            __syncthreads();
        }
        for (int t = 0; t < T; ++t) {
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < RS_MAXJ; ++j) {
                const int i = c0 + lane * 4 + 256 * j;
                if (i < d) {
                    const float4 xv = *(const float4 *)(xs + t * d + i);
                    acc += wv[j].x * xv.x + wv[j].y * xv.y + wv[j].z * xv.z + wv[j].w * xv.w;
                }
            }
            acc = wave_sum(acc);
            if (lane == 0 && e < E) {
                if (c0 == 0) a.z[t * E + e] = acc;
                else a.z[t * E + e] += acc;
            }
        }
    }
}

// Routing only, T <= 8: one block takes the top-k and writes every output.
__global__ __launch_bounds__(256) void route_small_finish_kernel(LayerArgs a) {
    extern __shared__ uint32_t lds_u[];
    const SmallRoute L(lds_u, a.E);
    small_route_compute(a, L);
    small_route_write(a, L);
}

// Router logits z[t][e] = inv_rms[t] * (x[t] . Wr[e]) + bias[e], fp32,
// 64x64 output tile per block, 16x16 threads with 4x4 outputs each.  Each
// 32-column slab is summed on its own and the slab sums are added with
// compensated (Kahan) summation, so the error stays near one fp32 rounding
// of the logit instead of growing with d.
__global__ __launch_bounds__(256) void route_logits_kernel(LayerArgs a) {
    __shared__ float xs[32][65];
    __shared__ float ws[32][65];
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    const int t0 = blockIdx.y * 64, e0 = blockIdx.x * 64;
    const int d = a.d;
    float acc[4][4] = {}, comp[4][4] = {};
    for (int k0 = 0; k0 < d; k0 += 32) {
        for (int i = threadIdx.x; i < 64 * 32; i += 256) {
            int r = i / 32, c = i % 32;
            int t = t0 + r, e = e0 + r;
            float xv = 0.f;
            if (t < a.T) {
                size_t o = (size_t)t * d + k0 + c;
                xv = a.x_is_bf16 ? bf16_to_float(((const uint16_t *)a.x)[o]) : ((const float *)a.x)[o];
            }
            xs[c][r] = xv;
            ws[c][r] = (e < a.E) ? a.Wr[(size_t)e * d + k0 + c] : 0.f;
        }
        __syncthreads();
        float part[4][4] = {};
#pragma unroll 8
        for (int c = 0; c < 32; ++c) {
            float xv[4], wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) { xv[i] = xs[c][ty + 16 * i]; wv[i] = ws[c][tx + 16 * i]; }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) part[i][j] = fmaf(xv[i], wv[j], part[i][j]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float y = part[i][j] - comp[i][j];
                const float t = acc[i][j] + y;
                comp[i][j] = (t - acc[i][j]) - y;
                acc[i][j] = t;
            }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int t = t0 + ty + 16 * i;
        if (t >= a.T) continue;
        float inv = a.inv_rms[t];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int e = e0 + tx + 16 * j;
            if (e < a.E) a.z[(size_t)t * a.E + e] = acc[i][j] * inv + (a.bias ? a.bias[e] : 0.f);
        }
    }
}

// One wave per token.
__global__ __launch_bounds__(256) void route_topk_kernel(LayerArgs a) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.T) return;
    wave_topk(a.z + (size_t)t * a.E, a.E, a.k, 1.f, nullptr, a.idx + (size_t)t * a.k, a.gate + (size_t)t * a.k,
              a.u_idx ? a.u_idx + (size_t)t * a.k : nullptr, a.u_gate ? a.u_gate + (size_t)t * a.k : nullptr,
              nullptr, nullptr);
}

// Any T: one block of 1024 threads.  Counts by LDS atomics (integer, so the
// result is order independent), exclusive scan, then a stable scatter over
// 512-token windows: within a window each expert's picks are marked in a
// bitmap and a pick's rank is the number of marked earlier tokens.
// Window of PW tokens (512, or 256 when E > 512 so the bitmaps fit in LDS).
__global__ __launch_bounds__(1024) void route_permute_kernel(LayerArgs a, int PW, int tile) {
    extern __shared__ int32_t sh[];
    const int th = threadIdx.x, nth = 1024;
    const int E = a.E, k = a.k, T = a.T;
    const int64_t n = (int64_t)T * k;
    int32_t *hist = sh;                 // [E]
    int32_t *run = sh + E;              // [E] running slot per expert
    int32_t *scan = sh + 2 * E;         // [1024]
    uint32_t *bm = (uint32_t *)(sh + 2 * E + 1024);  // [E][PW/32]
    const int BW = PW / 32;
    for (int e = th; e < E; e += nth) hist[e] = 0;
    __syncthreads();
    for (int64_t i = th; i < n; i += nth) atomicAdd(&hist[a.idx[i]], 1);
    __syncthreads();
    // exclusive scan over experts (E <= 1024, one per thread)
    int v = th < E ? hist[th] : 0;
    scan[th] = v;
    __syncthreads();
    for (int o = 1; o < nth; o <<= 1) {
        int add = th >= o ? scan[th - o] : 0;
        __syncthreads();
        scan[th] += add;
        __syncthreads();
    }
    int excl = scan[th] - v;
    if (th < E) {
        run[th] = excl;
        a.counts[th] = v;
        a.offsets[th] = excl;
        if (a.u_counts) a.u_counts[th] = v;
        if (a.u_offsets) a.u_offsets[th] = excl;
    }
    if (th == nth - 1) {
        a.offsets[E] = scan[th];
        if (a.u_offsets) a.u_offsets[E] = scan[th];
    }
    __syncthreads();
    for (int w0 = 0; w0 < T; w0 += PW) {
        for (int i = th; i < E * BW; i += nth) bm[i] = 0;
        __syncthreads();
        int wn = min(PW, T - w0);
        for (int i = th; i < wn * k; i += nth) {
            int tl = i / k;
            int e = a.idx[(int64_t)(w0 + tl) * k + i % k];
            atomicOr(&bm[e * BW + tl / 32], 1u << (tl % 32));
        }
        __syncthreads();
        for (int i = th; i < wn * k; i += nth) {
            int tl = i / k;
            int64_t gi = (int64_t)(w0 + tl) * k + i % k;
            int e = a.idx[gi];
            int rank = 0;
            for (int w = 0; w < tl / 32; ++w) rank += __popc(bm[e * BW + w]);
            rank += __popc(bm[e * BW + tl / 32] & ((1u << (tl % 32)) - 1u));
            int slot = run[e] + rank;
            a.perm[slot] = (int32_t)gi;
            a.pos[gi] = slot;
            if (a.u_perm) a.u_perm[slot] = (int32_t)gi;
            if (a.u_pos) a.u_pos[gi] = slot;
        }
        __syncthreads();
        for (int e = th; e < E; e += nth) {
            int c = 0;
            for (int w = 0; w < BW; ++w) c += __popc(bm[e * BW + w]);
            run[e] += c;
        }
        __syncthreads();
    }
    // miss list in (t, r) order
    int total = 0;
    for (int64_t b0 = 0; b0 < n; b0 += nth) {
        int64_t i = b0 + th;
        int e = i < n ? a.idx[i] : 0;
        int f = (i < n && !is_resident(a.mask, e)) ? 1 : 0;
        scan[th] = f;
        __syncthreads();
        for (int o = 1; o < nth; o <<= 1) {
            int add = th >= o ? scan[th - o] : 0;
            __syncthreads();
            scan[th] += add;
            __syncthreads();
        }
        int p = total + scan[th] - f;
        if (f && a.miss_te && p < a.miss_cap) {
            a.miss_te[2 * (int64_t)p] = (int32_t)(i / k);
            a.miss_te[2 * (int64_t)p + 1] = e;
            a.miss_w[p] = a.gate[i];
        }
        total += scan[nth - 1];
        __syncthreads();
    }
    if (th == 0 && a.miss_count) *a.miss_count = total;
    // work list: ceil(count/tile) items per resident expert with picks, then the shared expert
    int ni = (th < E && is_resident(a.mask, th)) ? (hist[th] + tile - 1) / tile : 0;
    scan[th] = ni;
    __syncthreads();
    for (int o = 1; o < nth; o <<= 1) {
        int add = th >= o ? scan[th - o] : 0;
        __syncthreads();
        scan[th] += add;
        __syncthreads();
    }
    int base = scan[th] - ni;
    if (th < E) {
        int off = scan[th] - ni;  // item base
        (void)off;
        int s0 = run[th] - hist[th];  // run[] now holds offsets + counts
        for (int j = 0; j < ni; ++j)
            a.items[base + j] = WorkItem{th, s0 + j * tile, min(tile, hist[th] - j * tile)};
    }
    int nr = scan[nth - 1];
    __syncthreads();
    if (th == 0) {
        int c = nr;
        for (int t0 = 0; t0 < T; t0 += tile)
            a.items[c++] = WorkItem{E, (int32_t)(n + t0), min(tile, T - t0)};
        *a.n_items = c;
    }
}

// ------------------------------------------------------------- launchers
hipError_t launch_route_logits_small(const LayerArgs &a, hipStream_t s) {
    const int blocks = (a.E + RS_WAVES - 1) / RS_WAVES + a.T;
    const size_t lds = sizeof(float) * (size_t)a.T * a.d;
    if (lds > LDS_LIMIT) return hipErrorInvalidValue;
    if (a.x_is_bf16)
        hipLaunchKernelGGL(route_logits_small_kernel<1>, dim3(blocks), dim3(256), lds, s, a);
    else
        hipLaunchKernelGGL(route_logits_small_kernel<0>, dim3(blocks), dim3(256), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_route_small_finish(const LayerArgs &a, hipStream_t s) {
    const size_t lds = 4 * (size_t)small_route_lds_words(a.E);
    if (lds > LDS_LIMIT) return hipErrorInvalidValue;
    hipLaunchKernelGGL(route_small_finish_kernel, dim3(1), dim3(256), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_route_logits(const LayerArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(route_logits_kernel, dim3((a.E + 63) / 64, (a.T + 63) / 64), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_route_topk(const LayerArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(route_topk_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_route_permute(const LayerArgs &a, int tile, hipStream_t s) {
    const int pw = a.E <= 512 ? 512 : 256;
    const size_t lds = sizeof(int32_t) * (size_t)(2 * a.E + 1024) + sizeof(uint32_t) * (size_t)a.E * (pw / 32);
    if (lds > LDS_LIMIT) return hipErrorInvalidValue;
    hipLaunchKernelGGL(route_permute_kernel, dim3(1), dim3(1024), lds, s, a, pw, tile);
    return hipGetLastError();
}

}  // namespace strata
