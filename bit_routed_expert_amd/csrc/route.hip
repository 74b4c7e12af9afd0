// Routing of one MoE layer: router logits, ordered top-k with gates, the
// stable per-expert permutation, the expert work list, the miss list of
// non-resident experts, and the fixed-point digit planes of the layer input.
//
// Per-layer routing of 10 of 512 experts (plus one shared expert) per token
// is the model the pages describe (greenbean-ai, "Strata 如何讓 12GB 顯卡跑
// Qwen3.8-Flash-Next？", section 一); the GPU runs the router (same page,
// section 二).  Logits are fp32; top-k is ordered by (logit desc, index asc);
// gates are the softmax renormalised over the k picks.
#include "common.hpp"

namespace strata {

// ----------------------------------------------------------------- top-k
// One wave picks the top-k of E logits (z already scaled and biased) and
// writes ordered ids and gates.  Lane l owns experts l, l+64, ...
__device__ void wave_topk(const float *z, int E, int k, int32_t *idx_out, float *gate_out, int32_t *idx_out2,
                          float *gate_out2) {
    const int lane = threadIdx.x & 63;
    constexpr int JM = 16;  // E <= 1024
    float v[JM];
    uint32_t taken = 0;
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        int e = lane + 64 * j;
        v[j] = (e < E) ? z[e] : -INFINITY;
        if (e >= E) taken |= 1u << j;
    }
    float selz0 = 0.f, myz = 0.f;
    int mye = 0;
    for (int r = 0; r < k; ++r) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            int e = lane + 64 * j;
            bool ok = !((taken >> j) & 1u);
            if (ok && (v[j] > bv || (v[j] == bv && e < be))) { bv = v[j]; be = e; }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            float ov = __shfl_xor(bv, o, WAVE);
            int oe = __shfl_xor(be, o, WAVE);
            if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (r == 0) selz0 = bv;
        if (lane == r) { myz = bv; mye = be; }
    }
    // gates: softmax over the k picks (the all-E normaliser cancels in the renormalisation)
    float p = (lane < k) ? expf(myz - selz0) : 0.f;
    float s = wave_sum(p);
    if (lane < k) {
        float g = p / s;
        idx_out[lane] = mye;
        gate_out[lane] = g;
        if (idx_out2) idx_out2[lane] = mye;
        if (gate_out2) gate_out2[lane] = g;
    }
}

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
        // digit sums per 128-column group (16 consecutive chunks)
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) sx += __shfl_xor(sx, o, WAVE);
        if (valid) {
            int U = c / 4, i = c % 4;
            uint32_t *dst = a.xq + ((size_t)t * (d / 32) + U) * (XPLANES * 4);
#pragma unroll
            for (int p = 0; p < XPLANES; ++p) dst[p * 4 + i] = word[p];
            if ((c & 15) == 0) a.xsum[(size_t)t * (d / 128) + c / 16] = sx;
            if ((c & 31) == 0) a.xscl[(size_t)t * G + c / 32] = ldexpf(1.f, -E);
        }
    }
    (void)red;
}

// Inverse RMS of token t's row (1 when the layer input is not normalised).
__device__ float token_inv_rms(const LayerArgs &a, int t, float *red) {
    if (!a.normalize) return 1.f;
    const int d = a.d, nth = blockDim.x, th = threadIdx.x;
    float ss = 0.f;
    for (int i = th; i < d; i += nth) {
        size_t o = (size_t)t * d + i;
        float xv = a.x_is_bf16 ? bf16_to_float(((const uint16_t *)a.x)[o]) : ((const float *)a.x)[o];
        ss += xv * xv;
    }
    ss = wave_sum(ss);
    __syncthreads();
    if ((th & 63) == 0) red[th >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < nth / 64; ++w) tot += red[w];
    __syncthreads();
    return 1.f / sqrtf(tot / (float)d + RMS_EPS);
}

__device__ __forceinline__ bool is_resident(const uint32_t *mask, int e) {
    return !mask || ((mask[e >> 5] >> (e & 31)) & 1u);
}

// --------------------------------------------- small-T permutation & lists
// One block; T*k <= blockDim.x.  Stable permutation (expert asc, token asc),
// work list (one item per resident expert with picks, then the shared expert
// in items of <= CHUNK_TOK tokens), miss list in (t, r) order.
__device__ void small_permute(const LayerArgs &a, int32_t *lds /* >= 2E+2+blockDim ints */) {
    const int th = threadIdx.x, nth = blockDim.x;
    const int E = a.E, n = a.T * a.k;
    int32_t *hist = lds;           // [E]
    int32_t *offs = lds + E;       // [E+1]
    int32_t *scan = lds + 2 * E + 1;  // [nth]
    for (int e = th; e < E; e += nth) hist[e] = 0;
    __syncthreads();
    int my_e = -1;
    if (th < n) {
        my_e = a.idx[th];
        atomicAdd(&hist[my_e], 1);
    }
    __syncthreads();
    if (th == 0) {
        int acc = 0;
        for (int e = 0; e < E; ++e) { offs[e] = acc; acc += hist[e]; }
        offs[E] = acc;
    }
    __syncthreads();
    for (int e = th; e < E; e += nth) {
        a.counts[e] = hist[e];
        a.offsets[e] = offs[e];
        if (a.u_counts) a.u_counts[e] = hist[e];
        if (a.u_offsets) a.u_offsets[e] = offs[e];
    }
    if (th == 0) {
        a.offsets[E] = offs[E];
        if (a.u_offsets) a.u_offsets[E] = offs[E];
    }
    if (th < n) {
        int t = th / a.k;
        int rank = 0;
        for (int j = 0; j < n; ++j)
            if (j / a.k < t && a.idx[j] == my_e) ++rank;
        int slot = offs[my_e] + rank;
        a.perm[slot] = th;
        a.pos[th] = slot;
        if (a.u_perm) a.u_perm[slot] = th;
        if (a.u_pos) a.u_pos[th] = slot;
    }
    // miss list: exclusive scan of non-resident flags in (t, r) order
    int miss = (th < n && !is_resident(a.mask, my_e)) ? 1 : 0;
    scan[th] = miss;
    __syncthreads();
    if (th == 0) {
        int acc = 0;
        for (int i = 0; i < nth; ++i) { int v = scan[i]; scan[i] = acc; acc += v; }
        if (a.miss_count) *a.miss_count = acc;
    }
    __syncthreads();
    if (miss && a.miss_te) {
        int p = scan[th];
        if (p < a.miss_cap) {
            a.miss_te[2 * p] = th / a.k;
            a.miss_te[2 * p + 1] = my_e;
            a.miss_w[p] = a.gate[th];
        }
    }
    __syncthreads();
    // work list
    if (th == 0) {
        int ni = 0;
        for (int e = 0; e < E; ++e)
            if (hist[e] > 0 && is_resident(a.mask, e)) {
                a.items[ni++] = WorkItem{e, offs[e], hist[e]};
            }
        for (int t0 = 0; t0 < a.T; t0 += CHUNK_TOK)
            a.items[ni++] = WorkItem{E, n + t0, min(CHUNK_TOK, a.T - t0)};
        *a.n_items = ni;
    }
}

// ------------------------------------------------------ decode-size route
// T <= 8.  Every block computes unnormalised logits of 8 experts (two per
// wave) for all T tokens; the last block to arrive scales them by the
// token's inverse RMS, adds the bias, picks the top-k, builds the
// permutation and lists, and writes the input digit planes.
constexpr int RS_EPB = 8;

// LDS floats of route_small: x rows, or logits + reduction scratch, or the
// permutation scratch, plus 4 words for the arrival flag.
__host__ __device__ inline int small_lds_floats(const LayerArgs &a) {
    int n = a.T * a.d;
    n = n > 64 + a.E ? n : 64 + a.E;
    n = n > 2 * a.E + 1 + 256 ? n : 2 * a.E + 1 + 256;
    return n + 4;
}

template <typename K> static void allow_lds(K kernel, size_t bytes) {
    if (bytes > 64 * 1024)
        (void)hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int XBF16>
__global__ __launch_bounds__(256) void route_small_kernel(LayerArgs a) {
    extern __shared__ float lds[];
    const int th = threadIdx.x, lane = th & 63, wave = th >> 6;
    const int d = a.d, T = a.T, E = a.E;
    float *xs = lds;  // [T][d]
    for (int i = th; i < T * d; i += 256)
        xs[i] = XBF16 ? bf16_to_float(((const uint16_t *)a.x)[i]) : ((const float *)a.x)[i];
    __syncthreads();
    for (int j = 0; j < RS_EPB / 4; ++j) {
        int e = blockIdx.x * RS_EPB + wave * (RS_EPB / 4) + j;
        if (e >= E) break;
        const float *w = a.Wr + (size_t)e * d;
        float acc[CHUNK_TOK];
#pragma unroll
        for (int t = 0; t < CHUNK_TOK; ++t) acc[t] = 0.f;
        for (int i = lane * 4; i < d; i += 256) {
            float4 wv = *(const float4 *)(w + i);
#pragma unroll
            for (int t = 0; t < CHUNK_TOK; ++t)
                if (t < T) {
                    const float *xr = xs + t * d + i;
                    acc[t] += wv.x * xr[0] + wv.y * xr[1] + wv.z * xr[2] + wv.w * xr[3];
                }
        }
#pragma unroll
        for (int t = 0; t < CHUNK_TOK; ++t)
            if (t < T) {
                float s = wave_sum(acc[t]);
                if (lane == 0) a.z[t * E + e] = s;
            }
    }
    // arrival: the flag lives just past the largest LDS use
    int &is_last = *(int *)(lds + small_lds_floats(a) - 4);
    __threadfence();
    __syncthreads();
    if (th == 0) is_last = (atomicAdd(a.counter, 1u) == gridDim.x - 1);
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    if (th == 0) *a.counter = 0;

    float *red = lds;  // reuse
    float *zs = lds + 64;  // [E] per token in turn
    for (int t = 0; t < T; ++t) {
        float inv = token_inv_rms(a, t, red);
        if (th == 0) a.inv_rms[t] = inv;
        for (int e = th; e < E; e += 256) {
            float v = a.z[t * E + e] * inv;
            if (a.bias) v += a.bias[e];
            zs[e] = v;
        }
        __syncthreads();
        if (wave == 0)
            wave_topk(zs, E, a.k, a.idx + t * a.k, a.gate + t * a.k, a.u_idx ? a.u_idx + t * a.k : nullptr,
                      a.u_gate ? a.u_gate + t * a.k : nullptr);
        __syncthreads();
        if (!a.route_only) prep_token(a, t, red, inv);
        __syncthreads();
    }
    __threadfence_block();
    small_permute(a, (int32_t *)lds);
}

// -------------------------------------------------------- large-T pieces
// One block of 256 threads per token: inverse RMS and input digit planes.
__global__ __launch_bounds__(256) void prep_x_kernel(LayerArgs a) {
    __shared__ float red[8];
    const int t = blockIdx.x;
    float inv = token_inv_rms(a, t, red);
    if (threadIdx.x == 0) a.inv_rms[t] = inv;
    if (!a.route_only) prep_token(a, t, red, inv);
}

// Router logits z[t][e] = inv_rms[t] * (x[t] . Wr[e]) + bias[e], fp32,
// 64x64 output tile per block, 16x16 threads with 4x4 outputs each.
__global__ __launch_bounds__(256) void route_logits_kernel(LayerArgs a) {
    __shared__ float xs[32][65];
    __shared__ float ws[32][65];
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    const int t0 = blockIdx.y * 64, e0 = blockIdx.x * 64;
    const int d = a.d;
    float acc[4][4] = {};
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
#pragma unroll 8
        for (int c = 0; c < 32; ++c) {
            float xv[4], wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) { xv[i] = xs[c][ty + 16 * i]; wv[i] = ws[c][tx + 16 * i]; }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += xv[i] * wv[j];
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
    wave_topk(a.z + (size_t)t * a.E, a.E, a.k, a.idx + (size_t)t * a.k, a.gate + (size_t)t * a.k,
              a.u_idx ? a.u_idx + (size_t)t * a.k : nullptr, a.u_gate ? a.u_gate + (size_t)t * a.k : nullptr);
}

// Any T: one block of 1024 threads.  Counts by LDS atomics (integer, so the
// result is order independent), exclusive scan, then a stable scatter over
// 512-token windows: within a window each expert's picks are marked in a
// bitmap and a pick's rank is the number of marked earlier tokens.
constexpr int PW = 512;  // tokens per window
__global__ __launch_bounds__(1024) void route_permute_kernel(LayerArgs a) {
    extern __shared__ int32_t sh[];
    const int th = threadIdx.x, nth = 1024;
    const int E = a.E, k = a.k, T = a.T;
    const int64_t n = (int64_t)T * k;
    int32_t *hist = sh;                 // [E]
    int32_t *run = sh + E;              // [E] running slot per expert
    int32_t *scan = sh + 2 * E;         // [1024]
    uint32_t *bm = (uint32_t *)(sh + 2 * E + 1024);  // [E][PW/32]
    constexpr int BW = PW / 32;
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
    // work list: ceil(count/CHUNK_TOK) items per resident expert with picks, then the shared expert
    int ni = (th < E && is_resident(a.mask, th)) ? (hist[th] + CHUNK_TOK - 1) / CHUNK_TOK : 0;
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
            a.items[base + j] = WorkItem{th, s0 + j * CHUNK_TOK, min(CHUNK_TOK, hist[th] - j * CHUNK_TOK)};
    }
    int nr = scan[nth - 1];
    __syncthreads();
    if (th == 0) {
        int c = nr;
        for (int t0 = 0; t0 < T; t0 += CHUNK_TOK)
            a.items[c++] = WorkItem{E, (int32_t)(n + t0), min(CHUNK_TOK, T - t0)};
        *a.n_items = c;
    }
}

// ------------------------------------------------------------- launchers
hipError_t launch_route_small(const LayerArgs &a, hipStream_t s) {
    int blocks = (a.E + RS_EPB - 1) / RS_EPB;
    size_t lds = sizeof(float) * (size_t)small_lds_floats(a);
    if (a.x_is_bf16) {
        allow_lds(route_small_kernel<1>, lds);
        hipLaunchKernelGGL(route_small_kernel<1>, dim3(blocks), dim3(256), lds, s, a);
    } else {
        allow_lds(route_small_kernel<0>, lds);
        hipLaunchKernelGGL(route_small_kernel<0>, dim3(blocks), dim3(256), lds, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_prep_x(const LayerArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(prep_x_kernel, dim3(a.T), dim3(256), 0, s, a);
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

hipError_t launch_route_permute(const LayerArgs &a, hipStream_t s) {
    size_t lds = sizeof(int32_t) * (size_t)(2 * a.E + 1024) + sizeof(uint32_t) * (size_t)a.E * (PW / 32);
    allow_lds(route_permute_kernel, lds);
    hipLaunchKernelGGL(route_permute_kernel, dim3(1), dim3(1024), lds, s, a);
    return hipGetLastError();
}

}  // namespace strata
