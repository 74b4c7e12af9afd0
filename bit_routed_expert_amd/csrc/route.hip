// Routing of one MoE layer: router logits, ordered top-k with gates, the
// stable per-expert permutation, the expert work list, the miss list of
// non-resident experts, and the fixed-point digit planes of the layer input.
//
// Per-layer routing of 10 of 512 experts (plus one shared expert) per token
// is the model the pages describe (greenbean-ai, "Strata 如何讓 12GB 顯卡跑
// Qwen3.8-Flash-Next？", section 一); the GPU runs the router (same page,
// section 二).  Logits are fp32; top-k is ordered by (logit desc, index asc);
// gates are the softmax renormalised over the k picks.
#include <algorithm>

#include "routing.hpp"
#include "mfma.hpp"

namespace strata {

// Every kernel here stays within the 64 KiB of LDS a block gets by default;
// a launch that would need more is refused rather than attempted.
constexpr size_t LDS_LIMIT = 64 * 1024;

// ------------------------------------------------------ input digit planes
// For token t: inverse RMS (or 1) and the digit planes of u = x * inv_rms:
// per 256-column group an exponent E with max|u| * 2^E inside the 4-digit
// range, X = rint(u * 2^E), and its balanced base-16 digits packed 8 columns
// per word (nibble n of word (unit U, plane p, i) = digit p of column 32U+8i+n).
// Runs on one block (any multiple of 64 threads); ld(i) = value i of the
// token's row as fp32.
template <typename Load>
__device__ void prep_token_row(const LayerArgs &a, int t, float inv, Load ld) {
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
            const float xv = valid ? ld(c * 8 + n) : 0.f;
            u[n] = xv * inv;
        }
        float m = 0.f;
#pragma unroll
        for (int n = 0; n < 8; ++n) m = fmaxf(m, fabsf(u[n]));
        // group max over the 32 chunks of a 256-column group (32 consecutive lanes)
        m = fmaxf(m, lane_xor<16>(m));
        m = fmaxf(m, lane_xor<8>(m));
        m = fmaxf(m, lane_xor<4>(m));
        m = fmaxf(m, lane_xor<2>(m));
        m = fmaxf(m, lane_xor<1>(m));
        int E = fixed_point_exponent<XPLANES>(m);
        int X[8];
        int sx = 0;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            X[n] = (int)rintf(ldexpf(u[n], E));
            sx += X[n];
        }
        uint32_t word[XPLANES];
        digit_words(X, word);
        // digit sums per 32-column unit (4 consecutive chunks)
        sx += lane_xor<1>(sx);
        sx += lane_xor<2>(sx);
        if (valid) {
            int U = c / 4, i = c % 4;
            uint32_t *dst = a.xq + ((size_t)t * (d / 32) + U) * (XPLANES * 4);
#pragma unroll
            for (int p = 0; p < XPLANES; ++p) dst[p * 4 + i] = word[p];
            if (i == 0) a.xsum[(size_t)t * (d / 32) + U] = sx;
            if ((c & 31) == 0) a.xscl[(size_t)t * G + c / 32] = ldexpf(1.f, -E);
        }
    }
}
__device__ void prep_token(const LayerArgs &a, int t, float inv) {
    prep_token_row(a, t, inv, [&](int i) { return x_value(a, t, i); });
}


// ------------------------------------------------------ decode-size route
// T <= 8.  Blocks [0, ceil(E/4)): one router row per wave, its loads issued
// before anything else, dotted with the T token rows staged in LDS; the
// unnormalised logits go to z.  Blocks past those: one per token, its
// inverse RMS and (unless routing only) its input digit planes.  The top-k
// is taken afterwards by every consumer block from z (a few KB), so no block
// waits on another inside this kernel.
//
// Order of a dot product x . Wr[e] (route_combine_small_kernel computes the
// same sums one 256-column chunk per block, so a stack of layers gets the
// logits of single-layer calls bit for bit): the columns are cut into
// 256-column chunks; lane s (0..7) of an 8-lane group takes columns
// 32i + 4s .. 32i + 4s + 3 (i = 0..7) of one chunk as one chain of fmas; the
// group's 8 partials are added in pairs, then quads, then halves (DPP, the
// same value in all 8 lanes); the chunk sums are added to 0 in chunk order.
constexpr int RS_WAVES = 4;     // router rows per block
constexpr int RS_CHUNK = 256;   // columns per chunk

template <typename XF>
__device__ __forceinline__ float chunk_part(const float4 (&w)[8], int ni, XF xf) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (i < ni) {
            const float4 x = xf(i);
            acc = fmaf(w[i].x, x.x, acc);
            acc = fmaf(w[i].y, x.y, acc);
            acc = fmaf(w[i].z, x.z, acc);
            acc = fmaf(w[i].w, x.w, acc);
        }
    }
    return acc;
}

__device__ __forceinline__ float group8_sum(float v) {
#define G8_DPP(CTRL) __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false))
    v += G8_DPP(0xB1);    // quad_perm [1,0,3,2]
    v += G8_DPP(0x4E);    // quad_perm [2,3,0,1]
    v += G8_DPP(0x141);   // row_half_mirror: quad 0 <-> quad 1 of each 8 lanes
#undef G8_DPP
    return v;
}

// LDS place of value v of the staged T x d rows: each 128-value block of an
// odd 256-value block is rotated by 32, so the 8 lane groups' 128-byte
// reads of one step fall on both halves of the banks.
__device__ __forceinline__ int xrot(int v) { return (v & ~127) | ((v + ((v >> 3) & 32)) & 127); }

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
        if (!a.route_only) prep_token(a, t, inv);
        return;
    }
    const int e = blockIdx.x * RS_WAVES + wave;
    const float *wrow = a.Wr + (size_t)(e < E ? e : 0) * d;
    const int g = lane >> 3, s4 = 4 * (lane & 7);
    float *xs = lds;  // [T][d], places by xrot
    float zacc[CHUNK_TOK];
#pragma unroll
    for (int t = 0; t < CHUNK_TOK; ++t) zacc[t] = 0.f;
    for (int c0 = 0; c0 < d; c0 += 8 * RS_CHUNK) {
        const int cb = c0 + RS_CHUNK * g;                 // this lane group's chunk
        const int ni = min(8, max(0, (d - cb) / 32));     // its 32-column steps inside d
        float4 wv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            wv[j] = (e < E && j < ni) ? *(const float4 *)(wrow + cb + 32 * j + s4) : make_float4(0.f, 0.f, 0.f, 0.f);
        if (c0 == 0) {
            // the T rows of x into LDS as fp32: 16-byte loads, eight per thread in flight
            constexpr int PER = XBF16 ? 8 : 4;   // values per 16-byte chunk
            const int nch = T * d / PER;
            for (int b = 0; b < nch; b += 8 * 256) {
                uint4 v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int c = b + th + 256 * j;
                    v[j] = c < nch ? ((const uint4 *)a.x)[c] : make_uint4(0u, 0u, 0u, 0u);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int c = b + th + 256 * j;
                    if (c < nch) {
                        const uint32_t q[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
                        if (XBF16) {
                            float4 *dst = (float4 *)(xs + xrot(8 * c));
                            dst[0] = make_float4(__uint_as_float(q[0] << 16), __uint_as_float(q[0] & 0xFFFF0000u),
                                                 __uint_as_float(q[1] << 16), __uint_as_float(q[1] & 0xFFFF0000u));
                            dst[1] = make_float4(__uint_as_float(q[2] << 16), __uint_as_float(q[2] & 0xFFFF0000u),
                                                 __uint_as_float(q[3] << 16), __uint_as_float(q[3] & 0xFFFF0000u));
                        } else {
                            *(float4 *)(xs + xrot(4 * c)) = make_float4(__uint_as_float(q[0]), __uint_as_float(q[1]),
                                                                        __uint_as_float(q[2]), __uint_as_float(q[3]));
                        }
                    }
                }
            }
            __syncthreads();
        }
        const int nch = min(8, (d - c0 + RS_CHUNK - 1) / RS_CHUNK);   // chunks of this pass
#pragma unroll
        for (int t = 0; t < CHUNK_TOK; ++t) {
            if (t < T) {
                const int rb = t * d + cb + s4;
                float p = chunk_part(wv, ni, [&](int i) { return *(const float4 *)(xs + xrot(rb + 32 * i)); });
                p = group8_sum(p);
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    if (c < nch)
                        zacc[t] += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), 8 * c));
            }
        }
    }
    if (lane == 0 && e < E) {
#pragma unroll
        for (int t = 0; t < CHUNK_TOK; ++t)
            if (t < T) a.z[t * E + e] = zacc[t];
    }
}

// ------------------------------------- decode-size route after a layer
// T <= 8, a layer after the first of a stack: the previous layer's combine
// and this layer's router in one kernel (the combine kernel's launch and
// the round trip of x through memory go).  Blocks [0, nr * ng): chunk c of
// router rows 64q .. 64q+63 (c = block mod nr, so the blocks of one chunk
// share an XCD): the chunk of every token's row x = x_prev + out_prev is
// formed in LDS exactly as combine_kernel forms it, then each wave dots 8
// router rows with it (one per 8-lane group, lanes as in
// route_logits_small_kernel) and writes the chunk sums as plane c of z.
// Blocks past those: one per token, its whole row x (also written to
// x_cur), its inverse RMS over 256 threads and its digit planes.
constexpr int RC_ROWS = 64;   // router rows per block: 8 waves x 8 lane groups

// x_prev + out_prev at columns i .. i+3 of token t, as combine_kernel
// forms them from rows in token order: the shared expert's row, then
// gate * row t*k + r of each resident pick in r order (fma), added to x.
// Every load is independent of the others (one round trip).
template <int PXBF16>
__device__ __forceinline__ float4 combine_x(const LayerArgs &a, int t, int i) {
    const int d = a.d, k = a.k;
    const float *__restrict__ Y = a.Y;
    float4 s = *(const float4 *)(Y + ((int64_t)a.T * k + t) * d + i);
    const uint32_t rb = a.pmask ? (uint32_t)a.rbits[t] : 0xFFFFFFFFu;
    for (int r0 = 0; r0 < k; r0 += 16) {
        float gr[16];
        float4 yv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const bool on = r0 + r < k && ((rb >> (r0 + r)) & 1u);
            gr[r] = on ? a.gate[t * k + r0 + r] : 0.f;
            yv[r] = on ? *(const float4 *)(Y + (int64_t)(t * k + r0 + r) * d + i) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (r0 + r < k && ((rb >> (r0 + r)) & 1u)) combine_acc(s, gr[r], yv[r]);
    }
    const int64_t row = (int64_t)t * d + i;
    float4 xv;
    if (PXBF16) {
        const uint2 q = *(const uint2 *)((const uint16_t *)a.px + row);
        xv = make_float4(__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xFFFF0000u),
                         __uint_as_float(q.y << 16), __uint_as_float(q.y & 0xFFFF0000u));
    } else {
        xv = *(const float4 *)((const float *)a.px + row);
    }
    return make_float4(xv.x + s.x, xv.y + s.y, xv.z + s.z, xv.w + s.w);
}

template <int PXBF16>
__global__ __launch_bounds__(512) void route_combine_small_kernel(LayerArgs a) {
    extern __shared__ float lds[];
    const int th = threadIdx.x, lane = th & 63, wave = th >> 6;
    const int d = a.d, T = a.T, E = a.E;
    const int nr = (d + RS_CHUNK - 1) / RS_CHUNK, ng = (E + RC_ROWS - 1) / RC_ROWS;
    float *xs = lds;   // router blocks: [T][256]; token blocks: [d] + 4 floats
    const bool router = (int)blockIdx.x < nr * ng;
    const int c = (int)blockIdx.x % nr;
    const int g = lane >> 3, s4 = 4 * (lane & 7);
    const int e = ((int)blockIdx.x / nr) * RC_ROWS + 8 * wave + g;
    const int cb = RS_CHUNK * c;
    const int ni = min(8, max(0, (d - cb) / 32));
    if (router) {
        float4 wv[8];
        const float *wrow = a.Wr + (size_t)(e < E ? e : 0) * d;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            wv[j] = (e < E && j < ni) ? *(const float4 *)(wrow + cb + 32 * j + s4) : make_float4(0.f, 0.f, 0.f, 0.f);
        const int w4 = min(RS_CHUNK / 4, (d - cb) / 4);   // float4 columns of this chunk inside d
        for (int u = th; u < T * (RS_CHUNK / 4); u += blockDim.x) {
            const int t = u / (RS_CHUNK / 4), q4 = u % (RS_CHUNK / 4);
            if (q4 < w4) *(float4 *)(xs + RS_CHUNK * t + 4 * q4) = combine_x<PXBF16>(a, t, cb + 4 * q4);
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < CHUNK_TOK; ++t) {
            if (t < T) {
                const float *xr = xs + RS_CHUNK * t + s4;
                float p = chunk_part(wv, ni, [&](int i) { return *(const float4 *)(xr + 32 * i); });
                p = group8_sum(p);
                if ((lane & 7) == 0 && e < E) a.z[((size_t)c * T + t) * E + e] = p;
            }
        }
    } else {
        const int t = (int)blockIdx.x - nr * ng;
        for (int u = th; u < d / 4; u += blockDim.x) {
            const float4 v = combine_x<PXBF16>(a, t, 4 * u);
            *(float4 *)(xs + 4 * u) = v;
            *(float4 *)(a.x_cur + (size_t)t * d + 4 * u) = v;
        }
        __syncthreads();
        const float inv = row_inv_rms(d, a.normalize, xs + d, 256, [&](int i) { return xs[i]; });
        if (th == 0) a.inv_rms[t] = inv;
        prep_token_row(a, t, inv, [&](int i) { return xs[i]; });
    }
}

// Routing only, T <= 8: one block takes the top-k and writes every output.
__global__ __launch_bounds__(256) void route_small_finish_kernel(LayerArgs a) {
    extern __shared__ uint32_t lds_u[];
    const SmallRoute L(lds_u, a.E);
    small_route_compute(a, L, a.z, a.inv_rms);
    small_route_write(a, L);
}

// Router dot products x[t] . Wr[e] on the bf16 matrix cores (the logit is
// inv_rms[t] times this plus bias[e], formed by the top-k kernel).  Wr (fp32)
// is split into three exact bf16 pieces as it is staged into LDS; x is one
// piece when it is bf16, else three (products
// of pieces below 2^-32 of the leading one are dropped).  Every product is
// exact in fp32; each 256-column block is summed on its own and the block
// sums are added in order.  The columns are cut into zsplit equal ranges of
// whole blocks (grid z), each written as its own partial plane of z, so the
// grid has enough blocks to hide memory latency; the top-k kernel adds the
// planes in order.  Block tile 256 tokens x 64 experts (8 waves, so each
// staged and split Wr tile feeds 256 tokens); wave w owns tokens 32*w .. +32
// against all 64 experts (two 32x32 MFMA tiles).
constexpr int RT_T = 256, RT_E = 64, RT_K = 32, RT_RS = RT_K + 8;   // LDS row: 32 bf16 + 16 B pad
constexpr int RT_THREADS = 2 * RT_T;                                 // two threads stage each x row
constexpr int RT_WC = RT_K * RT_E / RT_THREADS;                      // Wr columns staged per thread (4)

template <int PX>
__global__ __launch_bounds__(RT_THREADS, PX == 1 ? 4 : 2) void route_logits_mfma_kernel(LayerArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[PX][RT_T * RT_RS];
    __shared__ __attribute__((aligned(16))) uint16_t ws[3][RT_E * RT_RS];
    const int th = threadIdx.x, lane = th & 63, wv = th >> 6;
    const int n = lane & 31, h = lane >> 5;
    // Blocks are dealt to the 8 XCDs round-robin by linear index; renumber
    // them so that XCD c runs the c-th eighth of the (expert block fastest,
    // then token block, then column range) order: the expert blocks sharing a
    // token tile share that XCD's L2, and so do the token blocks of one column
    // range of the router pieces.
    const int nbx = gridDim.x, nby = gridDim.y, nb = nbx * nby * gridDim.z;
    const int id = blockIdx.x + nbx * (blockIdx.y + nby * blockIdx.z);
    const int li = (nb % 8 == 0) ? (id % 8) * (nb / 8) + id / 8 : id;
    const int bx = li % nbx, by = (li / nbx) % nby, bz = li / (nbx * nby);
    const int t0 = by * RT_T, e0 = bx * RT_E;
    const int d = a.d, T = a.T, E = a.E;
    const int kspan = d / a.zsplit, kbeg = bz * kspan, kend = kbeg + kspan;
    // staging: x rows th/2 (16 columns each), Wr rows th/8 (4 columns each)
    const int xr = th >> 1, xc = (th & 1) * 16;
    const int wr = th / (RT_K / RT_WC), wc = (th % (RT_K / RT_WC)) * RT_WC;
    const int64_t xoff = (int64_t)min(t0 + xr, T - 1) * d + xc;
    const int64_t woff = (int64_t)min(e0 + wr, E - 1) * d + wc;
    const bool wvalid = e0 + wr < E;
    float xv[16];
    float4 wf;      // 4 columns of this thread's Wr row (fp32)
    auto load = [&](int k0) __attribute__((always_inline)) {
        if (a.x_is_bf16) {
            const uint4 *p = (const uint4 *)((const uint16_t *)a.x + xoff + k0);
            const uint4 q0 = p[0], q1 = p[1];
            const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                xv[2 * j] = __uint_as_float(w[j] << 16);
                xv[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
            }
        } else {
            const float4 *p = (const float4 *)((const float *)a.x + xoff + k0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 q = p[j];
                xv[4 * j] = q.x; xv[4 * j + 1] = q.y; xv[4 * j + 2] = q.z; xv[4 * j + 3] = q.w;
            }
        }
        wf = *(const float4 *)(a.Wr + woff + k0);
    };
    f32x16_t P[2], acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) P[j][v] = acc[j][v] = 0.f;
    load(kbeg);
    for (int k0 = kbeg; k0 < kend; k0 += RT_K) {
        __syncthreads();
        {   // pieces into LDS: Wr = hi + mid + lo exactly, two columns packed per word
            const float w[4] = {wf.x, wf.y, wf.z, wf.w};
            uint32_t u[3][2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                uint16_t a0, b0, c0, a1, b1, c1;
                split3(w[2 * j], a0, b0, c0);
                split3(w[2 * j + 1], a1, b1, c1);
                u[0][j] = wvalid ? ((uint32_t)a0 | ((uint32_t)a1 << 16)) : 0u;
                u[1][j] = wvalid ? ((uint32_t)b0 | ((uint32_t)b1 << 16)) : 0u;
                u[2][j] = wvalid ? ((uint32_t)c0 | ((uint32_t)c1 << 16)) : 0u;
            }
#pragma unroll
            for (int q = 0; q < 3; ++q) *(uint2 *)(ws[q] + wr * RT_RS + wc) = make_uint2(u[q][0], u[q][1]);
            uint16_t hx[PX][16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (PX == 1) hx[0][j] = (uint16_t)(__float_as_uint(xv[j]) >> 16);
                else split3(xv[j], hx[0][j], hx[PX > 1 ? 1 : 0][j], hx[PX > 2 ? 2 : 0][j]);
            }
#pragma unroll
            for (int p = 0; p < PX; ++p) {
                uint32_t w[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) w[j] = (uint32_t)hx[p][2 * j] | ((uint32_t)hx[p][2 * j + 1] << 16);
                uint4 *dst = (uint4 *)(xs[p] + xr * RT_RS + xc);
                dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
                dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
            }
        }
        __syncthreads();
        if (k0 + RT_K < kend) load(k0 + RT_K);
#pragma unroll
        for (int kk = 0; kk < RT_K; kk += 16) {
            bf16x8_t A[PX], B[2][3];
#pragma unroll
            for (int p = 0; p < PX; ++p)
                A[p] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(xs[p] + (wv * 32 + n) * RT_RS + kk + 8 * h));
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 3; ++q)
                    B[j][q] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(ws[q] + (j * 32 + n) * RT_RS + kk + 8 * h));
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                P[j] = mfma(A[0], B[j][0], P[j]);
                P[j] = mfma(A[0], B[j][1], P[j]);
                P[j] = mfma(A[0], B[j][2], P[j]);
                if (PX == 3) {
                    P[j] = mfma(A[PX > 1 ? 1 : 0], B[j][0], P[j]);
                    P[j] = mfma(A[PX > 1 ? 1 : 0], B[j][1], P[j]);
                    P[j] = mfma(A[PX > 2 ? 2 : 0], B[j][0], P[j]);
                }
            }
        }
        if (((k0 + RT_K) & 255) == 0 || k0 + RT_K >= kend) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    acc[j][v] += P[j][v];
                    P[j][v] = 0.f;
                }
        }
    }
    float *zp = a.z + (int64_t)bz * T * E;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = e0 + j * 32 + n;
        if (e >= E) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int t = t0 + wv * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
            if (t < T) zp[(int64_t)t * E + e] = acc[j][v];
        }
    }
}

// One wave per token: the partial planes of z added in order into LDS, then
// the logits inv_rms[t] * z + bias and their top-k.
__global__ __launch_bounds__(256) void route_topk_kernel(LayerArgs a) {
    __shared__ float zrow[4][1024];
    __shared__ __attribute__((aligned(16))) uint32_t cand[4][TOPK_LDS_WORDS];
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (t >= a.T) return;
    const int E = a.E, ns = a.zsplit;
    float *zr = zrow[threadIdx.x >> 6];
    // every load of the token's planes issued before the first add (E <= 1024, at most 4 planes)
    float v[4][16];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int e = lane + 64 * j;
            v[q][j] = (q < ns && e < E) ? a.z[((size_t)q * a.T + t) * E + e] : 0.f;
        }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int e = lane + 64 * j;
        float acc = v[0][j];
#pragma unroll
        for (int q = 1; q < 4; ++q)
            if (q < ns) acc += v[q][j];
        if (e < E) zr[e] = acc;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // the row is read back by other lanes
    wave_topk(zr, E, a.k, a.inv_rms[t], a.bias, cand[threadIdx.x >> 6], a.idx + (size_t)t * a.k,
              a.gate + (size_t)t * a.k, a.u_idx ? a.u_idx + (size_t)t * a.k : nullptr,
              a.u_gate ? a.u_gate + (size_t)t * a.k : nullptr, nullptr, nullptr);
}

// ------------------------------------------------ permutation (larger T)
// Slots are ordered by (expert asc, token asc): three passes over blocks
// of PERM_T tokens.  route_count: per-block expert histogram and miss
// count; route_scan: totals, offsets, each block's first slot per expert,
// each block's first miss-list entry, and the work list; route_scatter:
// the stable rank of every pick inside its block (per-expert token
// bitmaps), perm/pos and the miss list in (t, r) order.
constexpr int PERM_T = 64;

__global__ __launch_bounds__(256) void route_count_kernel(LayerArgs a) {
    __shared__ int hist[1024];
    __shared__ int tmp[16];
    const int th = threadIdx.x, b = blockIdx.x, E = a.E, k = a.k;
    const int t0 = b * PERM_T, nt = min(PERM_T, a.T - t0);
    for (int e = th; e < E; e += 256) hist[e] = 0;
    __syncthreads();
    int nmiss = 0;
    for (int i = th; i < nt * k; i += 256) {
        const int e = a.idx[(int64_t)t0 * k + i];
        atomicAdd(&hist[e], 1);
        nmiss += is_resident(a.mask, e) ? 0 : 1;
    }
    __syncthreads();
    for (int e = th; e < E; e += 256) a.bcnt[(int64_t)b * E + e] = hist[e];
    int tot = 0;
    if (a.mask) block_excl_scan(nmiss, tmp, &tot);
    if (th == 0) a.bmiss[b] = tot;
}

__global__ __launch_bounds__(1024) void route_scan_kernel(LayerArgs a, int nb, int tile) {
    __shared__ int tmp[16];
    const int th = threadIdx.x, E = a.E, T = a.T;
    const int64_t n = (int64_t)T * a.k;
    // up to SCAN_REG count blocks (T <= 4096): every count is requested at
    // once and kept in registers for the rewrite below (one memory round trip)
    constexpr int SCAN_REG = 64;
    const bool inreg = nb <= SCAN_REG;
    int v[SCAN_REG];
    int c = 0;
    if (th < E) {
        if (inreg) {
#pragma unroll
            for (int b = 0; b < SCAN_REG; ++b) v[b] = b < nb ? a.bcnt[(int64_t)b * E + th] : 0;
#pragma unroll
            for (int b = 0; b < SCAN_REG; ++b) c += v[b];
        } else {
#pragma unroll 16
            for (int b = 0; b < nb; ++b) c += a.bcnt[(int64_t)b * E + th];
        }
    }
    int tot;
    const int off = block_excl_scan(c, tmp, &tot);
    if (th < E) {
        a.counts[th] = c;
        a.offsets[th] = off;
        if (a.u_counts) a.u_counts[th] = c;
        if (a.u_offsets) a.u_offsets[th] = off;
        int run = off;   // in place: count -> first slot of the block
        if (inreg) {
#pragma unroll
            for (int b = 0; b < SCAN_REG; ++b) {
                if (b < nb) a.bcnt[(int64_t)b * E + th] = run;
                run += v[b];
            }
        } else {
#pragma unroll 8
            for (int b = 0; b < nb; ++b) {
                const int cb = a.bcnt[(int64_t)b * E + th];
                a.bcnt[(int64_t)b * E + th] = run;
                run += cb;
            }
        }
    }
    if (th == 0) {
        a.offsets[E] = (int32_t)n;
        if (a.u_offsets) a.u_offsets[E] = (int32_t)n;
    }
    // first miss-list entry of every block
    int mbase = 0;
    for (int b0 = 0; b0 < nb; b0 += 1024) {
        const int b = b0 + th;
        const int v = b < nb ? a.bmiss[b] : 0;
        int sum;
        const int ex = block_excl_scan(v, tmp, &sum);
        __syncthreads();
        if (b < nb) a.bmiss[b] = mbase + ex;
        mbase += sum;
    }
    if (th == 0 && a.miss_count) *a.miss_count = mbase;
    // work list: ceil(count/tile) items per resident expert with picks, then the shared expert
    const int ni = (th < E && is_resident(a.mask, th)) ? (c + tile - 1) / tile : 0;
    int nr;
    const int base = block_excl_scan(ni, tmp, &nr);
    for (int j = 0; j < ni; ++j) a.items[base + j] = WorkItem{th, off + j * tile, min(tile, c - j * tile)};
    const int ns = (T + tile - 1) / tile;
    for (int j = th; j < ns; j += 1024)
        a.items[nr + j] = WorkItem{E, (int32_t)(n + (int64_t)j * tile), min(tile, T - j * tile)};
    if (th == 0) *a.n_items = nr + ns;
}

__global__ __launch_bounds__(256) void route_scatter_kernel(LayerArgs a) {
    extern __shared__ uint32_t lds_u[];
    constexpr int BW = PERM_T / 32;
    const int th = threadIdx.x, b = blockIdx.x, E = a.E, k = a.k;
    uint32_t *bm = lds_u;                           // [E][BW] token bitmaps
    int *base = (int *)(lds_u + E * BW);            // [E] first slot of this block
    int *tmp = base + E;                            // [16]
    const int t0 = b * PERM_T, nt = min(PERM_T, a.T - t0);
    for (int i = th; i < E * BW; i += 256) bm[i] = 0;
    for (int e = th; e < E; e += 256) base[e] = a.bcnt[(int64_t)b * E + e];
    __syncthreads();
    const int64_t g0 = (int64_t)t0 * k;
    for (int i = th; i < nt * k; i += 256) {
        const int tl = i / k, e = a.idx[g0 + i];
        atomicOr(&bm[e * BW + (tl >> 5)], 1u << (tl & 31));
    }
    __syncthreads();
    for (int i = th; i < nt * k; i += 256) {
        const int tl = i / k, e = a.idx[g0 + i];
        int rank = __popc(bm[e * BW + (tl >> 5)] & ((1u << (tl & 31)) - 1u));
        for (int w = 0; w < (tl >> 5); ++w) rank += __popc(bm[e * BW + w]);
        const int slot = base[e] + rank;
        a.perm[slot] = (int32_t)(g0 + i);
        a.pos[g0 + i] = slot;
        if (a.u_perm) a.u_perm[slot] = (int32_t)(g0 + i);
        if (a.u_pos) a.u_pos[g0 + i] = slot;
    }
    // miss list entries of this block, in pick order (t asc, r asc)
    if (!a.mask) return;
    int mrun = a.bmiss[b];
    for (int i0 = 0; i0 < nt * k; i0 += 256) {
        const int i = i0 + th;
        const int e = i < nt * k ? a.idx[g0 + i] : 0;
        const int f = (i < nt * k && !is_resident(a.mask, e)) ? 1 : 0;
        int sum;
        const int p = mrun + block_excl_scan(f, tmp, &sum);
        if (f && a.miss_te && p < a.miss_cap) {
            a.miss_te[2 * (int64_t)p] = (int32_t)((g0 + i) / k);
            a.miss_te[2 * (int64_t)p + 1] = e;
            a.miss_w[p] = a.gate[g0 + i];
        }
        mrun += sum;
        __syncthreads();
    }
}

// ------------------------------------------------------------- launchers
hipError_t launch_route_logits_small(const LayerArgs &a, hipStream_t s) {
    const int blocks = (a.E + RS_WAVES - 1) / RS_WAVES + a.T;
    const size_t lds = sizeof(float) * (size_t)a.T * a.d;
    if (lds > LDS_LIMIT) return hipErrorInvalidValue;
    if (a.x_is_bf16)
        STRATA_LAUNCH(route_logits_small_kernel<1>, dim3(blocks), dim3(256), lds, s, a);
    else
        STRATA_LAUNCH(route_logits_small_kernel<0>, dim3(blocks), dim3(256), lds, s, a);
    return hipGetLastError();
}

int route_logit_planes(int d) { return (d + RS_CHUNK - 1) / RS_CHUNK; }

hipError_t launch_route_combine_small(const LayerArgs &a, hipStream_t s) {
    const int nr = route_logit_planes(a.d), ng = (a.E + RC_ROWS - 1) / RC_ROWS;
    const size_t lds = sizeof(float) * std::max((size_t)a.T * RS_CHUNK, (size_t)a.d + 4);
    if (lds > LDS_LIMIT || a.T > CHUNK_TOK || a.k > 32 || !a.px || !a.x_cur || a.zplanes != nr || !a.ytok)
        return hipErrorInvalidValue;
    if (a.px_is_bf16)
        STRATA_LAUNCH(route_combine_small_kernel<1>, dim3(nr * ng + a.T), dim3(512), lds, s, a);
    else
        STRATA_LAUNCH(route_combine_small_kernel<0>, dim3(nr * ng + a.T), dim3(512), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_route_small_finish(const LayerArgs &a, hipStream_t s) {
    const size_t lds = 4 * (size_t)small_route_lds_words(a.E);
    if (lds > LDS_LIMIT) return hipErrorInvalidValue;
    STRATA_LAUNCH(route_small_finish_kernel, dim3(1), dim3(256), lds, s, a);
    return hipGetLastError();
}

// Column ranges of the larger-T router: up to 4, each a whole number of 256-column blocks.
int route_logit_splits(int d) {
    int ks = 4;
    while (ks > 1 && d % (ks * 256)) ks >>= 1;
    return ks;
}

hipError_t launch_route_logits(const LayerArgs &a, hipStream_t s) {
    const dim3 grid((a.E + RT_E - 1) / RT_E, (a.T + RT_T - 1) / RT_T, a.zsplit);
    if (a.d % RT_K || a.zsplit < 1 || a.d % a.zsplit || (a.d / a.zsplit) % RT_K || a.E > 1024) return hipErrorInvalidValue;
    if (a.x_is_bf16)
        STRATA_LAUNCH(route_logits_mfma_kernel<1>, grid, dim3(RT_THREADS), 0, s, a);
    else
        STRATA_LAUNCH(route_logits_mfma_kernel<3>, grid, dim3(RT_THREADS), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_route_topk(const LayerArgs &a, hipStream_t s) {
    if (a.E > 1024 || a.zsplit < 1 || a.zsplit > 4) return hipErrorInvalidValue;
    STRATA_LAUNCH(route_topk_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a);
    return hipGetLastError();
}

int route_perm_blocks(int T) { return (T + PERM_T - 1) / PERM_T; }

hipError_t launch_route_permute(const LayerArgs &a, int tile, hipStream_t s) {
    const int nb = route_perm_blocks(a.T);
    if (a.E > 1024) return hipErrorInvalidValue;
    const size_t lds = 4 * ((size_t)a.E * (PERM_T / 32) + a.E + 16);
    if (lds > LDS_LIMIT) return hipErrorInvalidValue;
    STRATA_LAUNCH(route_count_kernel, dim3(nb), dim3(256), 0, s, a);
    STRATA_LAUNCH(route_scan_kernel, dim3(1), dim3(1024), 0, s, a, nb, tile);
    STRATA_LAUNCH(route_scatter_kernel, dim3(nb), dim3(256), lds, s, a);
    return hipGetLastError();
}

}  // namespace strata
