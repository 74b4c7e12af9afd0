// Device helpers and the internal launch interface of the MoE layer library.
// gfx950 only (64-wide wavefronts).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "strata_moe.h"

namespace strata {

constexpr int WAVE = 64;
constexpr int CHUNK_TOK = 8;      // most tokens a GEMV-path kernel call takes
constexpr int ITEM_TOK = 2;       // tokens one GEMV-path work item carries (an expert's slots in pairs)
constexpr int XPLANES = 6;        // base-16 digit planes of an activation (24-bit fixed point)
constexpr int GEMM_BM = 96;       // tokens per expert tile (GEMM path)
constexpr int GEMM_MAX_K = 4096;  // largest d and f the GEMM path stages
constexpr float RMS_EPS = 1e-6f;

// Largest |X| that P balanced base-16 digits in [-8, 7] represent symmetrically:
// 7 * (16^P - 1) / 15.
__host__ __device__ constexpr int digit_limit(int P) {
    int s = 0, m = 1;
    for (int i = 0; i < P; ++i) { s += m; m *= 16; }
    return 7 * s;
}

__device__ __forceinline__ float half_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float bf16_to_float(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// The value of a 32-bit v in lane (lane ^ O), O a power of two up to 32,
// without the LDS crossbar: DPP inside 16-lane rows (quad permutes for 1
// and 2, the two 4-lane banks swapped by masked row shifts for 4, a row
// rotation by 8 for 8) and the gfx950 row / half swaps for 16 and 32.  The
// same partner as __shfl_xor(v, O), so sums and maxima keep their bits.
template <int O> __device__ __forceinline__ int lane_xor(int v) {
    static_assert(O == 1 || O == 2 || O == 4 || O == 8 || O == 16 || O == 32, "lane_xor: O");
    if constexpr (O == 1) {
        return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    } else if constexpr (O == 2) {
        return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    } else if constexpr (O == 4) {
        const int up = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xA, false);   // row_shr:4 into banks 1, 3
        return __builtin_amdgcn_update_dpp(up, v, 0x104, 0xF, 0x5, false);          // row_shl:4 into banks 0, 2
    } else if constexpr (O == 8) {
        return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
    } else if constexpr (O == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);   // [0]: even rows twice, [1]: odd
        return (threadIdx.x & 16) ? (int)r[0] : (int)r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);   // [0]: low half twice, [1]: high
        return (threadIdx.x & 32) ? (int)r[0] : (int)r[1];
    }
}
template <int O> __device__ __forceinline__ float lane_xor(float v) {
    return __builtin_bit_cast(float, lane_xor<O>(__builtin_bit_cast(int, v)));
}

// The value in lane + 4 (inside each 16-lane row; lanes 12..15 get 0).
__device__ __forceinline__ float lane_down4(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x104, 0xF, 0xF, false));
}

template <typename T> __device__ __forceinline__ T wave_sum(T v) {
    v += lane_xor<32>(v);
    v += lane_xor<16>(v);
    v += lane_xor<8>(v);
    v += lane_xor<4>(v);
    v += lane_xor<2>(v);
    v += lane_xor<1>(v);
    return v;
}
// Sum over the wave by DPP (no LDS round trips): row sums by quad permutes
// and row rotations, then row 0 into row 1, row 2 into row 3, and lane 31
// into rows 2 and 3; the total is complete in lanes 48..63.
__device__ __forceinline__ float wave_sum_dpp(float v) {
#define WS_DPP(CTRL, ROWS) __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false))
    v += WS_DPP(0xB1, 0xF);    // quad_perm [1,0,3,2]
    v += WS_DPP(0x4E, 0xF);    // quad_perm [2,3,0,1]
    v += WS_DPP(0x124, 0xF);   // row_ror:4
    v += WS_DPP(0x128, 0xF);   // row_ror:8
    v += WS_DPP(0x142, 0xA);   // row_bcast:15 into rows 1 and 3
    v += WS_DPP(0x143, 0xC);   // row_bcast:31 into rows 2 and 3
#undef WS_DPP
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, lane_xor<32>(v));
    v = fmaxf(v, lane_xor<16>(v));
    v = fmaxf(v, lane_xor<8>(v));
    v = fmaxf(v, lane_xor<4>(v));
    v = fmaxf(v, lane_xor<2>(v));
    v = fmaxf(v, lane_xor<1>(v));
    return v;
}

// Exponent E such that max_abs * 2^E fits the P-digit range, as large as possible.
template <int P> __device__ __forceinline__ int fixed_point_exponent(float max_abs) {
    if (!(max_abs > 0.f)) return 0;
    int e;
    frexpf(max_abs, &e);              // max_abs < 2^e
    int E = 4 * P - 1 - e;            // max_abs * 2^E < 2^(4P-1)
    if (ldexpf(max_abs, E) > (float)digit_limit(P)) E -= 1;
    return E;
}

// Digit-plane words of 8 fixed-point values X[n] (|X| <= digit_limit(6)):
// word[p] nibble n = balanced digit p of X[n] as a signed 4-bit field.
// Y = X + 0x888888 has plain base-16 digits d_p + 8, so each field is
// nibble p of Y xor 8; the nibbles are moved into place with byte permutes.
__device__ __forceinline__ void digit_words(const int X[8], uint32_t word[6]) {
    uint32_t ev[4], od[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t y0 = (uint32_t)(X[2 * q] + 0x888888), y1 = (uint32_t)(X[2 * q + 1] + 0x888888);
        ev[q] = (y0 & 0x0F0F0Fu) | ((y1 & 0x0F0F0Fu) << 4);          // byte b: nibble 2b of values 2q, 2q+1
        od[q] = ((y0 >> 4) & 0x0F0F0Fu) | (((y1 >> 4) & 0x0F0F0Fu) << 4);
    }
#pragma unroll
    for (int b = 0; b < 3; ++b) {
        const uint32_t lo_sel = (uint32_t)b | ((uint32_t)(b + 4) << 8) | 0x0C0C0000u;
        const uint32_t hi_sel = 0x00000C0Cu | ((uint32_t)b << 16) | ((uint32_t)(b + 4) << 24);
        word[2 * b] = (__builtin_amdgcn_perm(ev[1], ev[0], lo_sel) | __builtin_amdgcn_perm(ev[3], ev[2], hi_sel)) ^
                      0x88888888u;
        word[2 * b + 1] =
            (__builtin_amdgcn_perm(od[1], od[0], lo_sel) | __builtin_amdgcn_perm(od[3], od[2], hi_sel)) ^ 0x88888888u;
    }
}

// 1 / sqrt(mean(x^2) + eps) of one row of d values (1 when the layer does
// not normalise), ld(i) = value i of the row.  Threads 0..nth-1 of the
// block (nth <= blockDim.x, a multiple of 64) accumulate, all threads take
// the barriers; red = LDS scratch of nth/64 floats.  The result depends on
// nth, not on the block size or on where the row is read from.
template <typename Load>
__device__ float row_inv_rms(int d, int normalize, float *red, int nth, Load ld) {
    if (!normalize) return 1.f;
    const int th = threadIdx.x;
    float ss = 0.f;
    if (th < nth) {
        for (int i0 = 0; i0 < d; i0 += 8 * nth) {  // 8 independent loads in flight per pass
            float xv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) xv[j] = ld(min(i0 + th + j * nth, d - 1));
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float v = (i0 + th + j * nth < d) ? xv[j] : 0.f;
                ss = fmaf(v, v, ss);
            }
        }
    }
    ss = wave_sum(ss);
    __syncthreads();
    if ((th & 63) == 0 && th < nth) red[th >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < nth / 64; ++w) tot += red[w];
    __syncthreads();
    return 1.f / sqrtf(tot / (float)d + RMS_EPS);
}

// Value i of token t's layer input as fp32.
template <typename Args> __device__ __forceinline__ float x_value(const Args &a, int t, int i) {
    const size_t o = (size_t)t * a.d + i;
    return a.x_is_bf16 ? bf16_to_float(((const uint16_t *)a.x)[o]) : ((const float *)a.x)[o];
}

// Inverse RMS of token t's layer input, over the whole block.
template <typename Args>
__device__ float token_inv_rms(const Args &a, int t, float *red) {
    return row_inv_rms(a.d, a.normalize, red, (int)blockDim.x, [&](int i) { return x_value(a, t, i); });
}

// silu(g) * u = g / (1 + e^-g) * u with the hardware 2^x and reciprocal
// (about 1 ulp each), the same expression in every expert kernel.
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g)) * u;
}

// Combine step of one pick: s += g * y, component by component (fma).
__device__ __forceinline__ void combine_acc(float4 &s, float g, const float4 &y) {
    s.x = fmaf(g, y.x, s.x);
    s.y = fmaf(g, y.y, s.y);
    s.z = fmaf(g, y.z, s.z);
    s.w = fmaf(g, y.w, s.w);
}

// Work item of the expert kernels: consecutive slots of one expert (up to
// ITEM_TOK on the GEMV path, GEMM_BM on the GEMM path).
struct WorkItem {
    int32_t expert;     // 0..E-1 routed, E shared
    int32_t slot0;      // first slot; slots slot0 .. slot0+ntok-1
    int32_t ntok;
};

// Everything the kernels of one layer call need; device pointers.
struct LayerArgs {
    // shape
    int E, k, d, f, bits, T;
    // layer data
    const float *Wr;
    const float *bias;
    const uint8_t *codes;
    const uint16_t *scales;
    const uint32_t *mask;
    // input of this layer: residual stream x (bf16 or fp32) and whether to normalise it
    const void *x;
    int x_is_bf16;
    int normalize;
    // routing state (internal)
    float *z;            // [T][E] logits; larger T: [zsplit][T][E] partial sums over column ranges
    int zsplit;          // column ranges of the larger-T router (1 on the decode path)
    int zplanes;         // decode path: planes [zplanes][T][E] of z, added in order (1, or one per 256 columns)
    int32_t *idx;        // [T][k]
    float *gate;         // [T][k]
    int32_t *counts;     // [E]
    int32_t *offsets;    // [E+1]
    int32_t *perm;       // [T*k]
    int32_t *pos;        // [T*k]
    float *inv_rms;      // [T]
    int32_t *bcnt;       // [T/256 blocks][E] per-block expert counts, then first slots (larger T)
    int32_t *bmiss;      // [T/256 blocks] per-block miss counts, then first miss-list entries
    WorkItem *items;     // work list
    int32_t *n_items;    // [1]
    // optional user copies of routing
    int32_t *u_idx;
    float *u_gate;
    int32_t *u_counts, *u_offsets, *u_perm, *u_pos;
    // miss list
    int32_t *miss_te;
    float *miss_w;
    int32_t miss_cap;
    int32_t *miss_count;
    // digit planes of the layer input: [T][d/32][XPLANES][4] words, per
    // (token, 32-column unit) digit sums, per (token, 256-column group) 2^-E
    uint32_t *xq;
    int32_t *xsum;
    float *xscl;
    float *hf;           // [slots][f] SwiGLU activation h of each slot (GEMV path)
    float *Y;            // [slots][d] expert outputs: row = slot, or with ytok row t*k + r for pick r of
                         // token t (the shared expert's rows stay at slot T*k + t)
    int ytok;            // decode path, T >= 2: Y rows in token order (combines read them without pos)
    int32_t *rbits;      // [T] bit r set when pick r of token t is resident (written when a mask is given)
    // GEMM path: bf16 hi/lo activations, columns permuted inside each
    // 128-column step, and their sums over each step (x) or 32-feature group (h)
    uint16_t *xa;        // [2][T][d]
    float *sx;           // [T][d/128]
    uint16_t *ha;        // [2][slots][f]
    float *hs;           // [slots][f/32]
    int xpasses;         // 1 when the lo half of xa is zero (bf16 input, no normalisation)
    // combine outputs
    float *out;          // [T][d] layer output
    float *x_next;       // [T][d] residual stream after this layer (nullable)
    int route_only;
    // decode path, a layer after the first: the previous layer's combine runs
    // inside this layer's router kernel.  px: that layer's input (bf16 or
    // fp32), pmask: its resident mask; idx, pos, gate and Y still hold its
    // routing and expert outputs; x_cur: where this layer's input (= a.x) is written.
    const void *px;
    int px_is_bf16;
    const uint32_t *pmask;
    float *x_cur;
};

// Optional HIP events around the next kernels of the calling thread: the
// first launch records `start` when it begins, every launch records `stop`
// when it ends (so after a group of launches `stop` marks the last one),
// both timed by the dispatch itself rather than by separate queue packets.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchEvents g_launch_events;

#define STRATA_LAUNCH(KER, GRID, BLOCK, LDS, STREAM, ...)                                                 \
    do {                                                                                                  \
        hipEvent_t ev0_ = g_launch_events.start;                                                          \
        g_launch_events.start = nullptr;                                                                  \
        hipExtLaunchKernelGGL(KER, GRID, BLOCK, LDS, STREAM, ev0_, g_launch_events.stop, 0, __VA_ARGS__); \
    } while (0)

// Status of a HIP call for the C ABI: STRATA_OK, or STRATA_EHIP with the
// error kept for strata_status_str (per thread).
strata_status hip_status(hipError_t e);

// Launchers (one file each); return hipGetLastError() of their launches.
hipError_t launch_route_logits_small(const LayerArgs &a, hipStream_t s);
hipError_t launch_route_small_finish(const LayerArgs &a, hipStream_t s);
// previous layer's combine + this layer's router (T <= 8, a layer after the first)
hipError_t launch_route_combine_small(const LayerArgs &a, hipStream_t s);
int route_logit_planes(int d);   // planes of z that kernel writes (one per 256 columns)
hipError_t launch_gemv_gateup_small(const LayerArgs &a, int max_items, hipStream_t s);
hipError_t launch_gemv_gateup_multi(const LayerArgs &a, int max_items, hipStream_t s);
hipError_t launch_route_logits(const LayerArgs &a, hipStream_t s);
int route_logit_splits(int d);
hipError_t launch_route_topk(const LayerArgs &a, hipStream_t s);
hipError_t launch_route_permute(const LayerArgs &a, int tile, hipStream_t s);
int route_perm_blocks(int T);
hipError_t launch_gemv_down_multi(const LayerArgs &a, int max_items, hipStream_t s);
hipError_t launch_gemv_down_one(const LayerArgs &a, hipStream_t s);
bool gemv_one_token(int T, int E, int k, int d, int f);   // T = 1 kernels apply
hipError_t launch_combine(const LayerArgs &a, hipStream_t s);
// out += add and x_next = x + out over the layer's T x d values (misses computed elsewhere)
hipError_t launch_add_rows(const LayerArgs &a, const float *add, hipStream_t s);
hipError_t launch_gemm_prep(const LayerArgs &a, hipStream_t s);
hipError_t launch_gemm_gateup(const LayerArgs &a, int max_items, hipStream_t s);
hipError_t launch_gemm_down(const LayerArgs &a, int max_items, hipStream_t s);
bool gemm_supported(int d, int f);
bool gemv_supported(int d, int f, int bits);

}  // namespace strata
