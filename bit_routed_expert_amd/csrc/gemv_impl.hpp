// Expert FFNs for small token counts per expert (decode and MTP verify):
// stream the packed 3-/2-bit codes of each needed expert from HBM once and
// reduce them against up to 8 tokens.
//
// The pages' engine computes the cached experts' FFNs on the GPU (wiselychen.com,
// technique 2 "專家快取與 CPU／GPU 分工"; greenbean-ai section 二).  Here every
// expert is resident and the kernels are bound by HBM: 3.0625 bit per weight
// leaves under two VALU operations per weight at full bandwidth, so the inner
// product does no per-weight float work:
//   * a 32-code unit unpacks into four words of 4-bit lanes with 3 ANDs and
//     one 6-op gather (codes 0..7 are valid signed 4-bit values);
//   * an activation is held as 24-bit fixed point X = rint(v * 2^E) per column
//     group (256 columns for the layer input, 32 for the SwiGLU activation h),
//     split into 6 balanced base-16 digit planes (digits in [-8, 7]);
//   * v_dot8_i32_i4 multiplies 8 codes by 8 digits with exact int32 sums, so
//     sum(c * X) over a run of columns is exact and the code offset is the
//     exact correction sum((c - c0) X) = sum(c X) - c0 * sum(X);
//   * the fp16 block scale and 2^-E are applied once per (row, group, token).
// Lane mapping: a wave covers R rows x S = 64/R column slices; lane
// (row r, slice s) reads up to 4 consecutive 32-column units of its row
// (one 128-column group is read with 16-byte loads) and keeps per-token
// partial sums; the S slices are summed with cross-lane adds.  Every
// kernel uses the same slicing for a given matrix width, so a token's
// result does not depend on how many tokens share the call.
//
// Kernels:
//   gate/up: a block owns 32 rows j of gate and the same rows of up for one
//     work item (<= 8 tokens of one expert), so it forms h = silu(g) * u and
//     writes h already quantised (digit planes per 32-column group).
//   down, T <= 8: a block owns R rows of Wd for every work item, so the
//     weighted combine with the shared expert and the residual add happen in
//     the block (fixed order, no cross-block step); one token takes one wave
//     per work item.
//   down, larger T: a block per (work item, 2R-row tile) writes expert
//     outputs; the combine kernel sums them.
#pragma once
#include <algorithm>

#include "routing.hpp"

namespace strata {

constexpr int HGROUP_UNITS = 1;   // h is quantised per 32 columns
constexpr int XGROUP_UNITS = 8;   // the layer input per 256 columns
constexpr int MAX_HUNITS = 24;    // f <= 768 on this path

template <int BITS> struct Fmt {
    static constexpr int UB = BITS == 3 ? 12 : 8;  // bytes per 32-code unit
    static constexpr int C2 = BITS == 3 ? 7 : 3;   // 2 * code offset
};

// 32 codes of one unit as four words of 4-bit lanes: nibble n of word i is
// the code at place 8i + n.
template <int BITS> __device__ __forceinline__ void unit_nibbles(const uint32_t *w, uint32_t N[4]) {
    if constexpr (BITS == 3) {
        N[0] = w[0] & 0x77777777u;
        N[1] = w[1] & 0x77777777u;
        N[2] = w[2] & 0x77777777u;
        N[3] = ((w[0] >> 3) & 0x11111111u) | ((w[1] >> 2) & 0x22222222u) | ((w[2] >> 1) & 0x44444444u);
    } else {
        N[0] = w[0] & 0x33333333u;
        N[1] = (w[0] >> 2) & 0x33333333u;
        N[2] = w[1] & 0x33333333u;
        N[3] = (w[1] >> 2) & 0x33333333u;
    }
}

// 2 * sum((c - c0) X) from the six digit-plane sums: each half of the
// digits combines exactly in int32, the halves and the offset correction in fp32.
__device__ __forceinline__ float digits_value(const int *acc, int C2, int sx) {
    const int lo = acc[0] + (acc[1] << 4) + (acc[2] << 8);
    const int hi = acc[3] + (acc[4] << 4) + (acc[5] << 8);
    const float I = fmaf((float)hi, 4096.f, (float)lo);
    return fmaf(2.f, I, -(float)C2 * (float)sx);
}

// LDS word offset of unit U's digit planes (4 words each), with 4 words of
// padding after each lane slice so the S slices read different banks.
__device__ __forceinline__ int dig_off(int U, int units_per_slice) {
    return U * XPLANES * 4 + (U / units_per_slice) * 4;
}

// Unit-granular tile for the decode kernels: lane (row r = lane % R, slice
// s = lane / R) holds units [s*upl, (s+1)*upl) of row row0 + r (upl <= 8;
// aligned runs of 4 units are 128-column groups, read with 16-byte loads),
// and each unit's fp16 block scale.
constexpr int UPL_MAX = 8;
template <int BITS> struct UTile {
    uint32_t w[UPL_MAX][Fmt<BITS>::UB / 4];
    uint32_t sc[UPL_MAX];

    __device__ __forceinline__ void load(const uint8_t *__restrict__ mat, const uint16_t *__restrict__ msc, int in,
                                         int row0, int R, int upl) {
        const int lane = threadIdx.x & 63;
        const int r = row0 + lane % R, U0 = (lane / R) * upl;
        constexpr int UB = Fmt<BITS>::UB;
        const int64_t rbase = ((int64_t)(r >> 4) * (in >> 7) * 16 + (r & 15)) * 4 * UB;
        if (upl % 4 == 0) {   // aligned groups: 48 or 32 contiguous bytes each
#pragma unroll
            for (int gq = 0; gq < UPL_MAX / 4; ++gq) {
                if (4 * gq < upl) {
                    const uint4 *p = (const uint4 *)(mat + rbase + (int64_t)((U0 >> 2) + gq) * 64 * UB);
#pragma unroll
                    for (int i = 0; i < UB / 4; ++i) {
                        const uint4 v = p[i];
                        const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            w[4 * gq + (4 * i + c) / (UB / 4)][(4 * i + c) % (UB / 4)] = q[c];
                    }
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < UPL_MAX; ++u) {
                if (u < upl) {
                    const int U = U0 + u;
                    const uint32_t *p = (const uint32_t *)(mat + rbase + ((int64_t)(U >> 2) * 64 + (U & 3)) * UB);
#pragma unroll
                    for (int i = 0; i < UB / 4; ++i) w[u][i] = p[i];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UPL_MAX; ++u)
            if (u < upl) sc[u] = msc[((int64_t)r * in + 32 * (U0 + u)) >> 8];
    }
};

// Row sums of a UTile against NT tokens (digit planes in LDS at dig +
// tmap[t]*dstride, laid out by dig_off with upl units per slice; unit sums
// usum[tmap[t]*ustride + U]; activation scales gscl[tmap[t]*gstride + U/upg]).
// Partial sums are flushed into res every `period` units (a period never
// spans two weight blocks or two activation groups) and at the slice end.
// res[t] is complete in lanes with s == 0 (lane < R).
template <int BITS, int NT>
__device__ __forceinline__ void utile_compute(const UTile<BITS> &wt, int R, int upl, int period,
                                              const uint32_t *__restrict__ dig, int dstride,
                                              const int *__restrict__ usum, int ustride, const float *__restrict__ gscl,
                                              int gstride, int upg, const int *tmap, float res[NT]) {
    const int lane = threadIdx.x & 63;
    const int U0 = (lane / R) * upl;
    int acc[NT][XPLANES];
    int sx[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        res[t] = 0.f;
        sx[t] = 0;
#pragma unroll
        for (int p = 0; p < XPLANES; ++p) acc[t][p] = 0;
    }
#pragma unroll
    for (int u = 0; u < UPL_MAX; ++u) {
        if (u < upl) {
            const int U = U0 + u;
            uint32_t N[4];
            unit_nibbles<BITS>(wt.w[u], N);
            const int off = dig_off(U, upl);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int tt = tmap ? tmap[t] : t;
                const uint4 *dp = (const uint4 *)(dig + tt * dstride + off);
#pragma unroll
                for (int p = 0; p < XPLANES; ++p) {
                    const uint4 dv = dp[p];
                    int a_ = acc[t][p];
                    a_ = __builtin_amdgcn_sdot8((int)N[0], (int)dv.x, a_, false);
                    a_ = __builtin_amdgcn_sdot8((int)N[1], (int)dv.y, a_, false);
                    a_ = __builtin_amdgcn_sdot8((int)N[2], (int)dv.z, a_, false);
                    a_ = __builtin_amdgcn_sdot8((int)N[3], (int)dv.w, a_, false);
                    acc[t][p] = a_;
                }
                sx[t] += usum[tt * ustride + U];
            }
            if (u == upl - 1 || (U + 1) % period == 0) {
                const float scl = 0.5f * half_to_float((uint16_t)wt.sc[u]);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int tt = tmap ? tmap[t] : t;
                    const float v = digits_value(acc[t], Fmt<BITS>::C2, sx[t]);
                    res[t] = fmaf(v, scl * gscl[tt * gstride + U / upg], res[t]);
                    sx[t] = 0;
#pragma unroll
                    for (int p = 0; p < XPLANES; ++p) acc[t][p] = 0;
                }
            }
        }
    }
    for (int o = R; o < 64; o <<= 1) {
#pragma unroll
        for (int t = 0; t < NT; ++t) res[t] += __shfl_xor(res[t], o, WAVE);
    }
}

// Lane slices of the decode kernels for a matrix with `in` columns: the most
// slices (a power of two up to smax) that split its 32-column units evenly
// with at most UPL_MAX units each (and whole groups once a slice has 4 or
// more units); 0 if none.
__host__ __device__ inline int unit_slices(int in, int smax) {
    const int units = in / 32;
    for (int S = smax; S >= 1; S >>= 1)
        if (units % S == 0 && units / S <= UPL_MAX && (units / S < 4 || (units / S) % 4 == 0)) return S;
    return 0;
}
// Flush period (units): within one weight block (8 units, or 4 when the row
// length is an odd multiple of 128 columns) and one activation group.
__host__ __device__ inline int unit_period(int in, int upg) {
    const int wp = (in % 256) ? 4 : 8;
    return upg < wp ? upg : wp;
}

// Quantise 8 consecutive values with exponent E into one word per digit
// plane (nibble n = digit of value n); returns the sum of the fixed-point values.
__device__ __forceinline__ int chunk_digits(const float v[8], int E, uint32_t word[XPLANES]) {
    static_assert(XPLANES == 6, "digit_words packs six planes");
    int X[8], sx = 0;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        X[n] = (int)rintf(ldexpf(v[n], E));
        sx += X[n];
    }
    digit_words(X, word);
    return sx;
}

__device__ __forceinline__ int slot_token(const LayerArgs &a, const WorkItem &it, int j) {
    const int slot = it.slot0 + j;
    return it.expert == a.E ? slot - a.T * a.k : a.perm[slot] / a.k;
}

// ---------------------------------------------------------- gate and up
// LDS of the gate/up kernel: digit planes, unit sums and group scales of all
// T tokens, then the gate/up results [2][NT][2R], then the routing state.
struct GuLds {
    int dstride, units, G;
    uint32_t *dig;
    int *sum;
    float *scl;
    float *gu;
    __device__ GuLds(uint32_t *lds, int d, int R, int T, int NT) {
        const int S = 64 / R;
        units = d / 32;
        G = (d + 255) / 256;
        dstride = units * XPLANES * 4 + S * 4;
        dig = lds;
        sum = (int *)(lds + T * dstride);
        scl = (float *)(sum + T * units);
        gu = scl + T * G;
    }
};
__host__ __device__ inline int gateup_lds_words(int d, int R, int T, int nt) {
    const int S = 64 / R;
    const int dstride = (d / 32) * XPLANES * 4 + S * 4;
    return T * dstride + T * (d / 32) + T * ((d + 255) / 256) + nt * 4 * R;
}

// Staging of every token's input digit planes into LDS by direct
// global->LDS loads, one lane-slice run (ups units, contiguous in both
// places) per load (two when a run exceeds 64 chunks), issued by the waves
// that do not take a top-k so they overlap the routing.
__device__ __forceinline__ void xstage_issue(const LayerArgs &a, const GuLds &g, int S, int ups) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, T = a.T, NW = blockDim.x >> 6;
    const int w0 = T < NW ? T : NW - 1;   // first staging wave
    if (wave < w0) return;
    const int nw = NW - w0, chunks = ups * XPLANES;   // 16-byte chunks per run
    const int per = (chunks + 63) / 64;
    for (int job = wave - w0; job < T * S * per; job += nw) {
        const int run = job / per, part = job % per, t = run / S, sl = run % S;
        const int c = part * 64 + lane;
        const uint32_t *src = a.xq + ((size_t)t * g.units + sl * ups) * XPLANES * 4 + 4 * (size_t)min(c, chunks - 1);
        uint32_t *dst = g.dig + t * g.dstride + dig_off(sl * ups, ups) + 4 * part * 64;
        if (c < chunks) __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    }
}
// Gate/up for the NT tokens toks[] of one work item: waves [0, G) take gate
// rows j0 + R*w .. +R, waves [G, 2G) the same rows of up; then h = silu(g)
// * u (fp32) of those G*R columns goes to hf.
template <int BITS, int NT>
__device__ __forceinline__ void gateup_body(const LayerArgs &a, const WorkItem &it, const int *toks, int R,
                                            int j0, const GuLds &g) {
    const int th = threadIdx.x, wave = th >> 6, lane = th & 63, G = blockDim.x >> 7;
    const int d = a.d, f = a.f;
    const int upl = (d / 32) / (64 / R);
    const int m = wave / G, row0 = j0 + (wave % G) * R;
    const size_t mat_bytes = (size_t)d * f * BITS / 8;
    const size_t mat_blocks = (size_t)d * f / 256;
    const size_t mi = (size_t)it.expert * 3 + m;
    UTile<BITS> wt;
    wt.load(a.codes + mi * mat_bytes, a.scales + mi * mat_blocks, d, row0, R, upl);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's staging loads have landed
    __syncthreads();                                  // every wave's staged digit planes visible
    float res[NT];
    utile_compute<BITS, NT>(wt, R, upl, unit_period(d, XGROUP_UNITS), g.dig, g.dstride, g.sum, g.units, g.scl, g.G,
                            XGROUP_UNITS, toks, res);
    if (m == 1 && lane < R) {
#pragma unroll
        for (int j = 0; j < NT; ++j) g.gu[j * G * R + (wave - G) * R + lane] = res[j];
    }
    __syncthreads();
    if (m == 0 && lane < R) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const float gv = res[j], u = g.gu[j * G * R + wave * R + lane];
            a.hf[(size_t)(it.slot0 + j) * f + row0 + lane] = gv / (1.f + expf(-gv)) * u;
        }
    }
}

#define NT_SWITCH(BODY)                                               \
    switch (it.ntok) {                                                \
        case 1: if constexpr (1 <= NTMAX) BODY(1); break;             \
        case 2: if constexpr (2 <= NTMAX) BODY(2); break;             \
        case 3: if constexpr (3 <= NTMAX) BODY(3); break;             \
        case 4: if constexpr (4 <= NTMAX) BODY(4); break;             \
        case 5: if constexpr (5 <= NTMAX) BODY(5); break;             \
        case 6: if constexpr (6 <= NTMAX) BODY(6); break;             \
        case 7: if constexpr (7 <= NTMAX) BODY(7); break;             \
        case 8: if constexpr (8 <= NTMAX) BODY(8); break;             \
        default: break;                                               \
    }

// T <= 8: every block (2G waves, G*R columns of h; G = 1 for one token, 4
// otherwise so the tokens' top-k run on separate waves) takes the top-k of
// the T tokens itself from the router logits (a few KB) while its input
// digit planes, unit sums and group scales load, derives its own work item
// and runs it; the last block writes the routing outputs and the work list
// instead.
template <int BITS, int NTMAX>
__global__ __launch_bounds__(NTMAX == 1 ? 128 : 512) void gemv_gateup_small_kernel(LayerArgs a, int R,
                                                                                   int route_off) {
    extern __shared__ uint32_t lds[];
    const GuLds g(lds, a.d, R, a.T, NTMAX);
    const SmallRoute L(lds + route_off, a.E);
    const int S = 64 / R, upl = (a.d / 32) / S;
    if (blockIdx.x == gridDim.x - 1) {
        small_route_compute(a, L, a.z, a.inv_rms);
        small_route_write(a, L);
        return;
    }
    xstage_issue(a, g, S, upl);
    // unit sums and group scales into registers now, LDS after the routing
    const int per = g.units + g.G, nq = a.T * per;
    int qv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int q = threadIdx.x + blockDim.x * u, j = q / per, i = q % per;
        qv[u] = q < nq ? (i < g.units ? a.xsum[(size_t)j * g.units + i] : __float_as_int(a.xscl[(size_t)j * g.G + i - g.units])) : 0;
    }
    small_route_compute(a, L, a.z, a.inv_rms);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int q = threadIdx.x + blockDim.x * u, j = q / per, i = q % per;
        if (q < nq) {
            if (i < g.units) g.sum[j * g.units + i] = qv[u];
            else g.scl[j * g.G + i - g.units] = __int_as_float(qv[u]);
        }
    }
    for (int q = threadIdx.x + 2 * blockDim.x; q < nq; q += blockDim.x) {   // large d
        const int j = q / per, i = q % per;
        if (i < g.units) g.sum[j * g.units + i] = a.xsum[(size_t)j * g.units + i];
        else g.scl[j * g.G + i - g.units] = a.xscl[(size_t)j * g.G + i - g.units];
    }
    const int cols = (blockDim.x >> 7) * R, wg_per_item = a.f / cols;
    WorkItem it;
    int toks[CHUNK_TOK];
    if (!small_route_item(a, L, blockIdx.x / wg_per_item, it, toks)) return;
    const int j0 = (blockIdx.x % wg_per_item) * cols;
#define GU(n) gateup_body<BITS, n>(a, it, toks, R, j0, g)
    NT_SWITCH(GU)
#undef GU
}

// ----------------------------------------------------------------- down
// h of NT consecutive slots (fp32, [slot][f]) staged through registers and
// quantised into one wave's LDS region: per 32-column unit, 24-bit fixed
// point with exponent E from the unit's max |h|, 6 balanced base-16 digit
// planes, the unit's digit sum and 2^-E.  A lane takes 8-column chunks
// c = lane + 64u; the 4 chunks of a unit sit in 4 neighbouring lanes.
// load() issues the global loads; store() quantises and writes (so a
// caller can issue other loads in between without the in-order load
// counter making store() wait for them).
template <int NT> struct HStage {
    static constexpr int PER = (NT * MAX_HUNITS * 4 + 63) / 64;   // chunks per lane
    float4 v[PER][2];

    __device__ __forceinline__ void load(const LayerArgs &a, int slot0) {
        const int lane = threadIdx.x & 63, nch = NT * (a.f / 8);
        const float4 *src = (const float4 *)(a.hf + (size_t)slot0 * a.f);
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int c = min(lane + 64 * u, nch - 1);
            v[u][0] = src[2 * c];
            v[u][1] = src[2 * c + 1];
        }
    }

    __device__ __forceinline__ void store(const LayerArgs &a, int ups, int dstride, uint32_t *wdig, int *wsum,
                                          float *wscl) const {
        const int lane = threadIdx.x & 63, units = a.f / 32, cps = a.f / 8, nch = NT * cps;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int c = lane + 64 * u;
            const float h[8] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w,
                                v[u][1].x, v[u][1].y, v[u][1].z, v[u][1].w};
            float mx = 0.f;
#pragma unroll
            for (int n = 0; n < 8; ++n) mx = fmaxf(mx, fabsf(h[n]));
            mx = fmaxf(mx, __shfl_xor(mx, 1, WAVE));
            mx = fmaxf(mx, __shfl_xor(mx, 2, WAVE));
            const int E = fixed_point_exponent<XPLANES>(mx);
            uint32_t word[XPLANES];
            int sx = chunk_digits(h, E, word);
            sx += __shfl_xor(sx, 1, WAVE);
            sx += __shfl_xor(sx, 2, WAVE);
            if (c < nch) {
                const int j = c / cps, cc = c % cps, U = cc / 4, q = cc % 4;
                uint32_t *dst = wdig + j * dstride + dig_off(U, ups);
#pragma unroll
                for (int p = 0; p < XPLANES; ++p) dst[4 * p + q] = word[p];
                if (q == 0) {
                    wsum[j * units + U] = sx;
                    wscl[j * units + U] = ldexpf(1.f, -E);
                }
            }
        }
        // the same wave reads these LDS words next: order the writes before the reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
};

__host__ __device__ inline int down_wave_lds_words(int f, int R, int nt) {
    const int S = 64 / R;
    return nt * ((f / 32) * XPLANES * 4 + S * 4) + 2 * nt * (f / 32);
}

// One work item on this wave's tile: stage h (its loads issued before the
// prefetch of the next tile's codes, so waiting for them does not wait for
// the prefetch), then run the tile.
template <int BITS, int NT>
__device__ __forceinline__ void down_item(const LayerArgs &a, const WorkItem &it, const UTile<BITS> &wt, int R,
                                          int row0, uint32_t *wdig, float res[CHUNK_TOK], UTile<BITS> &next,
                                          bool do_next, int next_expert) {
    const int d = a.d, f = a.f, units = f / 32;
    const int S = 64 / R, upl = units / S;
    const int dstride = units * XPLANES * 4 + S * 4;
    int *wsum = (int *)(wdig + NT * dstride);
    float *wscl = (float *)(wsum + NT * units);
    HStage<NT> st;
    st.load(a, it.slot0);
    if (do_next)
        next.load(a.codes + ((size_t)next_expert * 3 + 2) * ((size_t)d * f * BITS / 8),
                  a.scales + ((size_t)next_expert * 3 + 2) * ((size_t)d * f / 256), f, row0, R, upl);
    st.store(a, upl, dstride, wdig, wsum, wscl);
    float r[NT];
    utile_compute<BITS, NT>(wt, R, upl, 1, wdig, dstride, wsum, units, wscl, units, HGROUP_UNITS, nullptr, r);
#pragma unroll
    for (int j = 0; j < NT; ++j) res[j] = r[j];
}

// T <= 8: block = NW waves on rows [row0, row0+R) of Wd for every work item;
// wave w runs items w, w+NW, ... (the next item's codes are loaded while the
// current one computes; with NW >= the number of items every wave has at
// most one, so all codes are requested at once), expert outputs land in
// LDS, then the block forms out[t] = y_shared[t] + sum_{r asc, resident}
// gate[t][r] * y[slot(t, r)] and x_next = x + out for those rows.
template <int BITS, int NTMAX>
__global__ __launch_bounds__(256) void gemv_down_rows_kernel(LayerArgs a, int R) {
    extern __shared__ uint32_t lds[];
    const int th = threadIdx.x, wave = th >> 6, lane = th & 63, NW = blockDim.x >> 6;
    const int d = a.d, f = a.f, T = a.T, k = a.k;
    const int row0 = blockIdx.x * R;
    const int nslots = T * k + T;
    float *ybuf = (float *)lds;  // [nslots][R]
    uint32_t *wdig = lds + nslots * R + wave * down_wave_lds_words(f, R, NTMAX);
    const int n = *a.n_items;
    const size_t mat_bytes = (size_t)d * f * BITS / 8;
    const size_t mat_blocks = (size_t)d * f / 256;
    // two register tiles used alternately (named, so no dynamic register
    // indexing); item `item` computes from one while item + NW's codes load into the other
    UTile<BITS> buf0, buf1;
    WorkItem cur = a.items[min(wave, n - 1)];
    if (wave < n)
        buf0.load(a.codes + ((size_t)cur.expert * 3 + 2) * mat_bytes,
                  a.scales + ((size_t)cur.expert * 3 + 2) * mat_blocks, f, row0, R, (f / 32) / (64 / R));
    for (int item = wave; item < n; item += 2 * NW) {
        {
            const WorkItem it = cur;
            const bool has = item + NW < n;
            if (has) cur = a.items[item + NW];
            float res[CHUNK_TOK];
#define DN(nn) down_item<BITS, nn>(a, it, buf0, R, row0, wdig, res, buf1, has, cur.expert)
            NT_SWITCH(DN)
#undef DN
            if (lane < R)
                for (int j = 0; j < it.ntok; ++j) ybuf[(it.slot0 + j) * R + lane] = res[j];
        }
        if (item + NW < n) {
            const WorkItem it = cur;
            const bool has = item + 2 * NW < n;
            if (has) cur = a.items[item + 2 * NW];
            float res[CHUNK_TOK];
#define DN(nn) down_item<BITS, nn>(a, it, buf1, R, row0, wdig, res, buf0, has, cur.expert)
            NT_SWITCH(DN)
#undef DN
            if (lane < R)
                for (int j = 0; j < it.ntok; ++j) ybuf[(it.slot0 + j) * R + lane] = res[j];
        }
    }
    __syncthreads();
    for (int q = th; q < T * R; q += blockDim.x) {
        const int t = q / R, i = q % R;
        float s = ybuf[(T * k + t) * R + i];
        for (int r = 0; r < k; ++r) {
            const int e = a.idx[t * k + r];
            if (is_resident(a.mask, e)) s = fmaf(a.gate[t * k + r], ybuf[a.pos[t * k + r] * R + i], s);
        }
        const size_t o = (size_t)t * d + row0 + i;
        a.out[o] = s;
        if (a.x_next) {
            const float xv = a.x_is_bf16 ? bf16_to_float(((const uint16_t *)a.x)[o]) : ((const float *)a.x)[o];
            a.x_next[o] = xv + s;
        }
    }
}

// One token: block = one wave per work item on rows [row0, row0+R) of Wd
// (R = 64/S, S lane slices of upl units, so every expert's rows of this
// tile are requested at once).  With no resident mask item w is slot w (the
// shared expert slot k), so h is loaded before the work list is read; the
// combine inputs load meanwhile too.
// Then out = y_shared + sum_{r asc, resident} gate[r] * y[slot(r)] and
// x_next = x + out for those rows.
__host__ __device__ inline int down_one_lds_words(int k, int f, int R) {
    const int S = 64 / R, units = f / 32;
    return (k + 1) * R + (k + 1) * (units * XPLANES * 4 + S * 4 + 2 * units) + 3 * k;
}

template <int BITS>
__global__ __launch_bounds__(768) void gemv_down_rows_one_kernel(LayerArgs a, int R) {
    extern __shared__ uint32_t lds[];
    const int th = threadIdx.x, wave = th >> 6, lane = th & 63, NW = blockDim.x >> 6;
    const int d = a.d, f = a.f, k = a.k;
    const int row0 = blockIdx.x * R;
    const int S = 64 / R, units = f / 32, upl = units / S;
    const int dstride = units * XPLANES * 4 + S * 4;
    float *ybuf = (float *)lds;  // [k + 1][R], by slot
    uint32_t *wdig = lds + (k + 1) * R + wave * (dstride + 2 * units);
    int *wsum = (int *)(wdig + dstride);
    float *wscl = (float *)(wsum + units);
    float *cg = (float *)(lds + (k + 1) * R + NW * (dstride + 2 * units));  // [k] gate of pick r
    int *cp = (int *)(cg + k);                                               // [k] slot of pick r
    int *con = cp + k;                                                       // [k] resident
    const bool fast = a.mask == nullptr;
    int slot = wave < k ? wave : k;
    HStage<1> st;
    if (fast) st.load(a, slot);
    int pe = 0, pp = 0;
    float pg = 0.f;
    if (wave == 0 && lane < k) {
        pe = a.idx[lane];
        pg = a.gate[lane];
        pp = a.pos[lane];
    }
    const int n = *a.n_items;
    if (wave < n) {
        const WorkItem it = a.items[wave];
        if (!fast) {
            slot = it.slot0;
            st.load(a, slot);
        }
        UTile<BITS> wt;
        wt.load(a.codes + ((size_t)it.expert * 3 + 2) * ((size_t)d * f * BITS / 8),
                a.scales + ((size_t)it.expert * 3 + 2) * ((size_t)d * f / 256), f, row0, R, upl);
        st.store(a, upl, dstride, wdig, wsum, wscl);
        float res[1];
        utile_compute<BITS, 1>(wt, R, upl, 1, wdig, dstride, wsum, units, wscl, units, HGROUP_UNITS, nullptr, res);
        if (lane < R) ybuf[slot * R + lane] = res[0];
    }
    if (wave == 0 && lane < k) {
        cg[lane] = pg;
        cp[lane] = pp;
        con[lane] = is_resident(a.mask, pe) ? 1 : 0;
    }
    __syncthreads();
    for (int i = th; i < R; i += blockDim.x) {
        float s = ybuf[k * R + i];
        for (int r = 0; r < k; ++r)
            if (con[r]) s = fmaf(cg[r], ybuf[cp[r] * R + i], s);
        const size_t o = (size_t)row0 + i;
        a.out[o] = s;
        if (a.x_next) {
            const float xv = a.x_is_bf16 ? bf16_to_float(((const uint16_t *)a.x)[o]) : ((const float *)a.x)[o];
            a.x_next[o] = xv + s;
        }
    }
}

// Any T: block = 2 waves = 2 row tiles of one work item; expert outputs to Y.
template <int BITS, int NTMAX>
__global__ __launch_bounds__(128) void gemv_down_items_kernel(LayerArgs a, int R) {
    extern __shared__ uint32_t lds[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int d = a.d, f = a.f;
    const int wg_per_item = d / (2 * R);
    const int item = blockIdx.x / wg_per_item;
    if (item >= *a.n_items) return;
    const WorkItem it = a.items[item];
    const int row0 = ((blockIdx.x % wg_per_item) * 2 + wave) * R;
    UTile<BITS> wt;
    wt.load(a.codes + ((size_t)it.expert * 3 + 2) * ((size_t)d * f * BITS / 8),
            a.scales + ((size_t)it.expert * 3 + 2) * ((size_t)d * f / 256), f, row0, R, (f / 32) / (64 / R));
    uint32_t *wdig = lds + wave * down_wave_lds_words(f, R, NTMAX);
    float res[CHUNK_TOK];
#define DN(nn) down_item<BITS, nn>(a, it, wt, R, row0, wdig, res, wt, false, 0)
    NT_SWITCH(DN)
#undef DN
    if (lane < R)
        for (int j = 0; j < it.ntok; ++j) a.Y[(size_t)(it.slot0 + j) * d + row0 + lane] = res[j];
}

// ------------------------------------------------------------- launchers
inline bool gemv_supported_impl(int d, int f, int bits) {
    if (bits != 3 && bits != 2) return false;
    if (unit_slices(d, 8) < 2 || unit_slices(f, 8) < 1) return false;   // decode tiles
    if (d % 128 || f % 128 || f > 32 * MAX_HUNITS || d > 8192) return false;
    const int Rd = 64 / unit_slices(f, 8);
    if (d % (2 * Rd)) return false;        // down blocks own R (rows kernel) or 2R rows
    return true;
}

static inline int ntmax_for(int T) { return T >= CHUNK_TOK ? CHUNK_TOK : T; }
// token capacity of a kernel instance: 1, 2, 4, 5 or 8
static inline int nt_round(int nt) { return nt <= 2 ? nt : (nt <= 4 ? 4 : (nt <= 5 ? 5 : 8)); }

// Every kernel here stays within the 64 KiB of LDS a block gets by default;
// a launch that would need more is refused rather than attempted.
constexpr size_t LDS_LIMIT = 64 * 1024;

#define LAUNCH_NT(KER, BITS, nt, grid, block, lds, s, ...)                                           \
    do {                                                                                             \
        if ((lds) > LDS_LIMIT) return hipErrorInvalidValue;                                          \
        switch (nt) {                                                                                \
            case 1: STRATA_LAUNCH((KER<BITS, 1>), grid, dim3(block), lds, s, __VA_ARGS__); break; \
            case 2: STRATA_LAUNCH((KER<BITS, 2>), grid, dim3(block), lds, s, __VA_ARGS__); break; \
            case 4: STRATA_LAUNCH((KER<BITS, 4>), grid, dim3(block), lds, s, __VA_ARGS__); break; \
            case 5: STRATA_LAUNCH((KER<BITS, 5>), grid, dim3(block), lds, s, __VA_ARGS__); break; \
            default: STRATA_LAUNCH((KER<BITS, 8>), grid, dim3(block), lds, s, __VA_ARGS__); break; \
        }                                                                                            \
    } while (0)

template <int BITS> hipError_t gateup_small_launch(const LayerArgs &a, int max_items, hipStream_t s) {
    const int R = 64 / unit_slices(a.d, 8);
    const int nt = nt_round(ntmax_for(a.T));
    const int off = gateup_lds_words(a.d, R, a.T, nt);
    const size_t lds = 4 * ((size_t)off + small_route_lds_words(a.E));
    const int G = (a.T == 1 || a.f % (4 * R)) ? 1 : 4;   // row groups per block
    const dim3 grid(max_items * (a.f / (G * R)) + 1);
    if (nt == 1 && G != 1) return hipErrorInvalidValue;
    LAUNCH_NT(gemv_gateup_small_kernel, BITS, nt, grid, 128 * G, lds, s, a, R, off);
    return hipGetLastError();
}

template <int BITS> hipError_t down_launch(const LayerArgs &a, int max_items, hipStream_t s) {
    const int R = 64 / unit_slices(a.f, 8);
    const int nt = nt_round(ntmax_for(a.T));
    const size_t lds = 4 * (size_t)2 * down_wave_lds_words(a.f, R, nt);
    const dim3 grid(max_items * (a.d / (2 * R)));
    LAUNCH_NT(gemv_down_items_kernel, BITS, nt, grid, 128, lds, s, a, R);
    return hipGetLastError();
}

// Waves of the down rows kernels: one token, one per work item (k + 1);
// else 4, or fewer when the LDS does not hold them.
static inline size_t down_rows_lds(int T, int k, int f, int R, int nt, int nw) {
    const int nslots = T * k + T;
    return 4 * ((size_t)nslots * R + (size_t)nw * down_wave_lds_words(f, R, nt));
}
static inline int down_rows_waves(int T, int k, int f, int R, int nt) {
    int nw = T == 1 ? k + 1 : 4;
    while (nw > 1 && down_rows_lds(T, k, f, R, nt, nw) > LDS_LIMIT) --nw;
    return nw;
}

template <int BITS> hipError_t down_rows_launch(const LayerArgs &a, hipStream_t s) {
    const int R = 64 / unit_slices(a.f, 8);
    const int nt = nt_round(ntmax_for(a.T));
    const int nw = down_rows_waves(a.T, a.k, a.f, R, nt);
    const size_t lds = down_rows_lds(a.T, a.k, a.f, R, nt, nw);
    const dim3 grid(a.d / R);
    if (a.T == 1) {
        const size_t lds1 = 4 * (size_t)down_one_lds_words(a.k, a.f, R);
        if (lds1 > LDS_LIMIT || a.k + 1 > 12) return hipErrorInvalidValue;
        STRATA_LAUNCH(gemv_down_rows_one_kernel<BITS>, grid, dim3(64 * (a.k + 1)), lds1, s, a, R);
        return hipGetLastError();
    }
    LAUNCH_NT(gemv_down_rows_kernel, BITS, nt, grid, 64 * nw, lds, s, a, R);
    return hipGetLastError();
}

}  // namespace strata
