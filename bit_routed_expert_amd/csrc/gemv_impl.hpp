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
template <int BITS, int UPLM = UPL_MAX> struct UTile {   // UPLM: capacity (upl <= UPLM)
    uint32_t w[UPLM][Fmt<BITS>::UB / 4];
    uint32_t sc[UPLM];
};

// A UTile filled with every code load issued unconditionally (units past
// upl re-read the lane's first unit, from cache), so filling it takes no
// branches and a prefetch into it needs no wait until its values are read.
// Scales are loaded only for the units utile_compute reads them at: the
// last unit of each flush period (`period`, as passed to utile_compute; a
// period never spans two weight blocks) and the lane's last unit; with a
// period of one unit every scale is read and the loads stay unconditional.
// GROUPED: upl is a multiple of 4 (16-byte group loads).
// r: this lane's row, U0: its first unit.
template <int BITS, bool GROUPED, int UPLM = UPL_MAX>
__device__ __forceinline__ void utile_load_all(UTile<BITS, UPLM> &t, const uint8_t *__restrict__ mat,
                                               const uint16_t *__restrict__ msc, int in, int r, int U0, int upl,
                                               int period) {
    constexpr int UB = Fmt<BITS>::UB;
    const int64_t rbase = ((int64_t)(r >> 4) * (in >> 7) * 16 + (r & 15)) * 4 * UB;
    if constexpr (GROUPED) {
#pragma unroll
        for (int gq = 0; gq < UPLM / 4; ++gq) {
            const int gg = 4 * gq < upl ? gq : 0;
            const uint4 *p = (const uint4 *)(mat + rbase + (int64_t)((U0 >> 2) + gg) * 64 * UB);
#pragma unroll
            for (int i = 0; i < UB / 4; ++i) {
                const uint4 v = p[i];
                const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int c = 0; c < 4; ++c) t.w[4 * gq + (4 * i + c) / (UB / 4)][(4 * i + c) % (UB / 4)] = q[c];
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < UPLM; ++u) {
            const int U = U0 + (u < upl ? u : 0);
            const uint32_t *p = (const uint32_t *)(mat + rbase + ((int64_t)(U >> 2) * 64 + (U & 3)) * UB);
#pragma unroll
            for (int i = 0; i < UB / 4; ++i) t.w[u][i] = p[i];
        }
    }
    if (period == 1) {   // every unit's scale is read: unconditional, like the codes
#pragma unroll
        for (int u = 0; u < UPLM; ++u) t.sc[u] = msc[((int64_t)r * in + 32 * (U0 + (u < upl ? u : 0))) >> 8];
    } else {
#pragma unroll
        for (int u = 0; u < UPLM; ++u)
            if (u < upl && (u == upl - 1 || (U0 + u + 1) % period == 0))
                t.sc[u] = msc[((int64_t)r * in + 32 * (U0 + u)) >> 8];
    }
}

// Row sums of a UTile against NT tokens (digit planes in LDS at dig +
// tok_of(tpk, t)*dstride, laid out by dig_off with upl units per slice; unit sums
// usum[tt*ustride + U]; activation scales gscl[tt*gstride + U/upg]; tt = tok_of(tpk, t)).
// Partial sums are flushed into res every `period` units (a period never
// spans two weight blocks or two activation groups) and at the slice end.
// res[t] is complete in lanes with s == 0 (lane < R).
template <int BITS, int NT, int UPLM = UPL_MAX>
__device__ __forceinline__ void utile_compute(const UTile<BITS, UPLM> &wt, int R, int upl, int period,
                                              const uint32_t *__restrict__ dig, int dstride,
                                              const int *__restrict__ usum, int ustride, const float *__restrict__ gscl,
                                              int gstride, int upg, uint32_t tpk, float res[NT]) {
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
    for (int u = 0; u < UPLM; ++u) {
        if (u < upl) {
            const int U = U0 + u;
            uint32_t N[4];
            unit_nibbles<BITS>(wt.w[u], N);
            const int off = dig_off(U, upl);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int tt = tok_of(tpk, t);
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
                    const int tt = tok_of(tpk, t);
                    const float v = digits_value(acc[t], Fmt<BITS>::C2, sx[t]);
                    res[t] = fmaf(v, scl * gscl[tt * gstride + U / upg], res[t]);
                    sx[t] = 0;
#pragma unroll
                    for (int p = 0; p < XPLANES; ++p) acc[t][p] = 0;
                }
            }
        }
    }
    // sum over the 64/R slices of each row (lane ^ R, ^ 2R, ...)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (R <= 8) res[t] += lane_xor<8>(res[t]);
        if (R <= 16) res[t] += lane_xor<16>(res[t]);
        if (R <= 32) res[t] += lane_xor<32>(res[t]);
    }
}

// utile_compute over the NT tokens one at a time (each token's result is
// the same as in a joint pass; the register footprint is that of one token,
// so kernels holding two code tiles keep every token count spill-free).
template <int BITS, int NT, int UPLM = UPL_MAX>
__device__ __forceinline__ void utile_compute_each(const UTile<BITS, UPLM> &wt, int R, int upl, int period,
                                                   const uint32_t *__restrict__ dig, int dstride,
                                                   const int *__restrict__ usum, int ustride,
                                                   const float *__restrict__ gscl, int gstride, int upg,
                                                   uint32_t tpk, float res[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float r[1];
        utile_compute<BITS, 1, UPLM>(wt, R, upl, period, dig, dstride, usum, ustride, gscl, gstride, upg,
                                     tpk >> (3 * t), r);
        res[t] = r[0];
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
__host__ __device__ constexpr int align4(int words) { return (words + 3) & ~3; }
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
// Gate/up for the NT tokens (token map tpk) of one work item: waves [0, G) take gate
// rows j0 + R*w .. +R, waves [G, 2G) the same rows of up; then h = silu(g)
// * u (fp32) of those G*R columns goes to hf.
template <int BITS, int NT>
__device__ __forceinline__ void gateup_body(const LayerArgs &a, const WorkItem &it, uint32_t tpk, int R,
                                            int j0, const GuLds &g) {
    const int th = threadIdx.x, wave = th >> 6, lane = th & 63, G = blockDim.x >> 7;
    const int d = a.d, f = a.f;
    const int upl = (d / 32) / (64 / R);
    const int m = wave / G, row0 = j0 + (wave % G) * R;
    const size_t mat_bytes = (size_t)d * f * BITS / 8;
    const size_t mat_blocks = (size_t)d * f / 256;
    const size_t mi = (size_t)it.expert * 3 + m;
    // this wave's staging loads (issued before the routing) have landed; the
    // code loads then go out unconditionally and stay in flight across the
    // barrier, which waits only for LDS (each use waits for its own unit)
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    UTile<BITS> wt;
    const int r = row0 + lane % R, U0 = (lane / R) * upl;
    if (upl % 4 == 0)
        utile_load_all<BITS, true>(wt, a.codes + mi * mat_bytes, a.scales + mi * mat_blocks, d, r, U0, upl,
                                   unit_period(d, XGROUP_UNITS));
    else
        utile_load_all<BITS, false>(wt, a.codes + mi * mat_bytes, a.scales + mi * mat_blocks, d, r, U0, upl,
                                    unit_period(d, XGROUP_UNITS));
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS stores are done
    __builtin_amdgcn_s_barrier();         // every wave's staged digit planes and sums visible
    float res[NT];
    utile_compute<BITS, NT>(wt, R, upl, unit_period(d, XGROUP_UNITS), g.dig, g.dstride, g.sum, g.units, g.scl, g.G,
                            XGROUP_UNITS, tpk, res);
    if (m == 1 && lane < R) {
#pragma unroll
        for (int j = 0; j < NT; ++j) g.gu[j * G * R + (wave - G) * R + lane] = res[j];
    }
    __syncthreads();
    if (m == 0 && lane < R) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const float gv = res[j], u = g.gu[j * G * R + wave * R + lane];
            a.hf[(size_t)(it.slot0 + j) * f + row0 + lane] = silu_mul(gv, u);
        }
    }
}

// One token: blocks of G gate waves and G up waves, G*R columns of h each
// (G = 2 when f allows).  The first f/(G*R) blocks take the shared expert
// and need no routing; every other group of f/(G*R) blocks takes one pick:
// each block takes the top-k itself from the router logits (a few KB, one
// wave) while the other waves stage the input digit planes, unit sums and
// group scales, and runs its pick's rows; the last block writes the routing
// outputs and the work list instead.
// Registers are held to three waves per SIMD, so a grid of about 2,100
// waves (ten picks plus the shared expert at f = 768) is resident at once.
template <int BITS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void gemv_gateup_small_kernel(LayerArgs a, int R, int route_off) {
    extern __shared__ uint32_t lds[];
    const GuLds g(lds, a.d, R, a.T, 1);
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
    const int cols = (blockDim.x >> 7) * R, wg_per_item = a.f / cols;
    const int b = blockIdx.x / wg_per_item;   // 0: shared expert, else pick b - 1
    if (b > 0 && threadIdx.x < 64) {
        WorkItem r{};
        const bool ok = one_token_item(a, b - 1, L.cand, r);
        if (threadIdx.x == 0) {
            L.tmp[0] = ok ? r.expert : -1;
            L.tmp[1] = r.slot0;
        }
    }
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
    WorkItem it{a.E, a.k, 1};
    if (b > 0) {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the item is in LDS
        __builtin_amdgcn_s_barrier();
        const int ex = L.tmp[0];
        if (ex < 0) return;   // a pick that is not resident (whole block)
        it = WorkItem{ex, L.tmp[1], 1};
    }
    const int j0 = (blockIdx.x % wg_per_item) * cols;
    gateup_body<BITS, 1>(a, it, TOK_IDENTITY, R, j0, g);
}

// Any T <= 8 (the path for T >= 2).  Blocks take the top-k of all T tokens
// once (from the router logits, while every token's input digit planes load
// into LDS) and list the work items (an expert's slots in pairs) in LDS;
// then every wave runs its own jobs, job = (work item, R/2 columns of h),
// jobs wave_id, wave_id + total waves, ..., the next job's codes loading
// into a second named tile while the current one computes.  In a job, lane
// rows r < R/2 are gate rows and r >= R/2 the same rows of up, so h =
// silu(g) * u forms inside the wave (no block barrier) and goes to hf; the
// down kernel quantises it.  The last block writes the routing outputs and
// the work list instead.
template <int BITS, int NT>
__device__ __forceinline__ void gateup_wave_job(const LayerArgs &a, const WorkItem &it, uint32_t tpk, int R, int c0,
                                                const GuLds &g, const UTile<BITS> &wt) {
    const int lane = threadIdx.x & 63, half = R / 2;
    const int upl = (a.d / 32) / (64 / R);
    float res[NT];
    utile_compute_each<BITS, NT>(wt, R, upl, unit_period(a.d, XGROUP_UNITS), g.dig, g.dstride, g.sum, g.units, g.scl,
                                 g.G, XGROUP_UNITS, tpk, res);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        // the up row's result sits half lanes above (lanes < half read it)
        const float gv = res[j], u = half == 4 ? lane_down4(res[j]) : half == 8 ? lane_xor<8>(res[j]) : lane_xor<16>(res[j]);
        if (lane < half) a.hf[(size_t)(it.slot0 + j) * a.f + c0 + lane] = silu_mul(gv, u);
    }
}

template <int BITS, bool GROUPED>
__global__ __launch_bounds__(512) void gemv_gateup_multi_kernel(LayerArgs a, int R, int route_off) {
    extern __shared__ uint32_t lds[];
    const GuLds g(lds, a.d, R, a.T, ITEM_TOK);
    const SmallRoute L(lds + route_off, a.E);
    const int S = 64 / R, upl = (a.d / 32) / S;
    if (blockIdx.x == gridDim.x - 1) {
        small_route_compute<true>(a, L, a.z, a.inv_rms);
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
    small_route_compute<true>(a, L, a.z, a.inv_rms);
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
    // this wave's staged digit planes have landed (every wave's are visible
    // after the table's barrier)
    __builtin_amdgcn_s_waitcnt(0);
    int32_t *itab = (int32_t *)(lds + ((route_off + small_route_lds_words(a.E) + 3) & ~3));   // 16-byte aligned
    const int half = R / 2, groups = a.f / half;
    const int nitems = small_route_table(a, L, itab);   // last block barrier
    const int njobs = nitems * groups;
    // jobs walk the table from its end: the shared expert's items (every
    // token, two per item) go out in the first rounds and the last rounds
    // hold one-token routed items, which shortens the tail
#define GU_ITEM(JOB_) (nitems - 1 - (JOB_) / groups)
    const int wpb = blockDim.x >> 6, nw = (gridDim.x - 1) * wpb;
    // job (and the item words read for it) are wave-uniform: say so, so the
    // job loop is scalar control flow
    int job = __builtin_amdgcn_readfirstlane(blockIdx.x * wpb + (threadIdx.x >> 6));
    if (job >= njobs) return;
    const int lane = threadIdx.x & 63, rl = lane % R, m = rl >= half ? 1 : 0, U0 = (lane / R) * upl;
    const int uper = unit_period(a.d, XGROUP_UNITS);
    const size_t mat_bytes = (size_t)a.d * a.f * BITS / 8, mat_blocks = (size_t)a.d * a.f / 256;
    // this lane's row of the job's expert: gate (m = 0) or up (m = 1) row c0 + rl - m*half
#define GU_LOAD(T_, IT_, JOB_)                                                                                         \
    utile_load_all<BITS, GROUPED>(T_, a.codes + ((size_t)(IT_).expert * 3 + m) * mat_bytes,                           \
                                  a.scales + ((size_t)(IT_).expert * 3 + m) * mat_blocks, a.d,                         \
                                  ((JOB_) % groups) * half + rl - m * half, U0, upl, uper)
    WorkItem it;
    uint32_t tpk;
    {
        const int4 v = *(const int4 *)(itab + 4 * GU_ITEM(job));
        it = WorkItem{__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                      __builtin_amdgcn_readfirstlane(v.z)};
        tpk = (uint32_t)__builtin_amdgcn_readfirstlane(v.w);
    }
    // two tiles used alternately (named, no copies): one computes while the
    // next job's codes load into the other
    UTile<BITS> b0, b1;
    GU_LOAD(b0, it, job);
#define GU_STEP(CUR, NXT)                                                                                              \
    {                                                                                                                  \
        const int next = job + nw;                                                                                     \
        const int nj = next < njobs ? next : job; /* past the end: re-read this job's tile (cached) */                 \
        const int4 v1 = *(const int4 *)(itab + 4 * GU_ITEM(nj));                                                       \
        GU_LOAD(NXT, (WorkItem{__builtin_amdgcn_readfirstlane(v1.x), 0, 0}), nj);                                      \
        const int c0 = (job % groups) * half;                                                                          \
        if (it.ntok == 1) gateup_wave_job<BITS, 1>(a, it, tpk, R, c0, g, CUR);                                         \
        else gateup_wave_job<BITS, 2>(a, it, tpk, R, c0, g, CUR);                                                      \
        if (next >= njobs) break;                                                                                      \
        job = next;                                                                                                    \
        it = WorkItem{__builtin_amdgcn_readfirstlane(v1.x), __builtin_amdgcn_readfirstlane(v1.y),                      \
                      __builtin_amdgcn_readfirstlane(v1.z)};                                                           \
        tpk = (uint32_t)__builtin_amdgcn_readfirstlane(v1.w);                                                          \
    }
    for (;;) {
        GU_STEP(b0, b1)
        GU_STEP(b1, b0)
    }
#undef GU_STEP
#undef GU_LOAD
#undef GU_ITEM
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
            mx = fmaxf(mx, lane_xor<1>(mx));
            mx = fmaxf(mx, lane_xor<2>(mx));
            const int E = fixed_point_exponent<XPLANES>(mx);
            uint32_t word[XPLANES];
            int sx = chunk_digits(h, E, word);
            sx += lane_xor<1>(sx);
            sx += lane_xor<2>(sx);
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

constexpr int DN1_MAX_WAVES = 12;   // one wave per pick plus the shared expert's (k + 1 <= 12)

template <int BITS, int UPLM>
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
    // residual input of this block's rows (threads th < R, R < blockDim.x),
    // loaded now so that the final combine waits for no memory round trip
    float xin = 0.f;
    if (a.x_next && th < R) {
        const size_t o = (size_t)row0 + th;
        xin = a.x_is_bf16 ? bf16_to_float(((const uint16_t *)a.x)[o]) : ((const float *)a.x)[o];
    }
    int pe = 0, pp = 0;
    float pg = 0.f;
    if (wave == 0 && lane < k) {
        pe = a.idx[lane];
        pg = a.gate[lane];
        pp = a.pos[lane];
    }
    // the work item is read together with the count (items holds k + 1 entries, so slot `wave` exists)
    const WorkItem it = a.items[wave < k ? wave : k];
    const int n = *a.n_items;
    if (wave < n) {
        if (!fast) {
            slot = it.slot0;
            st.load(a, slot);
        }
        UTile<BITS, UPLM> wt;   // loads issued unconditionally: the waits that follow cover only what they need
        utile_load_all<BITS, UPLM % 4 == 0, UPLM>(wt, a.codes + ((size_t)it.expert * 3 + 2) * ((size_t)d * f * BITS / 8),
                                                  a.scales + ((size_t)it.expert * 3 + 2) * ((size_t)d * f / 256), f,
                                                  row0 + lane % R, (lane / R) * upl, upl, 1);
        st.store(a, upl, dstride, wdig, wsum, wscl);
        float res[1];
        utile_compute<BITS, 1, UPLM>(wt, R, upl, 1, wdig, dstride, wsum, units, wscl, units, HGROUP_UNITS,
                                     TOK_IDENTITY, res);
        if (lane < R) ybuf[slot * R + lane] = res[0];
    }
    if (wave == 0 && lane < k) {
        cg[lane] = pg;
        cp[lane] = pp;
        con[lane] = is_resident(a.mask, pe) ? 1 : 0;
    }
    __syncthreads();
    if (th < R) {   // row i = th: shared expert, then the picks in order (every LDS read issued before the sums)
        const int i = th;
        int sl[DN1_MAX_WAVES];
        float gv[DN1_MAX_WAVES], yv[DN1_MAX_WAVES];
        bool on[DN1_MAX_WAVES];
#pragma unroll
        for (int r = 0; r < DN1_MAX_WAVES; ++r) {
            sl[r] = r < k ? cp[r] : k;
            gv[r] = r < k ? cg[r] : 0.f;
            on[r] = r < k && con[r] != 0;
        }
#pragma unroll
        for (int r = 0; r < DN1_MAX_WAVES; ++r) yv[r] = ybuf[sl[r] * R + i];
        float s = ybuf[k * R + i];
#pragma unroll
        for (int r = 0; r < DN1_MAX_WAVES; ++r)
            if (on[r]) s = fmaf(gv[r], yv[r], s);
        const size_t o = (size_t)row0 + i;
        a.out[o] = s;
        if (a.x_next) a.x_next[o] = xin + s;
    }
}

// Any T <= 8 (the path for T >= 2): block = one work item (<= 2 slots) x
// 8R rows of Wd (8 waves, one tile of R rows each, every tile's codes
// requested at once; 64-row blocks of 8 waves measured faster than 64 rows
// of 4 waves, 128 rows and 32 rows).  The item's h rows are quantised into LDS
// while the codes load, exactly as the one-token kernel quantises them
// (per 32-column unit: exponent from the unit's max |h|, 6 balanced base-16
// digit planes, digit sum, 2^-E; the 4 chunks of a unit in 4 neighbouring
// lanes), and shared by the waves; expert outputs go to Y and the combine
// kernel sums them.  Per (slot, row) the arithmetic is the one-token
// kernel's, so results do not depend on T.
constexpr int DN_WAVES = 8, DN_QMAX = 1;   // Q = 1 tile of R rows per wave
constexpr int DN_THREADS = 64 * DN_WAVES;

__host__ __device__ inline int down_multi_lds_words(int f, int R) {
    const int S = 64 / R, units = f / 32;
    return ITEM_TOK * (units * XPLANES * 4 + S * 4) + 2 * ITEM_TOK * units;
}

template <int BITS, int NT, int UPLM>
__device__ __forceinline__ void down_multi_tiles(const LayerArgs &a, const WorkItem &it, const UTile<BITS, UPLM> *wt,
                                                 int R, int Q, int row0, const uint32_t *dig, int dstride,
                                                 const int *hsum, const float *hscl, const int *yrow) {
    const int lane = threadIdx.x & 63, units = a.f / 32, upl = units / (64 / R);
#pragma unroll
    for (int q = 0; q < DN_QMAX; ++q) {
        if (q >= Q) break;
        float res[NT];
        utile_compute_each<BITS, NT, UPLM>(wt[q], R, upl, 1, dig, dstride, hsum, units, hscl, units, HGROUP_UNITS,
                                           TOK_IDENTITY, res);
        if (lane < R) {
#pragma unroll
            for (int j = 0; j < NT; ++j) a.Y[(size_t)yrow[j] * a.d + row0 + q * R + lane] = res[j];
        }
    }
}

template <int BITS, int UPLM>
__global__ __launch_bounds__(DN_THREADS) void gemv_down_multi_kernel(LayerArgs a, int R, int Q) {
    extern __shared__ uint32_t lds[];
    const int th = threadIdx.x, wave = th >> 6, lane = th & 63;
    const int d = a.d, f = a.f, units = f / 32, S = 64 / R, upl = units / S;
    const int rows_blk = DN_WAVES * Q * R, chunks = d / rows_blk;
    const int item = blockIdx.x / chunks;   // < max_items: the list slot exists
    const WorkItem it = a.items[item];      // read together with the count (one round trip)
    if (item >= *a.n_items) return;
    // Y row of each slot (token order: pick r of token t at t*k + r); needed
    // only by the stores at the end, so its load overlaps the code stream
    int yrow[ITEM_TOK];
#pragma unroll
    for (int j = 0; j < ITEM_TOK; ++j) {
        const int sl = it.slot0 + min(j, it.ntok - 1);
        yrow[j] = (a.ytok && sl < a.T * a.k) ? a.perm[sl] : sl;
    }
    const int row0 = (blockIdx.x % chunks) * rows_blk + wave * Q * R;
    // loads in the order they are used: this thread's h chunk, then the code
    // tiles (all unconditional, so each wait covers only what it needs)
    const int cps = f / 8, nch = it.ntok * cps;   // 8-column chunks of the item's h rows
    constexpr int HPER = (ITEM_TOK * MAX_HUNITS * 4 + DN_THREADS - 1) / DN_THREADS;   // chunks per thread
    float4 hv[2 * HPER];
#pragma unroll
    for (int u = 0; u < HPER; ++u) {
        const int cc = min(th + DN_THREADS * u, nch - 1);
        const float4 *src = (const float4 *)(a.hf + (size_t)it.slot0 * f) + 2 * cc;
        hv[2 * u] = src[0];
        hv[2 * u + 1] = src[1];
    }
    const size_t mi = (size_t)it.expert * 3 + 2;
    const uint8_t *mcodes = a.codes + mi * ((size_t)d * f * BITS / 8);
    const uint16_t *mscl = a.scales + mi * ((size_t)d * f / 256);
    UTile<BITS, UPLM> wt[DN_QMAX];
#pragma unroll
    for (int q = 0; q < DN_QMAX; ++q) {
        const int r = row0 + (q < Q ? q : 0) * R + lane % R;
        if constexpr (UPLM % 4 == 0)
            utile_load_all<BITS, true, UPLM>(wt[q], mcodes, mscl, f, r, (lane / R) * upl, upl, 1);
        else
            utile_load_all<BITS, false, UPLM>(wt[q], mcodes, mscl, f, r, (lane / R) * upl, upl, 1);
    }
    const int dstride = units * XPLANES * 4 + S * 4;
    uint32_t *dig = lds;
    int *hsum = (int *)(lds + ITEM_TOK * dstride);
    float *hscl = (float *)(hsum + ITEM_TOK * units);
    // quantise the item's h rows: chunk c (8 columns) of slot j = c / (f/8);
    // the 4 chunks of a unit sit in 4 neighbouring lanes
#pragma unroll
    for (int u = 0; u < HPER; ++u) {
        const int c = th + DN_THREADS * u;
        const float h[8] = {hv[2 * u].x, hv[2 * u].y, hv[2 * u].z, hv[2 * u].w,
                            hv[2 * u + 1].x, hv[2 * u + 1].y, hv[2 * u + 1].z, hv[2 * u + 1].w};
        float mx = 0.f;
#pragma unroll
        for (int n = 0; n < 8; ++n) mx = fmaxf(mx, fabsf(h[n]));
        mx = fmaxf(mx, lane_xor<1>(mx));
        mx = fmaxf(mx, lane_xor<2>(mx));
        const int E = fixed_point_exponent<XPLANES>(mx);
        uint32_t word[XPLANES];
        int sx = chunk_digits(h, E, word);
        sx += lane_xor<1>(sx);
        sx += lane_xor<2>(sx);
        if (c < nch) {
            const int j = c / cps, U = (c % cps) / 4, qq = c % 4;
            uint32_t *dst = dig + j * dstride + dig_off(U, upl);
#pragma unroll
            for (int p = 0; p < XPLANES; ++p) dst[4 * p + qq] = word[p];
            if (qq == 0) {
                hsum[j * units + U] = sx;
                hscl[j * units + U] = ldexpf(1.f, -E);
            }
        }
    }
    // LDS-only barrier: the code tiles stay in flight, so the first tile's
    // products start as soon as its own loads land
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS stores are done
    __builtin_amdgcn_s_barrier();
    if (it.ntok == 1) down_multi_tiles<BITS, 1, UPLM>(a, it, wt, R, Q, row0, dig, dstride, hsum, hscl, yrow);
    else down_multi_tiles<BITS, 2, UPLM>(a, it, wt, R, Q, row0, dig, dstride, hsum, hscl, yrow);
}

// ------------------------------------------------------------- launchers
inline bool gemv_supported_impl(int d, int f, int bits) {
    if (bits != 3 && bits != 2) return false;
    if (unit_slices(d, 8) < 2 || unit_slices(f, 8) < 1) return false;   // decode tiles (R = 64/S in 8..32)
    if (d % 128 || f % 128 || f > 32 * MAX_HUNITS || d > 8192) return false;
    return true;
}

// Every kernel here stays within the 64 KiB of LDS a block gets by default;
// a launch that would need more is refused rather than attempted.
constexpr size_t LDS_LIMIT = 64 * 1024;

// One token: blocks of G gate + G up waves (G*R columns of h) per work
// item, plus the routing writer.  Two wave pairs per block halve the input
// staging and the top-k waves per column (measured faster than one pair and
// than four).
template <int BITS> hipError_t gateup_small_launch(const LayerArgs &a, int max_items, hipStream_t s) {
    const int R = 64 / unit_slices(a.d, 8);
    const int G = a.f % (2 * R) == 0 ? 2 : 1;   // the result area holds up to four wave pairs' rows
    const int off = align4(gateup_lds_words(a.d, R, 1, 1));   // the routing state is 16-byte aligned
    const size_t lds = 4 * ((size_t)off + small_route_lds_words(a.E));
    if (a.T != 1 || lds > LDS_LIMIT) return hipErrorInvalidValue;
    STRATA_LAUNCH(gemv_gateup_small_kernel<BITS>, dim3(max_items * (a.f / (G * R)) + 1), dim3(128 * G), lds, s, a,
                  R, off);
    return hipGetLastError();
}

// T <= 8: 8-wave job-loop blocks, one per compute unit (a wave holds two
// code tiles, ~200 VGPRs), plus the routing writer.
template <int BITS> hipError_t gateup_multi_launch(const LayerArgs &a, int max_items, int cus, hipStream_t s) {
    const int R = 64 / unit_slices(a.d, 8), upl = (a.d / 32) / (64 / R);
    const int off = align4(gateup_lds_words(a.d, R, a.T, ITEM_TOK));
    const size_t lds = 4 * ((size_t)off + small_route_lds_words(a.E) + 3 + small_route_table_words(a.T, a.k));
    const int jobs = max_items * (a.f / (R / 2)), wpb = 8;
    const int grid = std::min((jobs + wpb - 1) / wpb, std::max(1, cus)) + 1;
    if (R % 2 || a.f % (R / 2) || lds > LDS_LIMIT || a.T > CHUNK_TOK) return hipErrorInvalidValue;
    if (upl % 4 == 0)
        STRATA_LAUNCH((gemv_gateup_multi_kernel<BITS, true>), dim3(grid), dim3(64 * wpb), lds, s, a, R, off);
    else
        STRATA_LAUNCH((gemv_gateup_multi_kernel<BITS, false>), dim3(grid), dim3(64 * wpb), lds, s, a, R, off);
    return hipGetLastError();
}

template <int BITS> hipError_t down_multi_launch(const LayerArgs &a, int max_items, hipStream_t s) {
    const int R = 64 / unit_slices(a.f, 8), Q = 1, rows = DN_WAVES * Q * R;
    const size_t lds = 4 * (size_t)down_multi_lds_words(a.f, R);
    const int upl = (a.f / 32) / (64 / R);
    if (Q > DN_QMAX || a.d % rows || lds > LDS_LIMIT) return hipErrorInvalidValue;
    const dim3 grid(max_items * (a.d / rows)), block(DN_THREADS);
    if (upl == 3)   // d_ff = 768: 3 units per lane
        STRATA_LAUNCH((gemv_down_multi_kernel<BITS, 3>), grid, block, lds, s, a, R, Q);
    else if (upl == 1)
        STRATA_LAUNCH((gemv_down_multi_kernel<BITS, 1>), grid, block, lds, s, a, R, Q);
    else
        STRATA_LAUNCH((gemv_down_multi_kernel<BITS, UPL_MAX>), grid, block, lds, s, a, R, Q);
    return hipGetLastError();
}

// One token: block = one wave per work item (k + 1 of them) on R rows.
template <int BITS> hipError_t down_one_launch(const LayerArgs &a, hipStream_t s) {
    const int R = 64 / unit_slices(a.f, 8);
    const size_t lds = 4 * (size_t)down_one_lds_words(a.k, a.f, R);
    if (a.T != 1 || lds > LDS_LIMIT || a.k + 1 > DN1_MAX_WAVES) return hipErrorInvalidValue;
    const int upl = (a.f / 32) / (64 / R);
    const dim3 grid(a.d / R), block(64 * (a.k + 1));
    if (upl == 3)   // d_ff = 768
        STRATA_LAUNCH((gemv_down_rows_one_kernel<BITS, 3>), grid, block, lds, s, a, R);
    else if (upl == 1)
        STRATA_LAUNCH((gemv_down_rows_one_kernel<BITS, 1>), grid, block, lds, s, a, R);
    else
        STRATA_LAUNCH((gemv_down_rows_one_kernel<BITS, UPL_MAX>), grid, block, lds, s, a, R);
    return hipGetLastError();
}

}  // namespace strata
