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
// (row r, slice s) reads its row's 4 units (48 or 32 bytes) of each
// 128-column group in its slice with 16-byte loads and keeps per-token
// partial sums; the S slices are summed with cross-lane adds.
//
// Kernels:
//   gate/up: a block owns 2R rows j of gate and the same rows of up for one
//     work item (<= 8 tokens of one expert), so it forms h = silu(g) * u and
//     writes h already quantised (digit planes per 32-column group).
//   down, T <= 8: a block owns R rows of Wd for every work item, so the
//     weighted combine with the shared expert and the residual add happen in
//     the block (fixed order, no cross-block step).
//   down, larger T: a block per (work item, 2R-row tile) writes expert
//     outputs; the combine kernel sums them.
#pragma once
#include "routing.hpp"

namespace strata {

constexpr int MAXQ = 4;           // 128-column groups per lane slice
constexpr int HGROUP_UNITS = 1;   // h is quantised per 32 columns
constexpr int XGROUP_UNITS = 8;   // the layer input per 256 columns
constexpr int MAX_HUNITS = 24;    // f <= 768 on this path

template <int BITS> struct Fmt {
    static constexpr int UB = BITS == 3 ? 12 : 8;  // bytes per 32-code unit
    static constexpr int DW = UB;                  // dwords per 128-column group (4 units)
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

// Codes and block scales of rows [row0, row0+R) of one packed matrix
// [out][in], for this lane's slice.
template <int BITS> struct WTile {
    uint32_t w[MAXQ][Fmt<BITS>::DW];
    uint32_t sc[MAXQ];  // fp16 scale bits per 128-column group (32-bit slots: packing
                        // 16-bit loads would stall the load stream)

    __device__ __forceinline__ void load(const uint8_t *__restrict__ mat, const uint16_t *__restrict__ msc,
                                         int in, int row0, int R) {
        const int lane = threadIdx.x & 63;
        const int S = 64 / R, Q = in / 128, QPS = Q / S;
        const int r = row0 + lane % R, s = lane / R;
        constexpr int UB = Fmt<BITS>::UB;
        const uint8_t *base = mat + ((size_t)((r / 16) * Q + s * QPS) * 16 + (r % 16)) * 4 * UB;
#pragma unroll
        for (int qq = 0; qq < MAXQ; ++qq) {
            if (qq < QPS) {
                const uint4 *p = (const uint4 *)(base + (size_t)qq * 16 * 4 * UB);
#pragma unroll
                for (int i = 0; i < Fmt<BITS>::DW / 4; ++i) {
                    const uint4 v = p[i];
                    w[qq][4 * i] = v.x;
                    w[qq][4 * i + 1] = v.y;
                    w[qq][4 * i + 2] = v.z;
                    w[qq][4 * i + 3] = v.w;
                }
                sc[qq] = (uint32_t)msc[((long)r * in + (s * QPS + qq) * 128) / 256];
            }
        }
    }
};

// Row sums of a loaded tile against NT tokens whose digit planes sit in LDS
// (dig + t*dstride, laid out by dig_off), with per-(token, unit) digit sums
// usum[t*ustride + U] and per-(token, group) scales gscl[t*gstride + U/upg].
// res[t] is complete in lanes with s == 0 (lane < R).
template <int BITS, int NT>
__device__ __forceinline__ void tile_compute(const WTile<BITS> &wt, int in, int R, const uint32_t *__restrict__ dig,
                                             int dstride, const int *__restrict__ usum, int ustride,
                                             const float *__restrict__ gscl, int gstride, int upg, float res[NT]) {
    const int lane = threadIdx.x & 63;
    const int S = 64 / R, Q = in / 128, QPS = Q / S;
    const int s = lane / R;
    const int ups = QPS * 4;
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
    for (int qq = 0; qq < MAXQ; ++qq) {
        if (qq < QPS) {
            const int q = s * QPS + qq;
            const float scl = 0.5f * half_to_float((uint16_t)wt.sc[qq]);
#pragma unroll
            for (int uu = 0; uu < 4; ++uu) {
                const int U = q * 4 + uu;
                uint32_t N[4];
                unit_nibbles<BITS>(&wt.w[qq][uu * Fmt<BITS>::UB / 4], N);
                const int off = dig_off(U, ups);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const uint4 *dp = (const uint4 *)(dig + t * dstride + off);
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
                    sx[t] += usum[t * ustride + U];
                }
                // flush at the end of a scale group or of the slice (a 128-column
                // group never straddles two weight blocks)
                if ((U + 1) % upg == 0 || (qq == QPS - 1 && uu == 3)) {
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const float v = digits_value(acc[t], Fmt<BITS>::C2, sx[t]);
                        res[t] = fmaf(v, scl * gscl[t * gstride + U / upg], res[t]);
                        sx[t] = 0;
#pragma unroll
                        for (int p = 0; p < XPLANES; ++p) acc[t][p] = 0;
                    }
                }
            }
        }
    }
    for (int o = R; o < 64; o <<= 1) {
#pragma unroll
        for (int t = 0; t < NT; ++t) res[t] += __shfl_xor(res[t], o, WAVE);
    }
}

// Quantise 8 consecutive values with exponent E into one word per digit
// plane (nibble n = digit of value n); returns the sum of the fixed-point values.
__device__ __forceinline__ int chunk_digits(const float v[8], int E, uint32_t word[XPLANES]) {
    int sx = 0;
#pragma unroll
    for (int p = 0; p < XPLANES; ++p) word[p] = 0;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const int X = (int)rintf(ldexpf(v[n], E));
        sx += X;
        int dg[XPLANES];
        to_digits<XPLANES>(X, dg);
#pragma unroll
        for (int p = 0; p < XPLANES; ++p) word[p] |= ((uint32_t)dg[p] & 15u) << (4 * n);
    }
    return sx;
}

__device__ __forceinline__ int slot_token(const LayerArgs &a, const WorkItem &it, int j) {
    const int slot = it.slot0 + j;
    return it.expert == a.E ? slot - a.T * a.k : a.perm[slot] / a.k;
}

// ---------------------------------------------------------- gate and up
// Block = 4 waves: waves 0,1 compute gate rows j0 .. j0+2R-1 (R each),
// waves 2,3 the same rows of up.  Then h = silu(g) * u for those 2R rows and
// the item's tokens, quantised per 32 columns, goes to hq/hsum/hscl.
template <int BITS, int NT>
__device__ __forceinline__ void gateup_body(const LayerArgs &a, const WorkItem &it, const int *toks, int R,
                                            int j0, uint32_t *lds) {
    const int th = threadIdx.x, wave = th >> 6, lane = th & 63;
    const int d = a.d, f = a.f;
    const int m = wave >> 1;  // 0 gate, 1 up
    const int row0 = j0 + (wave & 1) * R;
    const size_t mat_bytes = (size_t)d * f * BITS / 8;
    const size_t mat_blocks = (size_t)d * f / 256;
    const size_t mi = (size_t)it.expert * 3 + m;
    WTile<BITS> wt;
    wt.load(a.codes + mi * mat_bytes, a.scales + mi * mat_blocks, d, row0, R);

    // stage the tokens' digit planes, unit sums and group scales (every
    // staging load of a pass is issued before any LDS write)
    const int Q = d / 128, G = (d + 255) / 256, units = d / 32;
    const int S = 64 / R, ups = (Q / S) * 4;
    const int dstride = units * XPLANES * 4 + S * 4;
    uint32_t *ldig = lds;
    int *lsum = (int *)(lds + NT * dstride);
    float *lscl = (float *)(lsum + NT * units);
    float *gu = lscl + NT * G;  // [2][NT][2R]
    const int n16 = units * XPLANES;  // uint4 per token
    for (int base = 0; base < NT * n16; base += 256 * 4) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = min(base + th + 256 * u, NT * n16 - 1), j = i / n16, q = i % n16;
            v[u] = ((const uint4 *)(a.xq + (size_t)toks[j] * units * XPLANES * 4))[q];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = base + th + 256 * u;
            if (i < NT * n16) {
                const int j = i / n16, q = i % n16, U = q / XPLANES, p = q % XPLANES;
                *(uint4 *)(ldig + j * dstride + dig_off(U, ups) + 4 * p) = v[u];
            }
        }
    }
    for (int q = th; q < NT * (units + G); q += 256) {
        const int j = q / (units + G), i = q % (units + G);
        if (i < units) lsum[j * units + i] = a.xsum[(size_t)toks[j] * units + i];
        else lscl[j * G + (i - units)] = a.xscl[(size_t)toks[j] * G + (i - units)];
    }
    __syncthreads();
    float res[NT];
    tile_compute<BITS, NT>(wt, d, R, ldig, dstride, lsum, units, lscl, G, XGROUP_UNITS, res);
    const int hb = 2 * R;
    if (lane < R) {
#pragma unroll
        for (int j = 0; j < NT; ++j) gu[(m * NT + j) * hb + (wave & 1) * R + lane] = res[j];
    }
    __syncthreads();
    // h for NT tokens x hb columns: one chunk of 8 columns per lane of wave 0
    if (wave == 0) {
        const int cpt = hb / 8;  // chunks per token
        const int c = lane % cpt, j = lane / cpt;
        const bool valid = j < NT;
        const int jj = valid ? j : 0;
        float h[8];
        float mx = 0.f;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const float g = gu[jj * hb + c * 8 + n];
            const float u = gu[(NT + jj) * hb + c * 8 + n];
            h[n] = valid ? g / (1.f + expf(-g)) * u : 0.f;
            mx = fmaxf(mx, fabsf(h[n]));
        }
        // a 32-column group is 4 consecutive lanes
        mx = fmaxf(mx, __shfl_xor(mx, 1, WAVE));
        mx = fmaxf(mx, __shfl_xor(mx, 2, WAVE));
        const int E = fixed_point_exponent<XPLANES>(mx);
        uint32_t word[XPLANES];
        int sx = chunk_digits(h, E, word);
        sx += __shfl_xor(sx, 1, WAVE);
        sx += __shfl_xor(sx, 2, WAVE);
        if (valid) {
            const int slot = it.slot0 + j;
            const int col = j0 + c * 8, U = col / 32, i = (col / 8) % 4;
            uint32_t *dst = a.hq + ((size_t)slot * (f / 32) + U) * (XPLANES * 4);
#pragma unroll
            for (int p = 0; p < XPLANES; ++p) dst[p * 4 + i] = word[p];
            if (i == 0) {
                a.hsum[(size_t)slot * (f / 32) + U] = sx;
                a.hscl[(size_t)slot * (f / 32) + U] = ldexpf(1.f, -E);
            }
        }
    }
}

__host__ __device__ inline int gateup_lds_words(int d, int R, int nt) {
    const int S = 64 / R;
    const int dstride = (d / 32) * XPLANES * 4 + S * 4;
    return nt * dstride + nt * (d / 32) + nt * ((d + 255) / 256) + 2 * nt * 2 * R;
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


// T <= 8: every block takes the top-k of the T tokens itself from the
// router logits (a few KB), derives its own work item and runs it; the last
// block writes the routing outputs and the work list instead.
template <int BITS, int NTMAX>
__global__ __launch_bounds__(256) void gemv_gateup_small_kernel(LayerArgs a, int R, int route_off) {
    extern __shared__ uint32_t lds[];
    const SmallRoute L(lds + route_off, a.E);
    small_route_compute(a, L);
    if (blockIdx.x == gridDim.x - 1) {
        small_route_write(a, L);
        return;
    }
    const int wg_per_item = a.f / (2 * R);
    WorkItem it;
    int toks[CHUNK_TOK];
    if (!small_route_item(a, L, blockIdx.x / wg_per_item, it, toks)) return;
    const int j0 = (blockIdx.x % wg_per_item) * 2 * R;
#define GU(n) gateup_body<BITS, n>(a, it, toks, R, j0, lds)
    NT_SWITCH(GU)
#undef GU
}

// ----------------------------------------------------------------- down
// The h digit planes, unit sums and group scales of NT consecutive slots,
// staged through registers into one wave's LDS region.  load() issues the
// global loads; store() writes them (so a caller can issue other loads in
// between without the in-order load counter making store() wait for them).
template <int NT> struct HStage {
    static constexpr int PER = (NT * MAX_HUNITS * XPLANES + 63) / 64;  // uint4 per lane
    static constexpr int PERS = (NT * MAX_HUNITS + 63) / 64;           // sums / scales per lane
    uint4 v[PER];
    int sv[PERS];
    float cv[PERS];

    __device__ __forceinline__ void load(const LayerArgs &a, int slot0) {
        const int lane = threadIdx.x & 63, units = a.f / 32;
        const int n16 = NT * units * XPLANES, ns = NT * units;
        const uint4 *src = (const uint4 *)(a.hq + (size_t)slot0 * units * XPLANES * 4);
#pragma unroll
        for (int u = 0; u < PER; ++u) v[u] = src[min(lane + 64 * u, n16 - 1)];
#pragma unroll
        for (int u = 0; u < PERS; ++u) {
            const int i = min(lane + 64 * u, ns - 1);
            sv[u] = a.hsum[(size_t)slot0 * units + i];
            cv[u] = a.hscl[(size_t)slot0 * units + i];
        }
    }

    __device__ __forceinline__ void store(const LayerArgs &a, int ups, int dstride, uint32_t *wdig, int *wsum,
                                          float *wscl) const {
        const int lane = threadIdx.x & 63, units = a.f / 32;
        const int n16u = units * XPLANES, n16 = NT * n16u, ns = NT * units;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int i = lane + 64 * u;
            if (i < n16) {
                const int j = i / n16u, q = i % n16u, U = q / XPLANES, p = q % XPLANES;
                *(uint4 *)(wdig + j * dstride + dig_off(U, ups) + 4 * p) = v[u];
            }
        }
#pragma unroll
        for (int u = 0; u < PERS; ++u) {
            const int i = lane + 64 * u;
            if (i < ns) {
                wsum[i] = sv[u];
                wscl[i] = cv[u];
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
__device__ __forceinline__ void down_item(const LayerArgs &a, const WorkItem &it, const WTile<BITS> &wt, int R,
                                          int row0, uint32_t *wdig, float res[CHUNK_TOK], WTile<BITS> &next,
                                          bool do_next, int next_expert) {
    const int d = a.d, f = a.f, units = f / 32;
    const int S = 64 / R, ups = ((f / 128) / S) * 4;
    const int dstride = units * XPLANES * 4 + S * 4;
    int *wsum = (int *)(wdig + NT * dstride);
    float *wscl = (float *)(wsum + NT * units);
    HStage<NT> st;
    st.load(a, it.slot0);
    if (do_next)
        next.load(a.codes + ((size_t)next_expert * 3 + 2) * ((size_t)d * f * BITS / 8),
                  a.scales + ((size_t)next_expert * 3 + 2) * ((size_t)d * f / 256), f, row0, R);
    st.store(a, ups, dstride, wdig, wsum, wscl);
    float r[NT];
    tile_compute<BITS, NT>(wt, f, R, wdig, dstride, wsum, units, wscl, units, HGROUP_UNITS, r);
#pragma unroll
    for (int j = 0; j < NT; ++j) res[j] = r[j];
}

// T <= 8: block = 4 waves on rows [row0, row0+R) of Wd for every work item;
// wave w runs items w, w+4, ... (the next item's codes are loaded while the
// current one computes), expert outputs land in LDS, then the block forms
// out[t] = y_shared[t] + sum_{r asc, resident} gate[t][r] * y[slot(t, r)] and
// x_next = x + out for those rows.
template <int BITS, int NTMAX>
__global__ __launch_bounds__(256) void gemv_down_rows_kernel(LayerArgs a, int R) {
    extern __shared__ uint32_t lds[];
    const int th = threadIdx.x, wave = th >> 6, lane = th & 63;
    const int d = a.d, f = a.f, T = a.T, k = a.k;
    const int row0 = blockIdx.x * R;
    const int nslots = T * k + T;
    float *ybuf = (float *)lds;  // [nslots][R]
    uint32_t *wdig = lds + nslots * R + wave * down_wave_lds_words(f, R, NTMAX);
    const int n = *a.n_items;
    const size_t mat_bytes = (size_t)d * f * BITS / 8;
    const size_t mat_blocks = (size_t)d * f / 256;
    // two register tiles used alternately (named, so no dynamic register
    // indexing); item `item` computes from one while item + 4's codes load into the other
    WTile<BITS> buf0, buf1;
    WorkItem cur = a.items[min(wave, n - 1)];
    if (wave < n)
        buf0.load(a.codes + ((size_t)cur.expert * 3 + 2) * mat_bytes,
                  a.scales + ((size_t)cur.expert * 3 + 2) * mat_blocks, f, row0, R);
    for (int item = wave; item < n; item += 8) {
        {
            const WorkItem it = cur;
            const bool has = item + 4 < n;
            if (has) cur = a.items[item + 4];
            float res[CHUNK_TOK];
#define DN(nn) down_item<BITS, nn>(a, it, buf0, R, row0, wdig, res, buf1, has, cur.expert)
            NT_SWITCH(DN)
#undef DN
            if (lane < R)
                for (int j = 0; j < it.ntok; ++j) ybuf[(it.slot0 + j) * R + lane] = res[j];
        }
        if (item + 4 < n) {
            const WorkItem it = cur;
            const bool has = item + 8 < n;
            if (has) cur = a.items[item + 8];
            float res[CHUNK_TOK];
#define DN(nn) down_item<BITS, nn>(a, it, buf1, R, row0, wdig, res, buf0, has, cur.expert)
            NT_SWITCH(DN)
#undef DN
            if (lane < R)
                for (int j = 0; j < it.ntok; ++j) ybuf[(it.slot0 + j) * R + lane] = res[j];
        }
    }
    __syncthreads();
    for (int q = th; q < T * R; q += 256) {
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
    WTile<BITS> wt;
    wt.load(a.codes + ((size_t)it.expert * 3 + 2) * ((size_t)d * f * BITS / 8),
            a.scales + ((size_t)it.expert * 3 + 2) * ((size_t)d * f / 256), f, row0, R);
    uint32_t *wdig = lds + wave * down_wave_lds_words(f, R, NTMAX);
    float res[CHUNK_TOK];
#define DN(nn) down_item<BITS, nn>(a, it, wt, R, row0, wdig, res, wt, false, 0)
    NT_SWITCH(DN)
#undef DN
    if (lane < R)
        for (int j = 0; j < it.ntok; ++j) a.Y[(size_t)(it.slot0 + j) * d + row0 + lane] = res[j];
}

// ------------------------------------------------------------- launchers
// Column slices per wave for an input width `in`: the most slices (up to 4)
// that split the 128-column groups evenly with at most MAXQ per slice.
static inline int pick_slices(int in) {
    const int Q = in / 128;
    for (int S = 4; S >= 1; S >>= 1)
        if (Q % S == 0 && Q / S <= MAXQ) return S;
    return 0;
}

inline bool gemv_supported_impl(int d, int f, int bits) {
    if (bits != 3 && bits != 2) return false;
    if (d % 128 || f % 128 || f > 32 * MAX_HUNITS || d > 8192) return false;
    const int Sg = pick_slices(d), Sd = pick_slices(f);
    if (!Sg || !Sd) return false;
    const int Rg = 64 / Sg, Rd = 64 / Sd;
    if (Rg > 32) return false;             // one wave forms h of 8 tokens x 2R columns
    if (f % (2 * Rg)) return false;        // gate/up blocks own 2R rows of f
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
            case 1: hipLaunchKernelGGL((KER<BITS, 1>), grid, dim3(block), lds, s, __VA_ARGS__); break; \
            case 2: hipLaunchKernelGGL((KER<BITS, 2>), grid, dim3(block), lds, s, __VA_ARGS__); break; \
            case 4: hipLaunchKernelGGL((KER<BITS, 4>), grid, dim3(block), lds, s, __VA_ARGS__); break; \
            case 5: hipLaunchKernelGGL((KER<BITS, 5>), grid, dim3(block), lds, s, __VA_ARGS__); break; \
            default: hipLaunchKernelGGL((KER<BITS, 8>), grid, dim3(block), lds, s, __VA_ARGS__); break; \
        }                                                                                            \
    } while (0)

template <int BITS> hipError_t gateup_small_launch(const LayerArgs &a, int max_items, hipStream_t s) {
    const int R = 64 / pick_slices(a.d);
    const int nt = nt_round(ntmax_for(a.T));
    const int off = gateup_lds_words(a.d, R, nt);
    const size_t lds = 4 * ((size_t)off + small_route_lds_words(a.E));
    const dim3 grid(max_items * (a.f / (2 * R)) + 1);
    LAUNCH_NT(gemv_gateup_small_kernel, BITS, nt, grid, 256, lds, s, a, R, off);
    return hipGetLastError();
}

template <int BITS> hipError_t down_launch(const LayerArgs &a, int max_items, hipStream_t s) {
    const int R = 64 / pick_slices(a.f);
    const int nt = nt_round(ntmax_for(a.T));
    const size_t lds = 4 * (size_t)2 * down_wave_lds_words(a.f, R, nt);
    const dim3 grid(max_items * (a.d / (2 * R)));
    LAUNCH_NT(gemv_down_items_kernel, BITS, nt, grid, 128, lds, s, a, R);
    return hipGetLastError();
}

static inline size_t down_rows_lds(int T, int k, int f, int R, int nt) {
    const int nslots = T * k + T;
    return 4 * ((size_t)nslots * R + 4 * (size_t)down_wave_lds_words(f, R, nt));
}

template <int BITS> hipError_t down_rows_launch(const LayerArgs &a, hipStream_t s) {
    const int R = 64 / pick_slices(a.f);
    const int nt = nt_round(ntmax_for(a.T));
    const size_t lds = down_rows_lds(a.T, a.k, a.f, R, nt);
    const dim3 grid(a.d / R);
    LAUNCH_NT(gemv_down_rows_kernel, BITS, nt, grid, 256, lds, s, a, R);
    return hipGetLastError();
}

}  // namespace strata
