// Host-CPU evaluation of the experts a GPU does not hold: for every missed
// (token t, expert e, gate) of a layer, y_add[t] += gate * FFN_e(u_t), where
// FFN_e(u) = Wd_e (silu(Wg_e u) * (Wu_e u)) over the packed 3-/2-bit blocks.
//
// The pages' engine computes the cached experts on the GPU and the ones that
// miss the cache on the CPU at the same time, then adds the two (wiselychen.com,
// technique 2 "專家快取與 CPU／GPU 分工"; digiland.tw, "Strata 實測", item 2 "CPU 與
// GPU 的協同運算（Co-processing）"; tutuge.me "⚙️ 125B 是怎么塞进游戏 PC 的").
//
// This file is compiled once per instruction set (AVX-512 and AVX2, the
// namespace named by HX_NS) and holds only the two task functions below,
// with no library templates, so nothing built for one instruction set can
// be shared with the other at link time; the caller picks one set at run
// time and runs the tasks on its threads.  Arithmetic is fp32 with fused
// multiply-adds: weights scale * (code - c0) are exact in fp32; every dot
// product keeps four 16-lane partial sums and adds them in a fixed tree,
// so results do not depend on the thread count.
//
// Two phases:
//   A. per (expert, rows of h): decode the gate and up rows once, then
//      h[m][j] = silu(g) * u for every miss m of that expert;
//   B. per block of output columns (rows of Wd): for every expert in
//      ascending order, decode its down rows once, then y_add[t_m][i] +=
//      gate_m * (Wd_i . h[m]) for its misses in list order.  Each task owns
//      its columns of y_add, so every sum is formed in a fixed order.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "host_experts.hpp"

#ifndef HX_NS
#error "compile with -DHX_NS=<namespace of this instruction set>"
#endif

namespace HX_NS {

typedef float vf __attribute__((vector_size(64)));      // 16 fp32 lanes
typedef uint32_t vu __attribute__((vector_size(64)));
typedef int32_t vi __attribute__((vector_size(64)));

// Exact value of an IEEE binary16 bit pattern: normal numbers by moving the
// exponent and mantissa fields into place, subnormals as m * 2^-24 (exact).
static inline float half_to_float(uint16_t h) {
    const uint32_t s = (uint32_t)(h & 0x8000u) << 16, e = (h >> 10) & 0x1F, m = h & 0x3FF;
    uint32_t u;
    if (e == 0) {
        const float v = (float)m * 0x1p-24f;
        memcpy(&u, &v, 4);
    } else if (e == 31) {
        u = m ? 0x7FC00000u : 0x7F800000u;
    } else {
        u = ((e + 112) << 23) | (m << 13);
    }
    u |= s;
    float v;
    memcpy(&v, &u, 4);
    return v;
}

static inline uint32_t rd32(const uint8_t *p) {
    uint32_t v;
    memcpy(&v, p, 4);
    return v;
}

// The 32 codes of one unit, minus c0, as two vectors (places 0-15, 16-31).
// 3-bit unit: words A, B, C; places j < 24 are the low 3 bits of nibble
// j % 8 of word j / 8; places 24 + n gather bit 3 of nibble n of A, B, C.
static inline void unit_codes3(const uint8_t *p, float c0, vf &lo, vf &hi) {
    const uint32_t A = rd32(p), B = rd32(p + 4), C = rd32(p + 8);
    const vu sh = {0, 4, 8, 12, 16, 20, 24, 28, 0, 4, 8, 12, 16, 20, 24, 28};
    const vu sh3 = {0, 4, 8, 12, 16, 20, 24, 28, 3, 7, 11, 15, 19, 23, 27, 31};
    const vu ab = {A, A, A, A, A, A, A, A, B, B, B, B, B, B, B, B};
    const vu ca = {C, C, C, C, C, C, C, C, A, A, A, A, A, A, A, A};
    const vu zb = {0, 0, 0, 0, 0, 0, 0, 0, B, B, B, B, B, B, B, B};
    const vu zc = {0, 0, 0, 0, 0, 0, 0, 0, C, C, C, C, C, C, C, C};
    const vu m7 = {7, 7, 7, 7, 7, 7, 7, 7, 1, 1, 1, 1, 1, 1, 1, 1};
    const vu c_lo = (ab >> sh) & 7u;
    const vu c_hi = ((ca >> sh3) & m7) | (((zb >> sh3) & 1u) << 1) | (((zc >> sh3) & 1u) << 2);
    lo = __builtin_convertvector((vi)c_lo, vf) - c0;
    hi = __builtin_convertvector((vi)c_hi, vf) - c0;
}

// 2-bit unit: words A (places 0-15) and B (16-31); place j of a word is
// bits [4 (j % 8) + 2 (j / 8), +2).
static inline void unit_codes2(const uint8_t *p, float c0, vf &lo, vf &hi) {
    const uint32_t A = rd32(p), B = rd32(p + 4);
    const vu sh = {0, 4, 8, 12, 16, 20, 24, 28, 2, 6, 10, 14, 18, 22, 26, 30};
    const vu a = {A, A, A, A, A, A, A, A, A, A, A, A, A, A, A, A};
    const vu b = {B, B, B, B, B, B, B, B, B, B, B, B, B, B, B, B};
    lo = __builtin_convertvector((vi)((a >> sh) & 3u), vf) - c0;
    hi = __builtin_convertvector((vi)((b >> sh) & 3u), vf) - c0;
}

// Row r of a packed matrix [out][in] as fp32 weights scale * (code - c0).
static void decode_row(int bits, const uint8_t *mat, const uint16_t *msc, int in, int r, float *w) {
    const int UB = bits == 3 ? 12 : 8;
    const float c0 = bits == 3 ? 3.5f : 1.5f;
    const int64_t rowbase = (int64_t)(r >> 4) * (in >> 7);
    for (int c = 0; c < in; c += 32) {
        const int64_t off = ((rowbase + (c >> 7)) * 16 + (r & 15)) * 4 * UB + ((c & 127) >> 5) * UB;
        vf lo, hi;
        if (bits == 3) unit_codes3(mat + off, c0, lo, hi);
        else unit_codes2(mat + off, c0, lo, hi);
        const float s = half_to_float(msc[((int64_t)r * in + c) >> 8]);
        lo *= s;
        hi *= s;
        memcpy(w + c, &lo, 64);
        memcpy(w + c + 16, &hi, 64);
    }
}

static inline float hsum(vf v) {
    // fixed tree: 16 -> 8 -> 4 -> 2 -> 1
    float a[16];
    memcpy(a, &v, 64);
    for (int s = 8; s >= 1; s >>= 1)
        for (int i = 0; i < s; ++i) a[i] += a[i + s];
    return a[0];
}

// 16 floats from any address, as one vector load (a single-vector copy; a
// copy into an array of vectors went through the stack as 16-byte pieces and
// stalled every reload of it).
static inline vf ldv(const float *p) {
    vf v;
    __builtin_memcpy(&v, p, sizeof v);
    return v;
}

// w . x over n (a multiple of 64) columns: four partial sums of 16 lanes
// (columns i % 64 in [16q, 16q + 16) go to sum q), added in a fixed order.
static inline float dot(const float *w, const float *x, int n) {
    vf a0 = {}, a1 = {}, a2 = {}, a3 = {};
    for (int i = 0; i < n; i += 64) {
        a0 += ldv(w + i) * ldv(x + i);
        a1 += ldv(w + i + 16) * ldv(x + i + 16);
        a2 += ldv(w + i + 32) * ldv(x + i + 32);
        a3 += ldv(w + i + 48) * ldv(x + i + 48);
    }
    return hsum((a0 + a1) + (a2 + a3));
}

// Two rows against one vector (the gate and up rows of one h column), each
// summed exactly as dot() sums it.
static inline void dot2(const float *w0, const float *w1, const float *x, int n, float &r0, float &r1) {
    vf a0 = {}, a1 = {}, a2 = {}, a3 = {}, c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < n; i += 64) {
        const vf b0 = ldv(x + i), b1 = ldv(x + i + 16), b2 = ldv(x + i + 32), b3 = ldv(x + i + 48);
        a0 += ldv(w0 + i) * b0;
        a1 += ldv(w0 + i + 16) * b1;
        a2 += ldv(w0 + i + 32) * b2;
        a3 += ldv(w0 + i + 48) * b3;
        c0 += ldv(w1 + i) * b0;
        c1 += ldv(w1 + i + 16) * b1;
        c2 += ldv(w1 + i + 32) * b2;
        c3 += ldv(w1 + i + 48) * b3;
    }
    r0 = hsum((a0 + a1) + (a2 + a3));
    r1 = hsum((c0 + c1) + (c2 + c3));
}

// The gate and up rows against two vectors, each of the four dot products
// summed exactly as dot() sums it (the row loads are shared).
static inline void dot2x2(const float *w0, const float *w1, const float *x, const float *y, int n, float r[4]) {
    vf a0 = {}, a1 = {}, a2 = {}, a3 = {}, c0 = {}, c1 = {}, c2 = {}, c3 = {};
    vf e0 = {}, e1 = {}, e2 = {}, e3 = {}, g0 = {}, g1 = {}, g2 = {}, g3 = {};
    for (int i = 0; i < n; i += 64) {
        const vf p0 = ldv(w0 + i), p1 = ldv(w0 + i + 16), p2 = ldv(w0 + i + 32), p3 = ldv(w0 + i + 48);
        const vf q0 = ldv(w1 + i), q1 = ldv(w1 + i + 16), q2 = ldv(w1 + i + 32), q3 = ldv(w1 + i + 48);
        const vf b0 = ldv(x + i), b1 = ldv(x + i + 16), b2 = ldv(x + i + 32), b3 = ldv(x + i + 48);
        a0 += p0 * b0;
        a1 += p1 * b1;
        a2 += p2 * b2;
        a3 += p3 * b3;
        c0 += q0 * b0;
        c1 += q1 * b1;
        c2 += q2 * b2;
        c3 += q3 * b3;
        const vf d0 = ldv(y + i), d1 = ldv(y + i + 16), d2 = ldv(y + i + 32), d3 = ldv(y + i + 48);
        e0 += p0 * d0;
        e1 += p1 * d1;
        e2 += p2 * d2;
        e3 += p3 * d3;
        g0 += q0 * d0;
        g1 += q1 * d1;
        g2 += q2 * d2;
        g3 += q3 * d3;
    }
    r[0] = hsum((a0 + a1) + (a2 + a3));
    r[1] = hsum((c0 + c1) + (c2 + c3));
    r[2] = hsum((e0 + e1) + (e2 + e3));
    r[3] = hsum((g0 + g1) + (g2 + g3));
}

// One row against four vectors, each summed exactly as dot() sums it.
static inline void dotx4(const float *w, const float *const x[4], int n, float r[4]) {
    vf a[4][4] = {};
    for (int i = 0; i < n; i += 64) {
        const vf p0 = ldv(w + i), p1 = ldv(w + i + 16), p2 = ldv(w + i + 32), p3 = ldv(w + i + 48);
#pragma GCC unroll 4
        for (int v = 0; v < 4; ++v) {
            a[v][0] += p0 * ldv(x[v] + i);
            a[v][1] += p1 * ldv(x[v] + i + 16);
            a[v][2] += p2 * ldv(x[v] + i + 32);
            a[v][3] += p3 * ldv(x[v] + i + 48);
        }
    }
#pragma GCC unroll 4
    for (int v = 0; v < 4; ++v) r[v] = hsum((a[v][0] + a[v][1]) + (a[v][2] + a[v][3]));
}

static inline float silu_mul(float g, float u) { return g / (1.f + expf(-g)) * u; }

// Phase A task: rows [j0, j1) of h for every miss of expert e.
void gateup_rows(const HostMissArgs &a, int e, int j0, int j1) {
    const int d = a.d, f = a.f;
    const int64_t mat_bytes = (int64_t)d * f * a.bits / 8, mat_blocks = (int64_t)d * f / 256;
    const uint8_t *cg = a.codes + (int64_t)e * 3 * mat_bytes, *cu = cg + mat_bytes;
    const uint16_t *sg = a.scales + (int64_t)e * 3 * mat_blocks, *su = sg + mat_blocks;
    alignas(64) float wg[HOST_MAX_D], wu[HOST_MAX_D];
    for (int j = j0; j < j1; ++j) {
        decode_row(a.bits, cg, sg, d, j, wg);
        decode_row(a.bits, cu, su, d, j, wu);
        int q = a.gstart[e];
        for (; q + 2 <= a.gstart[e + 1]; q += 2) {   // two misses per pass over the rows
            const int m0 = a.order[q], m1 = a.order[q + 1];
            float r[4];
            dot2x2(wg, wu, a.u + (int64_t)a.miss_te[2 * m0] * d, a.u + (int64_t)a.miss_te[2 * m1] * d, d, r);
            a.h[(int64_t)m0 * f + j] = silu_mul(r[0], r[1]);
            a.h[(int64_t)m1 * f + j] = silu_mul(r[2], r[3]);
        }
        for (; q < a.gstart[e + 1]; ++q) {
            const int m = a.order[q], t = a.miss_te[2 * m];
            float g, u;
            dot2(wg, wu, a.u + (int64_t)t * d, d, g, u);
            a.h[(int64_t)m * f + j] = silu_mul(g, u);
        }
    }
}

// Phase B task: columns [i0, i1) of y_add, experts[0..ne) in order, each
// expert's misses in list order.
void down_cols(const HostMissArgs &a, const int32_t *experts, int ne, int i0, int i1) {
    const int d = a.d, f = a.f;
    const int64_t mat_bytes = (int64_t)d * f * a.bits / 8, mat_blocks = (int64_t)d * f / 256;
    for (int t = 0; t < a.T; ++t)
        for (int i = i0; i < i1; ++i) a.y_add[(int64_t)t * d + i] = 0.f;
    alignas(64) float wd[HOST_MAX_F];
    for (int x = 0; x < ne; ++x) {
        const int e = experts[x];
        const uint8_t *cd = a.codes + ((int64_t)e * 3 + 2) * mat_bytes;
        const uint16_t *sd = a.scales + (int64_t)e * 3 * mat_blocks + 2 * mat_blocks;
        for (int i = i0; i < i1; ++i) {
            decode_row(a.bits, cd, sd, f, i, wd);
            int q = a.gstart[e];
            for (; q + 4 <= a.gstart[e + 1]; q += 4) {   // four misses per pass over the row, added in list order
                const float *hx[4];
                for (int v = 0; v < 4; ++v) hx[v] = a.h + (int64_t)a.order[q + v] * f;
                float r[4];
                dotx4(wd, hx, f, r);
                for (int v = 0; v < 4; ++v) {
                    const int m = a.order[q + v];
                    a.y_add[(int64_t)a.miss_te[2 * m] * d + i] += a.miss_w[m] * r[v];
                }
            }
            for (; q < a.gstart[e + 1]; ++q) {
                const int m = a.order[q], t = a.miss_te[2 * m];
                a.y_add[(int64_t)t * d + i] += a.miss_w[m] * dot(wd, a.h + (int64_t)m * f, f);
            }
        }
    }
}

}  // namespace HX_NS
