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
// product keeps two 16-lane partial sums and adds them in a fixed tree,
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

// The 32 codes of one unit as two vectors (places 0-15, 16-31) of integers.
// 3-bit unit: words A, B, C; places j < 24 are the low 3 bits of nibble
// j % 8 of word j / 8; places 24 + n gather bit 3 of nibble n of A, B, C,
// which one scalar word D holds as its nibble n: then both vectors are two
// words spread over 8 lanes each, shifted and masked.
static inline void unit_codes3(const uint8_t *p, vi &lo, vi &hi) {
    const uint32_t A = rd32(p), B = rd32(p + 4), C = rd32(p + 8);
    const uint32_t D = ((A >> 3) & 0x11111111u) | ((B >> 2) & 0x22222222u) | ((C >> 1) & 0x44444444u);
    const vu sh = {0, 4, 8, 12, 16, 20, 24, 28, 0, 4, 8, 12, 16, 20, 24, 28};
    const vu ab = {A, A, A, A, A, A, A, A, B, B, B, B, B, B, B, B};
    const vu cd = {C, C, C, C, C, C, C, C, D, D, D, D, D, D, D, D};
    lo = (vi)((ab >> sh) & 7u);
    hi = (vi)((cd >> sh) & 7u);
}

// 2-bit unit: words A (places 0-15) and B (16-31); place j of a word is
// bits [4 (j % 8) + 2 (j / 8), +2).
static inline void unit_codes2(const uint8_t *p, vi &lo, vi &hi) {
    const uint32_t A = rd32(p), B = rd32(p + 4);
    const vu sh = {0, 4, 8, 12, 16, 20, 24, 28, 2, 6, 10, 14, 18, 22, 26, 30};
    const vu a = {A, A, A, A, A, A, A, A, A, A, A, A, A, A, A, A};
    const vu b = {B, B, B, B, B, B, B, B, B, B, B, B, B, B, B, B};
    lo = (vi)((a >> sh) & 3u);
    hi = (vi)((b >> sh) & 3u);
}

// Row r of a packed matrix [out][in] as fp32 weights scale * (code - c0),
// formed as code * scale - c0 * scale in one fused multiply-add (both
// products are exact in fp32, so the result is the exact weight).  Unit
// (r, c / 32) sits at the row's first unit + (c / 128) * 64 units + (c % 128)
// / 32 units; the scale of the 256-element block holding (r, c) is read once
// per block.
static void decode_row(int bits, const uint8_t *mat, const uint16_t *msc, int in, int r, float *w) {
    const int UB = bits == 3 ? 12 : 8;
    const float c0 = bits == 3 ? 3.5f : 1.5f;
    const uint8_t *row = mat + ((int64_t)(r >> 4) * (in >> 7) * 16 + (r & 15)) * 4 * UB;
    const int64_t e0 = (int64_t)r * in;
    int64_t blk = -1;
    vf s = {}, ms = {};
    for (int c = 0; c < in; c += 32) {
        const uint8_t *u = row + (int64_t)(c >> 7) * 64 * UB + ((c & 127) >> 5) * UB;
        if (((e0 + c) >> 8) != blk) {
            blk = (e0 + c) >> 8;
            const float sv = half_to_float(msc[blk]);
            s = vf{} + sv;
            ms = vf{} - c0 * sv;
        }
        vi lo, hi;
        if (bits == 3) unit_codes3(u, lo, hi);
        else unit_codes2(u, lo, hi);
        const vf wl = __builtin_convertvector(lo, vf) * s + ms, wh = __builtin_convertvector(hi, vf) * s + ms;
        memcpy(w + c, &wl, 64);
        memcpy(w + c + 16, &wh, 64);
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

// Rows w0 and w1 against NV vectors x[v] over n (a multiple of 32) columns.
// Every dot product keeps two partial sums of 16 lanes (columns i % 32 in
// [16p, 16p + 16) go to sum p) and ends with hsum(sum0 + sum1), whatever NV
// is, so a result does not depend on how the vectors were grouped; the row
// loads are shared by the NV vectors (0.75 loads per multiply-add at NV = 4).
// r[2v] = w0 . x[v], r[2v + 1] = w1 . x[v].
template <int NV> static inline void dots2(const float *w0, const float *w1, const float *const *x, int n, float *r) {
    vf a[NV][4];   // [vector][row 0 sum 0, row 0 sum 1, row 1 sum 0, row 1 sum 1]
#pragma GCC unroll 4
    for (int v = 0; v < NV; ++v) a[v][0] = a[v][1] = a[v][2] = a[v][3] = vf{};
    for (int i = 0; i < n; i += 32) {
        const vf p0 = ldv(w0 + i), p1 = ldv(w0 + i + 16), q0 = ldv(w1 + i), q1 = ldv(w1 + i + 16);
#pragma GCC unroll 4
        for (int v = 0; v < NV; ++v) {
            const vf b0 = ldv(x[v] + i), b1 = ldv(x[v] + i + 16);
            a[v][0] += p0 * b0;
            a[v][1] += p1 * b1;
            a[v][2] += q0 * b0;
            a[v][3] += q1 * b1;
        }
    }
#pragma GCC unroll 4
    for (int v = 0; v < NV; ++v) {
        r[2 * v] = hsum(a[v][0] + a[v][1]);
        r[2 * v + 1] = hsum(a[v][2] + a[v][3]);
    }
}

// dots2 over the misses q0 .. q1 of the list order (vector of miss m: base + its
// row offset), four at a time, then the remainder one at a time; fn(m, r0, r1)
// takes the two results of each miss in list order.
template <typename RowOf, typename Fn>
static inline void dots2_misses(const float *w0, const float *w1, int q0, int q1, const int32_t *order, int n,
                                RowOf row_of, Fn fn) {
    int q = q0;
    for (; q + 4 <= q1; q += 4) {
        const float *xs[4];
        for (int v = 0; v < 4; ++v) xs[v] = row_of(order[q + v]);
        float r[8];
        dots2<4>(w0, w1, xs, n, r);
        for (int v = 0; v < 4; ++v) fn(order[q + v], r[2 * v], r[2 * v + 1]);
    }
    for (; q < q1; ++q) {
        const float *xs[1] = {row_of(order[q])};
        float r[2];
        dots2<1>(w0, w1, xs, n, r);
        fn(order[q], r[0], r[1]);
    }
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
        dots2_misses(wg, wu, a.gstart[e], a.gstart[e + 1], a.order, d,
                     [&](int m) { return a.u + (int64_t)a.miss_te[2 * m] * d; },
                     [&](int m, float g, float u) { a.h[(int64_t)m * f + j] = silu_mul(g, u); });
    }
}

// Phase B task: columns [i0, i1) of y_add, experts[0..ne) in order, each
// expert's misses in list order.
void down_cols(const HostMissArgs &a, const int32_t *experts, int ne, int i0, int i1) {
    const int d = a.d, f = a.f;
    const int64_t mat_bytes = (int64_t)d * f * a.bits / 8, mat_blocks = (int64_t)d * f / 256;
    for (int t = 0; t < a.T; ++t)
        for (int i = i0; i < i1; ++i) a.y_add[(int64_t)t * d + i] = 0.f;
    alignas(64) float wd0[HOST_MAX_F], wd1[HOST_MAX_F];
    for (int x = 0; x < ne; ++x) {
        const int e = experts[x];
        const uint8_t *cd = a.codes + ((int64_t)e * 3 + 2) * mat_bytes;
        const uint16_t *sd = a.scales + (int64_t)e * 3 * mat_blocks + 2 * mat_blocks;
        for (int i = i0; i < i1; i += 2) {   // rows i and i + 1 of Wd (i1 - i0 is even), each column's adds in list order
            decode_row(a.bits, cd, sd, f, i, wd0);
            decode_row(a.bits, cd, sd, f, i + 1, wd1);
            dots2_misses(wd0, wd1, a.gstart[e], a.gstart[e + 1], a.order, f,
                         [&](int m) { return a.h + (int64_t)m * f; },
                         [&](int m, float y0, float y1) {
                             float *yr = a.y_add + (int64_t)a.miss_te[2 * m] * d;
                             yr[i] += a.miss_w[m] * y0;
                             yr[i + 1] += a.miss_w[m] * y1;
                         });
        }
    }
}

}  // namespace HX_NS
