/*
 * ORACLE for the sparse MoE layer forward.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The product path (the HIP library and its Python
 * binding) never calls it, and the two share no code, header or table.
 *
 * Plain, slow, obviously correct CPU C.  Floating point is double unless a
 * step's definition fixes float (the router logits and the gates are
 * defined as fp32 values; the layer output is fp32).  Loops run in the
 * order the definition states; OpenMP only splits independent items
 * (tokens, (token, expert) pairs), each of which one thread computes alone,
 * so results do not depend on the thread count.
 *
 * What the layer computes (per token t; E routed experts, top-k, one shared
 * expert): the model structure -- 512 routed experts per layer, 10 picked
 * per token per layer, plus 1 shared expert -- is the one described on
 * greenbean-ai, "Strata 如何讓 12GB 顯卡跑 Qwen3.8-Flash-Next？", section 一,
 * and wiselychen.com, "Strata ... RTX 5090 ... 1M context", the "30 秒定位"
 * fact table; the router, the shared expert and the cached experts run on
 * the GPU (greenbean-ai, section 二; wiselychen.com, technique 2 "專家快取與
 * CPU／GPU 分工"), and experts that are not resident on the GPU are left to
 * another processor (same passages; tutuge.me "⚙️ 125B 是怎么塞进游戏 PC 的").
 * The pages name the ~3-bit / ~2-bit classes (IQ3_XXS ≈3.06 bit/weight,
 * wiselychen.com technique 1 "低位元量化"; Q2_0, greenbean-ai section 四) but
 * give no byte layout, FFN form or router normalisation.  The library fixes
 * them as follows, and this file is written from that definition:
 *
 *   z[t][e]  = fp32( sum_i Wr[e][i] * u[t][i]  (+ bias[e]) )        (logits)
 *   idx[t][] = the k experts with the largest z, ordered by (z desc, e asc)
 *   p_e      = softmax over all E of z;  gate_r = p_idx_r / sum_r p_idx_r  (fp32)
 *   per expert e: g = Wg u, v = Wu u, h_j = silu(g_j) * v_j, y = Wd h
 *   out[t]   = y_shared + sum_{r<k, resident} gate_r * y_idx_r   (r ascending)
 *   weights  = fp16 scale of the 256-element block * (code - c0),
 *              c0 = 3.5 for 3-bit codes, 1.5 for 2-bit codes
 *
 * Byte layout of one matrix [out][in] (out % 16 == 0, in % 128 == 0):
 *   element (r, c) lives in "unit" (32 consecutive columns of one row)
 *     unit byte offset = (((r/16) * (in/128) + c/128) * 16 + r%16) * 4*UB + ((c%128)/32) * UB
 *     with UB = 12 bytes (3-bit) or 8 bytes (2-bit), j = c % 32 its place in the unit.
 *   3-bit unit: little-endian 32-bit words A, B, C.
 *     j <  24: code = bits [4n, 4n+3) of word (A, B, C)[j/8], n = j % 8
 *     j >= 24: n = j - 24; code = A bit (4n+3) | B bit (4n+3) << 1 | C bit (4n+3) << 2
 *   2-bit unit: little-endian 32-bit words A, B.
 *     word = A for j < 16 else B; jj = j % 16; n = jj % 8; half = jj / 8
 *     code = bits [4n + 2*half, 4n + 2*half + 2) of the word
 *   scales: one fp16 per 256 consecutive elements of the row-major flattened
 *     matrix (logical order), i.e. scale index (r*in + c) / 256.
 *   an expert's codes are gate [f][d], up [f][d], down [d][f], in that order;
 *   experts are stored 0..E-1 (routed) then E (shared); scales likewise.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ fp16 */
/* Exact value of an IEEE binary16 bit pattern. */
double oracle_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1F;
    int man = h & 0x3FF;
    double v;
    if (ex == 0) v = ldexp((double)man, -24);                 /* subnormal */
    else if (ex == 31) v = man ? NAN : INFINITY;
    else v = ldexp((double)(1024 + man), ex - 25);            /* 1.m * 2^(ex-15) */
    return sign ? -v : v;
}

/* ----------------------------------------------------------------- codes */
static uint32_t rd32(const uint8_t *p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

/* Code of element (r, c) of one packed matrix [out][in]. */
int oracle_code_at(int bits, const uint8_t *mat, int64_t out, int64_t in, int64_t r, int64_t c) {
    (void)out;
    int64_t ub = (bits == 3) ? 12 : 8;
    int64_t unit = (((r / 16) * (in / 128) + c / 128) * 16 + r % 16) * 4 * ub + ((c % 128) / 32) * ub;
    const uint8_t *u = mat + unit;
    int j = (int)(c % 32);
    if (bits == 3) {
        uint32_t A = rd32(u), B = rd32(u + 4), C = rd32(u + 8);
        if (j < 24) {
            uint32_t w = (j < 8) ? A : (j < 16) ? B : C;
            int n = j % 8;
            return (int)((w >> (4 * n)) & 7u);
        }
        int n = j - 24;
        return (int)(((A >> (4 * n + 3)) & 1u) | (((B >> (4 * n + 3)) & 1u) << 1) |
                     (((C >> (4 * n + 3)) & 1u) << 2));
    } else {
        uint32_t w = (j < 16) ? rd32(u) : rd32(u + 4);
        int jj = j % 16, n = jj % 8, half = jj / 8;
        return (int)((w >> (4 * n + 2 * half)) & 3u);
    }
}

/* All codes of one matrix, row-major [out][in]. */
void oracle_unpack_codes(int bits, const uint8_t *mat, int64_t out, int64_t in, uint8_t *codes) {
    for (int64_t r = 0; r < out; ++r)
        for (int64_t c = 0; c < in; ++c) codes[r * in + c] = (uint8_t)oracle_code_at(bits, mat, out, in, r, c);
}

/* Inverse of oracle_unpack_codes (used only to build hand-made test blocks). */
void oracle_pack_codes(int bits, const uint8_t *codes, int64_t out, int64_t in, uint8_t *mat) {
    int64_t ub = (bits == 3) ? 12 : 8;
    memset(mat, 0, (size_t)(out * in * bits / 8));
    for (int64_t r = 0; r < out; ++r)
        for (int64_t c = 0; c < in; ++c) {
            uint32_t v = codes[r * in + c];
            int64_t unit = (((r / 16) * (in / 128) + c / 128) * 16 + r % 16) * 4 * ub + ((c % 128) / 32) * ub;
            uint8_t *u = mat + unit;
            int j = (int)(c % 32);
            if (bits == 3) {
                if (j < 24) {
                    int w = j / 8, n = j % 8;
                    int bit0 = 4 * n;
                    for (int b = 0; b < 3; ++b)
                        if ((v >> b) & 1u) u[4 * w + (bit0 + b) / 8] |= (uint8_t)(1u << ((bit0 + b) % 8));
                } else {
                    int n = j - 24, bit = 4 * n + 3;
                    for (int b = 0; b < 3; ++b)
                        if ((v >> b) & 1u) u[4 * b + bit / 8] |= (uint8_t)(1u << (bit % 8));
                }
            } else {
                int w = j / 16, jj = j % 16, n = jj % 8, half = jj / 8;
                int bit0 = 4 * n + 2 * half;
                for (int b = 0; b < 2; ++b)
                    if ((v >> b) & 1u) u[4 * w + (bit0 + b) / 8] |= (uint8_t)(1u << ((bit0 + b) % 8));
            }
        }
}

static double code_offset(int bits) { return bits == 3 ? 3.5 : 1.5; }

/* Dequantised matrix [out][in] in double: scale(block) * (code - c0).
 * Every element is computed on its own, so rows may be split over threads. */
static void dequant_rows(int bits, const uint8_t *mat, const uint16_t *scales, int64_t out, int64_t in, double *w,
                         int threads) {
    double c0 = code_offset(bits);
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t r = 0; r < out; ++r)
        for (int64_t c = 0; c < in; ++c) {
            int64_t n = r * in + c;
            w[n] = oracle_half_to_double(scales[n / 256]) * ((double)oracle_code_at(bits, mat, out, in, r, c) - c0);
        }
}

void oracle_dequant(int bits, const uint8_t *mat, const uint16_t *scales, int64_t out, int64_t in, double *w) {
    dequant_rows(bits, mat, scales, out, in, w, 1);
}

/* ---------------------------------------------------------------- router */
/* z[t][e] = fp32(sum_i Wr[e][i] * u[t][i] + bias[e]), summed in double, i ascending. */
void oracle_logits(const float *u, int T, int d, const float *Wr, const float *bias, int E, float *z,
                   int threads) {
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int i = 0; i < d; ++i) s += (double)Wr[(int64_t)e * d + i] * (double)u[(int64_t)t * d + i];
            if (bias) s += (double)bias[e];
            z[(int64_t)t * E + e] = (float)s;
        }
}

/* "a ranks before b": larger logit first, lower index on ties. */
static int ranks_before(float za, int a, float zb, int b) { return za > zb || (za == zb && a < b); }

/* Top-k by (z desc, e asc), then gates: softmax over all E in double,
 * renormalised over the selected k, rounded to fp32. */
void oracle_select(const float *z, int T, int E, int k, int32_t *idx, float *gate) {
    char *taken = (char *)malloc((size_t)E);
    for (int t = 0; t < T; ++t) {
        const float *zt = z + (int64_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int r = 0; r < k; ++r) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || ranks_before(zt[e], e, zt[best], best))) best = e;
            taken[best] = 1;
            idx[(int64_t)t * k + r] = best;
        }
        double m = zt[idx[(int64_t)t * k]];
        double S = 0.0;
        for (int e = 0; e < E; ++e) S += exp((double)zt[e] - m);
        double q[64], Q = 0.0;
        for (int r = 0; r < k; ++r) {
            q[r] = exp((double)zt[idx[(int64_t)t * k + r]] - m) / S;
            Q += q[r];
        }
        for (int r = 0; r < k; ++r) gate[(int64_t)t * k + r] = (float)(q[r] / Q);
    }
    free(taken);
}

/* Smallest gap between adjacent logits of the sorted top-(k+1): the margin
 * that decides whether the ordered top-k is robust to rounding. */
void oracle_topk_margin(const float *z, int T, int E, int k, float *margin) {
    char *taken = (char *)malloc((size_t)E);
    for (int t = 0; t < T; ++t) {
        const float *zt = z + (int64_t)t * E;
        memset(taken, 0, (size_t)E);
        double prev = 0, mg = INFINITY;
        int kk = k + 1 <= E ? k + 1 : E;
        for (int r = 0; r < kk; ++r) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || ranks_before(zt[e], e, zt[best], best))) best = e;
            taken[best] = 1;
            if (r > 0 && prev - zt[best] < mg) mg = prev - zt[best];
            prev = zt[best];
        }
        margin[t] = (float)mg;
    }
    free(taken);
}

/* ----------------------------------------------------------- permutation */
/* counts[e], offsets[e] (exclusive prefix sum, offsets[E] = T*k), and slots
 * enumerated by (e asc, t asc): perm[slot] = t*k + r, pos[t*k + r] = slot. */
void oracle_permute(const int32_t *idx, int T, int k, int E, int32_t *counts, int32_t *offsets, int32_t *perm,
                    int32_t *pos) {
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t i = 0; i < (int64_t)T * k; ++i) counts[idx[i]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int t = 0; t < T; ++t)          /* t ascending gives t-ascending slots within each expert */
        for (int r = 0; r < k; ++r) {
            int e = idx[(int64_t)t * k + r];
            int32_t slot = offsets[e] + fill[e]++;
            perm[slot] = t * k + r;
            pos[(int64_t)t * k + r] = slot;
        }
    free(fill);
}

static int resident(const uint32_t *mask, int e) { return !mask || ((mask[e / 32] >> (e % 32)) & 1u); }

/* Miss list: every (t, r) whose expert is not resident, in (t asc, r asc)
 * order; the first `cap` are written, the return value is the full count. */
int oracle_misses(const int32_t *idx, const float *gate, int T, int k, const uint32_t *mask, int32_t *miss_te,
                  float *miss_w, int cap) {
    int n = 0;
    for (int t = 0; t < T; ++t)
        for (int r = 0; r < k; ++r) {
            int e = idx[(int64_t)t * k + r];
            if (!resident(mask, e)) {
                if (n < cap) {
                    miss_te[2 * n] = t;
                    miss_te[2 * n + 1] = e;
                    miss_w[n] = gate[(int64_t)t * k + r];
                }
                n++;
            }
        }
    return n;
}

/* ---------------------------------------------------------------- expert */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One expert FFN on one input vector, weights dequantised element by
 * element as they are used: y = Wd (silu(Wg u) * (Wu u)), double throughout. */
void oracle_expert_ffn(int bits, const uint8_t *codes, const uint16_t *scales, int d, int f, const double *u,
                       double *y) {
    int64_t mat_bytes = (int64_t)d * f * bits / 8;
    int64_t mat_blocks = (int64_t)d * f / 256;
    const uint8_t *cg = codes, *cu = codes + mat_bytes, *cd = codes + 2 * mat_bytes;
    const uint16_t *sg = scales, *su = scales + mat_blocks, *sd = scales + 2 * mat_blocks;
    double c0 = code_offset(bits);
    double *h = (double *)malloc(sizeof(double) * (size_t)f);
    for (int j = 0; j < f; ++j) {
        double g = 0.0, v = 0.0;
        for (int i = 0; i < d; ++i) {
            int64_t n = (int64_t)j * d + i;
            double wg = oracle_half_to_double(sg[n / 256]) * (oracle_code_at(bits, cg, f, d, j, i) - c0);
            double wu = oracle_half_to_double(su[n / 256]) * (oracle_code_at(bits, cu, f, d, j, i) - c0);
            g += wg * u[i];
            v += wu * u[i];
        }
        h[j] = silu(g) * v;
    }
    for (int i = 0; i < d; ++i) {
        double s = 0.0;
        for (int j = 0; j < f; ++j) {
            int64_t n = (int64_t)i * f + j;
            double wd = oracle_half_to_double(sd[n / 256]) * (oracle_code_at(bits, cd, d, f, i, j) - c0);
            s += wd * h[j];
        }
        y[i] = s;
    }
    free(h);
}

/* Same FFN for several inputs with the expert dequantised once up front
 * (the "grouped" evaluation).  Inputs are taken TB at a time so that TB
 * independent sums advance together, but every sum is still formed in the
 * order oracle_expert_ffn uses (i ascending for g and v, j ascending for y;
 * one rounded product, then one rounded add, per term), so each input's
 * result is bit-for-bit the one oracle_expert_ffn computes. */
#define TB 32
void oracle_expert_ffn_grouped(int bits, const uint8_t *codes, const uint16_t *scales, int d, int f, int n_in,
                               const double *u /*[n_in][d]*/, double *y /*[n_in][d]*/, int threads) {
    int64_t mat_bytes = (int64_t)d * f * bits / 8;
    int64_t mat_blocks = (int64_t)d * f / 256;
    double *Wg = (double *)malloc(sizeof(double) * (size_t)d * f);
    double *Wu = (double *)malloc(sizeof(double) * (size_t)d * f);
    double *Wd = (double *)malloc(sizeof(double) * (size_t)d * f);
    dequant_rows(bits, codes, scales, f, d, Wg, threads);
    dequant_rows(bits, codes + mat_bytes, scales + mat_blocks, f, d, Wu, threads);
    dequant_rows(bits, codes + 2 * mat_bytes, scales + 2 * mat_blocks, d, f, Wd, threads);
    int nblk = (n_in + TB - 1) / TB;
#pragma omp parallel for schedule(dynamic) num_threads(threads > 0 ? threads : 1)
    for (int b = 0; b < nblk; ++b) {
        int t0 = b * TB, nt = n_in - t0 < TB ? n_in - t0 : TB;
        double *ub = (double *)calloc((size_t)d * TB, sizeof(double));   /* [i][t]: input i of token t0+t */
        double *h = (double *)calloc((size_t)f * TB, sizeof(double));    /* [j][t] */
        for (int t = 0; t < nt; ++t)
            for (int i = 0; i < d; ++i) ub[(int64_t)i * TB + t] = u[(int64_t)(t0 + t) * d + i];
        for (int j = 0; j < f; ++j) {
            double g[TB], v[TB];
            for (int t = 0; t < TB; ++t) g[t] = v[t] = 0.0;
            for (int i = 0; i < d; ++i) {
                double wg = Wg[(int64_t)j * d + i], wu = Wu[(int64_t)j * d + i];
                for (int t = 0; t < TB; ++t) {
                    g[t] += wg * ub[(int64_t)i * TB + t];
                    v[t] += wu * ub[(int64_t)i * TB + t];
                }
            }
            for (int t = 0; t < TB; ++t) h[(int64_t)j * TB + t] = silu(g[t]) * v[t];
        }
        for (int i = 0; i < d; ++i) {
            double s[TB];
            for (int t = 0; t < TB; ++t) s[t] = 0.0;
            for (int j = 0; j < f; ++j) {
                double wd = Wd[(int64_t)i * f + j];
                for (int t = 0; t < TB; ++t) s[t] += wd * h[(int64_t)j * TB + t];
            }
            for (int t = 0; t < nt; ++t) y[(int64_t)(t0 + t) * d + i] = s[t];
        }
        free(ub);
        free(h);
    }
    free(Wg);
    free(Wu);
    free(Wd);
}
#undef TB

/* ----------------------------------------------------------------- layer */
/* Grouped evaluation of expert e (e == E: the shared expert, all T tokens)
 * for its n_in (token, pick) pairs, written to ys[(t*(k+1) + r)*d ...]. */
#define GROUP_BIG 256
static void group_expert(int bits, int e, int E, int k, int d, int f, int n_in, const int32_t *perm,
                         const int32_t *offsets, const uint8_t *codes, const uint16_t *scales, const double *ud,
                         double *ys, int threads) {
    double *ug = (double *)malloc(sizeof(double) * (size_t)n_in * d);
    double *yg = (double *)malloc(sizeof(double) * (size_t)n_in * d);
    for (int i = 0; i < n_in; ++i) {
        int t = (e == E) ? i : perm[offsets[e] + i] / k;
        memcpy(ug + (int64_t)i * d, ud + (int64_t)t * d, sizeof(double) * (size_t)d);
    }
    oracle_expert_ffn_grouped(bits, codes, scales, d, f, n_in, ug, yg, threads);
    for (int i = 0; i < n_in; ++i) {
        int t, r;
        if (e == E) { t = i; r = k; }
        else { t = perm[offsets[e] + i] / k; r = perm[offsets[e] + i] % k; }
        memcpy(ys + ((int64_t)t * (k + 1) + r) * d, yg + (int64_t)i * d, sizeof(double) * (size_t)d);
    }
    free(ug);
    free(yg);
}

/* Full layer for T tokens.  codes/scales hold E+1 experts (E = shared).
 * Writes routing (idx, gate), the permutation, the miss list, and
 * out[T][d] = fp32(y_shared + sum over resident r, ascending, of gate_r * y_r).
 * grouped = 0: each (token, expert) FFN on its own (dequant on the fly);
 * grouped = 1: each needed expert dequantised once, then all its tokens. */
int oracle_moe_layer(int bits, int E, int k, int d, int f, int T, const float *u, const float *Wr,
                     const float *bias, const uint8_t *codes, const uint16_t *scales, const uint32_t *mask,
                     int32_t *idx, float *gate, int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *pos,
                     float *out, int32_t *miss_te, float *miss_w, int miss_cap, int grouped, int threads) {
    int64_t exp_bytes = 3LL * d * f * bits / 8;
    int64_t exp_blocks = 3LL * d * f / 256;
    float *z = (float *)malloc(sizeof(float) * (size_t)T * E);
    oracle_logits(u, T, d, Wr, bias, E, z, threads);
    oracle_select(z, T, E, k, idx, gate);
    free(z);
    oracle_permute(idx, T, k, E, counts, offsets, perm, pos);
    int n_miss = oracle_misses(idx, gate, T, k, mask, miss_te, miss_w, miss_cap);

    /* per (t, r) expert outputs; column k holds the shared expert */
    double *ys = (double *)calloc((size_t)T * (k + 1) * d, sizeof(double));
    double *ud = (double *)malloc(sizeof(double) * (size_t)T * d);
    for (int64_t i = 0; i < (int64_t)T * d; ++i) ud[i] = (double)u[i];

    if (!grouped) {
#pragma omp parallel for schedule(dynamic) num_threads(threads > 0 ? threads : 1)
        for (int64_t p = 0; p < (int64_t)T * (k + 1); ++p) {
            int t = (int)(p / (k + 1)), r = (int)(p % (k + 1));
            int e = (r == k) ? E : idx[(int64_t)t * k + r];
            if (r < k && !resident(mask, e)) continue;
            oracle_expert_ffn(bits, codes + e * exp_bytes, scales + e * exp_blocks, d, f, ud + (int64_t)t * d,
                              ys + p * d);
        }
    } else {
        /* experts with many inputs one after another, each on every thread;
         * then the others side by side, one thread each (each expert writes
         * only its own (t, r) rows of ys, so the order does not matter) */
        for (int e = 0; e <= E; ++e) {
            int n_in = (e == E) ? T : counts[e];
            if (n_in >= GROUP_BIG && (e == E || resident(mask, e)))
                group_expert(bits, e, E, k, d, f, n_in, perm, offsets, codes + e * exp_bytes,
                             scales + e * exp_blocks, ud, ys, threads);
        }
#pragma omp parallel for schedule(dynamic) num_threads(threads > 0 ? threads : 1)
        for (int e = 0; e <= E; ++e) {
            int n_in = (e == E) ? T : counts[e];
            if (n_in > 0 && n_in < GROUP_BIG && (e == E || resident(mask, e)))
                group_expert(bits, e, E, k, d, f, n_in, perm, offsets, codes + e * exp_bytes,
                             scales + e * exp_blocks, ud, ys, 1);
        }
    }
    for (int t = 0; t < T; ++t)
        for (int i = 0; i < d; ++i) {
            double s = ys[((int64_t)t * (k + 1) + k) * d + i];
            for (int r = 0; r < k; ++r) {
                int e = idx[(int64_t)t * k + r];
                if (resident(mask, e)) s += (double)gate[(int64_t)t * k + r] * ys[((int64_t)t * (k + 1) + r) * d + i];
            }
            out[(int64_t)t * d + i] = (float)s;
        }
    free(ys);
    free(ud);
    return n_miss;
}

/* RMS normalisation of each row (no learnt gain): x / sqrt(mean(x^2) + eps),
 * in double, rounded to fp32.  Applied to the fp32 residual stream before
 * every layer after the first. */
void oracle_rmsnorm(const float *x, int T, int d, double eps, float *u) {
    for (int t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int i = 0; i < d; ++i) ss += (double)x[(int64_t)t * d + i] * (double)x[(int64_t)t * d + i];
        double inv = 1.0 / sqrt(ss / d + eps);
        for (int i = 0; i < d; ++i) u[(int64_t)t * d + i] = (float)((double)x[(int64_t)t * d + i] * inv);
    }
}
