/*
 * Seeded synthetic input generator shared by the tests, the oracle's
 * checks and the benchmark.
 *
 * It holds none of the MoE layer's arithmetic: it only turns a key and a
 * counter into bytes, normal deviates and uniform deviates, and rounds them
 * into the storage types the layer consumes (bf16, fp32, fp16).
 *
 * Counter-based: every output element is a pure function of
 * (key, element index), so any slice (one expert of one layer, say) can be
 * regenerated without producing the rest, and any thread split gives the
 * same bytes.
 *
 * Mixing function: the SplitMix64 output finaliser (Steele, Lea, Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014; constants
 * as published by Vigna for splitmix64.c).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Word i of the stream named by key. */
static inline uint64_t word_at(uint64_t key, uint64_t i) {
    return mix64(key + (i + 1) * GOLDEN);
}

/* Derive a stream key from a seed and up to four integer labels. */
uint64_t synth_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c, uint64_t d) {
    uint64_t k = mix64(seed ^ 0x5EED5EED5EED5EEDULL);
    k = mix64(k ^ (a + 1) * GOLDEN);
    k = mix64(k ^ (b + 3) * GOLDEN);
    k = mix64(k ^ (c + 5) * GOLDEN);
    k = mix64(k ^ (d + 7) * GOLDEN);
    return k;
}

/* Uniform double in the open interval (0, 1) from the top 53 bits. */
static inline double unit_open(uint64_t w) {
    return ((double)(w >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* Bytes [offset, offset + n) of the stream: little-endian words. */
void synth_bytes(uint64_t key, uint64_t offset, uint64_t n, uint8_t *out, int threads) {
    (void)threads;
    uint64_t end = offset + n;
    uint64_t w0 = offset >> 3, w1 = (end + 7) >> 3;
    int64_t nw = (int64_t)(w1 - w0);
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t j = 0; j < nw; ++j) {
        uint64_t wi = w0 + (uint64_t)j;
        uint64_t w = word_at(key, wi);
        uint64_t base = wi << 3;
        for (int b = 0; b < 8; ++b) {
            uint64_t pos = base + (uint64_t)b;
            if (pos >= offset && pos < end) out[pos - offset] = (uint8_t)(w >> (8 * b));
        }
    }
}

/* Standard normal deviate number i of the stream (Box-Muller, cosine branch,
 * double precision). */
static inline double normal_at(uint64_t key, uint64_t i) {
    double u1 = unit_open(word_at(key, 2 * i));
    double u2 = unit_open(word_at(key, 2 * i + 1));
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

void synth_normal_f64(uint64_t key, uint64_t offset, uint64_t n, double *out, int threads) {
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t j = 0; j < (int64_t)n; ++j) out[j] = normal_at(key, offset + (uint64_t)j);
}

/* fp32 value rounded to nearest-even from the double (C conversion). */
void synth_normal_f32(uint64_t key, uint64_t offset, uint64_t n, double stddev, float *out, int threads) {
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t j = 0; j < (int64_t)n; ++j)
        out[j] = (float)(stddev * normal_at(key, offset + (uint64_t)j));
}

/* fp32 -> bf16 bit pattern, round to nearest even (finite inputs). */
static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* bf16 standard normal: double -> fp32 (RNE) -> bf16 (RNE). */
void synth_normal_bf16(uint64_t key, uint64_t offset, uint64_t n, uint16_t *out, int threads) {
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t j = 0; j < (int64_t)n; ++j)
        out[j] = f32_to_bf16_rne((float)normal_at(key, offset + (uint64_t)j));
}

/* double -> IEEE binary16 bit pattern with one rounding to nearest even.
 * Finite inputs; values beyond the fp16 range saturate to infinity. */
static uint16_t f64_to_f16_rne(double v) {
    uint16_t sign = 0;
    if (v < 0) { sign = 0x8000; v = -v; }
    if (v == 0) return sign;
    int e;
    double m = frexp(v, &e);              /* v = m * 2^e, m in [0.5, 1) */
    if (e < -13) {                        /* subnormal range: units of 2^-24 */
        double q = nearbyint(ldexp(v, 24));
        return (uint16_t)(sign | (uint16_t)q);  /* q == 1024 lands on the smallest normal */
    }
    double q = nearbyint(ldexp(m, 11));   /* 11 significant bits */
    if (q >= 2048.0) { q = 1024.0; e += 1; }
    int ef = e + 14;
    if (ef >= 31) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (uint16_t)(ef << 10) | (uint16_t)((int)q - 1024));
}

/* fp16 bit patterns of (lo + (hi - lo) * U(0,1)) * mult. */
void synth_uniform_f16(uint64_t key, uint64_t offset, uint64_t n, double lo, double hi, double mult,
                       uint16_t *out, int threads) {
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t j = 0; j < (int64_t)n; ++j) {
        double u = unit_open(word_at(key, offset + (uint64_t)j));
        out[j] = f64_to_f16_rne((lo + (hi - lo) * u) * mult);
    }
}

/* Uniform doubles in (0, 1). */
void synth_uniform_f64(uint64_t key, uint64_t offset, uint64_t n, double *out, int threads) {
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t j = 0; j < (int64_t)n; ++j) out[j] = unit_open(word_at(key, offset + (uint64_t)j));
}

/* Raw 64-bit words (used for seeded permutations). */
void synth_words(uint64_t key, uint64_t offset, uint64_t n, uint64_t *out) {
    for (uint64_t j = 0; j < n; ++j) out[j] = word_at(key, offset + j);
}
