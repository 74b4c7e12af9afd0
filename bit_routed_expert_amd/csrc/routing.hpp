// Wave- and block-level routing helpers shared by the routing kernels and
// the decode-size gate/up kernel: ordered top-k with gates, and the small-T
// routing state (picks, per-expert token masks, work items, outputs).
//
// Top-k selection is by (logit desc, expert index asc); gates are the softmax
// renormalised over the k picks (per-layer routing of 10 of 512 experts:
// greenbean-ai, "Strata 如何讓 12GB 顯卡跑 Qwen3.8-Flash-Next？", section 一).
#pragma once
#include "common.hpp"

namespace strata {

// Monotone map of fp32 to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t f32_key(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Butterfly over the whole wave, every lane ending with the result and no
// scalar hand-off: quad permutes and row mirrors combine each 16-lane row,
// then the row swaps of gfx950 (16-lane rows, then 32-lane halves) pair each
// lane with its partner row.  Every lane combines the same two operands, so
// the result is the same bit pattern in all lanes.
#define WAVE_BFLY(V, OP)                                                                                   \
    {                                                                                                      \
        V = OP(V, (decltype(V))__builtin_bit_cast(decltype(V), __builtin_amdgcn_update_dpp(              \
                      0, __builtin_bit_cast(int, V), 0xB1, 0xF, 0xF, false))); /* quad_perm [1,0,3,2] */  \
        V = OP(V, (decltype(V))__builtin_bit_cast(decltype(V), __builtin_amdgcn_update_dpp(              \
                      0, __builtin_bit_cast(int, V), 0x4E, 0xF, 0xF, false))); /* quad_perm [2,3,0,1] */  \
        V = OP(V, (decltype(V))__builtin_bit_cast(decltype(V), __builtin_amdgcn_update_dpp(              \
                      0, __builtin_bit_cast(int, V), 0x141, 0xF, 0xF, false))); /* row_half_mirror */     \
        V = OP(V, (decltype(V))__builtin_bit_cast(decltype(V), __builtin_amdgcn_update_dpp(              \
                      0, __builtin_bit_cast(int, V), 0x140, 0xF, 0xF, false))); /* row_mirror */          \
        const auto p16 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, V),                 \
                                                          __builtin_bit_cast(uint32_t, V), false, false);  \
        V = OP(__builtin_bit_cast(decltype(V), (uint32_t)p16[0]), __builtin_bit_cast(decltype(V), (uint32_t)p16[1])); \
        const auto p32 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, V),                 \
                                                          __builtin_bit_cast(uint32_t, V), false, false);  \
        V = OP(__builtin_bit_cast(decltype(V), (uint32_t)p32[0]), __builtin_bit_cast(decltype(V), (uint32_t)p32[1])); \
    }
__device__ __forceinline__ uint32_t bfly_umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t bfly_umin(uint32_t a, uint32_t b) { return a < b ? a : b; }
__device__ __forceinline__ float bfly_fadd(float a, float b) { return a + b; }
__device__ __forceinline__ uint32_t wave_allmax_u32(uint32_t v) {
    WAVE_BFLY(v, bfly_umax)
    return v;
}
__device__ __forceinline__ uint32_t wave_allmin_u32(uint32_t v) {
    WAVE_BFLY(v, bfly_umin)
    return v;
}
__device__ __forceinline__ float wave_allsum_f32(float v) {
    WAVE_BFLY(v, bfly_fadd)
    return v;
}
#undef WAVE_BFLY

// LDS scratch of one wave's top-k (16-byte aligned): TOPK_CAND candidate
// entries of 64 bits, value key << 32 | ~expert index, so a larger entry is
// an earlier pick.
constexpr int TOPK_CAND = 64;
constexpr int TOPK_LDS_WORDS = 2 * TOPK_CAND;

// Selection by rounds (any number of equal keys; few registers): a round
// takes each lane's best remaining key (value desc, index asc) by a scan,
// the wave maximum of those values, then the smallest index among the lanes
// holding it; the owning lane clears that key.  Lane r < k ends with pick r
// in (*my_e, *my_k).  Keys are nonzero except for empty places.
// Expert held in place j of a lane: lane + 64j (strided), or with CONTIG
// 4*lane + (j mod 4) + 256*(j / 4), so a lane's places are four runs of 4
// consecutive experts (16-byte loads).  Either way the places of one lane
// rise with j, so "place ascending" inside a lane is "index ascending".
template <bool CONTIG> __device__ __forceinline__ int topk_place(int lane, int j) {
    return CONTIG ? 4 * lane + (j & 3) + 256 * (j >> 2) : lane + 64 * j;
}

template <int JM, bool CONTIG = false>
__device__ __forceinline__ void topk_rounds(uint32_t (&kv)[JM], int k, int *my_e, uint32_t *my_k) {
    const int lane = threadIdx.x & 63;
    for (int r = 0; r < k; ++r) {
        uint32_t bk = 0u;
        int bj = 0;
#pragma unroll
        for (int j = 0; j < JM; ++j) {   // a strict > keeps the lowest index among equal values
            bj = kv[j] > bk ? j : bj;
            bk = kv[j] > bk ? kv[j] : bk;
        }
        const uint32_t m = wave_allmax_u32(bk);
        const uint32_t e = wave_allmin_u32(bk == m ? (uint32_t)topk_place<CONTIG>(lane, bj) : 0xFFFFFFFFu);
        if (lane == r) {
            *my_e = (int)e;
            *my_k = m;
        }
        if (bk == m && (uint32_t)topk_place<CONTIG>(lane, bj) == e) {   // the owner clears its key
#pragma unroll
            for (int j = 0; j < JM; ++j)
                if (j == bj) kv[j] = 0u;
        }
    }
}

// Inclusive prefix sum over the wave (row shifts, then the row broadcasts).
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
    return v;
}

// Ordered top-k (k <= 32) of E logits z[e] * scale + bias[e] by one wave
// (JM = E/64 rounded up to 8 or 16), by (value desc, index asc); lane r < k
// ends with pick r: *e_out, *z_out.  cand: this wave's TOPK_LDS_WORDS of LDS.
//   1. P = the k-th largest of the 64 lane maxima, cut to its top 16 bits:
//      at least k keys are >= P, so every pick is >= P.  Found two bits at a
//      time from the top (a value is kept while k lanes reach it, counted
//      with wave ballots).
//   2. The keys >= P (usually a few more than k) are packed into LDS at a
//      wave prefix sum of the per-lane counts; when no lane holds more than
//      two (the usual case) they are its two largest keys, found as the keys
//      are formed.
//   3. Each candidate's rank is the number of larger entries (LDS reads that
//      every lane shares); rank r < k is pick r.
// More than TOPK_CAND candidates (many equal values) take the rounds above.
// planes > 1: z[e] is 0 + z[e] + z[pstride + e] + ... (planes terms, in
// order), the loads of up to 64 values per lane issued before their adds
// (16-byte loads with CONTIG, which needs E a multiple of 4).
template <int JM, bool CONTIG = false>
__device__ __forceinline__ void wave_topk_picks_fast(const float *z, int E, int k, float scale, const float *bias,
                                                     uint32_t *cand, int *e_out, float *z_out, int planes = 1,
                                                     int pstride = 0) {
    const int lane = threadIdx.x & 63;
    float zv[JM], bv[JM];
    if (CONTIG) {
        // places 4q .. 4q+3 of this lane are experts 4*lane + 256q .. +3 (16 bytes, inside
        // [0, E) or clamped into it; experts >= E are empty places below)
#pragma unroll
        for (int j = 0; j < JM; ++j) zv[j] = 0.f;
        // one buffer resource over the planes (base and size in scalar registers), each load
        // the lane's byte offset plus the plane's offset in a scalar register
        const uint64_t zb = (uint64_t)z;
        const uint32_t zlo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)zb);
        const uint32_t zhi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(zb >> 32));
        const __amdgpu_buffer_rsrc_t zr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(((uint64_t)zhi << 32) | zlo), 0, (int)(4u * (uint32_t)((planes - 1) * pstride + E)), 0x00020000);
        const uint32_t pbytes = (uint32_t)__builtin_amdgcn_readfirstlane(4 * pstride);
        uint32_t off4[JM / 4];
#pragma unroll
        for (int q = 0; q < JM / 4; ++q) off4[q] = 4u * (uint32_t)min(4 * lane + 256 * q, E - 4);
        for (int p0 = 0; p0 < planes; p0 += 64 / JM) {
            typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
            u32x4v pv[64 / JM][JM / 4];
#pragma unroll
            for (int p = 0; p < 64 / JM; ++p) {
                const uint32_t so = (uint32_t)min(p0 + p, planes - 1) * pbytes;
#pragma unroll
                for (int q = 0; q < JM / 4; ++q)
                    pv[p][q] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(zr, off4[q], so, 0));
            }
#pragma unroll
            for (int p = 0; p < 64 / JM; ++p)
#pragma unroll
                for (int q = 0; q < JM / 4; ++q)
                    if (p0 + p < planes) {
                        zv[4 * q] += __uint_as_float(pv[p][q][0]);
                        zv[4 * q + 1] += __uint_as_float(pv[p][q][1]);
                        zv[4 * q + 2] += __uint_as_float(pv[p][q][2]);
                        zv[4 * q + 3] += __uint_as_float(pv[p][q][3]);
                    }
        }
    } else if (planes == 1) {
#pragma unroll
        for (int j = 0; j < JM; ++j) zv[j] = z[min(lane + 64 * j, E - 1)];
    } else {
#pragma unroll
        for (int j = 0; j < JM; ++j) zv[j] = 0.f;
        constexpr int NPG = 64 / JM;   // planes per group of loads (64 values per lane)
        typedef const float __attribute__((address_space(1))) gfloat;
        int off[JM];
#pragma unroll
        for (int j = 0; j < JM; ++j) off[j] = min(lane + 64 * j, E - 1);
        for (int p0 = 0; p0 < planes; p0 += NPG) {
            // every load of the group issued, none behind a branch (planes past the
            // last re-read the last one); only planes < `planes` are added
            float pv[NPG][JM];
#pragma unroll
            for (int p = 0; p < NPG; ++p) {
                // the plane's base in scalar registers (each half through uint32_t:
                // readfirstlane returns int, which would sign-extend)
                const uint64_t b = (uint64_t)(z + (size_t)min(p0 + p, planes - 1) * pstride);
                const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
                const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
                gfloat *zp = (gfloat *)(((uint64_t)hi << 32) | lo);
#pragma unroll
                for (int j = 0; j < JM; ++j) pv[p][j] = zp[off[j]];
            }
#pragma unroll
            for (int p = 0; p < NPG; ++p)
#pragma unroll
                for (int j = 0; j < JM; ++j)
                    if (p0 + p < planes) zv[j] += pv[p][j];
        }
    }
#pragma unroll
    for (int j = 0; j < JM; ++j) bv[j] = 0.f;
    if (bias) {
#pragma unroll
        for (int j = 0; j < JM; ++j) bv[j] = bias[min(topk_place<CONTIG>(lane, j), E - 1)];
    }
    uint32_t kv[JM];   // value key (0 = empty)
    // the lane's two largest keys in order (value desc, place asc) and their places
    uint32_t mx = 0u, sx = 0u;
    int jm = 0, js = 0;
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        const int e = topk_place<CONTIG>(lane, j);
        kv[j] = (e < E) ? f32_key(zv[j] * scale + bv[j]) : 0u;
        const bool top = kv[j] > mx, second = !top && kv[j] > sx;
        js = top ? jm : (second ? j : js);
        sx = top ? mx : (second ? kv[j] : sx);
        jm = top ? j : jm;
        mx = top ? kv[j] : mx;
    }
    const uint32_t ku = (uint32_t)k;
    uint32_t P = 0u;
#pragma unroll
    for (int sh = 30; sh >= 16; sh -= 2) {
        const uint32_t c1 = P | (1u << sh), c2 = P | (2u << sh), c3 = P | (3u << sh);
        const bool b1 = __popcll(__ballot(mx >= c1)) >= ku;
        const bool b2 = __popcll(__ballot(mx >= c2)) >= ku;
        const bool b3 = __popcll(__ballot(mx >= c3)) >= ku;
        P = b3 ? c3 : (b2 ? c2 : (b1 ? c1 : P));
    }
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < JM; ++j) cnt += kv[j] >= P ? 1 : 0;
    uint64_t *c64 = (uint64_t *)cand;
    int C;
    if (__ballot(cnt > 2) == 0) {   // the usual case: the candidates are the lanes' two largest keys
        const int incl = wave_incl_scan(cnt);
        C = __builtin_amdgcn_readlane(incl, 63);
        const int pos = incl - cnt;
        if (cnt >= 1 && pos < TOPK_CAND) c64[pos] = ((uint64_t)mx << 32) | (uint32_t)~(uint32_t)topk_place<CONTIG>(lane, jm);
        if (cnt == 2 && pos + 1 < TOPK_CAND)
            c64[pos + 1] = ((uint64_t)sx << 32) | (uint32_t)~(uint32_t)topk_place<CONTIG>(lane, js);
    } else {
        const int incl = wave_incl_scan(cnt);
        C = __builtin_amdgcn_readlane(incl, 63);
        int pos = incl - cnt;
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            if (kv[j] >= P) {
                if (pos < TOPK_CAND) c64[pos] = ((uint64_t)kv[j] << 32) | (uint32_t)~(uint32_t)topk_place<CONTIG>(lane, j);
                ++pos;
            }
        }
    }
    int my_e = 0;
    uint32_t my_k = 0x80000000u;   // key of 0.0 for lanes past k
    if (C <= TOPK_CAND) {
        // entries are read 16 (or four) at a time: zero ones rank below every key
        const int Cp = C <= 16 ? 16 : (C + 3) & ~3;
        if (lane >= C && lane < Cp) c64[lane] = 0u;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint64_t key = lane < C ? c64[lane] : 0u;
        int rank = 0;
        if (C <= 16) {
            ulonglong2 q[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = *(const ulonglong2 *)(c64 + 2 * i);
#pragma unroll
            for (int i = 0; i < 8; ++i) rank += (q[i].x > key ? 1 : 0) + (q[i].y > key ? 1 : 0);
        } else {
            for (int i = 0; i < Cp; i += 4) {
                const ulonglong2 a = *(const ulonglong2 *)(c64 + i), b = *(const ulonglong2 *)(c64 + i + 2);
                rank += (a.x > key ? 1 : 0) + (a.y > key ? 1 : 0) + (b.x > key ? 1 : 0) + (b.y > key ? 1 : 0);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < C && rank < k) c64[rank] = key;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < k) {
            const uint64_t v = c64[lane];
            my_k = (uint32_t)(v >> 32);
            my_e = (int)~(uint32_t)v;
        }
    } else {
        topk_rounds<JM, CONTIG>(kv, k, &my_e, &my_k);
    }
    *e_out = my_e;
    *z_out = __uint_as_float((my_k & 0x80000000u) ? (my_k & 0x7FFFFFFFu) : ~my_k);
}

// Ordered top-k and gates of one token by one wave; lanes r < k write pick r.
// PLANES: z may be several planes (added in order); E a multiple of 4 up to
// 512 then takes the 16-byte-load layout.  Without it z is one plane.
template <bool PLANES = false>
__device__ __forceinline__ void wave_topk(const float *z, int E, int k, float scale, const float *bias,
                                          uint32_t *cand, int32_t *idx_out, float *gate_out, int32_t *idx_out2,
                                          float *gate_out2, int32_t *idx_lds, float *gate_lds, int planes = 1,
                                          int pstride = 0) {
    const int lane = threadIdx.x & 63;
    int e;
    float v;
    if (PLANES) {
        if (E <= 512 && (E & 3) == 0) wave_topk_picks_fast<8, true>(z, E, k, scale, bias, cand, &e, &v, planes, pstride);
        else if (E <= 512) wave_topk_picks_fast<8>(z, E, k, scale, bias, cand, &e, &v, planes, pstride);
        else wave_topk_picks_fast<16>(z, E, k, scale, bias, cand, &e, &v, planes, pstride);
    } else {
        if (E <= 512) wave_topk_picks_fast<8>(z, E, k, scale, bias, cand, &e, &v);
        else wave_topk_picks_fast<16>(z, E, k, scale, bias, cand, &e, &v);
    }
    const float top = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float p = (lane < k) ? expf(v - top) : 0.f;
    const float s = wave_allsum_f32(p);
    if (lane < k) {
        const float g = p / s;
        if (idx_out) idx_out[lane] = e;
        if (gate_out) gate_out[lane] = g;
        if (idx_out2) idx_out2[lane] = e;
        if (gate_out2) gate_out2[lane] = g;
        if (idx_lds) idx_lds[lane] = e;
        if (gate_lds) gate_lds[lane] = g;
    }
}

__device__ __forceinline__ bool is_resident(const uint32_t *mask, int e) {
    return !mask || ((mask[e >> 5] >> (e & 31)) & 1u);
}

// Exclusive scan of one int per thread over the block; *total = block sum.
__device__ __forceinline__ int block_excl_scan(int v, int *tmp /* >= 16 ints */, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int inc = wave_incl_scan(v);
    __syncthreads();
    if (lane == 63) tmp[wave] = inc;
    __syncthreads();
    int base = 0, tot = 0;
    for (int w = 0; w < nw; ++w) {
        const int sw = tmp[w];
        base += (w < wave) ? sw : 0;
        tot += sw;
    }
    *total = tot;
    return base + inc - v;
}

// ----------------------------------------------------- small-T routing state
// LDS words (base 16-byte aligned): top-k scratch of up to 8 waves
// [8][TOPK_LDS_WORDS], per-expert token masks [E], resident-picked bitmap
// [32], picks [256] (ids), gates [256], scratch [16].
constexpr int SMALL_ROUTE_WAVES = 8;
__host__ __device__ constexpr int small_route_lds_words(int E) {
    return SMALL_ROUTE_WAVES * TOPK_LDS_WORDS + E + 32 + 256 + 256 + 16;
}

struct SmallRoute {
    uint32_t *cand;
    int32_t *tokmask;
    uint32_t *picked;
    int32_t *sidx;
    float *sgate;
    int32_t *tmp;
    __device__ SmallRoute(uint32_t *base, int E)
        : cand(base),
          tokmask((int32_t *)(base + SMALL_ROUTE_WAVES * TOPK_LDS_WORDS)),
          picked(base + SMALL_ROUTE_WAVES * TOPK_LDS_WORDS + E),
          sidx((int32_t *)(base + SMALL_ROUTE_WAVES * TOPK_LDS_WORDS + E + 32)),
          sgate((float *)(base + SMALL_ROUTE_WAVES * TOPK_LDS_WORDS + E + 32 + 256)),
          tmp((int32_t *)(base + SMALL_ROUTE_WAVES * TOPK_LDS_WORDS + E + 32 + 512)) {}
};

// Top-k of T <= 8 tokens (one wave per token, blocks of at most
// SMALL_ROUTE_WAVES waves) from the unnormalised logits z[t][E] and the
// tokens' inverse RMS inv[t] (both may sit in LDS), then per-expert token
// masks and the bitmap of picked resident experts.
template <bool PLANES = false>
__device__ __forceinline__ void small_route_compute(const LayerArgs &a, const SmallRoute &L, const float *z,
                                                    const float *inv) {
    const int th = threadIdx.x, wave = th >> 6, nw = blockDim.x >> 6;
    const int E = a.E, k = a.k, T = a.T;
    for (int i = th; i < E; i += blockDim.x) L.tokmask[i] = 0;
    if (th < 32) L.picked[th] = 0;
    for (int t = wave; t < T; t += nw)
        wave_topk<PLANES>(z + t * E, E, k, inv[t], a.bias, L.cand + (wave % SMALL_ROUTE_WAVES) * TOPK_LDS_WORDS,
                          nullptr, nullptr, nullptr, nullptr, L.sidx + t * k, L.sgate + t * k, PLANES ? a.zplanes : 1,
                          T * E);
    __syncthreads();
    if (th < T * k) {
        const int e = L.sidx[th];
        atomicOr(&L.tokmask[e], 1 << (th / k));
        if (is_resident(a.mask, e)) atomicOr(&L.picked[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
}

// Token of slot j of a work item from its packed token map: 3 bits per
// slot (tokens < 8), slot j in bits [3j, 3j+3).
constexpr uint32_t TOK_IDENTITY = 0xFAC688u;   // slot j -> token j
__host__ __device__ __forceinline__ int tok_of(uint32_t tpk, int j) { return (int)((tpk >> (3 * j)) & 7u); }

// One token, one wave: the picks alone (no gates, no LDS state) and the
// work item of pick r (in top-k order): its expert and, as first slot, the
// number of picks of lower experts (the slot small_route_write gives it).
// Returns false when that expert is not resident.  Results are wave-uniform.
// cand: this wave's TOPK_LDS_WORDS of LDS.
__device__ __forceinline__ bool one_token_item(const LayerArgs &a, int r, uint32_t *cand, WorkItem &it) {
    const int lane = threadIdx.x & 63, k = a.k;
    int e;
    float v;
    if (a.E <= 512)
        wave_topk_picks_fast<8>(a.z, a.E, k, a.inv_rms[0], a.bias, cand, &e, &v);
    else
        wave_topk_picks_fast<16>(a.z, a.E, k, a.inv_rms[0], a.bias, cand, &e, &v);
    const int er = __builtin_amdgcn_readlane(e, r);
    if (!is_resident(a.mask, er)) return false;
    it = WorkItem{er, (int)__popcll(__ballot(lane < k && e < er)), 1};
    return true;
}

// Every work item of this routing, in the order small_route_write lists
// them, into LDS (whole block): itab[4i .. 4i+3] = expert, first slot,
// token count, packed token map.  Returns the number of items.
__host__ __device__ constexpr int small_route_table_words(int T, int k) {
    return 4 * (T * k + (T + ITEM_TOK - 1) / ITEM_TOK);
}
__device__ __forceinline__ int small_route_table(const LayerArgs &a, const SmallRoute &L, int32_t *itab) {
    const int th = threadIdx.x, nth = blockDim.x;
    const int E = a.E, T = a.T, n = T * a.k;
    const int ept = (E + nth - 1) / nth;
    int c_loc = 0, a_loc = 0;
    for (int j = 0; j < ept; ++j) {
        const int e = th * ept + j;
        if (e < E) {
            const int c = __popc((uint32_t)L.tokmask[e]);
            c_loc += c;
            a_loc += is_resident(a.mask, e) ? (c + ITEM_TOK - 1) / ITEM_TOK : 0;
        }
    }
    int tot;
    const int ex = block_excl_scan((a_loc << 16) | c_loc, L.tmp, &tot);
    int off = ex & 0xFFFF, ai = ex >> 16;
    for (int j = 0; j < ept; ++j) {
        const int e = th * ept + j;
        if (e < E) {
            const uint32_t mk = (uint32_t)L.tokmask[e];
            const int c = __popc(mk);
            if (is_resident(a.mask, e)) {
                uint32_t rest = mk;
                for (int q = 0; q < c; q += ITEM_TOK) {
                    uint32_t tpk = 0;
                    for (int i = 0; i < ITEM_TOK && rest; ++i) {
                        tpk |= (uint32_t)(__ffs(rest) - 1) << (3 * i);
                        rest &= rest - 1u;
                    }
                    *(int4 *)(itab + 4 * ai) = make_int4(e, off + q, min(ITEM_TOK, c - q), (int)tpk);
                    ++ai;
                }
            }
            off += c;
        }
    }
    if (th == 0) {
        for (int q = 0; q < T; q += ITEM_TOK)
            *(int4 *)(itab + 4 * ((tot >> 16) + q / ITEM_TOK)) =
                make_int4(E, n + q, min(ITEM_TOK, T - q), (int)(TOK_IDENTITY >> (3 * q)));
    }
    __syncthreads();
    return (tot >> 16) + (T + ITEM_TOK - 1) / ITEM_TOK;
}

// One block: write the routing outputs (ids, gates, counts, offsets,
// permutation, work list for the down kernel, miss list, user copies).
__device__ __forceinline__ void small_route_write(const LayerArgs &a, const SmallRoute &L) {
    const int th = threadIdx.x, nth = blockDim.x;
    const int E = a.E, k = a.k, T = a.T, n = T * k;
    if (th < n) {
        a.idx[th] = L.sidx[th];
        a.gate[th] = L.sgate[th];
        if (a.u_idx) a.u_idx[th] = L.sidx[th];
        if (a.u_gate) a.u_gate[th] = L.sgate[th];
    }
    const int ept = (E + nth - 1) / nth;
    int c_loc = 0, a_loc = 0;
    for (int j = 0; j < ept; ++j) {
        const int e = th * ept + j;
        if (e < E) {
            const int c = __popc((uint32_t)L.tokmask[e]);
            c_loc += c;
            a_loc += is_resident(a.mask, e) ? (c + ITEM_TOK - 1) / ITEM_TOK : 0;
        }
    }
    int tot;
    const int ex = block_excl_scan((a_loc << 16) | c_loc, L.tmp, &tot);
    int off = ex & 0xFFFF, ai = ex >> 16;
    for (int j = 0; j < ept; ++j) {
        const int e = th * ept + j;
        if (e < E) {
            const int c = __popc((uint32_t)L.tokmask[e]);
            a.counts[e] = c;
            a.offsets[e] = off;
            if (a.u_counts) a.u_counts[e] = c;
            if (a.u_offsets) a.u_offsets[e] = off;
            if (is_resident(a.mask, e))
                for (int q = 0; q < c; q += ITEM_TOK) a.items[ai++] = WorkItem{e, off + q, min(ITEM_TOK, c - q)};
            off += c;
        }
    }
    if (th == 0) {
        a.offsets[E] = tot & 0xFFFF;
        if (a.u_offsets) a.u_offsets[E] = tot & 0xFFFF;
        for (int q = 0; q < T; q += ITEM_TOK) a.items[(tot >> 16) + q / ITEM_TOK] = WorkItem{E, n + q, min(ITEM_TOK, T - q)};
        *a.n_items = (tot >> 16) + (T + ITEM_TOK - 1) / ITEM_TOK;
    }
    // slot of pick (t, r): offset of its expert + earlier tokens of that expert
    if (th < n) {
        const int e = L.sidx[th], t = th / k;
        int below = 0;
        for (int j = 0; j < n; ++j) below += L.sidx[j] < e ? 1 : 0;
        const int slot = below + __popc((uint32_t)L.tokmask[e] & ((1u << t) - 1u));
        a.perm[slot] = th;
        a.pos[th] = slot;
        if (a.u_perm) a.u_perm[slot] = th;
        if (a.u_pos) a.u_pos[th] = slot;
    }
    const int miss = (th < n && !is_resident(a.mask, L.sidx[th])) ? 1 : 0;
    int mt;
    const int mp = block_excl_scan(miss, L.tmp, &mt);
    if (miss && a.miss_te && mp < a.miss_cap) {
        a.miss_te[2 * mp] = th / k;
        a.miss_te[2 * mp + 1] = L.sidx[th];
        a.miss_w[mp] = L.sgate[th];
    }
    if (th == 0 && a.miss_count) *a.miss_count = mt;
    if (a.mask && th < T) {
        uint32_t b = 0;
        for (int r = 0; r < k; ++r) b |= is_resident(a.mask, L.sidx[th * k + r]) ? 1u << r : 0u;
        a.rbits[th] = (int32_t)b;
    }
}

}  // namespace strata
