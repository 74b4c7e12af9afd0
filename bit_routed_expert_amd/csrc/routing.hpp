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

// Ordered top-k of E logits z[e] * scale + bias[e] by one wave (JM = E/64
// rounded up to 8 or 16); lane r < k ends with pick r: *e_out, *z_out.  Each
// lane sorts its JM candidates by (value desc, index asc); a round takes the
// wave maximum of the lanes' head values (32-bit), then the smallest head
// index among the lanes holding it; the owning lane pops its head.
template <int JM>
__device__ __forceinline__ void wave_topk_picks_fast(const float *z, int E, int k, float scale, const float *bias,
                                                     int *e_out, float *z_out) {
    const int lane = threadIdx.x & 63;
    float zv[JM], bv[JM];
#pragma unroll
    for (int j = 0; j < JM; ++j) zv[j] = z[min(lane + 64 * j, E - 1)];
#pragma unroll
    for (int j = 0; j < JM; ++j) bv[j] = 0.f;
    if (bias) {
#pragma unroll
        for (int j = 0; j < JM; ++j) bv[j] = bias[min(lane + 64 * j, E - 1)];
    }
    uint32_t kv[JM], ki[JM];   // value key (0 = empty), expert index
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        const int e = lane + 64 * j;
        kv[j] = (e < E) ? f32_key(zv[j] * scale + bv[j]) : 0u;
        ki[j] = (uint32_t)e;
    }
    // bitonic sort, descending by (kv, -ki); indices of one lane increase with j
#pragma unroll
    for (int kk = 2; kk <= JM; kk <<= 1)
#pragma unroll
        for (int jj = kk >> 1; jj > 0; jj >>= 1)
#pragma unroll
            for (int i = 0; i < JM; ++i) {
                const int l = i ^ jj;
                if (l > i) {
                    const bool desc = (i & kk) == 0;
                    const bool a_first = kv[i] > kv[l] || (kv[i] == kv[l] && ki[i] < ki[l]);
                    const bool sw = desc ? !a_first : a_first;
                    const uint32_t tv = kv[i], ti = ki[i];
                    kv[i] = sw ? kv[l] : tv;
                    ki[i] = sw ? ki[l] : ti;
                    kv[l] = sw ? tv : kv[l];
                    ki[l] = sw ? ti : ki[l];
                }
            }
    int my_e = 0;
    uint32_t my_k = 0x80000000u;   // key of 0.0 for lanes past k
    for (int r = 0; r < k; ++r) {
        // largest head value, then the smallest expert index among the
        // lanes holding it; both land in every lane
        const uint32_t m = wave_allmax_u32(kv[0]);
        const uint32_t e = wave_allmin_u32(kv[0] == m ? ki[0] : 0xFFFFFFFFu);
        if (lane == r) {
            my_e = (int)e;
            my_k = m;
        }
        if (kv[0] == m && ki[0] == e) {  // the owner pops its head
#pragma unroll
            for (int j = 0; j < JM - 1; ++j) {
                kv[j] = kv[j + 1];
                ki[j] = ki[j + 1];
            }
            kv[JM - 1] = 0u;
        }
    }
    *e_out = my_e;
    *z_out = __uint_as_float((my_k & 0x80000000u) ? (my_k & 0x7FFFFFFFu) : ~my_k);
}

// Ordered top-k and gates of one token by one wave; lanes r < k write pick r.
__device__ __forceinline__ void wave_topk(const float *z, int E, int k, float scale, const float *bias,
                                          int32_t *idx_out, float *gate_out, int32_t *idx_out2, float *gate_out2,
                                          int32_t *idx_lds, float *gate_lds) {
    const int lane = threadIdx.x & 63;
    int e;
    float v;
    if (E <= 512)
        wave_topk_picks_fast<8>(z, E, k, scale, bias, &e, &v);
    else
        wave_topk_picks_fast<16>(z, E, k, scale, bias, &e, &v);
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
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o, WAVE);
        if (lane >= o) inc += t;
    }
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
// LDS words: per-expert token masks [E], resident-picked bitmap [32],
// picks [256] (ids), gates [256], scratch [16].
__host__ __device__ constexpr int small_route_lds_words(int E) { return E + 32 + 256 + 256 + 16; }

struct SmallRoute {
    int32_t *tokmask;
    uint32_t *picked;
    int32_t *sidx;
    float *sgate;
    int32_t *tmp;
    __device__ SmallRoute(uint32_t *base, int E)
        : tokmask((int32_t *)base),
          picked(base + E),
          sidx((int32_t *)(base + E + 32)),
          sgate((float *)(base + E + 32 + 256)),
          tmp((int32_t *)(base + E + 32 + 512)) {}
};

// Top-k of T <= 8 tokens (one wave per token) from the unnormalised logits
// z[t][E] and the tokens' inverse RMS inv[t] (both may sit in LDS), then
// per-expert token masks and the bitmap of picked resident experts.
__device__ __forceinline__ void small_route_compute(const LayerArgs &a, const SmallRoute &L, const float *z,
                                                    const float *inv) {
    const int th = threadIdx.x, wave = th >> 6, nw = blockDim.x >> 6;
    const int E = a.E, k = a.k, T = a.T;
    for (int i = th; i < E; i += blockDim.x) L.tokmask[i] = 0;
    if (th < 32) L.picked[th] = 0;
    for (int t = wave; t < T; t += nw)
        wave_topk(z + t * E, E, k, inv[t], a.bias, nullptr, nullptr, nullptr, nullptr, L.sidx + t * k,
                  L.sgate + t * k);
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
__device__ __forceinline__ bool one_token_item(const LayerArgs &a, int r, WorkItem &it) {
    const int lane = threadIdx.x & 63, k = a.k;
    int e;
    float v;
    if (a.E <= 512)
        wave_topk_picks_fast<8>(a.z, a.E, k, a.inv_rms[0], a.bias, &e, &v);
    else
        wave_topk_picks_fast<16>(a.z, a.E, k, a.inv_rms[0], a.bias, &e, &v);
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
}

}  // namespace strata
