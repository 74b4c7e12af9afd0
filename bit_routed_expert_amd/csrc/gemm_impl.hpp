// Expert FFNs for larger token counts: grouped GEMMs on the gfx950 matrix
// cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Every routed expert with n_e tokens, and the shared expert with all T
// tokens, computes g = W_g x, u = W_u x, h = silu(g) * u, y = W_d h
// (greenbean-ai, "Strata 如何讓 12GB 顯卡跑 Qwen3.8-Flash-Next？", section 一:
// 512 experts per layer, 10 routed + 1 shared per token; the block-quantised
// weights of section 四 are expanded only inside the kernel).  Work is cut
// into tiles of up to GEMM_BM tokens of one expert; a 256-thread block takes
// one tile and one slice of output features, each wave owning 32 (gate/up:
// 32 gate + the same 32 up rows) or 64 (down) features for all tile rows.
//
// Operands.  A (activations) is bf16, staged through LDS by direct
// global->LDS loads; the layer input and h are carried as a hi/lo bf16
// pair when they are not exactly bf16 (both pieces accumulate into the
// same fp32 tile, about 16 significant bits).  B (weights) is decoded in
// registers straight from the packed codes: a code c becomes the bf16
// number OFF8 + c (8 + c for 3-bit, 4 + c for 2-bit, both exact) with two
// integer ops per pair of codes.  The MFMA partial over one scale block
// (128 or 256 columns) is P = sum x (OFF8 + c); the true block product is
// sum x (c - c0) = P - (OFF8 + c0) * S with S = sum x over the block,
// which the producers of A also store, and it is folded in fp32 as
// acc += scale * (P - OFF * S).
//
// K order.  Inside each 128-column step the activations are stored
// permuted so that the 8 values a lane feeds to one MFMA are exactly the 8
// codes it unpacks from one 32-bit code word; the codes of one 32-column
// unit sit in four groups of 8 (words A, B, C and the bit-3 word of the
// 3-bit format; the low and high pairs of words A and B in the 2-bit
// format), each group in nibble order [0,4,1,5,2,6,3,7].
#pragma once
#include "mfma.hpp"

namespace strata {

constexpr int GM_NM = GEMM_BM / 32;   // 32-row token subtiles per tile
constexpr int GSUB = 64;              // K positions per LDS stage
constexpr int GROW = GSUB * 2;        // bytes per staged A row
constexpr int GMAX_STEPS = GEMM_MAX_K / 128;

// Position of column offset cc (0..127) inside its 128-column step.
__host__ __device__ __forceinline__ int step_pos(int cc) {
    const int u = cc >> 5, g = (cc >> 3) & 3, jj = cc & 7;
    const int j = (jj & 3) * 2 + (jj >> 2);   // inverse of [0,4,1,5,2,6,3,7]
    return 16 * (4 * (u & 1) + g) + 8 * (u >> 1) + j;
}

// 16-byte chunk swizzle of staged A rows (conflict-free 16-byte LDS reads
// of 32 consecutive rows at one logical chunk).
__device__ __forceinline__ int a_swz(int m) { return (m ^ (m >> 3)) & 7; }

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

__device__ __forceinline__ void lds_dma16(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// ---------------------------------------------------------------- decode
// M, B: 0x00700070 / 0x41004100 (3-bit) or 0x00600060 / 0x40804080 (2-bit);
// both 0 turn every decoded weight into 0 (a block whose scale is zero).
__device__ __forceinline__ u32x4_t pairs3(uint32_t W, uint32_t M, uint32_t B) {
    u32x4_t r;
    r[0] = ((W << 4) & M) | B;
    r[1] = (W & M) | B;
    r[2] = ((W >> 4) & M) | B;
    r[3] = ((W >> 8) & M) | B;
    return r;
}
template <int HP> __device__ __forceinline__ u32x4_t pairs2(uint32_t W, uint32_t M, uint32_t B) {
    u32x4_t r;
    r[0] = ((W << (5 - 2 * HP)) & M) | B;
    r[1] = ((HP == 0 ? (W << 1) : (W >> 1)) & M) | B;
    r[2] = ((W >> (3 + 2 * HP)) & M) | B;
    r[3] = ((W >> (7 + 2 * HP)) & M) | B;
    return r;
}

template <int BITS> struct Raw;
template <> struct Raw<3> { uint32_t w0, w1, w2; };
template <> struct Raw<2> { uint32_t w0, w1; };

template <int BITS> __device__ __forceinline__ Raw<BITS> load_unit(const uint8_t *p);
template <> __device__ __forceinline__ Raw<3> load_unit<3>(const uint8_t *p) {
    const uint32_t *q = (const uint32_t *)p;
    return Raw<3>{q[0], q[1], q[2]};
}
template <> __device__ __forceinline__ Raw<2> load_unit<2>(const uint8_t *p) {
    const uint2 v = *(const uint2 *)p;
    return Raw<2>{v.x, v.y};
}

// Buffer resources: a block-uniform base and size (scalar registers), so a
// load is the lane's 32-bit offset plus a uniform offset in a scalar
// register, with no per-lane address arithmetic; reads past the size return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
template <int BITS> __device__ __forceinline__ Raw<BITS> load_unit_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                                     uint32_t soff);
template <> __device__ __forceinline__ Raw<3> load_unit_buf<3>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0);
    return Raw<3>{v[0], v[1], v[2]};
}
template <> __device__ __forceinline__ Raw<2> load_unit_buf<2>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    return Raw<2>{v[0], v[1]};
}
// A pointer known to be the same in every lane, in scalar registers.
__device__ __forceinline__ const uint8_t *uniform_ptr(const void *p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint8_t *)(((uint64_t)hi << 32) | lo);
}

template <int G> __device__ __forceinline__ bf16x8_t decode_group3(const Raw<3> &r, uint32_t M, uint32_t B) {
    uint32_t W;
    if (G == 0) W = r.w0;
    else if (G == 1) W = r.w1;
    else if (G == 2) W = r.w2;
    else W = ((r.w0 >> 3) & 0x11111111u) | ((r.w1 >> 2) & 0x22222222u) | ((r.w2 >> 1) & 0x44444444u);
    return __builtin_bit_cast(bf16x8_t, pairs3(W, M, B));
}
template <int G> __device__ __forceinline__ bf16x8_t decode_group2(const Raw<2> &r, uint32_t M, uint32_t B) {
    return __builtin_bit_cast(bf16x8_t, pairs2<G & 1>(G < 2 ? r.w0 : r.w1, M, B));
}

template <int BITS> struct Dec;
template <> struct Dec<3> {
    static constexpr uint32_t MASK = 0x00700070u, BASE = 0x41004100u;   // bf16 8 + c, c in mantissa bits 4..6
    static constexpr float OFF = 11.5f;                                 // 8 + c0, c0 = 3.5
    template <int G> static __device__ __forceinline__ bf16x8_t get(const Raw<3> &r, uint32_t M, uint32_t B) {
        return decode_group3<G>(r, M, B);
    }
};
template <> struct Dec<2> {
    static constexpr uint32_t MASK = 0x00600060u, BASE = 0x40804080u;   // bf16 4 + c, c in mantissa bits 5..6
    static constexpr float OFF = 5.5f;                                  // 4 + c0, c0 = 1.5
    template <int G> static __device__ __forceinline__ bf16x8_t get(const Raw<2> &r, uint32_t M, uint32_t B) {
        return decode_group2<G>(r, M, B);
    }
};

// byte offset of the 32-column unit U of row r in a packed [out][in] matrix
template <int BITS> __device__ __forceinline__ int64_t unit_off(int r, int U, int in) {
    constexpr int UB = BITS == 3 ? 12 : 8;
    return ((((int64_t)(r >> 4) * (in >> 7) + (U >> 2)) * 16 + (r & 15)) * 4 + (U & 3)) * UB;
}

// Staged A row m of the block, logical 16-byte chunk c (0..7).
__device__ __forceinline__ bf16x8_t lds_a_read(const uint8_t *buf, int m, int c) {
    return __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(buf + m * GROW + 16 * (c ^ a_swz(m))));
}

// Block -> (tile, feature slice), all slices of a tile on one XCD (blocks
// are dealt to the 8 XCDs round-robin).  Returns false for spare blocks.
__device__ __forceinline__ bool pick_tile(int nft, int n_items, int &tile, int &ft) {
    const int total = nft * n_items;
    const int per = (total + 7) >> 3;
    const int b = blockIdx.x;
    const int q = b >> 3;
    const int bb = (b & 7) * per + q;
    if (q >= per || bb >= total) return false;
    tile = bb / nft;
    ft = bb - tile * nft;
    return true;
}

// Stage LDS step s (64 K positions) of the block's A rows into dst: each
// wave moves three groups of 8 rows per pass, 16 bytes per lane, straight
// into LDS (rows of pass p at dst + p * GEMM_BM * GROW).  Addresses are a
// block-uniform base (scalar registers) plus this lane's 32-bit byte offset.
template <int PASSES>
__device__ __forceinline__ void stage_a(__amdgpu_buffer_rsrc_t ar, const uint32_t aoff[3], uint32_t pass_bytes, int s,
                                        uint8_t *__restrict__ dst, int wv) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
        for (int q = 0; q < 3; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ar, (__attribute__((address_space(3))) void *)(dst + p * GEMM_BM * GROW + (wv * 3 + q) * 8 * GROW), 16,
                aoff[q], p * pass_bytes + (uint32_t)s * GSUB * 2, 0, 0);
}

// byte offset of the code unit a lane reads at LDS step s (relative to unit 2h of step 0)
template <int BITS> __device__ __forceinline__ int64_t b_off(int s) {
    constexpr int UB = BITS == 3 ? 12 : 8;
    return (int64_t)(s >> 1) * 64 * UB + (s & 1) * UB;
}

// Two weight slices (32 features each) against NMT token subtiles.  The
// accumulators hold the sum over the scale blocks seen so far divided by
// the current block's scale (Horner form): entering block c multiplies them
// by s_{c-1} / s_c, the block's MFMAs then add sum x (OFF8 + c) and one
// more MFMA adds -OFF * S; the result is acc * s_last.  A block with a zero
// scale is skipped by decoding its codes (and the offset weight) as 0 and
// keeping the previous scale.
template <int BITS, int NMT> struct Acc2 {
    f32x16_t A0[NMT], A1[NMT];
    float s0, s1;            // current scale of each slice (nonzero)
    uint32_t m0, b0, m1, b1; // decode mask / base of each slice (0 for a zero-scale block)
};

// MFMAs of one LDS step: the 4 code groups of this lane's unit for both
// slices, each against every token subtile and A pass.  Reads rd only.
template <int BITS, int PASSES, int NMT>
__device__ __forceinline__ void mfma_step(const uint8_t *__restrict__ rd, const Raw<BITS> &c0, const Raw<BITS> &c1,
                                          Acc2<BITS, NMT> &acc, int n, int h) {
#define MFMA_GROUP(G)                                                                    \
    {                                                                                    \
        const bf16x8_t w0 = Dec<BITS>::template get<G>(c0, acc.m0, acc.b0);              \
        const bf16x8_t w1 = Dec<BITS>::template get<G>(c1, acc.m1, acc.b1);              \
        _Pragma("unroll") for (int mi = 0; mi < NMT; ++mi) {                             \
            _Pragma("unroll") for (int p = 0; p < PASSES; ++p) {                         \
                const bf16x8_t av = lds_a_read(rd + p * GEMM_BM * GROW, mi * 32 + n, 2 * (G) + h); \
                acc.A0[mi] = mfma(av, w0, acc.A0[mi]);                                   \
                acc.A1[mi] = mfma(av, w1, acc.A1[mi]);                                   \
            }                                                                            \
        }                                                                                \
    }
    MFMA_GROUP(0) MFMA_GROUP(1) MFMA_GROUP(2) MFMA_GROUP(3)
#undef MFMA_GROUP
}

__device__ __forceinline__ uint32_t bf16_bits(float v) { return __float_as_uint(v) >> 16; }  // exact for bf16 values

// -OFF * S as three bf16 pieces (hi + mid + lo carry fp32's 24 bits), packed
// as the first K columns of an A fragment: {hi | mid << 16, lo}.
template <int BITS> __device__ __forceinline__ uint2 offset_pieces(float S) {
    const float t = -Dec<BITS>::OFF * S;
    const uint32_t hi = f2bf(t);
    const float t1 = t - __uint_as_float(hi << 16);
    const uint32_t mid = f2bf(t1);
    const uint32_t lo = f2bf(t1 - __uint_as_float(mid << 16));
    return make_uint2(hi | (mid << 16), lo);
}

// Enter scale block cb with raw fp16 scales q0, q1 of the two slices.
template <int BITS, int NMT>
__device__ __forceinline__ void enter_block(Acc2<BITS, NMT> &acc, const uint2 *__restrict__ lds_s, int cb,
                                            uint16_t q0, uint16_t q1, int n, int h) {
    const float f0 = half_to_float(q0), f1 = half_to_float(q1);
    const bool z0 = f0 == 0.f, z1 = f1 == 0.f;
    // ratio of the previous scale to this one (hardware reciprocal, 1 ulp)
    const float r0 = z0 ? 1.f : acc.s0 * __builtin_amdgcn_rcpf(f0), r1 = z1 ? 1.f : acc.s1 * __builtin_amdgcn_rcpf(f1);
    acc.s0 = z0 ? acc.s0 : f0;
    acc.s1 = z1 ? acc.s1 : f1;
    acc.m0 = z0 ? 0u : Dec<BITS>::MASK;
    acc.b0 = z0 ? 0u : Dec<BITS>::BASE;
    acc.m1 = z1 ? 0u : Dec<BITS>::MASK;
    acc.b1 = z1 ? 0u : Dec<BITS>::BASE;
    // offset weights: 1, 1, 1 in K rows 0..2 of the extra MFMA (lanes of half 0)
    const uint32_t one = 0x3F80u;
    const uint32_t o0 = (h == 0 && !z0) ? (one | (one << 16)) : 0u, o1 = (h == 0 && !z1) ? (one | (one << 16)) : 0u;
    const bf16x8_t w0 = __builtin_bit_cast(bf16x8_t, u32x4_t{o0, o0 & 0xFFFFu, 0u, 0u});
    const bf16x8_t w1 = __builtin_bit_cast(bf16x8_t, u32x4_t{o1, o1 & 0xFFFFu, 0u, 0u});
#pragma unroll
    for (int mi = 0; mi < NMT; ++mi) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            acc.A0[mi][v] *= r0;
            acc.A1[mi][v] *= r1;
        }
        // -OFF * S of row mi*32 + n as three bf16 pieces in K columns 0..2
        const uint2 pc = lds_s[cb * GEMM_BM + mi * 32 + n];
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, u32x4_t{pc.x, pc.y, 0u, 0u});
        acc.A0[mi] = mfma(av, w0, acc.A0[mi]);
        acc.A1[mi] = mfma(av, w1, acc.A1[mi]);
    }
}

// Main K loop shared by both GEMMs: stage s+1 (A by DMA, codes into
// registers) while step s runs on the matrix cores; enter a new scale
// block every CH columns.  cr0 + co0 / cr1 + co1: code unit of this lane for the two slices
// at step 0; sc0p/sc1p + (row*in + c) / 256: their scales.
template <int BITS, int PASSES, int NMT>
__device__ __forceinline__ void k_loop(Acc2<BITS, NMT> &acc, uint8_t *__restrict__ buf0, uint8_t *__restrict__ buf1,
                                       const uint2 *__restrict__ lds_s, __amdgpu_buffer_rsrc_t ar,
                                       const uint32_t aoff[3], uint32_t pass_bytes, __amdgpu_buffer_rsrc_t cr0,
                                       uint32_t co0, __amdgpu_buffer_rsrc_t cr1, uint32_t co1,
                                       const uint16_t *sc0p, const uint16_t *sc1p, int64_t rin0, int64_t rin1,
                                       int in, bool active, int wv, int n, int h) {
    const int nsub = in / GSUB;
    const int CH = (in & 255) ? 128 : 256;   // scale block along K
    const int spc = CH / GSUB;               // LDS steps per scale block (2 or 4: blocks start at even steps)
#pragma unroll
    for (int mi = 0; mi < NMT; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc.A0[mi][v] = acc.A1[mi][v] = 0.f;
    acc.s0 = acc.s1 = 1.f;
    Raw<BITS> ra0 = load_unit_buf<BITS>(cr0, co0, 0), rb0 = load_unit_buf<BITS>(cr1, co1, 0);
    Raw<BITS> ra1 = ra0, rb1 = rb0;
    uint16_t q0 = sc0p[rin0 >> 8], q1 = sc1p[rin1 >> 8];
    stage_a<PASSES>(ar, aoff, pass_bytes, 0, buf0, wv);
    wait_vmem();
    __syncthreads();
    for (int s = 0; s < nsub; s += 2) {
        // even step: compute from buf0, stage into buf1
        stage_a<PASSES>(ar, aoff, pass_bytes, s + 1, buf1, wv);
        if (active) {
            ra1 = load_unit_buf<BITS>(cr0, co0, (uint32_t)b_off<BITS>(s + 1));
            rb1 = load_unit_buf<BITS>(cr1, co1, (uint32_t)b_off<BITS>(s + 1));
            if (s % spc == 0) {
                enter_block<BITS, NMT>(acc, lds_s, s / spc, q0, q1, n, h);
                if (s + spc < nsub) {   // next block's scales
                    const int64_t c = (int64_t)(s + spc) * GSUB;
                    q0 = sc0p[(rin0 + c) >> 8];
                    q1 = sc1p[(rin1 + c) >> 8];
                }
            }
            mfma_step<BITS, PASSES, NMT>(buf0, ra0, rb0, acc, n, h);
        }
        wait_vmem();
        __syncthreads();
        // odd step: compute from buf1, stage into buf0
        const bool more = s + 2 < nsub;
        if (more) stage_a<PASSES>(ar, aoff, pass_bytes, s + 2, buf0, wv);
        if (active) {
            if (more) {
                ra0 = load_unit_buf<BITS>(cr0, co0, (uint32_t)b_off<BITS>(s + 2));
                rb0 = load_unit_buf<BITS>(cr1, co1, (uint32_t)b_off<BITS>(s + 2));
            }
            mfma_step<BITS, PASSES, NMT>(buf1, ra1, rb1, acc, n, h);
        }
        wait_vmem();
        __syncthreads();
    }
#pragma unroll
    for (int mi = 0; mi < NMT; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            acc.A0[mi][v] *= acc.s0;
            acc.A1[mi][v] *= acc.s1;
        }
}

// Token of tile row m (rows past ntok repeat the last token; their results are dropped).
__device__ __forceinline__ int tile_token(const LayerArgs &a, const WorkItem &it, int m) {
    const int64_t Tk = (int64_t)a.T * a.k;
    const int64_t slot = it.slot0 + min(m, it.ntok - 1);
    return slot < Tk ? a.perm[slot] / a.k : (int)(slot - Tk);
}

// ------------------------------------------------------------ gate / up
// Slices: gate rows j0 + n and up rows j0 + n, j0 = 128 * ft + 32 * wave.
template <int BITS, int PASSES, int NMT>
__device__ __forceinline__ void gateup_tile(const LayerArgs &a, const WorkItem &it, int ft,
                                            uint8_t *__restrict__ buf0, uint8_t *__restrict__ buf1,
                                            uint2 *__restrict__ lds_s, const int *__restrict__ lds_tok) {
    const int th = threadIdx.x, lane = th & 63, wv = th >> 6;
    const int n = lane & 31, h = lane >> 5;
    const int d = a.d, f = a.f, T = a.T;
    const int64_t Tk = (int64_t)T * a.k;
    const int ntok = it.ntok;
    // S per scale block (128 or 256 columns) and row, from the per-step sums
    const int nsteps = d >> 7, spb = (d & 255) ? 1 : 2, nblk = nsteps / spb;
    for (int i = th; i < nblk * GEMM_BM; i += 256) {
        const int cb = i / GEMM_BM, m = i - cb * GEMM_BM;
        const float *p = a.sx + (int64_t)lds_tok[m] * nsteps + cb * spb;
        lds_s[i] = offset_pieces<BITS>(spb == 2 ? p[0] + p[1] : p[0]);
    }
    uint32_t aoff[3];   // byte offsets into xa (< 2^31: checked by the launcher)
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const int m = (wv * 3 + q) * 8 + (lane >> 3);
        aoff[q] = 2u * ((uint32_t)lds_tok[m] * (uint32_t)d + 8u * ((lane & 7) ^ a_swz(m)));
    }
    const int j0 = ft * 128 + wv * 32, r = j0 + n;
    const uint32_t mbytes = (uint32_t)((int64_t)f * d * BITS / 8);   // one packed matrix
    const uint8_t *cg = uniform_ptr(a.codes + (int64_t)it.expert * 3 * mbytes);
    const uint8_t *cu = cg + mbytes;
    const uint16_t *sg = a.scales + (int64_t)it.expert * ((int64_t)3 * d * f / 256);
    const uint16_t *su = sg + (int64_t)f * d / 256;
    Acc2<BITS, NMT> acc;
    const uint32_t co = (uint32_t)unit_off<BITS>(r, 2 * h, d);
    k_loop<BITS, PASSES, NMT>(acc, buf0, buf1, lds_s, buf_rsrc(a.xa, (uint32_t)PASSES * T * d * 2), aoff,
                              (uint32_t)T * d * 2, buf_rsrc(cg, mbytes), co, buf_rsrc(cu, mbytes), co, sg, su, (int64_t)r * d, (int64_t)r * d, d, true,
                              wv, n, h);
    // h = silu(g) * u as a bf16 hi/lo pair at its permuted position, and
    // per-row sums of hi + lo over this wave's 32 features
    const int64_t slots = Tk + T;
    const int pos = (r & ~127) + step_pos(r & 127);
    // stores go through buffer resources spanning the tile's ntok rows, so
    // rows past ntok fall outside them and are dropped by the hardware
    const uint32_t rowb = 2u * f, nf = f / 32;
    const __amdgpu_buffer_rsrc_t rhi = buf_rsrc(uniform_ptr(a.ha + (int64_t)it.slot0 * f), ntok * rowb);
    const __amdgpu_buffer_rsrc_t rlo = buf_rsrc(uniform_ptr(a.ha + (slots + it.slot0) * f), ntok * rowb);
    const __amdgpu_buffer_rsrc_t rhs = buf_rsrc(uniform_ptr(a.hs + (int64_t)it.slot0 * nf), ntok * nf * 4);
    const uint32_t vo = 4u * h * rowb + 2u * pos, vs = 4u * (4u * h * nf + (j0 >> 5));
#pragma unroll
    for (int mi = 0; mi < NMT; ++mi) {
        float ssum[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const uint32_t ml = mi * 32 + 8 * (v >> 2) + (v & 3);   // tile row minus 4h
            const float g = acc.A0[mi][v], u = acc.A1[mi][v];
            const float hv = silu_mul(g, u);
            const uint16_t hi = f2bf(hv);
            const float hif = bf16_to_float(hi);
            const uint16_t lo = f2bf(hv - hif);
            ssum[v] = hif + bf16_to_float(lo);
            __builtin_amdgcn_raw_buffer_store_b16(hi, rhi, vo + ml * rowb, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b16(lo, rlo, vo + ml * rowb, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) ssum[v] = half_wave_sum(ssum[v]);
        if (n == 31) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const uint32_t ml = mi * 32 + 8 * (v >> 2) + (v & 3);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ssum[v]), rhs, vs + ml * nf * 4, 0, 0);
            }
        }
    }
}

template <int BITS, int PASSES>
__global__ __launch_bounds__(256, PASSES == 1 ? 3 : 2) void gemm_gateup_kernel(LayerArgs a, int nft) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_a0[PASSES * GEMM_BM * GROW];
    __shared__ __attribute__((aligned(16))) uint8_t lds_a1[PASSES * GEMM_BM * GROW];
    __shared__ uint2 lds_s[GMAX_STEPS * GEMM_BM];   // [scale block][row]: -OFF * S as bf16 pieces
    __shared__ int lds_tok[GEMM_BM];
    int tile, ft;
    if (!pick_tile(nft, *a.n_items, tile, ft)) return;
    const WorkItem it = a.items[tile];
    if (threadIdx.x < GEMM_BM) lds_tok[threadIdx.x] = tile_token(a, it, threadIdx.x);
    __syncthreads();
    switch ((it.ntok + 31) >> 5) {
        case 1: gateup_tile<BITS, PASSES, 1>(a, it, ft, lds_a0, lds_a1, lds_s, lds_tok); break;
        case 2: gateup_tile<BITS, PASSES, 2>(a, it, ft, lds_a0, lds_a1, lds_s, lds_tok); break;
        default: gateup_tile<BITS, PASSES, GM_NM>(a, it, ft, lds_a0, lds_a1, lds_s, lds_tok); break;
    }
}

// ------------------------------------------------------------------ down
// Slices: down rows j0 + n and j0 + 32 + n, j0 = 256 * ft + 64 * wave
// (waves past d take part in staging only).
template <int BITS, int NMT>
__device__ __forceinline__ void down_tile(const LayerArgs &a, const WorkItem &it, int ft,
                                          uint8_t *__restrict__ buf0, uint8_t *__restrict__ buf1,
                                          uint2 *__restrict__ lds_s) {
    const int th = threadIdx.x, lane = th & 63, wv = th >> 6;
    const int n = lane & 31, h = lane >> 5;
    const int d = a.d, f = a.f, T = a.T;
    const int64_t slots = (int64_t)T * a.k + T;
    const int ntok = it.ntok;
    // S per scale block (128 or 256 features) and row, from the 32-feature sums
    const int gpb = (f & 255) ? 4 : 8, nblk = f / (32 * gpb);
    for (int i = th; i < nblk * GEMM_BM; i += 256) {
        const int cb = i / GEMM_BM, m = i - cb * GEMM_BM;
        const float *p = a.hs + (it.slot0 + min(m, ntok - 1)) * (f / 32) + gpb * cb;
        float acc = 0.f;
        for (int q = 0; q < gpb; ++q) acc += p[q];
        lds_s[i] = offset_pieces<BITS>(acc);
    }
    uint32_t aoff[3];   // byte offsets into ha (< 2^31: checked by the launcher)
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const int m = (wv * 3 + q) * 8 + (lane >> 3);
        aoff[q] = 2u * ((uint32_t)(it.slot0 + min(m, ntok - 1)) * (uint32_t)f + 8u * ((lane & 7) ^ a_swz(m)));
    }
    const int j0 = ft * 256 + wv * 64;
    const bool active = j0 < d;
    const int r0 = min(j0, d - 64) + n, r1 = r0 + 32;
    const uint32_t mbytes = (uint32_t)((int64_t)f * d * BITS / 8);   // one packed matrix
    const uint8_t *cd = uniform_ptr(a.codes + ((int64_t)it.expert * 3 + 2) * mbytes);
    const uint16_t *sd = a.scales + (int64_t)it.expert * ((int64_t)3 * d * f / 256) + (int64_t)2 * f * d / 256;
    Acc2<BITS, NMT> acc;
    const __amdgpu_buffer_rsrc_t cr = buf_rsrc(cd, mbytes);
    k_loop<BITS, 2, NMT>(acc, buf0, buf1, lds_s, buf_rsrc(a.ha, (uint32_t)(2 * slots * f * 2)), aoff,
                         (uint32_t)(slots * f * 2), cr, (uint32_t)unit_off<BITS>(r0, 2 * h, f), cr,
                         (uint32_t)unit_off<BITS>(r1, 2 * h, f), sd, sd, (int64_t)r0 * f, (int64_t)r1 * f, f, active,
                         wv, n, h);
    if (!active) return;
    // rows past ntok fall outside the resource and are dropped
    const uint32_t rowb = 4u * d;
    const __amdgpu_buffer_rsrc_t ry = buf_rsrc(uniform_ptr(a.Y + (int64_t)it.slot0 * d), ntok * rowb);
    const uint32_t vo = 4u * h * rowb + 4u * r0;
#pragma unroll
    for (int mi = 0; mi < NMT; ++mi) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const uint32_t ml = mi * 32 + 8 * (v >> 2) + (v & 3);   // tile row minus 4h
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc.A0[mi][v]), ry, vo + ml * rowb, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc.A1[mi][v]), ry, vo + ml * rowb + 128, 0, 0);
        }
    }
}

template <int BITS>
__global__ __launch_bounds__(256, 3) void gemm_down_kernel(LayerArgs a, int nft) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_a0[2 * GEMM_BM * GROW];
    __shared__ __attribute__((aligned(16))) uint8_t lds_a1[2 * GEMM_BM * GROW];
    extern __shared__ uint2 lds_s[];   // [scale block of the f features][row]: -OFF * S as bf16 pieces
    int tile, ft;
    if (!pick_tile(nft, *a.n_items, tile, ft)) return;
    const WorkItem it = a.items[tile];
    switch ((it.ntok + 31) >> 5) {
        case 1: down_tile<BITS, 1>(a, it, ft, lds_a0, lds_a1, lds_s); break;
        case 2: down_tile<BITS, 2>(a, it, ft, lds_a0, lds_a1, lds_s); break;
        default: down_tile<BITS, GM_NM>(a, it, ft, lds_a0, lds_a1, lds_s); break;
    }
}

template <int BITS, int PASSES> hipError_t gemm_gateup_launch(const LayerArgs &a, int max_items, hipStream_t s) {
    const int nft = a.f / 128;
    const int64_t blocks = ((int64_t)nft * max_items + 7) / 8 * 8;
    if ((int64_t)PASSES * a.T * a.d * 2 > (int64_t)INT32_MAX) return hipErrorInvalidValue;   // 32-bit buffer offsets into xa
    STRATA_LAUNCH((gemm_gateup_kernel<BITS, PASSES>), dim3((unsigned)blocks), dim3(256), 0, s, a, nft);
    return hipGetLastError();
}

template <int BITS> hipError_t gemm_down_launch(const LayerArgs &a, int max_items, hipStream_t s) {
    const int nft = (a.d + 255) / 256;
    const int64_t blocks = ((int64_t)nft * max_items + 7) / 8 * 8;
    const size_t lds_s = sizeof(uint2) * GEMM_BM * (a.f / ((a.f & 255) ? 128 : 256));   // per scale block and row
    if (((int64_t)a.T * a.k + a.T) * a.f * 4 > (int64_t)INT32_MAX) return hipErrorInvalidValue;   // buffer offsets into ha
    STRATA_LAUNCH((gemm_down_kernel<BITS>), dim3((unsigned)blocks), dim3(256), lds_s, s, a, nft);
    return hipGetLastError();
}

}  // namespace strata
