// Expert FFN for small token counts per expert (decode and MTP verify):
// stream the packed 3-/2-bit codes of each needed expert from HBM once and
// reduce them against up to 8 tokens held in LDS.
//
// The pages' engine computes the cached experts' FFNs on the GPU (wiselychen.com,
// technique 2 "專家快取與 CPU／GPU 分工"; greenbean-ai section 二).  Here every
// expert is resident and the kernel is bound by HBM: 3.0625 bit per weight
// leaves under two VALU operations per weight at full bandwidth, so the inner
// product avoids per-weight float work:
//   * a 32-code unit unpacks into four words of 4-bit lanes with 3 ANDs and
//     one 6-op gather (codes 0..7 are valid signed 4-bit values);
//   * the activation is held as fixed point X = rint(v * 2^E) per 256-column
//     group, split into P balanced base-16 digit planes (digits in [-8, 7]);
//   * v_dot8_i32_i4 multiplies 8 codes by 8 digits with exact int32 sums, so
//     a block's sum(c * X) is exact and the code offset is the exact
//     correction sum((c - c0) X) = sum(c X) - c0 * sum(X);
//   * the fp16 block scale and 2^-E are applied once per (row, block, token).
// Lane mapping: a wave covers R rows x S = 64/R column slices; lane
// (row r, slice s) reads its row's 4 units (48 or 32 bytes) of each
// 128-column group in its slice with 16-byte loads and keeps per-token
// partial sums; the S slices are summed with two cross-lane adds.
#include "common.hpp"

namespace strata {

constexpr int MAXQ = 4;  // 128-column groups per lane slice

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

// sum_p 16^p acc[p] as a float (exact in int32 for P <= 4).
template <int P> __device__ __forceinline__ float digits_value(const int *acc, int C2, int sx) {
    if constexpr (P <= 4) {
        int I = 0;
#pragma unroll
        for (int p = P - 1; p >= 0; --p) I = (I << 4) + acc[p];
        return (float)(2 * I - C2 * sx);
    } else {
        int lo = 0, hi = 0;
#pragma unroll
        for (int p = 2; p >= 0; --p) lo = (lo << 4) + acc[p];
#pragma unroll
        for (int p = P - 1; p >= 3; --p) hi = (hi << 4) + acc[p];
        float I = fmaf((float)hi, 4096.f, (float)lo);
        return 2.f * I - (float)C2 * (float)sx;
    }
}

// LDS word offset of unit U's digit planes (P planes x 4 words), with 4 words
// of padding after each lane slice so the S slices read different banks.
__device__ __forceinline__ int dig_off(int U, int P, int units_per_slice) {
    return U * P * 4 + (U / units_per_slice) * 4;
}

// Rows [row0, row0+R) of one packed matrix [out][in] against NT tokens.
// Loads are issued first (so callers can stage LDS while they fly); the
// compute reads digit planes, per-(token,128-group) digit sums and
// per-(token,256-group) scales from LDS.  res[t] is valid in lanes with s == 0.
template <int BITS, int NT, int P> struct RowTile {
    uint32_t w[MAXQ][Fmt<BITS>::DW];
    int R, S, Q, QPS, r, s, in;
    const uint16_t *msc;

    __device__ __forceinline__ void load(const uint8_t *__restrict__ mat, const uint16_t *__restrict__ msc_,
                                         int in_, int row0, int R_) {
        const int lane = threadIdx.x & 63;
        R = R_;
        S = 64 / R;
        in = in_;
        Q = in / 128;
        QPS = Q / S;
        r = row0 + lane % R;
        s = lane / R;
        msc = msc_;
        constexpr int UB = Fmt<BITS>::UB;
        const uint8_t *base = mat + ((size_t)((r / 16) * Q + s * QPS) * 16 + (r % 16)) * 4 * UB;
#pragma unroll
        for (int qq = 0; qq < MAXQ; ++qq) {
            if (qq < QPS) {
                const uint4 *p = (const uint4 *)(base + (size_t)qq * 16 * 4 * UB);
#pragma unroll
                for (int i = 0; i < Fmt<BITS>::DW / 4; ++i) {
                    uint4 v = p[i];
                    w[qq][4 * i] = v.x;
                    w[qq][4 * i + 1] = v.y;
                    w[qq][4 * i + 2] = v.z;
                    w[qq][4 * i + 3] = v.w;
                }
            }
        }
    }

    __device__ __forceinline__ void compute(const uint32_t *__restrict__ dig, int dig_stride,
                                            const int *__restrict__ xsum, int sum_stride,
                                            const float *__restrict__ xscl, int scl_stride, float res[NT]) {
        int acc[NT][P];
        int sx[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            res[t] = 0.f;
            sx[t] = 0;
#pragma unroll
            for (int p = 0; p < P; ++p) acc[t][p] = 0;
        }
        const int ups = QPS * 4;
#pragma unroll
        for (int qq = 0; qq < MAXQ; ++qq) {
            if (qq < QPS) {
                const int q = s * QPS + qq;
#pragma unroll
                for (int uu = 0; uu < 4; ++uu) {
                    uint32_t N[4];
                    unit_nibbles<BITS>(&w[qq][uu * Fmt<BITS>::UB / 4], N);
                    const int off = dig_off(q * 4 + uu, P, ups);
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const uint4 *dp = (const uint4 *)(dig + t * dig_stride + off);
#pragma unroll
                        for (int p = 0; p < P; ++p) {
                            uint4 dv = dp[p];
                            int a_ = acc[t][p];
                            a_ = __builtin_amdgcn_sdot8((int)N[0], (int)dv.x, a_, false);
                            a_ = __builtin_amdgcn_sdot8((int)N[1], (int)dv.y, a_, false);
                            a_ = __builtin_amdgcn_sdot8((int)N[2], (int)dv.z, a_, false);
                            a_ = __builtin_amdgcn_sdot8((int)N[3], (int)dv.w, a_, false);
                            acc[t][p] = a_;
                        }
                    }
                }
#pragma unroll
                for (int t = 0; t < NT; ++t) sx[t] += xsum[t * sum_stride + q];
                // flush at the end of a (weight block, input group) run
                const long n0 = (long)r * in + q * 128;
                const bool last = (qq == QPS - 1);
                const bool newblk = ((n0 + 128) / 256 != n0 / 256) || ((q + 1) / 2 != q / 2);
                if (last || newblk) {
                    const float sc = 0.5f * half_to_float(msc[n0 / 256]);
                    const int g = q / 2;
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        float v = digits_value<P>(acc[t], Fmt<BITS>::C2, sx[t]);
                        res[t] = fmaf(v, sc * xscl[t * scl_stride + g], res[t]);
                        sx[t] = 0;
#pragma unroll
                        for (int p = 0; p < P; ++p) acc[t][p] = 0;
                    }
                }
            }
        }
        // sum the S column slices of each row
        for (int o = R; o < 64; o <<= 1) {
#pragma unroll
            for (int t = 0; t < NT; ++t) res[t] += __shfl_xor(res[t], o, WAVE);
        }
    }
};

__device__ __forceinline__ int slot_token(const LayerArgs &a, const WorkItem &it, int j) {
    int slot = it.slot0 + j;
    return it.expert == a.E ? slot - a.T * a.k : a.perm[slot] / a.k;
}

// ---------------------------------------------------------- gate and up
// Block = 4 waves = 4 row tiles of R rows; tiles [0, f/R) are gate rows,
// [f/R, 2f/R) up rows.  Outputs G/U[slot][row] (fp32).
template <int BITS, int NT>
__device__ __forceinline__ void gateup_body(const LayerArgs &a, const WorkItem &it, int R, int wg_per_item,
                                            uint32_t *lds) {
    const int th = threadIdx.x, wave = th >> 6, lane = th & 63;
    const int d = a.d, f = a.f;
    const int tiles_m = f / R;
    const int tile = (blockIdx.x % wg_per_item) * 4 + wave;
    const int m = tile < tiles_m ? 0 : 1;
    const int row0 = (tile % tiles_m) * R;
    const size_t mat_bytes = (size_t)d * f * BITS / 8;
    const size_t mat_blocks = (size_t)d * f / 256;
    const size_t mi = (size_t)it.expert * 3 + m;
    RowTile<BITS, NT, XPLANES> rt;
    rt.load(a.codes + mi * mat_bytes, a.scales + mi * mat_blocks, d, row0, R);

    // stage the tokens' digit planes, digit sums and group scales
    const int Q = d / 128, G = (d + 255) / 256, units = d / 32;
    const int S = 64 / R, ups = (Q / S) * 4;
    const int dig_stride = units * XPLANES * 4 + S * 4;
    uint32_t *ldig = lds;
    int *lsum = (int *)(lds + NT * dig_stride);
    float *lscl = (float *)(lsum + NT * Q);
    for (int j = 0; j < NT; ++j) {
        const int t = slot_token(a, it, j);
        const uint4 *src = (const uint4 *)(a.xq + (size_t)t * units * XPLANES * 4);
        for (int i = th; i < units * XPLANES; i += 256) {
            int U = i / XPLANES, p = i % XPLANES;
            *(uint4 *)(ldig + j * dig_stride + dig_off(U, XPLANES, ups) + 4 * p) = src[i];
        }
        for (int i = th; i < Q; i += 256) lsum[j * Q + i] = a.xsum[(size_t)t * Q + i];
        for (int i = th; i < G; i += 256) lscl[j * G + i] = a.xscl[(size_t)t * G + i];
    }
    __syncthreads();
    float res[NT];
    rt.compute(ldig, dig_stride, lsum, Q, lscl, G, res);
    if (lane < R) {
        float *dst = (m == 0 ? a.G : a.U) + (size_t)it.slot0 * f + row0 + lane;
#pragma unroll
        for (int j = 0; j < NT; ++j) dst[(size_t)j * f] = res[j];
    }
}

template <int BITS, int NTMAX>
__global__ __launch_bounds__(256) void gemv_gateup_kernel(LayerArgs a, int R) {
    extern __shared__ uint32_t lds[];
    const int wg_per_item = (2 * a.f / R) / 4;
    const int item = blockIdx.x / wg_per_item;
    if (item >= *a.n_items) return;
    const WorkItem it = a.items[item];
    switch (it.ntok) {
#define GU_CASE(n) \
    case n:        \
        if constexpr (n <= NTMAX) gateup_body<BITS, n>(a, it, R, wg_per_item, lds); \
        break;
        GU_CASE(1) GU_CASE(2) GU_CASE(3) GU_CASE(4) GU_CASE(5) GU_CASE(6) GU_CASE(7) GU_CASE(8)
#undef GU_CASE
        default: break;
    }
}

// ----------------------------------------------------------------- down
// Block = 2 waves = 2 row tiles of R rows of Wd [d][f].  Each block first
// forms h = silu(g) * u of its tokens and its 6-plane digits (24-bit fixed
// point per 256-column group), then reduces.  Outputs Y[slot][row] (fp32).
template <int BITS, int NT>
__device__ __forceinline__ void down_body(const LayerArgs &a, const WorkItem &it, int R, int wg_per_item,
                                          uint32_t *lds) {
    const int th = threadIdx.x, wave = th >> 6, lane = th & 63, nth = blockDim.x;
    const int d = a.d, f = a.f;
    const int row0 = ((blockIdx.x % wg_per_item) * 2 + wave) * R;
    const size_t mat_bytes = (size_t)d * f * BITS / 8;
    const size_t mat_blocks = (size_t)d * f / 256;
    const size_t mi = (size_t)it.expert * 3 + 2;
    RowTile<BITS, NT, HPLANES> rt;
    rt.load(a.codes + mi * mat_bytes, a.scales + mi * mat_blocks, f, row0, R);

    const int Q = f / 128, G = (f + 255) / 256, units = f / 32;
    const int S = 64 / R, ups = (Q / S) * 4;
    const int dig_stride = units * HPLANES * 4 + S * 4;
    uint32_t *ldig = lds;
    int *lsum = (int *)(lds + NT * dig_stride);
    float *lscl = (float *)(lsum + NT * Q);
    const int nchunk = f / 8;
    for (int j = 0; j < NT; ++j) {
        const float *g = a.G + (size_t)(it.slot0 + j) * f;
        const float *u = a.U + (size_t)(it.slot0 + j) * f;
        for (int base = 0; base < nchunk; base += nth) {
            const int c = base + th;
            const bool valid = c < nchunk;
            float h[8];
            float mx = 0.f;
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                float hv = 0.f;
                if (valid) {
                    float gv = g[c * 8 + n], uv = u[c * 8 + n];
                    hv = gv / (1.f + expf(-gv)) * uv;
                }
                h[n] = hv;
                mx = fmaxf(mx, fabsf(hv));
            }
#pragma unroll
            for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, WAVE));
            const int E = fixed_point_exponent<HPLANES>(mx);
            uint32_t word[HPLANES];
#pragma unroll
            for (int p = 0; p < HPLANES; ++p) word[p] = 0;
            int sx = 0;
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                int X = (int)rintf(ldexpf(h[n], E));
                sx += X;
                int dg[HPLANES];
                to_digits<HPLANES>(X, dg);
#pragma unroll
                for (int p = 0; p < HPLANES; ++p) word[p] |= ((uint32_t)dg[p] & 15u) << (4 * n);
            }
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) sx += __shfl_xor(sx, o, WAVE);
            if (valid) {
                const int U = c / 4, i = c % 4;
                uint32_t *dst = ldig + j * dig_stride + dig_off(U, HPLANES, ups);
#pragma unroll
                for (int p = 0; p < HPLANES; ++p) dst[p * 4 + i] = word[p];
                if ((c & 15) == 0) lsum[j * Q + c / 16] = sx;
                if ((c & 31) == 0) lscl[j * G + c / 32] = ldexpf(1.f, -E);
            }
        }
    }
    __syncthreads();
    float res[NT];
    rt.compute(ldig, dig_stride, lsum, Q, lscl, G, res);
    if (lane < R) {
        float *dst = a.Y + (size_t)it.slot0 * d + row0 + lane;
#pragma unroll
        for (int j = 0; j < NT; ++j) dst[(size_t)j * d] = res[j];
    }
}

template <int BITS, int NTMAX>
__global__ __launch_bounds__(128) void gemv_down_kernel(LayerArgs a, int R) {
    extern __shared__ uint32_t lds[];
    const int wg_per_item = a.d / (2 * R);
    const int item = blockIdx.x / wg_per_item;
    if (item >= *a.n_items) return;
    const WorkItem it = a.items[item];
    switch (it.ntok) {
#define DN_CASE(n) \
    case n:        \
        if constexpr (n <= NTMAX) down_body<BITS, n>(a, it, R, wg_per_item, lds); \
        break;
        DN_CASE(1) DN_CASE(2) DN_CASE(3) DN_CASE(4) DN_CASE(5) DN_CASE(6) DN_CASE(7) DN_CASE(8)
#undef DN_CASE
        default: break;
    }
}

// ------------------------------------------------------------- launchers
// Column slices per wave for an input width `in`: the most slices (up to 4)
// that split the 128-column groups evenly with at most MAXQ per slice.
static int pick_slices(int in) {
    const int Q = in / 128;
    for (int S = 4; S >= 1; S >>= 1)
        if (Q % S == 0 && Q / S <= MAXQ) return S;
    return 0;
}

bool gemv_supported(int d, int f, int bits) {
    if (bits != 3 && bits != 2) return false;
    if (d % 128 || f % 128) return false;
    int Sg = pick_slices(d), Sd = pick_slices(f);
    if (!Sg || !Sd) return false;
    int Rg = 64 / Sg, Rd = 64 / Sd;
    if ((2 * f / Rg) % 4 || f % Rg) return false;
    if (d % (2 * Rd)) return false;
    if (f / 8 > 4096 || d > 8192) return false;
    return true;
}

template <int BITS>
static hipError_t gateup_dispatch(const LayerArgs &a, int ntmax, int grid, int R, size_t lds, hipStream_t s) {
    switch (ntmax) {
        case 1: hipLaunchKernelGGL((gemv_gateup_kernel<BITS, 1>), dim3(grid), dim3(256), lds, s, a, R); break;
        case 2: hipLaunchKernelGGL((gemv_gateup_kernel<BITS, 2>), dim3(grid), dim3(256), lds, s, a, R); break;
        case 3:
        case 4: hipLaunchKernelGGL((gemv_gateup_kernel<BITS, 4>), dim3(grid), dim3(256), lds, s, a, R); break;
        default: hipLaunchKernelGGL((gemv_gateup_kernel<BITS, 8>), dim3(grid), dim3(256), lds, s, a, R); break;
    }
    return hipGetLastError();
}

template <int BITS>
static hipError_t down_dispatch(const LayerArgs &a, int ntmax, int grid, int R, size_t lds, hipStream_t s) {
    switch (ntmax) {
        case 1: hipLaunchKernelGGL((gemv_down_kernel<BITS, 1>), dim3(grid), dim3(128), lds, s, a, R); break;
        case 2: hipLaunchKernelGGL((gemv_down_kernel<BITS, 2>), dim3(grid), dim3(128), lds, s, a, R); break;
        case 3:
        case 4: hipLaunchKernelGGL((gemv_down_kernel<BITS, 4>), dim3(grid), dim3(128), lds, s, a, R); break;
        default: hipLaunchKernelGGL((gemv_down_kernel<BITS, 8>), dim3(grid), dim3(128), lds, s, a, R); break;
    }
    return hipGetLastError();
}

static int ntmax_for(int T) { return T >= CHUNK_TOK ? CHUNK_TOK : T; }

hipError_t launch_gemv_gateup(const LayerArgs &a, int max_items, hipStream_t s) {
    const int R = 64 / pick_slices(a.d);
    const int wg_per_item = (2 * a.f / R) / 4;
    const int ntmax = ntmax_for(a.T);
    const int S = 64 / R;
    const size_t dig_stride = (size_t)(a.d / 32) * XPLANES * 4 + S * 4;
    const int nt = ntmax <= 2 ? ntmax : (ntmax <= 4 ? 4 : 8);
    const size_t lds = 4 * (nt * dig_stride + nt * (a.d / 128) + nt * ((a.d + 255) / 256));
    const int grid = max_items * wg_per_item;
    return a.bits == 3 ? gateup_dispatch<3>(a, ntmax, grid, R, lds, s) : gateup_dispatch<2>(a, ntmax, grid, R, lds, s);
}

hipError_t launch_gemv_down(const LayerArgs &a, int max_items, hipStream_t s) {
    const int R = 64 / pick_slices(a.f);
    const int wg_per_item = a.d / (2 * R);
    const int ntmax = ntmax_for(a.T);
    const int S = 64 / R;
    const size_t dig_stride = (size_t)(a.f / 32) * HPLANES * 4 + S * 4;
    const int nt = ntmax <= 2 ? ntmax : (ntmax <= 4 ? 4 : 8);
    const size_t lds = 4 * (nt * dig_stride + nt * (a.f / 128) + nt * ((a.f + 255) / 256));
    const int grid = max_items * wg_per_item;
    return a.bits == 3 ? down_dispatch<3>(a, ntmax, grid, R, lds, s) : down_dispatch<2>(a, ntmax, grid, R, lds, s);
}

}  // namespace strata
