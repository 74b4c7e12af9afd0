// Matrix-core helpers shared by the GEMM and router kernels (gfx950).
#pragma once
#include "common.hpp"

namespace strata {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// D[32x32] += A[32x16] B[16x32]; lane l supplies A row l%32 and B column
// l%32, K elements 8*(l/32) .. +8; it holds D rows 8*(v/4) + 4*(l/32) + v%4
// of column l%32 in element v.
__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp32 -> bf16, round to nearest even (the hardware conversion, v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f2bf(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

// Sum of v over the 32 lanes of each half-wave (lanes 0-31 and 32-63) by DPP:
// row sums by quad permutes and row rotations, then row 0's sum broadcast
// into row 1 and row 2's into row 3; complete in lanes 16-31 and 48-63.
__device__ __forceinline__ float half_wave_sum(float v) {
#define HW_DPP(CTRL, ROWS) __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false))
    v += HW_DPP(0xB1, 0xF);    // quad_perm [1,0,3,2]
    v += HW_DPP(0x4E, 0xF);    // quad_perm [2,3,0,1]
    v += HW_DPP(0x124, 0xF);   // row_ror:4
    v += HW_DPP(0x128, 0xF);   // row_ror:8
    v += HW_DPP(0x142, 0xA);   // row_bcast:15 into rows 1 and 3
#undef HW_DPP
    return v;
}

// v = hi + mid + lo exactly (three bf16 pieces carry fp32's 24 bits).
__device__ __forceinline__ void split3(float v, uint16_t &hi, uint16_t &mid, uint16_t &lo) {
    hi = f2bf(v);
    const float r1 = v - bf16_to_float(hi);
    mid = f2bf(r1);
    lo = f2bf(r1 - bf16_to_float(mid));
}

}  // namespace strata
