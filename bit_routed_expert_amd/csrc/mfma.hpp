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

__device__ __forceinline__ uint16_t f2bf(float v) {   // round to nearest even (finite inputs)
    const uint32_t u = __float_as_uint(v);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// v = hi + mid + lo exactly (three bf16 pieces carry fp32's 24 bits).
__device__ __forceinline__ void split3(float v, uint16_t &hi, uint16_t &mid, uint16_t &lo) {
    hi = f2bf(v);
    const float r1 = v - bf16_to_float(hi);
    mid = f2bf(r1);
    lo = f2bf(r1 - bf16_to_float(mid));
}

}  // namespace strata
