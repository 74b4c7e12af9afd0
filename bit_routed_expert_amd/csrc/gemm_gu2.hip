// Instantiation of the 2-bit gate/up GEMM kernels.
#include "gemm_impl.hpp"

namespace strata {
template hipError_t gemm_gateup_launch<2, 1>(const LayerArgs &, int, hipStream_t);
template hipError_t gemm_gateup_launch<2, 2>(const LayerArgs &, int, hipStream_t);
}  // namespace strata
