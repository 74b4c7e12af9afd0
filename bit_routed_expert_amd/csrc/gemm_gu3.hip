// Instantiation of the 3-bit gate/up GEMM kernels.
#include "gemm_impl.hpp"

namespace strata {
template hipError_t gemm_gateup_launch<3, 1>(const LayerArgs &, int, hipStream_t);
template hipError_t gemm_gateup_launch<3, 2>(const LayerArgs &, int, hipStream_t);
}  // namespace strata
