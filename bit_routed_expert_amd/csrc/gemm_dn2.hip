// Instantiation of the 2-bit down GEMM kernel.
#include "gemm_impl.hpp"

namespace strata {
template hipError_t gemm_down_launch<2>(const LayerArgs &, int, hipStream_t);
}  // namespace strata
