// Down expert kernels for 3-bit codes (one translation unit per
// kernel family and code width, so the instantiations compile in parallel).
#include "gemv_impl.hpp"

namespace strata {
template hipError_t down_multi_launch<3>(const LayerArgs &, int, hipStream_t);
template hipError_t down_one_launch<3>(const LayerArgs &, hipStream_t);
}  // namespace strata
