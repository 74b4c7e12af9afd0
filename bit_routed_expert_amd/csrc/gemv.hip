// Public launchers of the expert GEMV kernels: dispatch on the code width
// to the instantiations in gemv_{gu,dn}{2,3}.hip.
#include "gemv_impl.hpp"

namespace strata {

extern template hipError_t gateup_small_launch<3>(const LayerArgs &, int, hipStream_t);
extern template hipError_t gateup_small_launch<2>(const LayerArgs &, int, hipStream_t);
extern template hipError_t down_launch<3>(const LayerArgs &, int, hipStream_t);
extern template hipError_t down_launch<2>(const LayerArgs &, int, hipStream_t);
extern template hipError_t down_rows_launch<3>(const LayerArgs &, hipStream_t);
extern template hipError_t down_rows_launch<2>(const LayerArgs &, hipStream_t);

bool gemv_supported(int d, int f, int bits) { return gemv_supported_impl(d, f, bits); }

bool down_rows_fits(int T, int k, int f) {
    const int R = 64 / unit_slices(f, 8);
    const int nt = nt_round(ntmax_for(T));
    if (T == 1) return k + 1 <= 12 && 4 * (size_t)down_one_lds_words(k, f, 64 / unit_slices(f, 8)) <= LDS_LIMIT;
    const int nw = down_rows_waves(T, k, f, R, nt);
    return T <= CHUNK_TOK && down_rows_lds(T, k, f, R, nt, nw) <= LDS_LIMIT;
}

hipError_t launch_gemv_gateup_small(const LayerArgs &a, int max_items, hipStream_t s) {
    return a.bits == 3 ? gateup_small_launch<3>(a, max_items, s) : gateup_small_launch<2>(a, max_items, s);
}

hipError_t launch_gemv_down(const LayerArgs &a, int max_items, hipStream_t s) {
    return a.bits == 3 ? down_launch<3>(a, max_items, s) : down_launch<2>(a, max_items, s);
}

hipError_t launch_gemv_down_rows(const LayerArgs &a, hipStream_t s) {
    return a.bits == 3 ? down_rows_launch<3>(a, s) : down_rows_launch<2>(a, s);
}

}  // namespace strata
