// Public launchers of the expert GEMV kernels: dispatch on the code width
// to the instantiations in gemv_{gu,dn}{2,3}.hip.
#include "gemv_impl.hpp"

namespace strata {

extern template hipError_t gateup_small_launch<3>(const LayerArgs &, int, hipStream_t);
extern template hipError_t gateup_small_launch<2>(const LayerArgs &, int, hipStream_t);
extern template hipError_t gateup_multi_launch<3>(const LayerArgs &, int, int, hipStream_t);
extern template hipError_t gateup_multi_launch<2>(const LayerArgs &, int, int, hipStream_t);
extern template hipError_t down_multi_launch<3>(const LayerArgs &, int, hipStream_t);
extern template hipError_t down_multi_launch<2>(const LayerArgs &, int, hipStream_t);
extern template hipError_t down_one_launch<3>(const LayerArgs &, hipStream_t);
extern template hipError_t down_one_launch<2>(const LayerArgs &, hipStream_t);

bool gemv_supported(int d, int f, int bits) { return gemv_supported_impl(d, f, bits); }

// The one-token kernels (R columns of h per gate/up block, one wave per work
// item in the down kernel) fit; otherwise a single token takes the T >= 2 path.
bool gemv_one_token(int T, int E, int k, int d, int f) {
    if (T != 1 || k + 1 > 12) return false;
    const int Rd = 64 / unit_slices(f, 8), Rg = 64 / unit_slices(d, 8);
    return 4 * (size_t)down_one_lds_words(k, f, Rd) <= LDS_LIMIT &&
           4 * ((size_t)align4(gateup_lds_words(d, Rg, 1, 1)) + small_route_lds_words(E)) <= LDS_LIMIT;
}

// Compute units of the current device (cached per device).
static int device_cus() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cache[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

hipError_t launch_gemv_gateup_small(const LayerArgs &a, int max_items, hipStream_t s) {
    return a.bits == 3 ? gateup_small_launch<3>(a, max_items, s) : gateup_small_launch<2>(a, max_items, s);
}

hipError_t launch_gemv_gateup_multi(const LayerArgs &a, int max_items, hipStream_t s) {
    const int cus = device_cus();
    return a.bits == 3 ? gateup_multi_launch<3>(a, max_items, cus, s) : gateup_multi_launch<2>(a, max_items, cus, s);
}

hipError_t launch_gemv_down_multi(const LayerArgs &a, int max_items, hipStream_t s) {
    return a.bits == 3 ? down_multi_launch<3>(a, max_items, s) : down_multi_launch<2>(a, max_items, s);
}

hipError_t launch_gemv_down_one(const LayerArgs &a, hipStream_t s) {
    return a.bits == 3 ? down_one_launch<3>(a, s) : down_one_launch<2>(a, s);
}

}  // namespace strata
