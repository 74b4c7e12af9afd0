// Internal interface of the host-CPU expert evaluation (host_experts.cpp,
// built once per instruction set; the C ABI picks one at run time).
#pragma once
#include <stddef.h>
#include <stdint.h>

struct HostMissArgs {
    int E, d, f, bits, T, n_miss, n_threads;
    const uint8_t *codes;      // (E+1) experts, packed as on the device
    const uint16_t *scales;    // fp16 block scales, same order
    const float *u;            // [T][d] layer input
    const int32_t *miss_te;    // [n_miss][2] (token, expert)
    const float *miss_w;       // [n_miss] gates
    float *h;                  // [n_miss][f] scratch: SwiGLU activations
    int32_t *gstart;           // [E+1] scratch: first miss of each expert in `order`
    int32_t *order;            // [n_miss] scratch: misses grouped by expert
    int32_t *experts;          // [E] scratch: experts with misses, ascending
    float *y_add;              // [T][d] result: sum of gate * FFN_e(u_t) over each token's misses
};

constexpr int HOST_MAX_D = 8192;   // longest row the tasks decode (d of gate/up)
constexpr int HOST_MAX_F = 4096;   // (f of down)
constexpr int HOST_RB_A = 32;      // rows of h per phase-A task
constexpr int HOST_RB_B = 32;      // output columns per phase-B task

namespace hx512 {
void gateup_rows(const HostMissArgs &a, int e, int j0, int j1);
void down_cols(const HostMissArgs &a, const int32_t *experts, int ne, int i0, int i1);
}
namespace hx256 {
void gateup_rows(const HostMissArgs &a, int e, int j0, int j1);
void down_cols(const HostMissArgs &a, const int32_t *experts, int ne, int i0, int i1);
}

// Host workspace layout (bytes, 64-byte aligned parts) for T tokens and
// up to cap misses: u, h, order, gstart, then the staging of the
// co-processing forward (raw layer input, miss list and count, y_add).
struct HostLayout {
    size_t u, h, order, gstart, experts, xstage, mte, mw, mcount, yadd, total;
};
inline HostLayout host_layout(int E, int d, int f, int64_t T, int64_t cap) {
    HostLayout l{};
    size_t o = 0;
    auto take = [&](size_t b) { size_t at = o; o += (b + 63) / 64 * 64; return at; };
    l.u = take(4 * (size_t)T * d);
    l.h = take(4 * (size_t)cap * f);
    l.order = take(4 * (size_t)cap);
    l.gstart = take(4 * (size_t)(E + 1));
    l.experts = take(4 * (size_t)E);
    l.xstage = take(4 * (size_t)T * d);
    l.mte = take(8 * (size_t)cap);
    l.mw = take(4 * (size_t)cap);
    l.mcount = take(4);
    l.yadd = take(4 * (size_t)T * d);
    l.total = o;
    return l;
}

#include "strata_moe.h"
namespace strata {
// Both phases over n_threads host threads; fills a.gstart, a.order, a.experts.
void run_host_misses(HostMissArgs &a);
strata_status check_shape(const strata_moe_shape *s);   // the C ABI's shape validation
bool host_supported(const strata_moe_shape &s);          // the host consumer handles this shape here
}
