// Host-CPU consumer of the miss list: the experts a resident mask leaves out
// of the GPU forward are computed on the host's cores, from the packed
// weights the host holds, and added to the GPU's output.  The pages' engine
// splits each layer this way -- experts in the GPU's cache run there, the
// others on the CPU at the same time, and the two partial results are added
// (wiselychen.com, technique 2 "專家快取與 CPU／GPU 分工"; digiland.tw, "Strata
// 實測", item 2 "CPU 與 GPU 的協同運算（Co-processing）"; greenbean-ai, "Strata
// 如何讓 12GB 顯卡跑 Qwen3.8-Flash-Next？", section 二).
//
// This file holds the instruction-set choice, the thread pool and the C
// entry points; the arithmetic is in host_experts.cpp (one build per
// instruction set).  Nothing here touches the GPU; it is built by the host
// compiler for the baseline x86-64 instruction set.
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <thread>
#include <vector>

#include "strata_moe.h"
#include "host_experts.hpp"

namespace strata {

namespace {

enum class Isa { NONE, AVX2, AVX512 };

// The widest set this CPU runs; STRATA_HOST_ISA=avx2 in the environment
// picks AVX2 on an AVX-512 machine (read once per process).
Isa host_isa() {
    static const Isa isa = [] {
        __builtin_cpu_init();
        const bool avx2 = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma");
        const bool avx512 = avx2 && __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                            __builtin_cpu_supports("avx512dq") && __builtin_cpu_supports("avx512vl");
        const char *want = getenv("STRATA_HOST_ISA");
        if (avx512 && !(want && strcmp(want, "avx2") == 0)) return Isa::AVX512;
        return avx2 ? Isa::AVX2 : Isa::NONE;
    }();
    return isa;
}

template <typename F> void parallel_tasks(int n_tasks, int n_threads, F &&fn) {
    std::atomic<int> next{0};
    auto worker = [&]() {
        for (int t = next.fetch_add(1); t < n_tasks; t = next.fetch_add(1)) fn(t);
    };
    const int nt = n_tasks < n_threads ? n_tasks : n_threads;
    std::vector<std::thread> pool;
    for (int i = 1; i < nt; ++i) pool.emplace_back(worker);
    worker();
    for (auto &th : pool) th.join();
}

}  // namespace

bool host_supported(const strata_moe_shape &s) {
    return host_isa() != Isa::NONE && s.d_model <= HOST_MAX_D && s.d_ff <= HOST_MAX_F && s.d_model % 64 == 0 &&
           s.d_ff % 64 == 0;
}

// y_add = sum over the misses of gate * FFN_e(u_t), every row of y_add
// written (rows of tokens without misses are zero).  a.gstart, a.order and
// a.experts are filled here.
void run_host_misses(HostMissArgs &a) {
    const int E = a.E, n = a.n_miss;
    for (int e = 0; e <= E; ++e) a.gstart[e] = 0;
    for (int m = 0; m < n; ++m) a.gstart[a.miss_te[2 * m + 1] + 1]++;
    for (int e = 0; e < E; ++e) a.gstart[e + 1] += a.gstart[e];
    int ne = 0;
    for (int e = 0; e < E; ++e)
        if (a.gstart[e + 1] > a.gstart[e]) a.experts[ne++] = e;
    {   // stable grouping: misses of each expert in list order
        std::vector<int32_t> fill(a.gstart, a.gstart + E);
        for (int m = 0; m < n; ++m) a.order[fill[a.miss_te[2 * m + 1]]++] = m;
    }
    const bool wide = host_isa() == Isa::AVX512;
    const int ja = (a.f + HOST_RB_A - 1) / HOST_RB_A;
    parallel_tasks(ne * ja, a.n_threads, [&](int task) {
        const int e = a.experts[task / ja], j0 = (task % ja) * HOST_RB_A;
        const int j1 = j0 + HOST_RB_A < a.f ? j0 + HOST_RB_A : a.f;
        if (wide) hx512::gateup_rows(a, e, j0, j1);
        else hx256::gateup_rows(a, e, j0, j1);
    });
    const int ib = (a.d + HOST_RB_B - 1) / HOST_RB_B;
    parallel_tasks(ib, a.n_threads, [&](int task) {
        const int i0 = task * HOST_RB_B, i1 = i0 + HOST_RB_B < a.d ? i0 + HOST_RB_B : a.d;
        if (wide) hx512::down_cols(a, a.experts, ne, i0, i1);
        else hx256::down_cols(a, a.experts, ne, i0, i1);
    });
}

}  // namespace strata

using namespace strata;

extern "C" {

size_t strata_moe_host_workspace_bytes(const strata_moe_shape *shape, int32_t T, int32_t miss_cap) {
    if (check_shape(shape) != STRATA_OK || T < 0 || miss_cap < 0 || !host_supported(*shape)) return 0;
    return host_layout(shape->n_experts, shape->d_model, shape->d_ff, T, miss_cap).total;
}

const char *strata_moe_host_isa(void) {
    switch (host_isa()) {
        case Isa::AVX512: return "avx512";
        case Isa::AVX2: return "avx2";
        default: return "none";
    }
}

strata_status strata_moe_host_misses(const strata_moe_shape *shape, const strata_moe_host_layer *layer,
                                     const float *u, int32_t T, const int32_t *miss_te, const float *miss_w,
                                     int32_t n_miss, float *y_add, void *host_ws, size_t host_ws_bytes,
                                     int32_t n_threads) {
    strata_status st = check_shape(shape);
    if (st != STRATA_OK) return st;
    if (!layer || T < 0 || n_miss < 0 || n_threads < 1) return STRATA_EINVAL;
    const int bits = layer->bits ? layer->bits : shape->bits;
    if (bits != 3 && bits != 2) return STRATA_EUNSUPPORTED;
    if (!host_supported(*shape)) return STRATA_EUNSUPPORTED;
    if (T == 0) return STRATA_OK;
    if (!layer->codes || !layer->scales || !u || !y_add || !host_ws || (n_miss > 0 && (!miss_te || !miss_w)))
        return STRATA_EINVAL;
    const HostLayout hl = host_layout(shape->n_experts, shape->d_model, shape->d_ff, T, n_miss);
    if (host_ws_bytes < hl.total) return STRATA_EWORKSPACE;
    for (int m = 0; m < n_miss; ++m)
        if (miss_te[2 * m] < 0 || miss_te[2 * m] >= T || miss_te[2 * m + 1] < 0 ||
            miss_te[2 * m + 1] >= shape->n_experts)
            return STRATA_EINVAL;
    char *w = (char *)host_ws;
    HostMissArgs a{};
    a.E = shape->n_experts;
    a.d = shape->d_model;
    a.f = shape->d_ff;
    a.bits = bits;
    a.T = T;
    a.n_miss = n_miss;
    a.n_threads = n_threads;
    a.codes = layer->codes;
    a.scales = layer->scales;
    a.u = u;
    a.miss_te = miss_te;
    a.miss_w = miss_w;
    a.h = (float *)(w + hl.h);
    a.gstart = (int32_t *)(w + hl.gstart);
    a.order = (int32_t *)(w + hl.order);
    a.experts = (int32_t *)(w + hl.experts);
    a.y_add = y_add;
    run_host_misses(a);
    return STRATA_OK;
}

}  // extern "C"
