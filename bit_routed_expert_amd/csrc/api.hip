// C ABI of the MoE layer library: host-side validation, workspace carving,
// kernel selection by token count, the per-layer loop and stream ordering.
// Nothing here allocates device memory or synchronises the stream.
#include <string.h>

#include "strata_moe.h"
#include "common.hpp"

using namespace strata;

namespace {

thread_local hipError_t g_last_hip = hipSuccess;

}  // namespace

namespace strata {
thread_local LaunchEvents g_launch_events;
}  // namespace strata

namespace {

constexpr size_t ALIGN = 256;
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
size_t up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

// Token counts up to this take the decode path (one work item per expert).
constexpr int SMALL_T = 8;

struct Layout {
    size_t counter, z, idx, gate, counts, offsets, perm, pos, inv_rms, items, n_items, xq, xsum, xscl, hf,
        xa, sx, ha, hs, bcnt, bmiss, Y, out, xres0, xres1, miss_count, total;
    int64_t max_items;
};

bool small_path(const strata_moe_shape &s, int64_t T) {
    return T <= SMALL_T && (size_t)T * s.d_model * sizeof(float) <= 64 * 1024;
}

// Work items: an expert's slots in pairs (decode path: at most one per
// pick, plus the shared expert's), else tiles of up to GEMM_BM tokens per
// resident expert with picks plus the shared expert's.
int64_t max_items_for(const strata_moe_shape &s, int64_t T) {
    if (small_path(s, T)) return T * s.top_k + (T + ITEM_TOK - 1) / ITEM_TOK;
    return (T * s.top_k + GEMM_BM - 1) / GEMM_BM + s.n_experts + (T + GEMM_BM - 1) / GEMM_BM + 2;
}

Layout layout(const strata_moe_shape &s, int64_t T) {
    Layout l{};
    const int64_t E = s.n_experts, k = s.top_k, d = s.d_model, f = s.d_ff;
    const int64_t slots = T * k + T;
    const bool sp = small_path(s, T);
    const int64_t Tq = sp ? T : 0, Sq = sp ? slots : 0;   // digit planes: decode path only
    const int64_t Tg = sp ? 0 : T, Sg = sp ? 0 : slots;   // bf16 operands: GEMM path only
    l.max_items = max_items_for(s, T);
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o += up(bytes); return at; };
    l.counter = take(ALIGN);
    l.z = take(sizeof(float) * T * E * (sp ? 1 : route_logit_splits((int)d)));
    l.idx = take(4 * T * k);
    l.gate = take(4 * T * k);
    l.counts = take(4 * E);
    l.offsets = take(4 * (E + 1));
    l.perm = take(4 * T * k);
    l.pos = take(4 * T * k);
    l.inv_rms = take(4 * T);
    l.items = take(sizeof(WorkItem) * l.max_items);
    l.n_items = take(4);
    l.xq = take((size_t)Tq * (d / 32) * XPLANES * 16);
    l.xsum = take(4 * Tq * (d / 32));
    l.xscl = take(4 * Tq * ((d + 255) / 256));
    l.hf = take(4 * Sq * f);
    l.xa = take((size_t)2 * Tg * d * 2);
    l.sx = take(4 * Tg * (d / 128));
    l.ha = take((size_t)2 * Sg * f * 2);
    l.hs = take(4 * Sg * (f / 32));
    const int64_t nb = sp ? 0 : route_perm_blocks((int)T);
    l.bcnt = take(4 * nb * E);
    l.bmiss = take(4 * nb);
    l.Y = take(sizeof(float) * slots * d);
    l.out = take(sizeof(float) * T * d);
    l.xres0 = take(sizeof(float) * T * d);
    l.xres1 = take(sizeof(float) * T * d);
    l.miss_count = take(4);
    l.total = o;
    return l;
}

strata_status check_shape(const strata_moe_shape *s) {
    if (!s) return STRATA_EINVAL;
    if (s->n_shared != 1 || s->top_k < 1 || s->top_k > 32 || s->n_experts < s->top_k || s->n_experts > 1024)
        return STRATA_EINVAL;
    if (s->d_model <= 0 || s->d_ff <= 0 || s->d_model % 128 || s->d_ff % 128) return STRATA_EINVAL;
    if (s->bits != 3 && s->bits != 2) return STRATA_EUNSUPPORTED;
    if (!gemv_supported(s->d_model, s->d_ff, s->bits)) return STRATA_EUNSUPPORTED;
    if (!gemm_supported(s->d_model, s->d_ff)) return STRATA_EUNSUPPORTED;
    return STRATA_OK;
}

void fill_common(LayerArgs &a, const strata_moe_shape &s, const Layout &l, char *ws, int T) {
    memset(&a, 0, sizeof(a));
    a.E = s.n_experts;
    a.k = s.top_k;
    a.d = s.d_model;
    a.f = s.d_ff;
    a.bits = s.bits;
    a.T = T;
    a.z = (float *)(ws + l.z);
    a.zsplit = small_path(s, T) ? 1 : route_logit_splits(s.d_model);
    a.idx = (int32_t *)(ws + l.idx);
    a.gate = (float *)(ws + l.gate);
    a.counts = (int32_t *)(ws + l.counts);
    a.offsets = (int32_t *)(ws + l.offsets);
    a.perm = (int32_t *)(ws + l.perm);
    a.pos = (int32_t *)(ws + l.pos);
    a.inv_rms = (float *)(ws + l.inv_rms);
    a.items = (WorkItem *)(ws + l.items);
    a.n_items = (int32_t *)(ws + l.n_items);
    a.counter = (uint32_t *)(ws + l.counter);
    a.xq = (uint32_t *)(ws + l.xq);
    a.xsum = (int32_t *)(ws + l.xsum);
    a.xscl = (float *)(ws + l.xscl);
    a.hf = (float *)(ws + l.hf);
    a.Y = (float *)(ws + l.Y);
    a.xa = (uint16_t *)(ws + l.xa);
    a.sx = (float *)(ws + l.sx);
    a.ha = (uint16_t *)(ws + l.ha);
    a.hs = (float *)(ws + l.hs);
    a.bcnt = (int32_t *)(ws + l.bcnt);
    a.bmiss = (int32_t *)(ws + l.bmiss);
}

void set_route_out(LayerArgs &a, const strata_route_out *r) {
    if (!r) return;
    a.u_idx = r->topk_idx;
    a.u_gate = r->topk_w;
    a.u_counts = r->counts;
    a.u_offsets = r->offsets;
    a.u_perm = r->perm;
    a.u_pos = r->pos;
}

// Caller events around each kernel group, attached to its launches.
struct Recorder {
    void *const *events;
    int n, i;
    hipStream_t s;
    void before() {
        if (events && i < n) g_launch_events = LaunchEvents{(hipEvent_t)events[2 * i], (hipEvent_t)events[2 * i + 1]};
    }
    void after() {
        g_launch_events = LaunchEvents{};
        ++i;
    }
};

#define RUN(call)                                   \
    do {                                            \
        rec.before();                               \
        hipError_t e_ = (call);                     \
        rec.after();                                \
        if (e_ != hipSuccess) {                     \
            g_last_hip = e_;                        \
            return STRATA_EHIP;                     \
        }                                           \
    } while (0)

// Route (and, unless route_only, prepare the input digit planes) of one
// layer.  On the decode path the top-k is taken inside the gate/up kernel
// (forward) or by a one-block finisher (routing only).
strata_status route_layer(LayerArgs &a, const strata_moe_shape &s, int T, Recorder &rec) {
    if (small_path(s, T)) {
        RUN(launch_route_logits_small(a, rec.s));
        if (a.route_only) RUN(launch_route_small_finish(a, rec.s));
    } else {
        RUN(launch_gemm_prep(a, rec.s));
        RUN(launch_route_logits(a, rec.s));
        RUN(launch_route_topk(a, rec.s));
        RUN(launch_route_permute(a, GEMM_BM, rec.s));
    }
    return STRATA_OK;
}

}  // namespace

extern "C" {

size_t strata_moe_workspace_bytes(const strata_moe_shape *shape, int32_t T, int32_t L) {
    (void)L;
    if (check_shape(shape) != STRATA_OK || T < 0) return 0;
    return layout(*shape, T > 0 ? T : 1).total;
}

const char *strata_status_str(strata_status s) {
    switch (s) {
        case STRATA_OK: return "ok";
        case STRATA_EINVAL: return "invalid argument";
        case STRATA_EUNSUPPORTED: return "unsupported shape or format";
        case STRATA_EWORKSPACE: return "workspace too small";
        case STRATA_EHIP: return hipGetErrorString(g_last_hip);
        default: return "unknown status";
    }
}

int32_t strata_moe_kernel_names(const strata_moe_shape *shape, int32_t T, const char **names, int32_t max) {
    static const char *one[] = {"route_logits", "route_gemv_gateup", "gemv_down_combine"};
    static const char *small[] = {"route_logits", "route_gemv_gateup", "gemv_down", "combine"};
    static const char *large[] = {"gemm_prep", "route_logits", "route_topk", "route_permute",
                                  "gemm_gateup", "gemm_down", "combine"};   // route_permute: three kernels
    if (check_shape(shape) != STRATA_OK) return 0;
    const bool sp = small_path(*shape, T);
    const bool t1 = sp && gemv_one_token(T, shape->n_experts, shape->top_k, shape->d_model, shape->d_ff);
    const char **src = sp ? (t1 ? one : small) : large;
    const int n = sp ? (t1 ? 3 : 4) : 7;
    for (int i = 0; i < n && i < max; ++i) names[i] = src[i];
    return n;
}

strata_status strata_moe_route(const strata_moe_shape *shape, const strata_moe_layer *layer, const void *x,
                               strata_xdtype xdtype, int32_t T, const strata_route_out *out, void *ws,
                               size_t ws_bytes, void *stream) {
    strata_status st = check_shape(shape);
    if (st != STRATA_OK) return st;
    if (T < 0 || !layer || (xdtype != STRATA_X_BF16 && xdtype != STRATA_X_F32)) return STRATA_EINVAL;
    if (T == 0) return STRATA_OK;
    if (!x || !layer->router_w || !ws) return STRATA_EINVAL;
    if (!aligned16(x) || !aligned16(ws) || !aligned16(layer->router_w)) return STRATA_EINVAL;
    const Layout l = layout(*shape, T);
    if (ws_bytes < l.total) return STRATA_EWORKSPACE;
    LayerArgs a;
    fill_common(a, *shape, l, (char *)ws, T);
    a.Wr = layer->router_w;
    a.bias = layer->router_bias;
    a.mask = nullptr;
    a.x = x;
    a.x_is_bf16 = xdtype == STRATA_X_BF16;
    a.normalize = 0;
    a.route_only = 1;
    set_route_out(a, out);
    Recorder rec{nullptr, 0, 0, (hipStream_t)stream};
    return route_layer(a, *shape, T, rec);
}

strata_status strata_moe_forward(const strata_moe_shape *shape, const strata_moe_layer *layers, int32_t L,
                                 const void *x, strata_xdtype xdtype, int32_t T, uint32_t flags, float *y_last,
                                 float *resid_out, const strata_route_out *route_out, int32_t *miss_te,
                                 float *miss_w, int32_t miss_cap, int32_t *miss_count, void *ws, size_t ws_bytes,
                                 void *const *events, int32_t n_events, void *stream) {
    strata_status st = check_shape(shape);
    if (st != STRATA_OK) return st;
    if (T < 0 || L < 1 || !layers || (xdtype != STRATA_X_BF16 && xdtype != STRATA_X_F32) || miss_cap < 0 ||
        (flags & ~(uint32_t)STRATA_NORM_FIRST) || n_events < 0 || (n_events > 0 && !events))
        return STRATA_EINVAL;
    if (T == 0) return STRATA_OK;
    if (!x || !y_last || !ws) return STRATA_EINVAL;
    if (!aligned16(x) || !aligned16(y_last) || !aligned16(ws) || (resid_out && !aligned16(resid_out)))
        return STRATA_EINVAL;
    bool any_mask = false;
    for (int l = 0; l < L; ++l) {
        if (!layers[l].router_w || !layers[l].codes || !layers[l].scales) return STRATA_EINVAL;
        if (!aligned16(layers[l].router_w) || !aligned16(layers[l].codes)) return STRATA_EINVAL;
        if (layers[l].bits != 0 && layers[l].bits != 3 && layers[l].bits != 2) return STRATA_EUNSUPPORTED;
        any_mask |= layers[l].resident_mask != nullptr;
    }
    if (any_mask && (!miss_te || !miss_w || !miss_count)) return STRATA_EINVAL;
    const Layout lay = layout(*shape, T);
    if (ws_bytes < lay.total) return STRATA_EWORKSPACE;
    char *w = (char *)ws;
    Recorder rec{events, n_events, 0, (hipStream_t)stream};

    for (int l = 0; l < L; ++l) {
        LayerArgs a;
        fill_common(a, *shape, lay, w, T);
        const strata_moe_layer &ly = layers[l];
        a.Wr = ly.router_w;
        a.bias = ly.router_bias;
        a.codes = ly.codes;
        a.scales = ly.scales;
        a.mask = ly.resident_mask;
        a.bits = ly.bits ? ly.bits : shape->bits;   // the workspace layout does not depend on it
        if (l == 0) {
            a.x = x;
            a.x_is_bf16 = xdtype == STRATA_X_BF16;
        } else {
            a.x = w + ((l - 1) % 2 ? lay.xres1 : lay.xres0);
            a.x_is_bf16 = 0;
        }
        a.normalize = (l > 0) || (flags & STRATA_NORM_FIRST);
        a.xpasses = (a.x_is_bf16 && !a.normalize) ? 1 : 2;
        a.route_only = 0;
        if (route_out) set_route_out(a, &route_out[l]);
        if (miss_te) {
            a.miss_te = miss_te + (size_t)l * miss_cap * 2;
            a.miss_w = miss_w + (size_t)l * miss_cap;
            a.miss_cap = miss_cap;
        }
        a.miss_count = miss_count ? miss_count + l : (int32_t *)(w + lay.miss_count);
        a.out = (l == L - 1) ? y_last : (float *)(w + lay.out);
        a.x_next = (l == L - 1) ? resid_out : (float *)(w + (l % 2 ? lay.xres1 : lay.xres0));
        st = route_layer(a, *shape, T, rec);
        if (st != STRATA_OK) return st;
        if (small_path(*shape, T)) {
            if (gemv_one_token(T, shape->n_experts, shape->top_k, shape->d_model, shape->d_ff)) {
                RUN(launch_gemv_gateup_small(a, (int)lay.max_items, rec.s));
                RUN(launch_gemv_down_one(a, rec.s));
            } else {
                RUN(launch_gemv_gateup_multi(a, (int)lay.max_items, rec.s));
                RUN(launch_gemv_down_multi(a, (int)lay.max_items, rec.s));
                RUN(launch_combine(a, rec.s));
            }
        } else {
            RUN(launch_gemm_gateup(a, (int)lay.max_items, rec.s));
            RUN(launch_gemm_down(a, (int)lay.max_items, rec.s));
            RUN(launch_combine(a, rec.s));
        }
    }
    return STRATA_OK;
}

}  // extern "C"
