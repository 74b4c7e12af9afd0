// C ABI of the MoE layer library: host-side validation, workspace carving,
// kernel selection by token count, the per-layer loop and stream ordering.
// Nothing here allocates device memory or synchronises the stream.
#include <string.h>

#include <mutex>

#include "strata_moe.h"
#include "common.hpp"
#include "host_experts.hpp"

using namespace strata;

namespace {

thread_local hipError_t g_last_hip = hipSuccess;

}  // namespace

namespace strata {
thread_local LaunchEvents g_launch_events;

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

strata_status hip_status(hipError_t e) {
    if (e == hipSuccess) return STRATA_OK;
    g_last_hip = e;
    return STRATA_EHIP;
}
}  // namespace strata

namespace {

constexpr size_t ALIGN = 256;
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
size_t up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

// Token counts up to this take the decode path (one work item per expert).
constexpr int SMALL_T = 8;

struct Layout {
    size_t z, idx, gate, counts, offsets, perm, pos, inv_rms, items, n_items, xq, xsum, xscl, hf,
        xa, sx, ha, hs, bcnt, bmiss, Y, rbits, out, xres0, xres1, miss_count, total;
    int64_t max_items;
};

bool small_path(const strata_moe_shape &s, int64_t T) {
    return T <= SMALL_T && (size_t)T * s.d_model * sizeof(float) <= 64 * 1024;
}

// Decode-path batches of 2..8 tokens (the item-major expert kernels, whose
// outputs a separate combine sums): in a stack, a layer's combine is folded
// into the next layer's router kernel.
bool fuse_combine(const strata_moe_shape &s, int64_t T) {
    return small_path(s, T) && !strata::gemv_one_token((int)T, s.n_experts, s.top_k, s.d_model, s.d_ff);
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
    l.z = take(sizeof(float) * T * E * (sp ? route_logit_planes((int)d) : route_logit_splits((int)d)));
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
    l.rbits = take(4 * T);
    l.out = take(sizeof(float) * T * d);
    l.xres0 = take(sizeof(float) * T * d);
    l.xres1 = take(sizeof(float) * T * d);
    l.miss_count = take(4);
    l.total = o;
    return l;
}

// The larger-T kernels address the bf16 layer input (hi and lo pieces) and
// h with 32-bit buffer offsets, and slots and permutation entries are int32:
// token counts whose arrays would not fit are refused before any launch.
bool fits_32bit(const strata_moe_shape &s, int64_t T) {
    if (small_path(s, T)) return true;
    const int64_t slots = T * s.top_k + T;
    return 2 * T * s.d_model * 2 <= (int64_t)INT32_MAX && slots * s.d_ff * 4 <= (int64_t)INT32_MAX &&
           slots <= (int64_t)INT32_MAX;
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
    a.zplanes = 1;
    a.idx = (int32_t *)(ws + l.idx);
    a.gate = (float *)(ws + l.gate);
    a.counts = (int32_t *)(ws + l.counts);
    a.offsets = (int32_t *)(ws + l.offsets);
    a.perm = (int32_t *)(ws + l.perm);
    a.pos = (int32_t *)(ws + l.pos);
    a.inv_rms = (float *)(ws + l.inv_rms);
    a.items = (WorkItem *)(ws + l.items);
    a.n_items = (int32_t *)(ws + l.n_items);
    a.xq = (uint32_t *)(ws + l.xq);
    a.xsum = (int32_t *)(ws + l.xsum);
    a.xscl = (float *)(ws + l.xscl);
    a.hf = (float *)(ws + l.hf);
    a.Y = (float *)(ws + l.Y);
    a.rbits = (int32_t *)(ws + l.rbits);
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
        if (e_ != hipSuccess) return hip_status(e_); \
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
    if (check_shape(shape) != STRATA_OK || T < 0 || !fits_32bit(*shape, T)) return 0;
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

int32_t strata_moe_kernel_names(const strata_moe_shape *shape, int32_t T, int32_t L, const char **names,
                                int32_t max) {
    static const char *one[] = {"route_logits", "route_gemv_gateup", "gemv_down_combine"};
    static const char *small[] = {"route_logits", "route_gemv_gateup", "gemv_down", "combine"};
    static const char *large[] = {"gemm_prep", "route_logits", "route_topk", "route_permute",
                                  "gemm_gateup", "gemm_down", "combine"};   // route_permute: three kernels
    if (check_shape(shape) != STRATA_OK || T < 1 || L < 1) return 0;
    int n = 0;
    auto put = [&](const char *s) {
        if (n < max) names[n] = s;
        ++n;
    };
    if (!small_path(*shape, T)) {
        for (int l = 0; l < L; ++l)
            for (const char *s : large) put(s);
    } else if (gemv_one_token(T, shape->n_experts, shape->top_k, shape->d_model, shape->d_ff)) {
        for (int l = 0; l < L; ++l)
            for (const char *s : one) put(s);
    } else {
        // layer l > 0 of a stack: the previous layer's combine and this router in one kernel
        for (int l = 0; l < L; ++l) {
            put(l == 0 || L == 1 ? small[0] : "combine_route_logits");
            put(small[1]);
            put(small[2]);
        }
        put(small[3]);
    }
    return n;
}

strata_status strata_moe_route(const strata_moe_shape *shape, const strata_moe_layer *layer, const void *x,
                               strata_xdtype xdtype, int32_t T, const strata_route_out *out, void *ws,
                               size_t ws_bytes, void *stream) {
    strata_status st = check_shape(shape);
    if (st != STRATA_OK) return st;
    if (T < 0 || !layer || (xdtype != STRATA_X_BF16 && xdtype != STRATA_X_F32)) return STRATA_EINVAL;
    if (T == 0) return STRATA_OK;
    if (!fits_32bit(*shape, T)) return STRATA_EUNSUPPORTED;
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

}  // extern "C"

namespace {

// Host side of a co-processing forward: per masked layer, the miss list and
// the layer input are copied to the host (on `aux`, after the kernel that
// completes the miss list), the host computes the missed experts while the
// GPU runs the resident ones, and the sum is added on the GPU.
struct Coproc {
    const strata_moe_host_layer *host_layers;
    char *hws;
    HostLayout hl;
    int n_threads;
    hipStream_t aux;
    hipEvent_t ev_miss = nullptr, ev_copied = nullptr;
    ~Coproc() {
        if (ev_miss) (void)hipEventDestroy(ev_miss);
        if (ev_copied) (void)hipEventDestroy(ev_copied);
    }
};

strata_status coproc_copy_out(Coproc &cp, const LayerArgs &a, hipStream_t s) {
    const size_t xb = (size_t)a.T * a.d * (a.x_is_bf16 ? 2 : 4);
    hipError_t e = hipEventRecord(cp.ev_miss, s);
    if (e == hipSuccess && cp.aux != s) e = hipStreamWaitEvent(cp.aux, cp.ev_miss, 0);
    if (e == hipSuccess)
        e = hipMemcpyAsync(cp.hws + cp.hl.mcount, a.miss_count, 4, hipMemcpyDeviceToHost, cp.aux);
    if (e == hipSuccess)
        e = hipMemcpyAsync(cp.hws + cp.hl.mte, a.miss_te, (size_t)a.miss_cap * 8, hipMemcpyDeviceToHost, cp.aux);
    if (e == hipSuccess)
        e = hipMemcpyAsync(cp.hws + cp.hl.mw, a.miss_w, (size_t)a.miss_cap * 4, hipMemcpyDeviceToHost, cp.aux);
    if (e == hipSuccess) e = hipMemcpyAsync(cp.hws + cp.hl.xstage, a.x, xb, hipMemcpyDeviceToHost, cp.aux);
    if (e == hipSuccess) e = hipEventRecord(cp.ev_copied, cp.aux);
    return hip_status(e);
}

// Wait for the copies, compute the layer's missed experts on the host, and
// enqueue their sum into the layer's output and residual stream.
strata_status coproc_finish(Coproc &cp, const LayerArgs &a, int bits, const strata_moe_host_layer &hl_,
                            float *yadd_dev, hipStream_t s) {
    hipError_t e = hipEventSynchronize(cp.ev_copied);
    if (e != hipSuccess) return hip_status(e);
    const int T = a.T, d = a.d;
    const int n = *(const int32_t *)(cp.hws + cp.hl.mcount);
    if (n < 0 || n > a.miss_cap) return STRATA_EINVAL;   // cannot happen with miss_cap >= T*k
    // the layer input the GPU used: x (bf16 or fp32), RMS-normalised when the layer normalises
    float *u = (float *)(cp.hws + cp.hl.u);
    const char *xs = cp.hws + cp.hl.xstage;
    for (int t = 0; t < T; ++t) {
        float *ur = u + (size_t)t * d;
        for (int i = 0; i < d; ++i) {
            if (a.x_is_bf16) {
                const uint32_t b = (uint32_t)((const uint16_t *)xs)[(size_t)t * d + i] << 16;
                memcpy(&ur[i], &b, 4);
            } else {
                ur[i] = ((const float *)xs)[(size_t)t * d + i];
            }
        }
        if (a.normalize) {
            double ss = 0.0;
            for (int i = 0; i < d; ++i) ss += (double)ur[i] * ur[i];
            const float inv = (float)(1.0 / sqrt(ss / d + (double)RMS_EPS));
            for (int i = 0; i < d; ++i) ur[i] *= inv;
        }
    }
    HostMissArgs h{};
    h.E = a.E;
    h.d = d;
    h.f = a.f;
    h.bits = bits;
    h.T = T;
    h.n_miss = n;
    h.n_threads = cp.n_threads;
    h.codes = hl_.codes;
    h.scales = hl_.scales;
    h.u = u;
    h.miss_te = (const int32_t *)(cp.hws + cp.hl.mte);
    h.miss_w = (const float *)(cp.hws + cp.hl.mw);
    h.h = (float *)(cp.hws + cp.hl.h);
    h.gstart = (int32_t *)(cp.hws + cp.hl.gstart);
    h.order = (int32_t *)(cp.hws + cp.hl.order);
    h.experts = (int32_t *)(cp.hws + cp.hl.experts);
    h.y_add = (float *)(cp.hws + cp.hl.yadd);
    run_host_misses(h);
    e = hipMemcpyAsync(yadd_dev, h.y_add, (size_t)T * d * 4, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(launch_add_rows(a, yadd_dev, s));
}

strata_status forward_impl(const strata_moe_shape *shape, const strata_moe_layer *layers, int32_t L, const void *x,
                           strata_xdtype xdtype, int32_t T, uint32_t flags, float *y_last, float *resid_out,
                           const strata_route_out *route_out, int32_t *miss_te, float *miss_w, int32_t miss_cap,
                           int32_t *miss_count, void *ws, size_t ws_bytes, void *const *events, int32_t n_events,
                           void *stream, Coproc *cp) {
    strata_status st = check_shape(shape);
    if (st != STRATA_OK) return st;
    if (T < 0 || L < 1 || !layers || (xdtype != STRATA_X_BF16 && xdtype != STRATA_X_F32) || miss_cap < 0 ||
        (flags & ~(uint32_t)STRATA_NORM_FIRST) || n_events < 0 || (n_events > 0 && !events))
        return STRATA_EINVAL;
    if (T == 0) return STRATA_OK;
    if (!fits_32bit(*shape, T)) return STRATA_EUNSUPPORTED;
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

    // T = 2..8 stacks: the combine of layer l runs inside layer l+1's router
    // kernel (same arithmetic), so only the last layer launches a combine
    const bool fuse = L > 1 && !cp && fuse_combine(*shape, T);
    const void *px = nullptr;          // previous layer's input and mask
    int px_bf16 = 0;
    const uint32_t *pmask = nullptr;
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
        a.ytok = fuse_combine(*shape, T) ? 1 : 0;   // item-major down kernel: Y rows in token order
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
        const bool co = cp && a.mask;   // this layer's misses go to the host
        if (fuse && l > 0) {
            a.px = px;
            a.px_is_bf16 = px_bf16;
            a.pmask = pmask;
            a.x_cur = (float *)const_cast<void *>(a.x);
            a.zplanes = route_logit_planes(shape->d_model);
            RUN(launch_route_combine_small(a, rec.s));
        } else {
            st = route_layer(a, *shape, T, rec);
            if (st != STRATA_OK) return st;
        }
        px = a.x;
        px_bf16 = a.x_is_bf16;
        pmask = a.mask;
        if (small_path(*shape, T)) {
            // the gate/up kernel completes the routing and the miss list
            if (gemv_one_token(T, shape->n_experts, shape->top_k, shape->d_model, shape->d_ff)) {
                RUN(launch_gemv_gateup_small(a, (int)lay.max_items, rec.s));
                if (co && (st = coproc_copy_out(*cp, a, rec.s)) != STRATA_OK) return st;
                RUN(launch_gemv_down_one(a, rec.s));
            } else {
                RUN(launch_gemv_gateup_multi(a, (int)lay.max_items, rec.s));
                if (co && (st = coproc_copy_out(*cp, a, rec.s)) != STRATA_OK) return st;
                RUN(launch_gemv_down_multi(a, (int)lay.max_items, rec.s));
                if (!fuse || l == L - 1) RUN(launch_combine(a, rec.s));
            }
        } else {
            if (co && (st = coproc_copy_out(*cp, a, rec.s)) != STRATA_OK) return st;
            RUN(launch_gemm_gateup(a, (int)lay.max_items, rec.s));
            RUN(launch_gemm_down(a, (int)lay.max_items, rec.s));
            RUN(launch_combine(a, rec.s));
        }
        // the host's sum is staged in the expert-output area: the combine has
        // read it (earlier on the stream) and the next layer writes it later
        if (co && (st = coproc_finish(*cp, a, a.bits, cp->host_layers[l], (float *)(w + lay.Y), rec.s)) != STRATA_OK)
            return st;
    }
    return STRATA_OK;
}

}  // namespace

extern "C" {

strata_status strata_moe_forward(const strata_moe_shape *shape, const strata_moe_layer *layers, int32_t L,
                                 const void *x, strata_xdtype xdtype, int32_t T, uint32_t flags, float *y_last,
                                 float *resid_out, const strata_route_out *route_out, int32_t *miss_te,
                                 float *miss_w, int32_t miss_cap, int32_t *miss_count, void *ws, size_t ws_bytes,
                                 void *const *events, int32_t n_events, void *stream) {
    return forward_impl(shape, layers, L, x, xdtype, T, flags, y_last, resid_out, route_out, miss_te, miss_w,
                        miss_cap, miss_count, ws, ws_bytes, events, n_events, stream, nullptr);
}

strata_status strata_moe_forward_coprocess(const strata_moe_shape *shape, const strata_moe_layer *layers,
                                           const strata_moe_host_layer *host_layers, int32_t L, const void *x,
                                           strata_xdtype xdtype, int32_t T, uint32_t flags, float *y_last,
                                           float *resid_out, const strata_route_out *route_out, int32_t *miss_te,
                                           float *miss_w, int32_t miss_cap, int32_t *miss_count, void *ws,
                                           size_t ws_bytes, void *host_ws, size_t host_ws_bytes, int32_t n_threads,
                                           void *aux_stream, void *stream) {
    strata_status st = check_shape(shape);
    if (st != STRATA_OK) return st;
    if (T < 0 || L < 1 || !layers || !host_layers || n_threads < 1) return STRATA_EINVAL;
    if (T == 0) return STRATA_OK;
    if (!host_supported(*shape)) return STRATA_EUNSUPPORTED;
    if ((int64_t)miss_cap < (int64_t)T * shape->top_k || !miss_te || !miss_w || !miss_count || !host_ws)
        return STRATA_EINVAL;
    for (int l = 0; l < L; ++l) {
        if (!layers[l].resident_mask) continue;
        if (!host_layers[l].codes || !host_layers[l].scales) return STRATA_EINVAL;
        const int hb = host_layers[l].bits ? host_layers[l].bits : shape->bits;
        const int db = layers[l].bits ? layers[l].bits : shape->bits;
        if (hb != db) return STRATA_EINVAL;
    }
    Coproc cp;
    cp.host_layers = host_layers;
    cp.hws = (char *)host_ws;
    cp.hl = host_layout(shape->n_experts, shape->d_model, shape->d_ff, T, miss_cap);
    if (host_ws_bytes < cp.hl.total) return STRATA_EWORKSPACE;
    cp.n_threads = n_threads;
    cp.aux = aux_stream ? (hipStream_t)aux_stream : (hipStream_t)stream;
    hipError_t e = hipEventCreateWithFlags(&cp.ev_miss, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&cp.ev_copied, hipEventDisableTiming);
    if (e != hipSuccess) return hip_status(e);
    return forward_impl(shape, layers, L, x, xdtype, T, flags, y_last, resid_out, route_out, miss_te, miss_w,
                        miss_cap, miss_count, ws, ws_bytes, nullptr, 0, stream, &cp);
}

// ------------------------------------------------ no-allocation variant
// The workspace of strata_moe_forward_noalloc: a fixed array in device
// memory, one copy per device (created when the library's code is loaded on
// that device, held until the process ends).  Host code must not use the
// name `scratch` as an address: each device's copy is found once with
// hipGetSymbolAddress and that address is what the kernels are given.
static __device__ __align__(256) uint8_t scratch[STRATA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];

// Address of the current device's scratch, looked up on its first use.
strata_status device_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= MAX_DEVICES) return STRATA_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!p) return hip_status(hipErrorInvalidSymbol);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return STRATA_OK;
}

}  // namespace

strata_status strata_moe_forward_noalloc(const strata_moe_shape *shape, const strata_moe_layer *layers, int32_t L,
                                         const void *x, strata_xdtype xdtype, int32_t T, uint32_t flags,
                                         float *y_last, float *resid_out, const strata_route_out *route_out,
                                         int32_t *miss_te, float *miss_w, int32_t miss_cap, int32_t *miss_count,
                                         void *const *events, int32_t n_events, void *stream) {
    strata_status st = check_shape(shape);
    if (st != STRATA_OK) return st;
    if (T < 0) return STRATA_EINVAL;
    if (T > 0) {
        if (!fits_32bit(*shape, T)) return STRATA_EUNSUPPORTED;
        if (layout(*shape, T).total > STRATA_NOALLOC_SCRATCH_BYTES) return STRATA_EWORKSPACE;
    }
    void *ws = nullptr;
    if (T > 0) {
        st = device_scratch(&ws);
        if (st != STRATA_OK) return st;
    }
    return strata_moe_forward(shape, layers, L, x, xdtype, T, flags, y_last, resid_out, route_out, miss_te, miss_w,
                              miss_cap, miss_count, ws, T > 0 ? STRATA_NOALLOC_SCRATCH_BYTES : 0, events, n_events,
                              stream);
}

}  // extern "C"
