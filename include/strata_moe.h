/*
 * strata_moe.h -- C ABI of the MI355X (gfx950) sparse MoE layer forward.
 *
 * What one layer computes, per token t (E routed experts, top-k, 1 shared):
 *   z[t][e]   = sum_i Wr[e][i] * u[t][i] (+ bias[e])              fp32 router logits
 *   idx[t][r] = the k experts with the largest z, ordered by (z desc, e asc)
 *   gate[t][r]= softmax over all E, renormalised over the k picked (fp32)
 *   per expert e:  h = silu(Wg_e u) * (Wu_e u),  y_e = Wd_e h          (SwiGLU)
 *   out[t]    = y_shared[t] + sum_{r<k, e=idx[t][r] resident} gate[t][r] * y_e[t]
 * The structure (512 routed experts per layer, 10 routed + 1 shared per
 * token per layer, 48 layers) is the model the pages describe:
 * greenbean-ai, "Strata 如何讓 12GB 顯卡跑 Qwen3.8-Flash-Next？", section 一;
 * wiselychen.com, "Strata ... RTX 5090 ... 1M context", "30 秒定位" table.
 * Experts that are not resident on the accelerator are computed elsewhere
 * (same page, technique 2 "專家快取與 CPU／GPU 分工"; greenbean-ai section 二;
 * tutuge.me "⚙️ 125B 是怎么塞进游戏 PC 的"): here a resident mask drops them
 * from the GPU sum and lists them, with their gates, in a miss list.
 *
 * Stacks of L layers (an MTP verify step runs the drafted tokens through all
 * layers in one batch: wiselychen.com technique 4 "MTP 推測解碼";
 * greenbean-ai section 三): x_0 = x; layer l consumes u_l = x_0 for l = 0
 * (or rmsnorm(x_0) with STRATA_NORM_FIRST) and u_l = rmsnorm(x_l) for
 * l > 0, where rmsnorm(v) = v / sqrt(mean(v^2) + 1e-6) (no learnt gain);
 * x_{l+1} = x_l + out_l in fp32.
 *
 * WEIGHT FORMAT (the pages name ~3-bit IQ3_XXS at about 3.06 bit/weight,
 * wiselychen.com technique 1 "低位元量化", and 2-bit Q2_0, greenbean-ai section
 * 四, but give no byte layout; this library fixes one):
 *   w = fp16 scale of its 256-element block * (code - c0),
 *   3-bit codes 0..7 with c0 = 3.5 (3.0625 bit/weight with the scale),
 *   2-bit codes 0..3 with c0 = 1.5 (2.0625 bit/weight).
 *   Per expert: gate [f][d], up [f][d], down [d][f] (out x in, row-major),
 *   experts 0..E-1 routed, then the shared expert E.  Requirements:
 *   d % 128 == 0 and f % 128 == 0.
 *   codes: element (r, c) of a matrix [out][in] sits in a 32-column "unit"
 *     at byte offset (((r/16)*(in/128) + c/128)*16 + r%16)*4*UB + ((c%128)/32)*UB
 *     (UB = 12 for 3-bit, 8 for 2-bit) at place j = c % 32.
 *     3-bit unit = little-endian u32 words A, B, C:
 *       j < 24 : code = bits [4n, 4n+3) of (A, B, C)[j/8], n = j % 8;
 *       j >= 24: n = j-24, code = A bit(4n+3) | B bit(4n+3)<<1 | C bit(4n+3)<<2.
 *     2-bit unit = little-endian u32 words A (j < 16), B (j >= 16):
 *       jj = j % 16: code = bits [4(jj%8) + 2(jj/8), +2) of the word.
 *     Matrix m of expert e starts at byte (3e + m) * d*f*bits/8.
 *   scales: IEEE binary16, one per 256 consecutive elements of the
 *     row-major flattened matrix: index (3e + m) * (d*f/256) + (r*in + c)/256.
 *
 * CONVENTIONS
 *   Pointers marked [dev] are device pointers, [host] host pointers.  The
 *   caller owns every buffer, including the workspace; the library never
 *   allocates on these entry points and keeps no per-call global state.
 *   Calls enqueue on `stream` (a hipStream_t, passed as void*) and return
 *   without a host synchronisation; outputs are valid once the stream is
 *   synchronised.  They enqueue kernel launches only (no memset, copy or
 *   event unless events are passed), so a call can be captured in a HIP
 *   graph and replayed with new contents in the same buffers.  Validation happens on the host before any launch and
 *   nothing is enqueued when it fails.  Calls that overlap on one workspace
 *   race.
 *   The workspace needs no initialisation: a call writes every part of it
 *   that it reads, so what a previous call (or anything else) left there
 *   does not change its results.
 *   x, y_last, resid_out, the workspace, router weights and codes must be
 *   16-byte aligned (hipMalloc and torch allocations are); a misaligned one
 *   is rejected with STRATA_EINVAL.
 */
#ifndef STRATA_MOE_H
#define STRATA_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    STRATA_OK = 0,
    STRATA_EINVAL = 1,       /* null required pointer or inconsistent argument */
    STRATA_EUNSUPPORTED = 2, /* shape or format this build does not handle */
    STRATA_EWORKSPACE = 3,   /* workspace smaller than strata_moe_workspace_bytes() */
    STRATA_EHIP = 4          /* a HIP launch failed; strata_status_str() names it */
} strata_status;

typedef enum { STRATA_X_BF16 = 0, STRATA_X_F32 = 1 } strata_xdtype;

enum { STRATA_NORM_FIRST = 1u }; /* forward flags: rmsnorm the first layer's input too */

/* [host] layer shape.  bits = 3 or 2.  n_shared must be 1.
 * Limits: 1 <= top_k <= 32, top_k <= n_experts <= 1024. */
typedef struct {
    int32_t n_experts, top_k, n_shared, d_model, d_ff, bits;
} strata_moe_shape;

/* [host] struct of [dev] pointers, one per layer. */
typedef struct {
    const float *router_w;          /* [E][d] fp32 */
    const float *router_bias;       /* [E] fp32, or NULL */
    const uint8_t *codes;           /* (E+1) experts, format above */
    const uint16_t *scales;         /* (E+1) experts, fp16 bit patterns */
    const uint32_t *resident_mask;  /* [ceil(E/32)] bitset (bit e%32 of word e/32), or NULL = all resident */
    int32_t bits;                   /* this layer's code width, 3 or 2 (codes and scales in that format),
                                       or 0 = the shape's bits.  Layers of one stack may differ: precision
                                       can change from layer to layer (greenbean-ai, "Strata 如何讓 12GB 顯卡跑
                                       Qwen3.8-Flash-Next？", §四).  Any other value: STRATA_EUNSUPPORTED. */
} strata_moe_layer;

/* [host] struct of optional [dev] outputs (any field may be NULL):
 *   topk_idx [T][k] int32, topk_w [T][k] fp32 (gates),
 *   counts [E] int32 (routed picks per expert), offsets [E+1] int32 (exclusive prefix sum),
 *   perm [T*k] int32: slot -> t*k + r, slots ordered by (expert asc, token asc),
 *   pos  [T*k] int32: t*k + r -> slot. */
typedef struct {
    int32_t *topk_idx;
    float *topk_w;
    int32_t *counts;
    int32_t *offsets;
    int32_t *perm;
    int32_t *pos;
} strata_route_out;

/* Bytes of workspace a call with this shape, T tokens and L layers needs
 * (the same for every L: layers reuse it in turn).  0 for an invalid or
 * unsupported shape or token count.  The workspace holds the per-call state
 * of one layer: router logits, picks, gates, the permutation, the work list,
 * the quantised layer input and the experts' intermediate outputs.
 * Larger-T calls (above 8 tokens) are limited to token counts whose bf16
 * layer input (2*T*d*2 bytes) and SwiGLU activations ((T*k + T)*f*4 bytes)
 * stay below 2^31 bytes (63,550 tokens for d = 2048, f = 768, k = 10). */
size_t strata_moe_workspace_bytes(const strata_moe_shape *shape, int32_t T, int32_t L);

/* Routing only, for one layer: the router logits, the ordered top-k with
 * its gates and the permutation that groups picks by expert (per-layer
 * routing of 10 of 512 experts: greenbean-ai, "Strata 如何讓 12GB 顯卡跑
 * Qwen3.8-Flash-Next？", section 一; the GPU runs the router: same page,
 * section 二).  x: [dev] [T][d], bf16 or fp32, used as given (no
 * normalisation).  out: [host] struct of [dev] outputs, any may be NULL.
 * ws: [dev] workspace of strata_moe_workspace_bytes(shape, T, 1) bytes.
 * EINVAL: a null x, router or workspace, T < 0, a bad dtype or a misaligned
 * pointer; EUNSUPPORTED: a shape or token count outside the limits above;
 * EWORKSPACE: ws_bytes too small; EHIP: a launch failed.
 * T = 0 is a no-op returning STRATA_OK. */
strata_status strata_moe_route(const strata_moe_shape *shape, const strata_moe_layer *layer, const void *x,
                               strata_xdtype xdtype, int32_t T, const strata_route_out *out, void *ws,
                               size_t ws_bytes, void *stream);

/* Forward of L stacked layers for T tokens: per layer the routing above,
 * the SwiGLU FFN of every picked resident expert and of the shared expert
 * over the packed blocks (the GPU computes the router, the shared expert and
 * the experts it holds: greenbean-ai, section 二; wiselychen.com technique 2
 * "專家快取與 CPU／GPU 分工"; ~3-bit and ~2-bit weights dequantised as they
 * are used: wiselychen.com technique 1 "低位元量化"), the weighted combine,
 * and the residual add that feeds the next layer (a verify step runs its
 * tokens through every layer in one batch: wiselychen.com technique 4 "MTP
 * 推測解碼").  Errors as for strata_moe_route, plus EINVAL for L < 1, a
 * null layer array, codes or scales, unknown flags or a mask without miss
 * buffers, and EUNSUPPORTED for a layer bits value other than 0, 2 or 3.
 *   layers     [host] array of L layer structs.
 *   x          [dev] [T][d] bf16 or fp32, the first layer's residual stream x_0.
 *   flags      STRATA_NORM_FIRST or 0.
 *   y_last     [dev] [T][d] fp32: out of the last layer (required).
 *   resid_out  [dev] [T][d] fp32: x_L (nullable).
 *   route_out  [host] array of L structs (nullable): routing of each layer.
 *   miss_te    [dev] [miss_cap][2] int32 (t, e); miss_w [dev] [miss_cap] fp32 gates;
 *   miss_count [dev] [L] int32: true number of misses per layer.  The first
 *              miss_cap misses of each layer, in (t asc, r asc) order, are written at
 *              miss_te + l*miss_cap*2 / miss_w + l*miss_cap.  The miss buffers may be
 *              NULL only when no layer has a resident mask; miss_cap = T*k never overflows.
 *   events     [host] array of 2*n_events hipEvent_t (as void*) or NULL: when given, the
 *              library records events[2i] before and events[2i+1] after the i-th kernel
 *              group it enqueues (i < n_events; strata_moe_kernel_names lists the groups of
 *              a call), for per-kernel timing by the caller.
 * The results do not depend on how the layers are split into calls: L layers in
 * one call give the bits of L one-layer calls chained through resid_out (with
 * STRATA_NORM_FIRST from the second on), although a T = 2..8 stack runs each
 * layer's combine inside the next layer's router kernel.
 * T = 0 is a no-op returning STRATA_OK. */
strata_status strata_moe_forward(const strata_moe_shape *shape, const strata_moe_layer *layers, int32_t L,
                                 const void *x, strata_xdtype xdtype, int32_t T, uint32_t flags, float *y_last,
                                 float *resid_out, const strata_route_out *route_out, int32_t *miss_te,
                                 float *miss_w, int32_t miss_cap, int32_t *miss_count, void *ws, size_t ws_bytes,
                                 void *const *events, int32_t n_events, void *stream);

/* strata_moe_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc.  The library keeps a fixed scratch
 * array of STRATA_NOALLOC_SCRATCH_BYTES in device memory, one per device it
 * runs on (its address found on the first call on that device), held until
 * the process ends; this entry point allocates nothing and frees nothing.
 * Every call on one GPU uses that GPU's array, so calls that overlap on one
 * GPU race, whatever their streams; calls in sequence on a stream are fine.
 * The array is never cleared: no part of it needs to start at zero (see the
 * workspace note above).  Arguments, results and errors are those of
 * strata_moe_forward, plus STRATA_EWORKSPACE when the call needs more than
 * the array holds (strata_moe_workspace_bytes(shape, T, L) >
 * STRATA_NOALLOC_SCRATCH_BYTES; for d = 2048, f = 768, top-10 that is
 * T > 403), returned before anything is enqueued. */
#define STRATA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
strata_status strata_moe_forward_noalloc(const strata_moe_shape *shape, const strata_moe_layer *layers, int32_t L,
                                         const void *x, strata_xdtype xdtype, int32_t T, uint32_t flags,
                                         float *y_last, float *resid_out, const strata_route_out *route_out,
                                         int32_t *miss_te, float *miss_w, int32_t miss_cap, int32_t *miss_count,
                                         void *const *events, int32_t n_events, void *stream);

/* ------------------------------------------------------------------------
 * Host-CPU consumer of the miss list.  The pages' engine computes the
 * experts its GPU holds on the GPU and the others on the CPU at the same
 * time, then adds the two (wiselychen.com, technique 2 "專家快取與 CPU／GPU 分工";
 * digiland.tw, "Strata 實測", item 2 "CPU 與 GPU 的協同運算（Co-processing）";
 * tutuge.me "⚙️ 125B 是怎么塞进游戏 PC 的").  Here the host evaluates, for
 * every listed miss (t, e, gate), gate * FFN_e(u_t) from packed weights in
 * host memory (the format above), in fp32 on host threads with AVX-512 when
 * the CPU has it, else AVX2 (strata_moe_host_isa() says which; neither:
 * STRATA_EUNSUPPORTED).  Results do not depend on the thread count.
 * Limits: d_model <= 8192, d_ff <= 4096.
 */

/* [host] struct of [host] pointers: one layer's weights as the host holds
 * them (same bytes as strata_moe_layer.codes / .scales). */
typedef struct {
    const uint8_t *codes;    /* (E+1) experts */
    const uint16_t *scales;  /* fp16 bit patterns */
    int32_t bits;            /* 3 or 2, or 0 = the shape's bits */
} strata_moe_host_layer;

/* Bytes of host workspace for T tokens and up to miss_cap misses per layer
 * (0 for an invalid shape or one the host consumer does not handle). */
size_t strata_moe_host_workspace_bytes(const strata_moe_shape *shape, int32_t T, int32_t miss_cap);

/* "avx512", "avx2" or "none": the instruction set the host consumer uses. */
const char *strata_moe_host_isa(void);

/* Host only, synchronous: y_add[t] = sum over the misses of token t of
 * gate * FFN_e(u_t) (rows of tokens without misses are set to 0).
 *   u        [host] [T][d] fp32: the layer input the experts consume.
 *   miss_te  [host] [n_miss][2] (t, e) with 0 <= t < T, 0 <= e < E; miss_w [host] [n_miss] gates.
 *   y_add    [host] [T][d] fp32, written.
 *   host_ws  [host] strata_moe_host_workspace_bytes(shape, T, n_miss) bytes.
 *   n_threads >= 1 host threads.
 * EINVAL: null pointers, a miss outside the ranges, n_threads < 1;
 * EWORKSPACE: host_ws too small; EUNSUPPORTED: see above. */
strata_status strata_moe_host_misses(const strata_moe_shape *shape, const strata_moe_host_layer *layer,
                                     const float *u, int32_t T, const int32_t *miss_te, const float *miss_w,
                                     int32_t n_miss, float *y_add, void *host_ws, size_t host_ws_bytes,
                                     int32_t n_threads);

/* strata_moe_forward with the misses of every masked layer computed on the
 * host and added in: per masked layer, once the kernel that completes the
 * miss list has been enqueued, the miss list and the layer input are copied
 * to host_ws on aux_stream (after an event on `stream`, so the copies
 * overlap the GPU's expert kernels; aux_stream may be NULL: then `stream`),
 * the calling thread waits for those copies, computes the misses as
 * strata_moe_host_misses does, and enqueues on `stream` a copy of their sum
 * to the workspace and a kernel that adds it to the layer's output
 * (y = y_resident + y_misses, then x_next = x + y).  The next layer starts
 * from that residual.  The call returns once the last layer's host work is
 * done and its add is enqueued: host_ws must stay untouched until `stream`
 * is synchronised.  host_layers: [host] array of L structs (used for masked
 * layers).  host_ws: [host] strata_moe_host_workspace_bytes(shape, T,
 * miss_cap) bytes, page-locked (hipHostMalloc) so that the copies run
 * asynchronously.  miss_cap must be at least T*k (no miss is left out).
 * Layers without a mask run as in strata_moe_forward.  Errors as for
 * strata_moe_forward and strata_moe_host_misses; the HIP events it needs are
 * created and destroyed inside the call. */
strata_status strata_moe_forward_coprocess(const strata_moe_shape *shape, const strata_moe_layer *layers,
                                           const strata_moe_host_layer *host_layers, int32_t L, const void *x,
                                           strata_xdtype xdtype, int32_t T, uint32_t flags, float *y_last,
                                           float *resid_out, const strata_route_out *route_out, int32_t *miss_te,
                                           float *miss_w, int32_t miss_cap, int32_t *miss_count, void *ws,
                                           size_t ws_bytes, void *host_ws, size_t host_ws_bytes, int32_t n_threads,
                                           void *aux_stream, void *stream);

/* Names of the kernel groups an L-layer strata_moe_forward call with T tokens
 * enqueues, in order (the i-th is what events[2i], events[2i+1] bracket):
 * static strings, the first max of them written to names.  Returns the
 * number of groups (which may exceed max), 0 for an invalid shape, T < 1 or
 * L < 1.  For T = 2..8 a stack folds each layer's combine into the next
 * layer's router kernel ("combine_route_logits"), so only the last layer
 * ends with "combine": 3L + 1 groups. */
int32_t strata_moe_kernel_names(const strata_moe_shape *shape, int32_t T, int32_t L, const char **names,
                                int32_t max);

/* Running expert popularity (the expert cache learns which experts are hot as
 * it is used: wiselychen.com, technique 2 "專家快取與 CPU／GPU 分工"; wiki.nginx.tw,
 * "Strata：把 1250 億參數的 Qwen3.8-Flash-Next 跑在遊戲顯卡上", dynamic expert cache item).
 * counts_acc[e] += counts[e] for e < n_experts: [dev] int64 [E] running totals (caller-owned, zeroed
 * by the caller before the first call) and [dev] int32 [E] per-call counts such as
 * strata_route_out.counts.  Enqueued on `stream`.  EINVAL: a null pointer or E outside 1..1024;
 * EHIP: the launch failed. */
strata_status strata_moe_counts_accumulate(int64_t *counts_acc, const int32_t *counts, int32_t n_experts,
                                           void *stream);

/* Resident set from running counts: mask_out ([dev] uint32 [ceil(E/32)], bit e%32 of word e/32, the
 * strata_moe_layer.resident_mask format) gets the n_resident experts with the largest counts, ties
 * to the lower index, so the mask is the same on every run.  Enqueued on `stream`.  EINVAL: a null
 * pointer, E outside 1..1024 or n_resident outside 0..E; EHIP: the launch failed. */
strata_status strata_moe_resident_topn(const int64_t *counts_acc, int32_t n_experts, int32_t n_resident,
                                       uint32_t *mask_out, void *stream);

/* Static description of a status (for STRATA_EHIP, of the last HIP error). */
const char *strata_status_str(strata_status s);

#ifdef __cplusplus
}
#endif
#endif /* STRATA_MOE_H */
