#!/usr/bin/env python3
"""Benchmark of the MI355X sparse MoE layer forward.

Default run (one JSON line): the headline is the full-size decode layer --
512 routed experts top-10 + 1 shared, d = 2048, f = 768, 3-bit 256-element
blocks, T = 1 token of bf16 N(0,1) input, random N(0, 1/d) router; one step
= one whole layer forward (router, top-k and gates, permutation, expert
FFNs over the packed codes, shared expert, combine).  Every step uses a new
token and the next of 48 resident layers (the model's depth), so the
~0.93 GB of codes per layer come from HBM, not the 256 MB Infinity Cache.
The same line carries the other two workloads the metric names, each
timed on its own with the same step and warmup counts:
  * "verify_T5": the verify step of multi-token prediction, 5 tokens
    (1 accepted + 4 drafts) through all 48 resident layers in one call,
    residual stream carried between layers (value = token-rows/s);
  * "prefill_4096_2bit": one 4096-token prefill chunk through a full-size
    2-bit layer (the matrix-core path; two resident layers alternate).
Before the warmup every resident layer has run once, so the timed steps see
no first touches, and untimed steps have run for --ramp-ms (100 ms), so the
GPU's clocks have left the idle of the host-side setup; the timed calls'
arguments are marshalled before the timed region starts.

`--workload NAME` times one workload alone (decode, mtp_verify,
prefill_2bit, or zipf_prefill: the 32K-token Zipf-skewed prompt with the
165-expert resident mask), e.g. under a profiler.

Each record reports the dominant kernel's roofline fraction (its time from
HIP events the library records around it, on the stream it runs on) against
the vendor peak and against probed peaks (a stream read of 4 GiB and bf16
matrix-core chains, measured in the same run), its HBM bytes from committed
rocprofv3 counter runs when those were taken on the current kernel source,
and the CPU oracle's rate on a bounded sample.

`--copy-calibration MIB` adds a plain fp32 elementwise copy of known size to
the run (reference kernel for the byte counters); `--traffic-from FETCH
WRITE` turns the counter CSVs of two such runs into
profiles/traffic_<kernel>_<workload>.md; `--counters-from CSV` turns a
matrix-core counter run into profiles/counters_<kernel>_<workload>.md.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "bit_routed_expert_amd", "csrc")

# Per workload: the dominant kernel (library kernel group and the symbol
# rocprofv3 reports), the source files that define it, the synthetic
# workload whose shapes and streams it uses, and the resident layers.
WORKLOADS = {
    "decode": dict(kernel="route_gemv_gateup", symbol="gemv_gateup_small_kernel", rotate=48, inputs=None,
                   synth="decode", sources=["common.hpp", "routing.hpp", "gemv_impl.hpp", "gemv_gu3.hip"]),
    "mtp_verify": dict(kernel="route_gemv_gateup", symbol="gemv_gateup_multi_kernel", rotate=48, inputs=4,
                       synth="mtp_verify", sources=["common.hpp", "routing.hpp", "gemv_impl.hpp", "gemv_gu3.hip"]),
    "prefill_2bit": dict(kernel="gemm_gateup", symbol="gemm_gateup_kernel", rotate=2, inputs=4,
                         synth="prefill_2bit", sources=["common.hpp", "mfma.hpp", "gemm_impl.hpp", "gemm_gu2.hip"]),
    # one step = the whole 32K prompt: its eight 4096-token chunks, in order
    "zipf_prefill": dict(kernel="gemm_gateup", symbol="gemm_gateup_kernel", rotate=2, inputs=8,
                         synth="zipf_prefill", sources=["common.hpp", "mfma.hpp", "gemm_impl.hpp", "gemm_gu3.hip"]),
}
# kernels whose counters the profiles may hold, by (kernel group, workload)
COUNTER_KERNELS = {
    "gemm_gateup": ("gemm_gateup_kernel", ["common.hpp", "mfma.hpp", "gemm_impl.hpp", "gemm_gu2.hip"]),
    "gemm_down": ("gemm_down_kernel", ["common.hpp", "mfma.hpp", "gemm_impl.hpp", "gemm_dn2.hip"]),
    "gemv_down": ("gemv_down_rows_one_kernel", ["common.hpp", "routing.hpp", "gemv_impl.hpp", "gemv_dn3.hip"]),
    "gemv_down_multi": ("gemv_down_multi_kernel", ["common.hpp", "routing.hpp", "gemv_impl.hpp", "gemv_dn3.hip"]),
    "route_gemv_gateup": None,   # filled per workload from WORKLOADS
}
COPY_SYMBOL = "MulFunctor"
SUB_RECORDS = (("verify_T5", "mtp_verify"), ("prefill_4096_2bit", "prefill_2bit"))
METRIC = "MoE-layer tokens/s (decode T=1,5; prefill 4096) + % of HBM/MFMA peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps of each workload (default: 2000 decode, 100 verify, 200 prefill, 30 Zipf)")
    p.add_argument("--warmup", type=int, default=None, help="untimed steps after the setup passes (default steps/10)")
    p.add_argument("--rotate", type=int, default=None, help="independent resident layers cycled through")
    p.add_argument("--cpu-sample-s", type=float, default=8.0, help="target seconds of oracle work per sample")
    p.add_argument("--ramp-ms", type=float, default=100.0,
                   help="untimed steps run for this long (batches of 8, synchronised) before the warmup steps")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-probes", action="store_true")
    p.add_argument("--profile-only", action="store_true", help="skip the CPU baseline, probes and event pass")
    p.add_argument("--workload", default="all", choices=["all"] + sorted(WORKLOADS),
                   help="all (decode headline + verify and prefill sub-records) or one workload alone")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="run a plain fp32 elementwise copy of MIB MiB (read + write) 5 times before the warmup")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write the traffic summary from two rocprofv3 counter CSVs of a --copy-calibration run")
    p.add_argument("--traffic-kernel", default=None,
                   help="kernel group the traffic summary is for (default: the workload's dominant kernel)")
    p.add_argument("--counters-from", metavar="CSV", help="write the matrix-core counter summary from a CSV")
    p.add_argument("--stats-from", metavar="CSV",
                   help="write profiles/kernel_stats_<workload>.md from a rocprofv3 --stats kernel_stats CSV")
    p.add_argument("--stats-cmd", default="", help="the profiled command, recorded in the stats summary")
    a = p.parse_args()
    return a


def _log(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def default_steps(workload):
    return {"decode": 2000, "mtp_verify": 100, "zipf_prefill": 30}.get(workload, 200)


def source_hash(files):
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


# ------------------------------------------------------------------ probes
def probe_peaks(dev):
    """Achievable peaks on this GPU: a 4 GiB stream read (16-byte loads,
    far beyond the Infinity Cache) and bf16 matrix-core chains."""
    import torch
    import bit_routed_expert_amd as brx
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(65536, dtype=torch.int32, device=dev)
    sinkf = torch.empty(65536, dtype=torch.float32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    best_read = 0.0
    for blocks in (2048, 4096, 8192):
        for rep in range(4):
            ev[0].record()
            brx.probe_hbm_read(buf, nbytes, sink, blocks)
            ev[1].record()
            torch.cuda.synchronize()
            if rep:
                best_read = max(best_read, nbytes / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9)
    del buf
    best_mfma = 0.0
    for blocks in (1024, 2048):
        for rep in range(3):
            ev[0].record()
            fl = brx.probe_mfma_bf16(4096, sinkf, blocks)
            ev[1].record()
            torch.cuda.synchronize()
            if rep:
                best_mfma = max(best_mfma, fl / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e12)
    return {"hbm_read_gbs": round(best_read, 1), "hbm_read_frac_of_nominal": round(best_read / HBM_PEAK_GBS, 4),
            "mfma_bf16_tflops": round(best_mfma, 1),
            "mfma_bf16_frac_of_nominal": round(best_mfma / BF16_MFMA_PEAK_TFLOPS, 4),
            "method": "best of repeated launches: stream read of a 4 GiB buffer (16-byte loads, 2048-8192 blocks); "
                      "4 independent v_mfma_f32_32x32x16_bf16 chains per wave, 4096 steps, 1024-2048 blocks"}


# ------------------------------------------------------------ resident data
class Resident:
    """Resident layers and input batches of one synthetic workload."""

    def __init__(self, name, nrot, n_in, dev):
        import torch
        import bit_routed_expert_amd as brx
        import synth
        w = synth.WORKLOADS[name]
        self.w = w
        self.T = w.tokens_per_call
        self.calls = w.calls
        self.bias = torch.from_numpy(synth.zipf_bias(w)).to(dev) if w.zipf_s > 0 else None
        self.mask_np = synth.resident_mask(w) if w.resident else None
        self.mask = torch.from_numpy(self.mask_np.view(np.int32)).to(dev) if self.mask_np is not None else None
        layer_bytes = w.experts_total * w.code_bytes_per_expert
        pinned = torch.empty(layer_bytes, dtype=torch.uint8, pin_memory=True)
        self.layers = []
        for l in range(nrot):
            synth.layer_codes_into(w, l, pinned.data_ptr())
            codes = torch.empty(layer_bytes, dtype=torch.uint8, device=dev)
            codes.copy_(pinned, non_blocking=False)
            scales = torch.from_numpy(synth.layer_scales(w, l).view(np.int16)).to(dev)
            wr = torch.from_numpy(synth.router_weights(w, l)).to(dev)
            self.layers.append(brx.LayerData(router_w=wr, codes=codes, scales=scales, router_bias=self.bias,
                                             resident_mask=self.mask))
        del pinned
        if self.calls > 1 and n_in % self.calls:
            sys.exit("the input batches must hold whole prompts")
        self.n_in = n_in
        self.xs = torch.from_numpy(synth.x_tokens(w, range(n_in * self.T), rep=1).view(np.int16)).to(dev).view(
            n_in, self.T, w.d_model)


def bench_workload(name, args, res, dev, probes, steps, warmup):
    """Time `steps` steps of one workload (after one setup pass per resident
    layer and `warmup` untimed steps) and build its record."""
    import torch
    import bit_routed_expert_amd as brx
    cfg = WORKLOADS[name]
    w = res.w
    T, calls = res.T, res.calls
    E, k, d, f = w.n_experts, w.top_k, w.d_model, w.d_ff
    sh = brx.shape(E, k, d, f, w.bits)
    depth = w.layers
    nrot = len(res.layers)
    if nrot < depth:
        sys.exit(f"--rotate must be at least the stack depth {depth}")
    ws_bytes = brx.workspace_bytes(sh, T, depth)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    resid = torch.empty((T, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    names = brx.kernel_names(sh, T, depth)   # kernel groups of one call, in launch order
    miss = {}
    if res.mask is not None:   # miss list of every (token, non-resident pick); T*k entries never overflow
        cap = T * k
        miss = dict(miss_te=torch.empty((cap, 2), dtype=torch.int32, device=dev),
                    miss_w=torch.empty(cap, dtype=torch.float32, device=dev), miss_cap=cap,
                    miss_count=torch.zeros(depth, dtype=torch.int32, device=dev))
    n_in = res.n_in

    def stack(i):
        return [res.layers[(i * depth + j) % nrot] for j in range(depth)]

    def step(i, events=None, route_outs=None, call=None):
        for c in (range(calls) if call is None else [call]):
            brx.forward(sh, stack(i), res.xs[(i * calls + c) % n_in], brx.X_BF16, T, y, ws, ws_bytes,
                        resid_out=resid, route_outs=route_outs, events=events, stream=stream, **miss)

    # the timed calls, their arguments marshalled ahead (the same calls as
    # step(), so the GPU's first kernel is not held back by Python)
    calls_timed = [brx.PreparedForward(sh, stack(i), res.xs[(i * calls + c) % n_in], brx.X_BF16, T, y, ws, ws_bytes,
                                       resid_out=resid, stream=stream, **miss)
                   for i in range(warmup, warmup + steps) for c in range(calls)]

    # ---- setup passes: every resident layer once; then untimed steps until
    # the GPU has run for args.ramp_ms (its clocks settle after an idle
    # host-side setup); then the warmup steps
    setup_passes = 0
    for i in range(max(1, nrot // depth)):
        step(i)
        setup_passes += depth * calls
    torch.cuda.synchronize()
    ramp_steps, t_ramp = 0, time.perf_counter()
    while (time.perf_counter() - t_ramp) * 1e3 < args.ramp_ms:
        for _ in range(8):
            step(ramp_steps)
            ramp_steps += 1
        torch.cuda.synchronize()
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        del src, dst
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps, no instrumentation
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for call in calls_timed:
        call()
    ev1.record()
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / steps
    tokens_per_s = T * calls * steps / (total_ms / 1e3)

    # ---- per-kernel durations: library-recorded HIP events around each
    # kernel group of a call, same steps (averaged over groups of one name)
    nk = len(names)
    kern_us = {n: [] for n in names}
    if not args.profile_only:
        hip = _Hip()
        ev_calls = min(steps * calls, max(1, 20000 // (2 * nk)))
        evs = [[hip.event() for _ in range(2 * nk)] for _ in range(ev_calls)]
        torch.cuda.synchronize()
        for j in range(ev_calls):   # one forward call per event set
            step(warmup + j // calls, events=evs[j], call=j % calls)
        torch.cuda.synchronize()
        for j in range(ev_calls):
            for g in range(nk):
                kern_us[names[g]].append(hip.elapsed_ms(evs[j][2 * g], evs[j][2 * g + 1]) * 1e3)
        for row in evs:
            for e in row:
                hip.destroy(e)
    kern_avg = {n: (float(np.mean(v)) if v else None) for n, v in kern_us.items()}

    per_mat_codes = d * f * w.bits // 8 + (d * f // 256) * 2   # one matrix: codes + fp16 scales
    dom = cfg["kernel"]
    dom_us = kern_avg.get(dom)
    roof = None
    extra = {}

    def roofline(bound, work, unit_work):
        if not dom_us:
            return None
        if bound == "hbm":
            achieved = work / (dom_us * 1e-6) / 1e9
            peak, unit, probed = HBM_PEAK_GBS, "GB/s", probes.get("hbm_read_gbs") if probes else None
        else:
            achieved = work / (dom_us * 1e-6) / 1e12
            peak, unit, probed = BF16_MFMA_PEAK_TFLOPS, "TFLOP/s", probes.get("mfma_bf16_tflops") if probes else None
        r = {"kernel": dom, "bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
             "frac": round(achieved / peak, 4), "traffic": _traffic_from_profiles(dom, name),
             unit_work: work, "avg_us": round(dom_us, 3)}
        if probed:
            r["probed_peak"] = probed
            r["frac_of_probed"] = round(achieved / probed, 4)
        return r

    if name in ("decode", "mtp_verify"):
        # gate and up codes + scales of the distinct experts the call's tokens
        # need, plus the shared one (logits and activations are a few KB and
        # are left out); for T > 1 the distinct count is read back from the
        # routing of every (input batch, layer) the steps cycle through
        n_exp = k + 1
        if T > 1:
            uniq = []
            for i in range(min(n_in, warmup + steps)):
                ro = [{"topk_idx": torch.empty((T, k), dtype=torch.int32, device=dev)} for _ in range(depth)]
                step(i, route_outs=ro)
                torch.cuda.synchronize()
                uniq += [len(np.unique(r["topk_idx"].cpu().numpy())) for r in ro]
            n_exp = float(np.mean(uniq)) + 1
        roof = roofline("hbm", n_exp * 2 * per_mat_codes, "algorithmic_bytes")
        layer_bytes_alg = n_exp * 3 * per_mat_codes + E * d * 4 + T * d * 2 + T * d * 4
        extra["layer_hbm_frac"] = round(depth * calls * layer_bytes_alg / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                        4)
        if probes:
            extra["layer_frac_of_probed_read"] = round(depth * calls * layer_bytes_alg / (ms_per_step * 1e-3) / 1e9
                                                       / probes["hbm_read_gbs"], 4)
        if name == "decode":
            metric = "MoE-layer tokens/s (decode T=1, full-size 3-bit layer)"
            wl = "decode layer: E=512 top-10 + 1 shared, d=2048, f=768, 3-bit blocks, T=1"
        else:
            metric = "MTP verify token-rows/s (T=5 through 48 full-size 3-bit layers)"
            wl = "MTP verify: T=5 through 48 layers of E=512 top-10 + 1 shared, d=2048, f=768, 3-bit blocks"
            if roof:
                roof["distinct_experts_per_layer"] = round(n_exp - 1, 2)
        dtype = "int4-dot/fp32"
    elif name == "zipf_prefill":
        # routing of every chunk, read back once: resident picks (the only
        # routed pairs computed), misses and per-expert load
        mask_np = res.mask_np
        res_bits = np.unpackbits(mask_np.view(np.uint8), bitorder="little")[:E].astype(bool)
        hits, loads, online = [], [], []
        acc = torch.zeros(E, dtype=torch.int64, device=dev)          # running popularity
        learnt = torch.zeros_like(res.mask)                           # resident set learnt from earlier chunks
        for c in range(calls):
            ro = [{"topk_idx": torch.empty((T, k), dtype=torch.int32, device=dev),
                   "counts": torch.empty(E, dtype=torch.int32, device=dev)}]
            step(warmup, route_outs=ro, call=c)
            torch.cuda.synchronize()
            idx = ro[0]["topk_idx"].cpu().numpy()
            cnt = ro[0]["counts"].cpu().numpy()
            hits.append(int(res_bits[idx].sum()))
            loads.append(float(cnt.max()) / (T * k / E))
            if c > 0:
                lbits = np.unpackbits(learnt.cpu().numpy().view(np.uint8), bitorder="little")[:E].astype(bool)
                online.append(float(lbits[idx].mean()))
            brx.counts_accumulate(acc, ro[0]["counts"], E, stream=stream)
            brx.resident_topn(acc, E, int(res_bits.sum()), learnt, stream=stream)
            torch.cuda.synchronize()
        # useful gate+up flops of the resident routed and the T shared token-expert pairs, per launch
        roof = roofline("mfma", 2.0 * (float(np.mean(hits)) + T) * d * (2 * f), "algorithmic_flops")
        n_res = int(res_bits.sum())
        metric = "MoE-layer tokens/s (32K-token Zipf-skewed prefill, 165-expert resident mask, 3-bit layer)"
        wl = (f"Zipf(1.1) prefill: 32768 tokens in {calls} chunks of {T}, E=512 top-10 + 1 shared, d=2048, f=768, "
              f"3-bit blocks, {n_res} resident experts")
        dtype = "bf16-mfma/fp32"
        layer_flops = 2.0 * (float(np.mean(hits)) + T) * 3 * d * f * calls
        extra["layer_mfma_frac"] = round(layer_flops / (ms_per_step * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)
        if not args.profile_only:
            extra["coprocess"] = _coprocess_timing(res, sh, ws, ws_bytes, dev, step_layer=warmup % nrot)
        extra["routing"] = {"hit_rate": round(sum(hits) / (calls * T * k), 4),
                            "misses_per_chunk": round(T * k - float(np.mean(hits)), 1),
                            "max_over_mean_load": round(float(np.max(loads)), 2),
                            "online_resident_hit_rate": round(float(np.mean(online)), 4) if online else None,
                            "static_hit_rate_same_chunks": round(sum(hits[1:]) / ((calls - 1) * T * k), 4)
                            if calls > 1 else None}
    else:
        # useful gate+up flops of the T*k routed and T shared token-expert pairs
        roof = roofline("mfma", 2.0 * (T * k + T) * d * (2 * f), "algorithmic_flops")
        layer_flops = 2.0 * (T * k + T) * 3 * d * f
        extra["layer_mfma_frac"] = round(layer_flops / (ms_per_step * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)
        metric = "MoE-layer tokens/s (4096-token prefill chunk, 2-bit layer)"
        wl = "prefill chunk: E=512 top-10 + 1 shared, d=2048, f=768, 2-bit blocks, T=4096"
        dtype = "bf16-mfma/fp32"

    cpu = None
    if not args.no_cpu_baseline and not args.profile_only:
        _log(f"{name}: timed, CPU baseline next")
        cpu = _cpu_baseline(name, w, args.cpu_sample_s, bias=None if res.bias is None else res.bias.cpu().numpy(),
                            mask=res.mask_np)
    rec = {
        "metric": metric,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "steps": steps,
        "warmup": warmup,
        "setup_layer_passes": setup_passes,
        "ramp_steps": ramp_steps,
        "ms_per_step": round(ms_per_step, 5),
        "dtype": dtype,
        "config": {"workload": wl, "tokens_per_step": T * calls, "layers_per_step": depth,
                   "resident_layers_rotated": nrot, "parallelism": "single GPU"},
        "roofline": roof,
        "kernels_us": {n: (round(v, 3) if v is not None else None) for n, v in kern_avg.items()},
        "cpu_baseline": cpu,
    }
    rec.update(extra)
    return rec


def _coprocess_timing(res, sh, ws, ws_bytes, dev, step_layer):
    """The masked prompt with its misses computed on the host and merged
    (strata_moe_forward_coprocess), chunk by chunk through one resident
    layer, and the host's share alone (strata_moe_host_misses on the first
    chunk's miss list)."""
    import torch
    import bit_routed_expert_amd as brx
    import oracle
    import synth
    w = res.w
    T, calls, k, d = res.T, res.calls, w.top_k, w.d_model
    codes = np.empty(w.experts_total * w.code_bytes_per_expert, dtype=np.uint8)
    synth.layer_codes_into(w, step_layer, codes.ctypes.data)
    scales = synth.layer_scales(w, step_layer)
    layer = res.layers[step_layer]
    cap = T * k
    hnb = brx.host_workspace_bytes(sh, T, cap)
    hws = torch.empty(hnb, dtype=torch.uint8, pin_memory=True)
    threads = oracle._threads()
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    resid = torch.empty((T, d), dtype=torch.float32, device=dev)
    mte = torch.empty((cap, 2), dtype=torch.int32, device=dev)
    mw = torch.empty(cap, dtype=torch.float32, device=dev)
    mc = torch.zeros(1, dtype=torch.int32, device=dev)
    aux = torch.cuda.Stream()
    times = []
    for rep in range(2):   # the first pass is untimed
        torch.cuda.synchronize()
        t0 = time.time()
        for c in range(calls):
            brx.forward_coprocess(sh, [layer], [(codes, scales, w.bits)], res.xs[c % res.n_in], brx.X_BF16, T, y, ws,
                                  ws_bytes, hws, hnb, threads, mte, mw, cap, mc, resid_out=resid, aux_stream=aux)
        torch.cuda.synchronize()
        times.append(time.time() - t0)
    # the host's share alone: chunk 0's misses (its miss list from a plain masked forward)
    brx.forward(sh, [layer], res.xs[0], brx.X_BF16, T, y, ws, ws_bytes, miss_te=mte, miss_w=mw, miss_cap=cap,
                miss_count=mc)
    torch.cuda.synchronize()
    n = int(mc.cpu()[0])
    te, gw = mte[:n].cpu().numpy(), mw[:n].cpu().numpy()
    u = synth.bf16_to_f32(res.xs[0].cpu().numpy().view(np.uint16))
    y_add = np.empty((T, d), np.float32)
    hws_np = np.empty(brx.host_workspace_bytes(sh, T, n), np.uint8)
    t0 = time.time()
    brx.host_misses(sh, codes, scales, w.bits, u, T, te, gw, n, y_add, hws_np, hws_np.nbytes, threads)
    host_s = time.time() - t0
    macs = n * 3 * d * w.d_ff
    return {"ms_per_prompt": round(times[-1] * 1e3, 2), "tokens_per_s": round(T * calls / times[-1], 1),
            "host_misses_ms_per_chunk": round(host_s * 1e3, 2), "misses_chunk0": n,
            "host_gflops": round(2 * macs / host_s / 1e9, 1), "host_isa": brx.host_isa(), "host_threads": threads, "cpu_topology": _cpu_topology(),
            "what": "each chunk: GPU routing and resident experts, miss list and input copied to the host on a "
                    "second stream, host FFNs of the misses from host-resident packed weights, merged on the GPU"}


def main():
    args = parse()
    if args.traffic_from:
        traffic_summary(args)
        return
    if args.counters_from:
        counters_summary(args)
        return
    if args.stats_from:
        stats_summary(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the MoE layer path here is single-GPU "
              "(expert-parallel sharding is a design note, not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda", 0)
    t0 = time.time()
    probes = None
    if not args.no_probes and not args.profile_only:
        probes = probe_peaks(dev)
        _log(f"probes {probes['hbm_read_gbs']} GB/s, {probes['mfma_bf16_tflops']} TFLOP/s")
    todo = [args.workload] if args.workload != "all" else ["decode"] + [wl for _, wl in SUB_RECORDS]
    recs = {}
    cache = {}
    for name in todo:
        cfg = WORKLOADS[name]
        steps = args.steps if args.steps is not None else default_steps(name)
        warmup = args.warmup if args.warmup is not None else max(1, steps // 10)
        nrot = args.rotate if args.rotate is not None else cfg["rotate"]
        synth_name = cfg["synth"]
        # the verify step runs through the decode line's 48 resident layers (same shape and format)
        if name == "mtp_verify" and "decode" in cache and len(cache["decode"].layers) >= 48:
            res = cache["decode"]
            import synth
            res_v = Resident.__new__(Resident)
            res_v.__dict__.update(res.__dict__)
            wv = synth.WORKLOADS["mtp_verify"]
            res_v.w, res_v.T, res_v.calls, res_v.n_in = wv, wv.tokens_per_call, wv.calls, cfg["inputs"]
            res_v.xs = torch.from_numpy(synth.x_tokens(wv, range(cfg["inputs"] * wv.tokens), rep=1)
                                        .view(np.int16)).to(dev).view(cfg["inputs"], wv.tokens, wv.d_model)
            res = res_v
        else:
            n_in = (warmup + steps) if cfg["inputs"] is None else cfg["inputs"]
            res = Resident(synth_name, nrot, n_in, dev)
        cache[name] = res
        _log(f"{name}: {len(res.layers)} resident layers ready ({time.time() - t0:.1f} s)")
        recs[name] = bench_workload(name, args, res, dev, probes, steps, warmup)
        _log(f"{name}: {recs[name]['value']} tokens/s, {recs[name]['ms_per_step']} ms/step ({time.time() - t0:.1f} s)")
        if name == "prefill_2bit":
            cache.clear()
    setup_s = time.time() - t0

    head = recs[todo[0]]
    line = {
        "metric": METRIC if args.workload == "all" else head["metric"],
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": head["warmup"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
    }
    for key in ("setup_layer_passes", "ramp_steps", "kernels_us", "layer_hbm_frac", "layer_frac_of_probed_read",
                "layer_mfma_frac", "routing", "coprocess"):
        if key in head:
            line[key] = head[key]
    if args.workload == "all":
        line["workloads"] = {label: recs[name] for label, name in SUB_RECORDS}
    line["probes"] = probes
    line["wall_s"] = round(setup_s, 1)
    print(json.dumps(line))


class _Hip:
    """hipEvent create / elapsed / destroy through the HIP runtime (events are
    recorded by the library on the stream its kernels run on)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        # same SONAME as the runtime torch already loaded, so events and streams agree
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = self.ct.c_void_p()
        if self.lib.hipEventCreate(self.ct.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.lib.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


# ------------------------------------------------------------ counter files
def _kernel_sources(kernel, workload):
    if kernel == WORKLOADS[workload]["kernel"]:
        return WORKLOADS[workload]["symbol"], WORKLOADS[workload]["sources"]
    return COUNTER_KERNELS[kernel]


def _traffic_path(kernel, workload):
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")


def _traffic_from_profiles(kernel, workload):
    """HBM bytes per launch of a kernel from the committed counter summary,
    only if it was taken on the current kernel source."""
    path = _traffic_path(kernel, workload)
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("TRAFFIC "):
            rec = json.loads(line[len("TRAFFIC "):])
            if rec.get("source_sha256") != source_hash(_kernel_sources(kernel, workload)[1]):
                return None
            return rec["bytes_per_launch"]
    return None


def _counter_rows(path):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _per_dispatch(rows, counter, symbol):
    """Counter value per dispatch of kernels named `symbol` (summed over the
    rows a dispatch has for that counter)."""
    by = {}
    for r in rows:
        if r["Counter_Name"] == counter and symbol in r["Kernel_Name"]:
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            by[key] = by.get(key, 0.0) + float(r["Counter_Value"])
    return list(by.values())


def _durations_ns(rows, symbol):
    """End - start of each dispatch of `symbol`, when the CSV has timestamps."""
    by = {}
    for r in rows:
        if symbol in r["Kernel_Name"] and r.get("Start_Timestamp") and r.get("End_Timestamp"):
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            by[key] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return list(by.values())


def traffic_summary(args):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of a kernel, scaled by what
    the same counters read for the calibration copy (which moves exactly MIB
    MiB each way)."""
    if not args.copy_calibration:
        sys.exit("--traffic-from needs the --copy-calibration size of the profiled run")
    wl = args.workload if args.workload != "all" else "decode"
    kernel = args.traffic_kernel or WORKLOADS[wl]["kernel"]
    symbol, sources = _kernel_sources(kernel, wl)
    copy_bytes = args.copy_calibration * (1 << 20)
    out = {}
    for counter, path in zip(("FETCH_SIZE", "WRITE_SIZE"), args.traffic_from):
        rows = _counter_rows(path)
        cp = _per_dispatch(rows, counter, COPY_SYMBOL)
        kv = _per_dispatch(rows, counter, symbol)
        if not cp or not kv:
            sys.exit(f"{path}: no {counter} rows for the calibration copy or {symbol}")
        factor = copy_bytes / (float(np.median(cp)) * 1024.0)
        out[counter] = dict(kib_per_dispatch=float(np.mean(kv)), dispatches=len(kv),
                            copy_kib=float(np.median(cp)), factor=factor,
                            bytes=float(np.mean(kv)) * 1024.0 * factor)
    rec = dict(kernel=kernel, symbol=symbol, workload=wl,
               fetch_bytes=round(out["FETCH_SIZE"]["bytes"]), write_bytes=round(out["WRITE_SIZE"]["bytes"]),
               bytes_per_launch=round(out["FETCH_SIZE"]["bytes"] + out["WRITE_SIZE"]["bytes"]),
               fetch_factor=round(out["FETCH_SIZE"]["factor"], 4), write_factor=round(out["WRITE_SIZE"]["factor"], 4),
               copy_mib=args.copy_calibration, source_sha256=source_hash(sources))
    path = _traffic_path(kernel, wl)
    kflag = f" --traffic-kernel {kernel}" if args.traffic_kernel else ""
    with open(path, "w") as fh:
        fh.write(f"# HBM traffic of `{kernel}` ({symbol}, {wl} workload)\n\n")
        fh.write("Counters: rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE (KiB per dispatch), one run each, on\n"
                 f"`bench.py --workload {wl} --profile-only --copy-calibration {args.copy_calibration}`;"
                 " every value is scaled by\nexpected / measured for the calibration copy"
                 f" (`torch.mul(src, 1.0, out=dst)`, {args.copy_calibration} MiB each way).\n\n")
        fh.write("| counter | kernel KiB/dispatch | dispatches | copy KiB | factor | bytes/launch |\n|---|---|---|---|---|---|\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            o = out[c]
            fh.write(f"| {c} | {o['kib_per_dispatch']:.1f} | {o['dispatches']} | {o['copy_kib']:.1f} | "
                     f"{o['factor']:.4f} | {o['bytes']:.0f} |\n")
        fh.write("\nCommands (from the repository root; each counter pass in its own run):\n\n```\n")
        for c, tag in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
            fh.write(f"cd /tmp && TMPDIR=/tmp timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv "
                     f"-d $REPO/gpurun_out/pmc_{wl}_{tag} -o run -- python3 $REPO/bench.py --workload {wl} "
                     f"--steps 20 --warmup 4 --profile-only --copy-calibration {args.copy_calibration}\n")
        fh.write(f"python3 bench.py --workload {wl}{kflag} --copy-calibration {args.copy_calibration} "
                 f"--traffic-from gpurun_out/pmc_{wl}_fetch/run_counter_collection.csv "
                 f"gpurun_out/pmc_{wl}_write/run_counter_collection.csv\n```\n\n")
        fh.write("TRAFFIC " + json.dumps(rec) + "\n")
    print(json.dumps(rec))


def stats_summary(args):
    """Kernel durations of a profiled run (rocprofv3 --kernel-trace --stats)."""
    wl = args.workload if args.workload != "all" else "decode"
    rows = _counter_rows(args.stats_from)
    path = os.path.join(ROOT, "profiles", f"kernel_stats_{wl}.md")
    with open(path, "w") as fh:
        fh.write(f"# Kernel durations under rocprofv3 ({wl} workload)\n\n")
        fh.write("Command (from the repository root, `$REPO` = its absolute path):\n\n```\n")
        fh.write((args.stats_cmd or "(not recorded)") + "\n")
        fh.write(f"python3 bench.py --workload {wl} --stats-from <that run's run_kernel_stats.csv>\n```\n\n")
        fh.write("| kernel | calls | avg us | min us | max us | % |\n|---|---|---|---|---|---|\n")
        for r in rows:
            name = r["Name"].replace("|", "\\|")
            if len(name) > 90:
                name = name[:87] + "..."
            fh.write(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |\n")
        srcs = sorted(set(sum((cfg["sources"] for cfg in WORKLOADS.values()), [])))
        fh.write("\nKERNELSTATS " + json.dumps(dict(workload=wl, source_sha256=source_hash(srcs))) + "\n")
    print(path)


MFMA_COUNTERS = ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_BUSY_CYCLES", "SQ_WAVES",
                 "GRBM_GUI_ACTIVE", "GRBM_COUNT")


def counters_summary(args):
    """Matrix-core utilisation of the larger-batch kernels from one
    rocprofv3 --pmc run of MFMA_COUNTERS: per dispatch, the MFMA
    instructions, matrix-core busy cycles, VALU instructions and the GPU's
    active cycles, and ratios of them."""
    wl = args.workload if args.workload != "all" else "prefill_2bit"
    rows = _counter_rows(args.counters_from)
    kernels = [("gemm_gateup", "gemm_gateup_kernel"), ("gemm_down", "gemm_down_kernel"),
               ("route_logits", "route_logits_mfma_kernel")]
    out = {}
    for label, symbol in kernels:
        vals = {c: _per_dispatch(rows, c, symbol) for c in MFMA_COUNTERS}
        if not vals["SQ_INSTS_MFMA"]:
            continue
        m = {c: float(np.mean(v)) if v else None for c, v in vals.items()}
        r = {"dispatches": len(vals["SQ_INSTS_MFMA"]), **{c: m[c] for c in MFMA_COUNTERS}}
        if m["SQ_INSTS_MFMA"]:
            r["mfma_busy_cycles_per_mfma"] = m["SQ_VALU_MFMA_BUSY_CYCLES"] / m["SQ_INSTS_MFMA"]
            r["valu_insts_per_mfma"] = m["SQ_INSTS_VALU"] / m["SQ_INSTS_MFMA"]
        if m["GRBM_GUI_ACTIVE"]:
            # GRBM_GUI_ACTIVE is summed over the 8 XCDs; 1024 SIMDs (256 CUs x 4)
            cyc = m["GRBM_GUI_ACTIVE"] / 8.0
            r["gpu_cycles"] = cyc
            r["mfma_busy_frac_of_simd_cycles"] = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * 1024.0)
            durs = _durations_ns(rows, symbol)
            if durs:
                r["duration_us"] = float(np.mean(durs)) / 1e3
                r["clock_ghz"] = cyc / float(np.mean(durs))
        out[label] = r
    srcs = source_hash(["common.hpp", "mfma.hpp", "gemm_impl.hpp", "gemm_gu2.hip", "gemm_dn2.hip", "gemm_gu3.hip",
                        "gemm_dn3.hip", "route.hip"])
    path = os.path.join(ROOT, "profiles", f"counters_mfma_{wl}.md")
    with open(path, "w") as fh:
        fh.write(f"# Matrix-core counters of the larger-batch kernels ({wl} workload)\n\n")
        fh.write("One rocprofv3 --pmc pass of " + ", ".join(MFMA_COUNTERS) + ", means per dispatch.\n"
                 "GRBM_GUI_ACTIVE is summed over the 8 XCDs (cycles = value / 8); the busy fraction divides\n"
                 "SQ_VALU_MFMA_BUSY_CYCLES by cycles x 1024 SIMDs.\n\n")
        fh.write("| kernel | dispatches | SQ_INSTS_MFMA | MFMA busy cycles | busy/MFMA | VALU/MFMA | GPU cycles | "
                 "busy frac | us (profiled) | GHz |\n|---|---|---|---|---|---|---|---|---|---|\n")
        for label, r in out.items():
            fh.write(f"| {label} | {r['dispatches']} | {r['SQ_INSTS_MFMA']:.4g} | {r['SQ_VALU_MFMA_BUSY_CYCLES']:.4g} | "
                     f"{r.get('mfma_busy_cycles_per_mfma', 0):.2f} | {r.get('valu_insts_per_mfma', 0):.2f} | "
                     f"{r.get('gpu_cycles', 0):.4g} | {r.get('mfma_busy_frac_of_simd_cycles', 0):.3f} | "
                     f"{r.get('duration_us', 0):.1f} | {r.get('clock_ghz', 0):.2f} |\n")
        fh.write("\nCommand (from the repository root):\n\n```\n")
        fh.write(f"cd /tmp && TMPDIR=/tmp timeout -s KILL 120 rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} "
                 f"--output-format csv -d $REPO/gpurun_out/pmc_{wl}_mfma -o run -- python3 $REPO/bench.py "
                 f"--workload {wl} --steps 20 --warmup 4 --profile-only\n")
        fh.write(f"python3 bench.py --workload {wl} --counters-from "
                 f"gpurun_out/pmc_{wl}_mfma/run_counter_collection.csv\n```\n\n")
        fh.write("COUNTERS " + json.dumps(dict(workload=wl, source_sha256=srcs, kernels=out)) + "\n")
    print(json.dumps(out))


# ---------------------------------------------------------------- CPU side
def _cpu_model():
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return platform.processor() or "unknown"


def _cpu_topology():
    """Sockets, cores per socket and threads per core as lscpu reports them."""
    keys = {"Socket(s):": "sockets", "Core(s) per socket:": "cores_per_socket", "Thread(s) per core:": "threads_per_core"}
    topo = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            for k, name in keys.items():
                if line.startswith(k):
                    try:
                        topo[name] = int(line.split(":", 1)[1].strip())
                    except ValueError:
                        pass
    except Exception:
        pass
    return topo


def _cpu_baseline(name, w, target_s, bias=None, mask=None):
    """The oracle (grouped evaluation: each needed expert dequantised once,
    then its tokens) on a bounded sample of the workload, with every thread
    of this job's CPU share, and once more on one thread for the decode and
    verify workloads.  Decode and verify calls carry the workload's T tokens
    through one full-size layer (a stack of 48 layers costs 48 such calls
    per step); the prefill sample is one whole 4096-token chunk."""
    import oracle
    import synth
    codes = np.empty(w.experts_total * w.code_bytes_per_expert, dtype=np.uint8)
    synth.layer_codes_into(w, 0, codes.ctypes.data)
    scales = synth.layer_scales(w, 0)
    Wr = synth.router_weights(w, 0)
    cores = oracle._threads()

    def run(tc, n_max, threads, limit_s):
        xs = synth.bf16_to_f32(synth.x_tokens(w, range(n_max * tc), rep=2))
        n = 0
        t0 = time.time()
        while n < n_max:
            oracle.moe_layer(w.bits, w.n_experts, w.top_k, w.d_model, w.d_ff, xs[n * tc:(n + 1) * tc], Wr, codes,
                             scales, bias=bias, mask=mask, grouped=True, threads=threads)
            n += 1
            if time.time() - t0 >= limit_s:
                break
        return n, time.time() - t0

    tc = w.tokens_per_call
    rec = {"unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu_model": _cpu_model(),
           "cpu_topology": _cpu_topology(), "host_cpus_visible": os.cpu_count()}
    if tc <= 8:
        n, el = run(tc, 64, cores, target_s)
        rec["value"] = round(n * tc / el / w.layers, 4)
        per = "" if w.layers == 1 else f", rate divided by the {w.layers}-layer stack depth"
        rec["sample"] = f"{n} calls of {tc} token(s) through one full-size layer ({cores} threads){per}"
        n1, el1 = run(tc, 64, 1, target_s)
        rec["single_thread"] = {"value": round(n1 * tc / el1 / w.layers, 4),
                                "sample": f"{n1} calls of {tc} token(s), 1 thread{per}"}
    else:
        n, el = run(tc, 1, cores, 0.0)
        rec["value"] = round(tc / el, 2)
        rec["sample"] = f"one whole {tc}-token call through one full-size layer ({cores} threads, {el:.1f} s)"
    return rec


if __name__ == "__main__":
    main()
