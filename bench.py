#!/usr/bin/env python3
"""Benchmark of the MI355X sparse MoE layer forward.

Default workload (the headline line; one step = one full layer forward:
router, top-k and gates, permutation, expert FFNs over packed 3-bit blocks,
shared expert, combine): the full-size decode layer -- 512 routed experts
top-10 + 1 shared, d = 2048, f = 768, 3-bit 256-element blocks, T = 1 token
of bf16 N(0,1) input, random N(0, 1/d) router.  Every step uses a new token
and the next of `--rotate` independent resident layers, so the ~0.93 GB of
codes per layer come from HBM, not from the 256 MB Infinity Cache.

`--workload mtp_verify` times the verify step of multi-token prediction:
5 tokens (1 accepted + 4 drafts) through a stack of 48 independent
full-size 3-bit layers in one call, residual stream carried between layers
(value = token-rows through the whole stack per second).  `--workload
prefill_2bit` times the 4096-token 2-bit prefill chunk (matrix-core GEMM
path).  Both are secondary lines; the decode layer is the headline.

Prints one JSON line: tokens/s, the dominant kernel's roofline fraction
(kernel time from HIP events the library records around that kernel, on the
stream the kernel runs on) with its HBM bytes from committed rocprofv3
counter runs when they were taken on the current kernel source, and the CPU
oracle's rate on a bounded sample.

`--copy-calibration MIB` adds a plain fp32 elementwise copy of known size to
the run (reference kernel for the byte counters); `--traffic-from FETCH
WRITE` turns the counter CSVs of two such runs (rocprofv3 --pmc FETCH_SIZE,
then WRITE_SIZE) into profiles/traffic_<kernel>_<workload>.md.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "bit_routed_expert_amd", "csrc")

# Per workload: the dominant kernel (library kernel name and the symbol
# rocprofv3 reports) and the source files that define it.
WORKLOADS = {
    "decode": dict(kernel="route_gemv_gateup", symbol="gemv_gateup_small_kernel", rotate=48, inputs=None,
                   sources=["common.hpp", "routing.hpp", "gemv_impl.hpp", "gemv_gu3.hip"]),
    "mtp_verify": dict(kernel="route_gemv_gateup", symbol="gemv_gateup_multi_kernel", rotate=48, inputs=4,
                       sources=["common.hpp", "routing.hpp", "gemv_impl.hpp", "gemv_gu3.hip"]),
    "prefill_2bit": dict(kernel="gemm_gateup", symbol="gemm_gateup_kernel", rotate=2, inputs=4,
                         sources=["common.hpp", "mfma.hpp", "gemm_impl.hpp", "gemm_gu2.hip"]),
    # one step = the whole 32K prompt: its eight 4096-token chunks, in order
    "zipf_prefill": dict(kernel="gemm_gateup", symbol="gemm_gateup_kernel", rotate=2, inputs=8,
                         sources=["common.hpp", "mfma.hpp", "gemm_impl.hpp", "gemm_gu3.hip"]),
}
COPY_SYMBOL = "MulFunctor"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps (default 2000 decode, 200 prefill, 100 verify, 30 Zipf prompts)")
    p.add_argument("--warmup", type=int, default=None, help="untimed steps (default steps / 10)")
    p.add_argument("--rotate", type=int, default=None, help="independent resident layers cycled through")
    p.add_argument("--cpu-sample-s", type=float, default=12.0, help="target seconds of oracle work")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--profile-only", action="store_true", help="skip the CPU baseline and event pass")
    p.add_argument("--workload", default="decode", choices=sorted(WORKLOADS),
                   help="decode (the headline line), the 48-layer T=5 verify step, the 4096-token 2-bit "
                        "prefill chunk or the 32K-token Zipf-skewed prefill with the 165-expert resident mask")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="run a plain fp32 elementwise copy of MIB MiB (read + write) 5 times before the warmup")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write the traffic summary from two rocprofv3 counter CSVs of a --copy-calibration run")
    a = p.parse_args()
    if a.steps is None:
        a.steps = {"decode": 2000, "mtp_verify": 100, "zipf_prefill": 30}.get(a.workload, 200)
    if a.warmup is None:
        a.warmup = max(1, a.steps // 10)
    if a.rotate is None:
        a.rotate = WORKLOADS[a.workload]["rotate"]
    return a


def source_hash(workload):
    h = hashlib.sha256()
    for name in WORKLOADS[workload]["sources"]:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def main():
    args = parse()
    if args.traffic_from:
        traffic_summary(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the MoE layer path here is single-GPU "
              "(expert-parallel sharding is a design note, not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_routed_expert_amd as brx
    import synth

    cfg = WORKLOADS[args.workload]
    w = synth.WORKLOADS[args.workload]
    T = w.tokens_per_call
    E, k, d, f = w.n_experts, w.top_k, w.d_model, w.d_ff
    sh = brx.shape(E, k, d, f, w.bits)
    dev = torch.device("cuda", 0)

    # ---- resident inputs: `rotate` independent layers + the token batches
    calls = w.calls                     # forward calls per step (the prompt's chunks)
    bias = torch.from_numpy(synth.zipf_bias(w)).to(dev) if w.zipf_s > 0 else None
    mask_np = synth.resident_mask(w) if w.resident else None
    mask = torch.from_numpy(mask_np.view(np.int32)).to(dev) if mask_np is not None else None
    nrot = args.rotate
    layer_bytes = w.experts_total * w.code_bytes_per_expert
    pinned = torch.empty(layer_bytes, dtype=torch.uint8, pin_memory=True)
    layers = []
    t0 = time.time()
    for l in range(nrot):
        synth.layer_codes_into(w, l, pinned.data_ptr())
        codes = torch.empty(layer_bytes, dtype=torch.uint8, device=dev)
        codes.copy_(pinned, non_blocking=False)
        scales = torch.from_numpy(synth.layer_scales(w, l).view(np.int16)).to(dev)
        wr = torch.from_numpy(synth.router_weights(w, l)).to(dev)
        layers.append(brx.LayerData(router_w=wr, codes=codes, scales=scales, router_bias=bias, resident_mask=mask))
    del pinned
    n_step = args.warmup + args.steps
    n_in = n_step if cfg["inputs"] is None else cfg["inputs"]   # a new token per decode step
    if calls > 1 and n_in % calls:
        sys.exit("the input batches must hold whole prompts")
    xs = torch.from_numpy(synth.x_tokens(w, range(n_in * T), rep=1).view(np.int16)).to(dev).view(n_in, T, d)
    setup_s = time.time() - t0

    depth = w.layers                    # layers one step runs through (48 for the verify stack)
    if nrot < depth:
        sys.exit(f"--rotate must be at least the stack depth {depth}")
    ws_bytes = brx.workspace_bytes(sh, T, depth)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    resid = torch.empty((T, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    names = brx.kernel_names(sh, T)
    miss = {}
    if mask is not None:   # miss list of every (token, non-resident pick); T*k entries never overflow
        cap = T * k
        miss = dict(miss_te=torch.empty((cap, 2), dtype=torch.int32, device=dev),
                    miss_w=torch.empty(cap, dtype=torch.float32, device=dev), miss_cap=cap,
                    miss_count=torch.zeros(depth, dtype=torch.int32, device=dev))

    def stack(i):
        return [layers[(i * depth + j) % nrot] for j in range(depth)]

    def step(i, events=None, route_outs=None, call=None):
        for c in (range(calls) if call is None else [call]):
            brx.forward(sh, stack(i), xs[(i * calls + c) % n_in], brx.X_BF16, T, y, ws, ws_bytes, resid_out=resid,
                        route_outs=route_outs, events=events, stream=stream, **miss)

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        del src, dst
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps, no instrumentation
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(args.warmup, n_step):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / args.steps
    tokens_per_s = T * calls * args.steps / (total_ms / 1e3)

    # ---- per-kernel durations: library-recorded HIP events around each kernel, same steps
    # (every layer of a stack: the i-th kernel group of layer l is group l*nk + i)
    nk = len(names)
    kern_us = {n: [] for n in names}
    if not args.profile_only:
        hip = _Hip()
        ev_calls = min(args.steps * calls, max(1, 20000 // (2 * nk * depth)))
        evs = [[hip.event() for _ in range(2 * nk * depth)] for _ in range(ev_calls)]
        torch.cuda.synchronize()
        for j in range(ev_calls):   # one forward call per event set
            step(args.warmup + j // calls, events=evs[j], call=j % calls)
        torch.cuda.synchronize()
        for j in range(ev_calls):
            for g in range(nk * depth):
                kern_us[names[g % nk]].append(hip.elapsed_ms(evs[j][2 * g], evs[j][2 * g + 1]) * 1e3)
        for row in evs:
            for e in row:
                hip.destroy(e)
    kern_avg = {n: (float(np.mean(v)) if v else None) for n, v in kern_us.items()}

    per_mat_codes = d * f * w.bits // 8 + (d * f // 256) * 2   # one matrix: codes + fp16 scales
    dom = cfg["kernel"]
    dom_us = kern_avg.get(dom)
    roof = None
    if args.workload in ("decode", "mtp_verify"):
        # gate and up codes + scales of the distinct experts the call's tokens
        # need, plus the shared one (logits and activations are a few KB and
        # are left out); for T > 1 the distinct count is read back from the
        # routing of every (input batch, layer) the steps cycle through
        n_exp = k + 1
        if T > 1:
            uniq = []
            for i in range(min(n_in, n_step)):
                ro = [{"topk_idx": torch.empty((T, k), dtype=torch.int32, device=dev)} for _ in range(depth)]
                step(i, route_outs=ro)
                torch.cuda.synchronize()
                uniq += [len(np.unique(r["topk_idx"].cpu().numpy())) for r in ro]
            n_exp = float(np.mean(uniq)) + 1
        dom_bytes = n_exp * 2 * per_mat_codes
        if dom_us:
            achieved = dom_bytes / (dom_us * 1e-6) / 1e9
            roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": _traffic_from_profiles(args.workload), "algorithmic_bytes": dom_bytes,
                    "avg_us": round(dom_us, 3)}
        layer_bytes_alg = n_exp * 3 * per_mat_codes + E * d * 4 + T * d * 2 + T * d * 4
        if args.workload == "decode":
            metric = "MoE-layer tokens/s (decode T=1, full-size 3-bit layer)"
            wl = "decode layer: E=512 top-10 + 1 shared, d=2048, f=768, 3-bit blocks, T=1"
        else:
            metric = "MTP verify token-rows/s (T=5 through 48 full-size 3-bit layers)"
            wl = "MTP verify: T=5 through 48 layers of E=512 top-10 + 1 shared, d=2048, f=768, 3-bit blocks"
            if roof:
                roof["distinct_experts_per_layer"] = round(n_exp - 1, 2)
        dtype = "int4-dot/fp32"
    elif args.workload == "zipf_prefill":
        # routing of every chunk, read back once: resident picks (the only
        # routed pairs computed), misses and per-expert load
        res_bits = np.unpackbits(mask_np.view(np.uint8), bitorder="little")[:E].astype(bool)
        hits, loads, online = [], [], []
        acc = torch.zeros(E, dtype=torch.int64, device=dev)          # running popularity
        learnt = torch.zeros_like(mask)                               # resident set learnt from earlier chunks
        for c in range(calls):
            ro = [{"topk_idx": torch.empty((T, k), dtype=torch.int32, device=dev),
                   "counts": torch.empty(E, dtype=torch.int32, device=dev)}]
            step(args.warmup, route_outs=ro, call=c)
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
        flops = 2.0 * (float(np.mean(hits)) + T) * d * (2 * f)
        if dom_us:
            achieved = flops / (dom_us * 1e-6) / 1e12
            roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4),
                    "traffic": _traffic_from_profiles(args.workload), "algorithmic_flops": flops,
                    "avg_us": round(dom_us, 3)}
        n_res = int(res_bits.sum())
        layer_bytes_alg = (n_res + 1) * 3 * per_mat_codes + E * d * 4 + T * d * 2 + T * d * 4
        metric = "MoE-layer tokens/s (32K-token Zipf-skewed prefill, 165-expert resident mask, 3-bit layer)"
        wl = (f"Zipf(1.1) prefill: 32768 tokens in {calls} chunks of {T}, E=512 top-10 + 1 shared, d=2048, f=768, "
              f"3-bit blocks, {n_res} resident experts")
        dtype = "bf16-mfma/fp32"
        zipf_stats = {"hit_rate": round(sum(hits) / (calls * T * k), 4),
                      "misses_per_chunk": round(T * k - float(np.mean(hits)), 1),
                      "max_over_mean_load": round(float(np.max(loads)), 2),
                      "online_resident_hit_rate": round(float(np.mean(online)), 4) if online else None,
                      "static_hit_rate_same_chunks": round(sum(hits[1:]) / ((calls - 1) * T * k), 4)
                      if calls > 1 else None}
    else:
        # useful gate+up flops of the T*k routed and T shared token-expert pairs
        flops = 2.0 * (T * k + T) * d * (2 * f)
        if dom_us:
            achieved = flops / (dom_us * 1e-6) / 1e12
            roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4),
                    "traffic": _traffic_from_profiles(args.workload), "algorithmic_flops": flops,
                    "avg_us": round(dom_us, 3)}
        layer_bytes_alg = (E + 1) * 3 * per_mat_codes + E * d * 4 + T * d * 2 + T * d * 4
        metric = "MoE-layer tokens/s (4096-token prefill chunk, 2-bit layer)"
        wl = "prefill chunk: E=512 top-10 + 1 shared, d=2048, f=768, 2-bit blocks, T=4096"
        dtype = "bf16-mfma/fp32"

    cpu = None
    if not args.no_cpu_baseline and not args.profile_only:
        cpu = _cpu_baseline(w, args.cpu_sample_s, bias=None if bias is None else bias.cpu().numpy(), mask=mask_np)

    rec = {
        "metric": metric,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": wl, "tokens_per_step": T * calls, "layers_per_step": depth,
                   "resident_layers_rotated": nrot, "parallelism": "single GPU"},
        "roofline": roof,
        "layer_hbm_frac": round(depth * calls * layer_bytes_alg / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernels_us": {n: (round(v, 3) if v is not None else None) for n, v in kern_avg.items()},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    if args.workload == "zipf_prefill":
        rec["routing"] = zipf_stats
    print(json.dumps(rec))


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


def _traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{WORKLOADS[workload]['kernel']}_{workload}.md")


def _traffic_from_profiles(workload):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, only if it was taken on the current kernel source."""
    path = _traffic_path(workload)
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("TRAFFIC "):
            rec = json.loads(line[len("TRAFFIC "):])
            if rec.get("source_sha256") != source_hash(workload):
                return None
            return rec["bytes_per_launch"]
    return None


def _counter_rows(path):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def traffic_summary(args):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the dominant kernel,
    scaled by what the same counters read for the calibration copy (which
    moves exactly MIB MiB each way)."""
    if not args.copy_calibration:
        sys.exit("--traffic-from needs the --copy-calibration size of the profiled run")
    cfg = WORKLOADS[args.workload]
    copy_bytes = args.copy_calibration * (1 << 20)
    out = {}
    for counter, path in zip(("FETCH_SIZE", "WRITE_SIZE"), args.traffic_from):
        rows = [r for r in _counter_rows(path) if r["Counter_Name"] == counter]
        cp = [float(r["Counter_Value"]) for r in rows if COPY_SYMBOL in r["Kernel_Name"]]
        kv = [float(r["Counter_Value"]) for r in rows if cfg["symbol"] in r["Kernel_Name"]]
        if not cp or not kv:
            sys.exit(f"{path}: no {counter} rows for the calibration copy or {cfg['symbol']}")
        factor = copy_bytes / (float(np.median(cp)) * 1024.0)
        out[counter] = dict(kib_per_dispatch=float(np.mean(kv)), dispatches=len(kv),
                            copy_kib=float(np.median(cp)), factor=factor,
                            bytes=float(np.mean(kv)) * 1024.0 * factor)
    rec = dict(kernel=cfg["kernel"], symbol=cfg["symbol"], workload=args.workload,
               fetch_bytes=round(out["FETCH_SIZE"]["bytes"]), write_bytes=round(out["WRITE_SIZE"]["bytes"]),
               bytes_per_launch=round(out["FETCH_SIZE"]["bytes"] + out["WRITE_SIZE"]["bytes"]),
               fetch_factor=round(out["FETCH_SIZE"]["factor"], 4), write_factor=round(out["WRITE_SIZE"]["factor"], 4),
               copy_mib=args.copy_calibration, source_sha256=source_hash(args.workload))
    path = _traffic_path(args.workload)
    with open(path, "w") as fh:
        fh.write(f"# HBM traffic of `{cfg['kernel']}` ({args.workload} workload)\n\n")
        fh.write("Counters: rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE (KiB per dispatch), one run each, on\n"
                 f"`bench.py --workload {args.workload} --profile-only --copy-calibration {args.copy_calibration}`;"
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
                     f"-d $REPO/gpurun_out/pmc_{tag} -o run -- python3 $REPO/bench.py --workload {args.workload} "
                     f"--steps 20 --warmup 4 --profile-only --copy-calibration {args.copy_calibration}\n")
        fh.write(f"python3 bench.py --workload {args.workload} --copy-calibration {args.copy_calibration} "
                 "--traffic-from gpurun_out/pmc_fetch/run_counter_collection.csv "
                 "gpurun_out/pmc_write/run_counter_collection.csv\n```\n\n")
        fh.write("TRAFFIC " + json.dumps(rec) + "\n")
    print(json.dumps(rec))


def _cpu_baseline(w, target_s, bias=None, mask=None):
    """The oracle (grouped evaluation: each needed expert dequantised once,
    then its tokens) on a bounded sample of the workload's tokens, for about
    target_s seconds.  Calls carry one token (T = 1 and the prefill chunk) or
    the workload's T <= 8 token batch; a stack of `layers` layers costs
    `layers` such calls per token row."""
    import oracle
    import synth
    codes = np.empty(w.experts_total * w.code_bytes_per_expert, dtype=np.uint8)
    synth.layer_codes_into(w, 0, codes.ctypes.data)
    scales = synth.layer_scales(w, 0)
    Wr = synth.router_weights(w, 0)
    tc = w.tokens_per_call if w.tokens_per_call <= 8 else 1
    xs = synth.bf16_to_f32(synth.x_tokens(w, range(64 * tc), rep=2))
    n = 0
    t0 = time.time()
    while n < 64:
        oracle.moe_layer(w.bits, w.n_experts, w.top_k, w.d_model, w.d_ff, xs[n * tc:(n + 1) * tc], Wr, codes,
                         scales, bias=bias, mask=mask, grouped=True)
        n += 1
        if time.time() - t0 >= target_s:
            break
    el = time.time() - t0
    cores = oracle._threads()
    rate = n * tc / el / w.layers
    if w.layers == 1:
        sample = f"{n * tc} tokens in {n} calls of {tc}, one full-size layer each (grouped oracle, {cores} threads)"
    else:
        sample = (f"{n} calls of {tc} tokens through one full-size layer (grouped oracle, {cores} threads), "
                  f"rate divided by the {w.layers}-layer stack depth")
    return {"value": round(rate, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle", "sample": sample}


if __name__ == "__main__":
    main()
