#!/usr/bin/env python3
"""Benchmark of the MI355X sparse MoE layer forward.

Workload (one step = one full layer forward: router, top-k and gates,
permutation, expert FFNs over packed 3-bit blocks, shared expert, combine):
the full-size decode layer -- 512 routed experts top-10 + 1 shared,
d = 2048, f = 768, 3-bit 256-element blocks, T = 1 token of bf16 N(0,1)
input, random N(0, 1/d) router.  Every step uses a new token and the next of
`--rotate` independent resident layers, so the ~0.93 GB of codes per layer
come from HBM, not from the 256 MB Infinity Cache.

Prints one JSON line: tokens/s, the dominant kernel's HBM roofline fraction
(kernel time from HIP events recorded by the library around that kernel) and
the CPU oracle's rate on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--rotate", type=int, default=16, help="independent resident layers cycled through")
    p.add_argument("--cpu-sample-s", type=float, default=12.0, help="target seconds of oracle work")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--profile-only", action="store_true", help="skip the CPU baseline and event pass")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the MoE layer path here is single-GPU "
              "(expert-parallel sharding is a design note, not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_routed_expert_amd as brx
    import synth

    w = synth.WORKLOADS["decode"]
    T, E, k, d, f = w.tokens, w.n_experts, w.top_k, w.d_model, w.d_ff
    sh = brx.shape(E, k, d, f, w.bits)
    dev = torch.device("cuda", 0)

    # ---- resident inputs: `rotate` independent layers + one token per step
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
        layers.append(brx.LayerData(router_w=wr, codes=codes, scales=scales))
    del pinned
    n_tok = args.warmup + args.steps
    xs = torch.from_numpy(synth.x_tokens(w, range(n_tok), rep=1).view(np.int16)).to(dev)
    setup_s = time.time() - t0

    ws_bytes = brx.workspace_bytes(sh, T, 1)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    resid = torch.empty((T, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    names = brx.kernel_names(sh, T)

    def step(i, events=None):
        brx.forward(sh, [layers[i % nrot]], xs[i], brx.X_BF16, T, y, ws, ws_bytes, resid_out=resid,
                    events=events, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps, no instrumentation
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(args.warmup, n_tok):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / args.steps
    tokens_per_s = T * args.steps / (total_ms / 1e3)

    # ---- per-kernel durations: library-recorded HIP events around each kernel, same steps
    nk = len(names)
    kern_us = {n: [] for n in names}
    if not args.profile_only:
        hip = _Hip()
        evs = [[hip.event() for _ in range(2 * nk)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for j, i in enumerate(range(args.warmup, n_tok)):
            step(i, events=evs[j])
        torch.cuda.synchronize()
        for j in range(args.steps):
            for q, n in enumerate(names):
                kern_us[n].append(hip.elapsed_ms(evs[j][2 * q], evs[j][2 * q + 1]) * 1e3)
        for row in evs:
            for e in row:
                hip.destroy(e)
    kern_avg = {n: (float(np.mean(v)) if v else None) for n, v in kern_us.items()}

    # dominant kernel: the gate/up expert kernel (it also takes the top-k from
    # the logits).  Algorithmic bytes per launch: the gate and up codes + fp16
    # scales of the 11 experts one token needs (logits and activations are
    # a few KB and are left out).
    per_expert_gu = 2 * (d * f * w.bits // 8 + (d * f // 256) * 2)
    n_exp = k + 1
    dom = "route_gemv_gateup"
    dom_bytes = n_exp * per_expert_gu
    dom_us = kern_avg.get(dom)
    roof = None
    if dom_us:
        achieved = dom_bytes / (dom_us * 1e-6) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "algorithmic_bytes": dom_bytes, "avg_us": round(dom_us, 3)}
        roof["traffic"] = _traffic_from_profiles(dom)

    # whole-layer algorithmic bytes: 11 experts (3 matrices) + router + x + y
    layer_bytes_alg = n_exp * (3 * d * f * w.bits // 8 + 3 * (d * f // 256) * 2) + E * d * 4 + d * 2 + d * 4

    cpu = None
    if not args.no_cpu_baseline and not args.profile_only:
        cpu = _cpu_baseline(w, args.cpu_sample_s)

    rec = {
        "metric": "MoE-layer tokens/s (decode T=1, full-size 3-bit layer)",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4-dot/fp32",
        "data": "synthetic",
        "config": {"workload": "decode layer: E=512 top-10 + 1 shared, d=2048, f=768, 3-bit blocks, T=1",
                   "tokens_per_step": T, "resident_layers_rotated": nrot, "parallelism": "single GPU"},
        "roofline": roof,
        "layer_hbm_frac": round(layer_bytes_alg / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernels_us": {n: (round(v, 3) if v is not None else None) for n, v in kern_avg.items()},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
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


def _traffic_from_profiles(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, only if they
    were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_decode.json")
    if not os.path.exists(path):
        return None
    try:
        import hashlib
        rec = json.load(open(path))
        src = os.path.join(ROOT, "bit_routed_expert_amd", "csrc", rec["source"])
        h = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if h != rec["source_sha256"]:
            return None
        return rec["bytes_per_launch"]
    except Exception:
        return None


def _cpu_baseline(w, target_s):
    """The oracle (grouped evaluation: each needed expert dequantised once,
    then its tokens) on single decode tokens, for about target_s seconds."""
    import oracle
    import synth
    L = {}
    codes = np.empty(w.experts_total * w.code_bytes_per_expert, dtype=np.uint8)
    synth.layer_codes_into(w, 0, codes.ctypes.data)
    scales = synth.layer_scales(w, 0)
    Wr = synth.router_weights(w, 0)
    xs = synth.bf16_to_f32(synth.x_tokens(w, range(64), rep=2))
    n = 0
    t0 = time.time()
    while n < 64:
        oracle.moe_layer(w.bits, w.n_experts, w.top_k, w.d_model, w.d_ff, xs[n:n + 1], Wr, codes, scales,
                         grouped=True)
        n += 1
        if time.time() - t0 >= target_s:
            break
    el = time.time() - t0
    cores = oracle._threads()
    return {"value": round(n / el, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} decode tokens, one full-size layer each (grouped oracle, {cores} threads)"}


if __name__ == "__main__":
    main()
