"""GPU forward with the misses computed on the host CPU and merged
(strata_moe_forward_coprocess) against the oracle's UNMASKED layer: the
resident experts on the GPU plus the missed ones on the host must give the
whole layer, y_full = y_masked + sum of missed gate * y_e, within the
output bar (max-abs <= 2e-3 x RMS), and the residual stream likewise.
Routing and the miss list are those of the masked forward, bit for bit."""
from __future__ import annotations

import time

import numpy as np
import pytest

import bit_routed_expert_amd as brx
import oracle
import synth
from tests import gpu_util as G
from tests import workloads as W

pytestmark = pytest.mark.gpu


def _coprocess(w, Ls, x, T, flags=0):
    """Run strata_moe_forward_coprocess on len(Ls) layers (host copies of
    the weights are the numpy arrays themselves)."""
    import torch as t
    sh = G.shape_of(w)
    L = len(Ls)
    k, E = w.top_k, w.n_experts
    layers = [G.layer_to_dev(Lr) for Lr in Ls]
    host = [(Lr["codes"], Lr["scales"], w.bits) for Lr in Ls]
    nb = brx.workspace_bytes(sh, T, L)
    ws = t.empty(nb, dtype=t.uint8, device="cuda")
    cap = T * k
    hnb = brx.host_workspace_bytes(sh, T, cap)
    hws = t.empty(hnb, dtype=t.uint8, pin_memory=True)
    y = t.empty((T, w.d_model), dtype=t.float32, device="cuda")
    resid = t.empty((T, w.d_model), dtype=t.float32, device="cuda")
    mte = t.full((L, cap, 2), -1, dtype=t.int32, device="cuda")
    mw = t.zeros((L, cap), dtype=t.float32, device="cuda")
    mc = t.zeros(L, dtype=t.int32, device="cuda")
    ros = [dict(topk_idx=t.empty((T, k), dtype=t.int32, device="cuda"),
                counts=t.empty(E, dtype=t.int32, device="cuda")) for _ in range(L)]
    aux = t.cuda.Stream()
    t0 = time.time()
    brx.forward_coprocess(sh, layers, host, G.dev(x), brx.X_BF16, T, y, ws, nb, hws, hnb, oracle._threads(), mte, mw,
                          cap, mc, resid_out=resid, route_outs=ros, flags=flags, aux_stream=aux)
    t.cuda.synchronize()
    el = time.time() - t0
    return dict(y=y.cpu().numpy(), resid=resid.cpu().numpy(), miss_count=mc.cpu().numpy(),
                miss_te=mte.cpu().numpy(), idx=[r["topk_idx"].cpu().numpy() for r in ros], seconds=el)


@pytest.mark.parametrize("call", [0, 5])
def test_zipf_chunk_gpu_plus_host_equals_full_layer(call):
    """A 4096-token chunk of the Zipf-skewed prompt with the 165-expert
    resident mask: ~6,000 misses computed on the host."""
    w = synth.WORKLOADS["zipf_prefill"]
    T = w.tokens_per_call
    L = W.layer_data(w, 0)
    x, _ = W.draw_tokens(w, L["Wr"], L["bias"], range(call * T, (call + 1) * T))
    u = synth.bf16_to_f32(x)
    t0 = time.time()
    full = oracle.moe_layer(w.bits, w.n_experts, w.top_k, w.d_model, w.d_ff, u, L["Wr"], L["codes"], L["scales"],
                            bias=L["bias"], grouped=True)
    print(f"zipf call {call}: unmasked oracle {time.time() - t0:.1f}s", flush=True)
    got = _coprocess(w, [L], x, T)
    np.testing.assert_array_equal(got["idx"][0], full["idx"])
    nm = int(got["miss_count"][0])
    idx = full["idx"]
    res = np.unpackbits(L["mask"].view(np.uint8), bitorder="little")[: w.n_experts].astype(bool)
    assert nm == int((~res[idx]).sum()) and nm > 1000
    r = G.assert_close(got["y"], full["out"], what="GPU + host misses vs unmasked oracle")
    G.assert_close(got["resid"], u + full["out"], what="residual")
    print(f"zipf call {call}: {nm} misses on the host ({brx.host_isa()}), call {got['seconds']:.2f}s, "
          f"max-abs/RMS {r:.2e}")


@pytest.mark.parametrize("T,rep", [(1, 0), (5, 2), (8, 5), (37, 1)])
def test_full_size_layer_half_resident(T, rep):
    """Full-size 3-bit layer with every other expert resident: the one-token,
    T <= 8 and matrix-core paths."""
    w = synth.WORKLOADS["decode"]
    L = W.layer_data(w, 2)
    bits = np.zeros(w.n_experts, bool)
    bits[::2] = True
    L["mask"] = np.packbits(bits, bitorder="little").view(np.uint32)
    x, _ = W.draw_tokens(w, L["Wr"], None, range(T), rep=rep)
    u = synth.bf16_to_f32(x)
    full = oracle.moe_layer(w.bits, w.n_experts, w.top_k, w.d_model, w.d_ff, u, L["Wr"], L["codes"], L["scales"])
    print(f"case coprocess full-size T={T}", flush=True)
    got = _coprocess(w, [L], x, T)
    np.testing.assert_array_equal(got["idx"][0], full["idx"])
    G.assert_close(got["y"], full["out"])
    G.assert_close(got["resid"], u + full["out"], what="residual")


@pytest.mark.parametrize("T", [4, 20])
def test_two_layer_stack_with_masks(T):
    """Small layer, two masked layers: layer 1 consumes rmsnorm of the full
    residual stream (GPU resident experts + host misses of layer 0)."""
    w = synth.WORKLOADS["tiny"]
    masks = [np.array([0b0110_1011_1001_0111], np.uint32), np.array([0b1001_0110_0111_1010], np.uint32)]
    x0 = None
    Ls, xl = [], None
    for l in range(2):
        attempt = 0
        while True:
            Lr = W.layer_data(w, l, attempt)
            if l == 0:
                x0, _ = W.draw_tokens(w, Lr["Wr"], None, range(T), rep=19)
                xl = synth.bf16_to_f32(x0)
            u = oracle.layer_input(xl, l)
            if oracle.topk_margin(oracle.logits(u, Lr["Wr"]), w.top_k).min() >= W.MARGIN:
                break
            attempt += 1
        full = oracle.moe_layer(w.bits, w.n_experts, w.top_k, w.d_model, w.d_ff, u, Lr["Wr"], Lr["codes"],
                                Lr["scales"])
        Lr["mask"] = masks[l]
        Ls.append(Lr)
        xl = oracle.residual_add(xl, full["out"])
        y_last = full["out"]
    print(f"case coprocess two-layer small T={T}", flush=True)
    got = _coprocess(w, Ls, x0, T)
    G.assert_close(got["y"], y_last, what="last layer output")
    G.assert_close(got["resid"], xl, what="residual")
    assert got["miss_count"].min() > 0
