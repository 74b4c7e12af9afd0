"""strata_moe_forward_noalloc (the library's fixed per-device scratch in
place of a workspace) against strata_moe_forward on a fresh zeroed
workspace: calls in a row with shrinking inputs on the one-token, T <= 8
and matrix-core paths, a two-layer stack and a masked layer with its miss
list, all bit for bit; the first call against the oracle; and the refusal
of a call that needs more than the scratch holds."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import bit_routed_expert_amd as brx
import oracle
import synth
from tests import gpu_util as G
from tests import workloads as W

pytestmark = pytest.mark.gpu


def _run(noalloc, w, layers, x_dev, T, masked):
    import torch as t
    k, E, L = w.top_k, w.n_experts, len(layers)
    y = t.full((T, w.d_model), float("nan"), dtype=t.float32, device="cuda")
    resid = t.full((T, w.d_model), float("nan"), dtype=t.float32, device="cuda")
    ros = [dict(topk_idx=t.empty((T, k), dtype=t.int32, device="cuda"),
                topk_w=t.empty((T, k), dtype=t.float32, device="cuda"),
                counts=t.empty(E, dtype=t.int32, device="cuda"),
                offsets=t.empty(E + 1, dtype=t.int32, device="cuda"),
                perm=t.empty(T * k, dtype=t.int32, device="cuda"),
                pos=t.empty(T * k, dtype=t.int32, device="cuda")) for _ in range(L)]
    miss = {}
    if masked:
        cap = T * k
        miss = dict(miss_te=t.full((L, cap, 2), -1, dtype=t.int32, device="cuda"),
                    miss_w=t.zeros((L, cap), dtype=t.float32, device="cuda"), miss_cap=cap,
                    miss_count=t.zeros(L, dtype=t.int32, device="cuda"))
    sh = G.shape_of(w)
    if noalloc:
        brx.forward_noalloc(sh, layers, x_dev, brx.X_BF16, T, y, resid_out=resid, route_outs=ros, **miss)
    else:
        nb = brx.workspace_bytes(sh, T, L)
        ws = t.zeros(nb, dtype=t.uint8, device="cuda")
        brx.forward(sh, layers, x_dev, brx.X_BF16, T, y, ws, nb, resid_out=resid, route_outs=ros, **miss)
    t.cuda.synchronize()
    out = dict(y=y.cpu().numpy(), resid=resid.cpu().numpy())
    for l, r in enumerate(ros):
        for key, v in r.items():
            out[f"{key}{l}"] = v.cpu().numpy()
    for key, v in miss.items():
        if key != "miss_cap":
            out[key] = v.cpu().numpy()
    return out


def _same(a, b, what):
    assert a.keys() == b.keys()
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=f"{what}: {key}")


def test_noalloc_equals_forward_in_a_row():
    """Three calls in a row on the full-size layer, each smaller than the
    one before (T = 37 on the matrix-core path, 5, then 1), then a two-layer
    stack and a masked small layer: each equals strata_moe_forward on a
    fresh workspace bit for bit, whatever the scratch held from the call
    before."""
    w = synth.WORKLOADS["decode"]
    L0 = W.layer_data(w, 3)
    ld = G.layer_to_dev(L0)
    first = True
    for T in (37, 5, 1):
        x, _ = W.draw_tokens(w, L0["Wr"], None, range(T), rep=41)
        print(f"case no-alloc full-size T={T}", flush=True)
        a = _run(True, w, [ld], G.dev(x), T, False)
        b = _run(False, w, [ld], G.dev(x), T, False)
        _same(a, b, f"T={T}")
        if first:   # and the oracle, to the parity bar
            ref = oracle.moe_layer(w.bits, w.n_experts, w.top_k, w.d_model, w.d_ff, synth.bf16_to_f32(x), L0["Wr"],
                                   L0["codes"], L0["scales"])
            G.assert_close(a["y"], ref["out"])
            np.testing.assert_array_equal(a["topk_idx0"], ref["idx"])
            first = False
    print("case no-alloc two-layer stack T=5", flush=True)
    L1 = W.layer_data(w, 4)
    layers = [ld, G.layer_to_dev(L1)]
    x, _ = W.draw_tokens(w, L0["Wr"], None, range(5), rep=43)
    _same(_run(True, w, layers, G.dev(x), 5, False), _run(False, w, layers, G.dev(x), 5, False), "stack")
    wt = synth.WORKLOADS["tiny"]
    Lt = W.layer_data(wt, 0)
    Lt["mask"] = np.array([0b0110_1011_1001_0111], np.uint32)
    lt = G.layer_to_dev(Lt)
    for T in (20, 3):
        print(f"case no-alloc masked small layer T={T}", flush=True)
        x, _ = W.draw_tokens(wt, Lt["Wr"], None, range(T), rep=45)
        _same(_run(True, wt, [lt], G.dev(x), T, True), _run(False, wt, [lt], G.dev(x), T, True), f"masked T={T}")


def test_noalloc_refuses_calls_larger_than_the_scratch():
    """A call that needs more than STRATA_NOALLOC_SCRATCH_BYTES is refused
    with STRATA_EWORKSPACE before anything is enqueued (its output keeps
    its contents); the next call that fits still runs."""
    import torch as t
    w = synth.WORKLOADS["decode"]
    sh = G.shape_of(w)
    T_big = 404
    assert brx.workspace_bytes(sh, T_big) > brx.NOALLOC_SCRATCH_BYTES >= brx.workspace_bytes(sh, 403)
    L0 = W.layer_data(w, 3)
    ld = G.layer_to_dev(L0)
    x = t.zeros((T_big, w.d_model), dtype=t.int16, device="cuda")
    y = t.full((T_big, w.d_model), 7.0, dtype=t.float32, device="cuda")
    lib = brx.load_library()
    c_layers = (brx.Layer * 1)(ld.as_c())
    st = lib.strata_moe_forward_noalloc(ctypes.byref(sh), c_layers, 1, x.data_ptr(), brx.X_BF16, T_big, 0,
                                        y.data_ptr(), None, None, None, None, 0, None, None, 0,
                                        t.cuda.current_stream().cuda_stream)
    assert st == brx.STRATA_EWORKSPACE
    t.cuda.synchronize()
    assert bool((y == 7.0).all())
    xs, _ = W.draw_tokens(w, L0["Wr"], None, range(2), rep=47)
    a = _run(True, w, [ld], G.dev(xs), 2, False)
    b = _run(False, w, [ld], G.dev(xs), 2, False)
    _same(a, b, "after refusal")
