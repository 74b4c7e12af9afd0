"""Helpers for the GPU parity tests: upload synthetic layers, call the
library through its C ABI, and compare with the oracle."""
from __future__ import annotations

import numpy as np

import bit_routed_expert_amd as brx

TOL = 2e-3          # max-abs error <= TOL * RMS of the reference output
GATE_TOL = 1e-6     # absolute gate error


def torch():
    import torch as _t
    return _t


def dev(a: np.ndarray):
    t = torch()
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return t.from_numpy(np.ascontiguousarray(a)).cuda()


def layer_to_dev(L: dict) -> brx.LayerData:
    return brx.LayerData(router_w=dev(L["Wr"]), codes=dev(L["codes"]), scales=dev(L["scales"]),
                         router_bias=None if L.get("bias") is None else dev(L["bias"]),
                         resident_mask=None if L.get("mask") is None else dev(L["mask"]))


def shape_of(w) -> brx.Shape:
    return brx.shape(w.n_experts, w.top_k, w.d_model, w.d_ff, w.bits)


def run_forward(w, layers, x_dev, xdtype, T, flags=0, miss_cap=None, want_route=True, ws_fill=0):
    """Run strata_moe_forward; returns numpy results.  ws_fill: byte value
    the workspace holds before the call."""
    t = torch()
    sh = shape_of(w)
    L = len(layers)
    nb = brx.workspace_bytes(sh, T, L)
    ws = t.full((nb,), ws_fill, dtype=t.uint8, device="cuda")
    y = t.empty((T, w.d_model), dtype=t.float32, device="cuda")
    resid = t.empty((T, w.d_model), dtype=t.float32, device="cuda")
    k, E = w.top_k, w.n_experts
    ros = None
    if want_route:
        ros = [dict(topk_idx=t.empty((T, k), dtype=t.int32, device="cuda"),
                    topk_w=t.empty((T, k), dtype=t.float32, device="cuda"),
                    counts=t.empty(E, dtype=t.int32, device="cuda"),
                    offsets=t.empty(E + 1, dtype=t.int32, device="cuda"),
                    perm=t.empty(T * k, dtype=t.int32, device="cuda"),
                    pos=t.empty(T * k, dtype=t.int32, device="cuda")) for _ in range(L)]
    cap = T * k if miss_cap is None else miss_cap
    any_mask = any(ly.resident_mask is not None for ly in layers)
    mte = mw = mc = None
    if any_mask:
        mte = t.full((L, max(cap, 1), 2), -1, dtype=t.int32, device="cuda")
        mw = t.zeros((L, max(cap, 1)), dtype=t.float32, device="cuda")
        mc = t.zeros(L, dtype=t.int32, device="cuda")
    brx.forward(sh, layers, x_dev, xdtype, T, y, ws, nb, resid_out=resid, route_outs=ros, miss_te=mte,
                miss_w=mw, miss_cap=cap, miss_count=mc, flags=flags)
    t.cuda.synchronize()
    out = dict(y=y.cpu().numpy(), resid=resid.cpu().numpy())
    if ros is not None:
        out["route"] = [{kk: v.cpu().numpy() for kk, v in r.items()} for r in ros]
    if any_mask:
        out["miss_te"] = mte.cpu().numpy()
        out["miss_w"] = mw.cpu().numpy()
        out["miss_count"] = mc.cpu().numpy()
    return out


def assert_close(got: np.ndarray, ref: np.ndarray, tol: float = TOL, what: str = "output"):
    ref = ref.astype(np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got.astype(np.float64) - ref)))
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert err <= tol * rms, f"{what}: max-abs error {err:.3e} > {tol} x RMS {rms:.3e} (ratio {err / rms:.2e})"
    return err / rms


def assert_route_equal(got: dict, ref: dict, rows=None):
    """Routing outputs: integers bit-exact, gates within GATE_TOL."""
    gi, ri = got["topk_idx"], ref["idx"]
    gg, rg = got["topk_w"], ref["gate"]
    if rows is not None:
        gi, gg = gi[rows], gg[rows]
    assert np.array_equal(gi, ri), "top-k ids differ"
    assert np.max(np.abs(gg - rg)) <= GATE_TOL, f"gates differ by {np.max(np.abs(gg - rg)):.2e}"
    if rows is None:
        for key in ("counts", "offsets", "perm", "pos"):
            assert np.array_equal(got[key], ref[key]), f"{key} differs"
