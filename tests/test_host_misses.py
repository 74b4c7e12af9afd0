"""The host-CPU consumer of the miss list (strata_moe_host_misses, host
code in the library: no GPU involved) against the oracle: for every listed
miss (t, e, gate), y_add[t] = sum of gate * FFN_e(u_t), with FFN_e the
oracle's expert FFN in double.  The bar is the parity bar of the layer
output: max-abs error <= 2e-3 x RMS (fp32 sums against double ones; the
measured error is near 1e-6)."""
from __future__ import annotations

import os

import numpy as np
import pytest

import bit_routed_expert_amd as brx
import oracle
import synth
from tests import workloads as W

TOL = 2e-3
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _oracle_y_add(w, L, u, te, mw):
    """sum of gate * oracle FFN_e(u_t), per token, in double."""
    ref = np.zeros((u.shape[0], w.d_model))
    for (t, e), g in zip(te, mw):
        ref[t] += float(g) * oracle.expert_ffn(w.bits, W.expert_slice(w, L["codes"], e, "codes"),
                                               W.expert_slice(w, L["scales"], e, "scales"), w.d_model, w.d_ff,
                                               u[t].astype(np.float64))
    return ref


def _run_host(w, L, u, te, mw, threads):
    sh = brx.shape(w.n_experts, w.top_k, w.d_model, w.d_ff, w.bits)
    T, n = u.shape[0], len(mw)
    nb = brx.host_workspace_bytes(sh, T, n)
    hws = np.zeros(nb, np.uint8)
    y = np.full((T, w.d_model), np.nan, np.float32)
    brx.host_misses(sh, L["codes"], L["scales"], w.bits, np.ascontiguousarray(u, np.float32), T,
                    np.ascontiguousarray(te, np.int32), np.ascontiguousarray(mw, np.float32), n, y, hws, nb, threads)
    return y


def _close(got, ref):
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref)))
    assert np.all(np.isfinite(got))
    assert err <= TOL * rms, f"max-abs {err:.3e} > {TOL} x RMS {rms:.3e}"
    return err / rms


def test_host_isa_is_known():
    assert brx.host_isa() in ("avx512", "avx2")


@pytest.mark.parametrize("bits", [3, 2])
def test_small_layer_misses_against_oracle(bits):
    """The 16-expert layer (its down matrix's 256-element scale blocks span
    two rows) with a mask: the host's sums equal the oracle's y_full -
    y_masked identity term by term."""
    base = synth.WORKLOADS["tiny"]
    w = synth.Workload(f"tiny_b{bits}", 16, 2, 256, 128, bits, 12, seed=base.seed + 0x300 + bits)
    L = W.layer_data(w, 0)
    mask = np.array([0b0110_1011_1001_0111], np.uint32)
    x, _ = W.draw_tokens(w, L["Wr"], None, range(12), rep=3)
    u = synth.bf16_to_f32(x)
    r = oracle.moe_layer(w.bits, 16, 2, 256, 128, u, L["Wr"], L["codes"], L["scales"], mask=mask)
    full = oracle.moe_layer(w.bits, 16, 2, 256, 128, u, L["Wr"], L["codes"], L["scales"])
    te, mw = r["miss_te"], r["miss_w"]
    assert len(mw) > 0
    y = _run_host(w, L, u, te, mw, 3)
    _close(y, _oracle_y_add(w, L, u, te, mw))
    # and the identity with the layer outputs: y_masked + y_add = y_full
    _close(r["out"] + y, full["out"])


def test_full_size_experts_and_thread_count():
    """Full-size 3-bit experts, several misses per expert and per token (in
    list order, as a GPU writes them), rows without misses zero; 1 and 5
    threads give the same bits."""
    w = synth.WORKLOADS["decode"]
    E, d, f = w.n_experts, w.d_model, w.d_ff
    codes = np.zeros(w.experts_total * w.code_bytes_per_expert, np.uint8)
    scales = np.zeros(w.experts_total * w.blocks_per_expert, np.uint16)
    experts = [3, 77, 500]
    for e in experts:
        codes[e * w.code_bytes_per_expert:(e + 1) * w.code_bytes_per_expert] = synth.expert_codes(w, 0, e)
        scales[e * w.blocks_per_expert:(e + 1) * w.blocks_per_expert] = synth.expert_scales(w, 0, e)
    L = dict(codes=codes, scales=scales)
    T = 5
    u = synth.bf16_to_f32(synth.x_tokens(w, range(T), rep=9))
    te = np.array([[0, 77], [0, 500], [1, 3], [3, 3], [3, 77], [3, 500], [4, 500]], np.int32)
    mw = np.array([0.3, 0.05, 0.2, 0.11, 0.07, 0.5, 0.01], np.float32)
    y1 = _run_host(w, L, u, te, mw, 1)
    y5 = _run_host(w, L, u, te, mw, 5)
    np.testing.assert_array_equal(y1, y5)
    assert np.all(y1[2] == 0)                    # token 2 has no misses
    r = _close(y1, _oracle_y_add(w, L, u, te, mw))
    print(f"host misses max-abs/RMS {r:.2e} ({brx.host_isa()})")


def test_avx2_build_gives_the_same_bits():
    """The AVX2 build (forced with STRATA_HOST_ISA=avx2 in a fresh process)
    runs the same 16-lane operations in the same order as the AVX-512 one."""
    import os
    import subprocess
    import sys
    if brx.host_isa() != "avx512":
        pytest.skip("this CPU has no AVX-512: only the AVX2 build runs here")
    code = (
        "import numpy as np, sys\n"
        "sys.path.insert(0, %r)\n"
        "import bit_routed_expert_amd as brx\n"
        "from tests import test_host_misses as H\n"
        "assert brx.host_isa() == 'avx2'\n"
        "w, L, u, te, mw = H._case()\n"
        "np.save(sys.argv[1], H._run_host(w, L, u, te, mw, 2))\n") % ROOT
    out = os.path.join(os.environ.get("TMPDIR", "/tmp"), f"host_avx2_{os.getpid()}.npy")
    env = dict(os.environ, STRATA_HOST_ISA="avx2")
    subprocess.run([sys.executable, "-c", code, out], check=True, env=env, cwd=ROOT)
    try:
        w, L, u, te, mw = _case()
        np.testing.assert_array_equal(np.load(out), _run_host(w, L, u, te, mw, 2))
    finally:
        os.remove(out)


def _case():
    w = synth.Workload("tiny_isa", 16, 2, 256, 128, 3, 6, seed=0x5EED0321)
    L = W.layer_data(w, 0)
    u = synth.bf16_to_f32(synth.x_tokens(w, range(6), rep=4))
    te = np.array([[0, 1], [0, 9], [2, 4], [5, 1], [5, 15]], np.int32)
    mw = np.array([0.5, 0.25, 0.75, 0.6, 0.4], np.float32)
    return w, L, u, te, mw


def test_host_misses_validation():
    import ctypes
    lib = brx.load_library()
    sh = brx.shape(16, 2, 256, 128, 3)
    hl = brx.HostLayer(0x1000, 0x2000, 0)
    ws = np.zeros(brx.host_workspace_bytes(sh, 4, 2), np.uint8)
    u = np.zeros((4, 256), np.float32)
    y = np.zeros((4, 256), np.float32)
    mw = np.ones(2, np.float32)

    def call(te, threads=2, wsb=ws.nbytes):
        te = np.asarray(te, np.int32)
        return lib.strata_moe_host_misses(ctypes.byref(sh), ctypes.byref(hl), u.ctypes.data, 4, te.ctypes.data,
                                          mw.ctypes.data, 2, y.ctypes.data, ws.ctypes.data, wsb, threads)

    assert call([[0, 1], [4, 1]]) == brx.STRATA_EINVAL       # token out of range
    assert call([[0, 1], [1, 16]]) == brx.STRATA_EINVAL      # a routed expert index only
    assert call([[0, 1], [1, 2]], threads=0) == brx.STRATA_EINVAL
    assert call([[0, 1], [1, 2]], wsb=ws.nbytes - 64) == brx.STRATA_EWORKSPACE
    bad = brx.HostLayer(0x1000, 0x2000, 4)
    assert lib.strata_moe_host_misses(ctypes.byref(sh), ctypes.byref(bad), u.ctypes.data, 4, None, None, 0,
                                      y.ctypes.data, ws.ctypes.data, ws.nbytes, 1) == brx.STRATA_EUNSUPPORTED
