"""Host-side checks of the C ABI that need no GPU: every declared symbol is
exported, workspace sizing, and the validation errors (nothing is launched
when validation fails)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import bit_routed_expert_amd as brx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            src = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b(strata_\w+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = brx.load_library()
    names = _declared_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    assert set(names) == set(brx.EXPORTED_SYMBOLS)


def test_workspace_sizes():
    sh = brx.shape(512, 10, 2048, 768, 3)
    assert brx.workspace_bytes(sh, 1) > 0
    assert brx.workspace_bytes(sh, 4096) > brx.workspace_bytes(sh, 5)
    # per slot ((T*k + T) of them): fp32 expert output row (d) + 16-bit digit planes of h (f)
    assert brx.workspace_bytes(sh, 4096) >= 4096 * 11 * (2048 * 4 + 768 * 2)


@pytest.mark.parametrize("bad", [
    dict(n_shared=0), dict(top_k=0), dict(top_k=33), dict(n_experts=5, top_k=10), dict(d_model=200),
    dict(d_ff=100), dict(n_experts=2048)])
def test_invalid_shapes_rejected(bad):
    kw = dict(n_experts=512, top_k=10, n_shared=1, d_model=2048, d_ff=768, bits=3)
    kw.update(bad)
    sh = brx.Shape(kw["n_experts"], kw["top_k"], kw["n_shared"], kw["d_model"], kw["d_ff"], kw["bits"])
    lib = brx.load_library()
    assert lib.strata_moe_workspace_bytes(ctypes.byref(sh), 1, 1) == 0
    st = lib.strata_moe_forward(ctypes.byref(sh), None, 1, None, 0, 1, 0, None, None, None, None, None, 0, None,
                                None, 0, None, 0, None)
    assert st == brx.STRATA_EINVAL


def test_unsupported_bits():
    sh = brx.shape(512, 10, 2048, 768, 4)
    lib = brx.load_library()
    st = lib.strata_moe_forward(ctypes.byref(sh), None, 1, None, 0, 1, 0, None, None, None, None, None, 0, None,
                                None, 0, None, 0, None)
    assert st == brx.STRATA_EUNSUPPORTED


@pytest.mark.parametrize("bits", [1, 4, -3])
def test_unsupported_layer_bits(bits):
    """A layer's own code width must be 0 (the shape's), 3 or 2."""
    lib = brx.load_library()
    sh = brx.shape(512, 10, 2048, 768, 3)
    ly = (brx.Layer * 2)(brx.Layer(0x1000, None, 0x2000, 0x3000, None, 2),
                         brx.Layer(0x1000, None, 0x2000, 0x3000, None, bits))
    st = lib.strata_moe_forward(ctypes.byref(sh), ly, 2, 0x4000, 0, 1, 0, 0x5000, None, None, None, None, 0, None,
                                0x6000, 1 << 30, None, 0, None)
    assert st == brx.STRATA_EUNSUPPORTED


def _fake_layer():
    # non-null placeholders: validation fails before anything touches them
    return brx.Layer(0x1000, None, 0x2000, 0x3000, None)


def test_forward_validation_errors():
    lib = brx.load_library()
    sh = brx.shape(512, 10, 2048, 768, 3)
    ly = (brx.Layer * 1)(_fake_layer())
    need = brx.workspace_bytes(sh, 4)

    def call(**kw):
        a = dict(layers=ly, L=1, x=0x4000, xd=0, T=4, flags=0, y=0x5000, ws=0x6000, wsb=need, cap=0, mte=None,
                 mw=None, mc=None, nev=0, ev=None)
        a.update(kw)
        return lib.strata_moe_forward(ctypes.byref(sh), a["layers"], a["L"], a["x"], a["xd"], a["T"], a["flags"],
                                      a["y"], None, None, a["mte"], a["mw"], a["cap"], a["mc"], a["ws"], a["wsb"],
                                      a["ev"], a["nev"], None)

    assert call(T=-1) == brx.STRATA_EINVAL
    assert call(T=0, x=None, y=None, ws=None) == brx.STRATA_OK          # T = 0 is a no-op
    assert call(L=0) == brx.STRATA_EINVAL
    assert call(x=None) == brx.STRATA_EINVAL
    assert call(y=None) == brx.STRATA_EINVAL
    assert call(ws=None) == brx.STRATA_EINVAL
    assert call(xd=7) == brx.STRATA_EINVAL
    assert call(flags=8) == brx.STRATA_EINVAL
    assert call(cap=-1) == brx.STRATA_EINVAL
    assert call(nev=2) == brx.STRATA_EINVAL
    assert call(wsb=need - 1) == brx.STRATA_EWORKSPACE
    masked = (brx.Layer * 1)(brx.Layer(0x1000, None, 0x2000, 0x3000, 0x7000))
    assert call(layers=masked) == brx.STRATA_EINVAL                   # mask needs miss buffers
    nocodes = (brx.Layer * 1)(brx.Layer(0x1000, None, None, 0x3000, None))
    assert call(layers=nocodes) == brx.STRATA_EINVAL


def test_route_validation_errors():
    lib = brx.load_library()
    sh = brx.shape(512, 10, 2048, 768, 3)
    ly = _fake_layer()
    need = brx.workspace_bytes(sh, 4)
    f = lib.strata_moe_route
    assert f(ctypes.byref(sh), ctypes.byref(ly), 0x4000, 0, -1, None, 0x6000, need, None) == brx.STRATA_EINVAL
    assert f(ctypes.byref(sh), ctypes.byref(ly), 0x4000, 0, 0, None, 0x6000, need, None) == brx.STRATA_OK
    assert f(ctypes.byref(sh), ctypes.byref(ly), None, 0, 4, None, 0x6000, need, None) == brx.STRATA_EINVAL
    assert f(ctypes.byref(sh), ctypes.byref(ly), 0x4000, 0, 4, None, 0x6000, need - 8, None) == \
        brx.STRATA_EWORKSPACE


def test_token_count_limit_of_the_larger_T_path():
    """Token counts whose bf16 layer input or SwiGLU activations would pass
    2^31 bytes (32-bit buffer offsets) are refused before any launch."""
    lib = brx.load_library()
    sh = brx.shape(512, 10, 2048, 768, 3)
    ok_T, bad_T = 63550, 63551                 # (T*10 + T) * 768 * 4 <= 2^31 - 1
    assert brx.workspace_bytes(sh, ok_T) > 0
    assert lib.strata_moe_workspace_bytes(ctypes.byref(sh), bad_T, 1) == 0
    ly = (brx.Layer * 1)(_fake_layer())
    st = lib.strata_moe_forward(ctypes.byref(sh), ly, 1, 0x4000, 0, bad_T, 0, 0x5000, None, None, None, None, 0,
                                None, 0x6000, 1 << 40, None, 0, None)
    assert st == brx.STRATA_EUNSUPPORTED
    lyr = _fake_layer()
    st = lib.strata_moe_route(ctypes.byref(sh), ctypes.byref(lyr), 0x4000, 0, bad_T, None, 0x6000, 1 << 40, None)
    assert st == brx.STRATA_EUNSUPPORTED


def test_probe_validation_errors():
    lib = brx.load_library()
    assert lib.strata_probe_hbm_read(None, 1024, 0x1000, 4, None) == brx.STRATA_EINVAL
    assert lib.strata_probe_hbm_read(0x1008, 1024, 0x1000, 4, None) == brx.STRATA_EINVAL   # misaligned
    assert lib.strata_probe_hbm_read(0x1000, 1000, 0x2000, 4, None) == brx.STRATA_EINVAL   # not whole 16 B
    assert lib.strata_probe_hbm_read(0x1000, 1024, 0x2000, 0, None) == brx.STRATA_EINVAL
    fl = ctypes.c_double()
    assert lib.strata_probe_mfma_bf16(0, 0x1000, 4, ctypes.byref(fl), None) == brx.STRATA_EINVAL
    assert lib.strata_probe_mfma_bf16(16, 0x1000, 0, ctypes.byref(fl), None) == brx.STRATA_EINVAL
    assert lib.strata_probe_mfma_bf16(16, None, 4, ctypes.byref(fl), None) == brx.STRATA_EINVAL


def test_status_strings():
    lib = brx.load_library()
    for s in range(4):
        assert lib.strata_status_str(s)


def test_kernel_names_by_path():
    sh = brx.shape(512, 10, 2048, 768, 3)
    assert brx.kernel_names(sh, 1)[0] == "route_logits"
    assert "route_permute" in brx.kernel_names(sh, 4096)


def test_kernel_names_list_every_group_of_a_call():
    """One name per event pair a forward call records, in launch order: three
    groups per layer at T = 1, four at T = 2..8 for one layer and 3L + 1 for
    a stack (each layer's combine runs in the next layer's router kernel),
    seven per layer on the matrix-core path; nothing for T < 1 or L < 1."""
    sh = brx.shape(512, 10, 2048, 768, 3)
    assert brx.kernel_names(sh, 1, 2) == ["route_logits", "route_gemv_gateup", "gemv_down_combine"] * 2
    assert brx.kernel_names(sh, 5, 1) == ["route_logits", "route_gemv_gateup", "gemv_down", "combine"]
    three = brx.kernel_names(sh, 5, 3)
    assert three == (["route_logits", "route_gemv_gateup", "gemv_down"]
                     + ["combine_route_logits", "route_gemv_gateup", "gemv_down"] * 2 + ["combine"])
    assert len(brx.kernel_names(sh, 5, 48)) == 3 * 48 + 1
    assert len(brx.kernel_names(sh, 4096, 2)) == 14
    lib = brx.load_library()
    assert lib.strata_moe_kernel_names(ctypes.byref(sh), 0, 1, None, 0) == 0
    assert lib.strata_moe_kernel_names(ctypes.byref(sh), 5, 0, None, 0) == 0
