"""Parity of the HIP path (called through the C ABI) with the oracle.

Integers (top-k ids, counts, offsets, permutation, miss list) bit-exact;
gates within 1e-6; float outputs within max-abs 2e-3 x RMS of the oracle's
output over the compared tensor.  Inputs are drawn with top-(k+1) logit
margins >= 1e-3 so the ordered routing is unique.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G
from tests import workloads as W

pytestmark = pytest.mark.gpu


def _layer_case(name, T=None, rep=0, with_mask=None, bits=None):
    w = synth.WORKLOADS[name]
    if bits is not None and bits != w.bits:
        w = synth.Workload(w.name + f"_b{bits}", w.n_experts, w.top_k, w.d_model, w.d_ff, bits, w.tokens,
                           seed=w.seed + 0x100)
    T = T or w.tokens_per_call
    L = W.layer_data(w, 0)
    if with_mask is not None:
        L["mask"] = with_mask
    x, _ = W.draw_tokens(w, L["Wr"], L["bias"], range(T), rep=rep)
    return w, L, x, T


def _oracle_layer(w, L, u, mask=None):
    return oracle.moe_layer(w.bits, w.n_experts, w.top_k, w.d_model, w.d_ff, u, L["Wr"], L["codes"],
                            L["scales"], bias=L["bias"], mask=mask if mask is not None else L.get("mask"))


@pytest.mark.parametrize("bits", [3, 2])
def test_tiny_layer(bits):
    w, L, x, T = _layer_case("tiny", bits=bits)
    print(f"case tiny bits={bits} T={T}", flush=True)
    ref = _oracle_layer(w, L, synth.bf16_to_f32(x))
    got = G.run_forward(w, [G.layer_to_dev(L)], G.dev(x), 0, T)
    G.assert_route_equal(got["route"][0], ref)
    G.assert_close(got["y"], ref["out"])
    np.testing.assert_array_equal(got["resid"], (synth.bf16_to_f32(x) + got["y"]).astype(np.float32))


def test_tiny_layer_with_mask_and_misses():
    mask = np.array([0b0110_1011_1001_0111], np.uint32)
    w, L, x, T = _layer_case("tiny", with_mask=mask)
    print(f"case tiny masked T={T}", flush=True)
    ref = _oracle_layer(w, L, synth.bf16_to_f32(x))
    got = G.run_forward(w, [G.layer_to_dev(L)], G.dev(x), 0, T)
    G.assert_route_equal(got["route"][0], ref)
    G.assert_close(got["y"], ref["out"])
    n = int(got["miss_count"][0])
    assert n == ref["miss_count"]
    np.testing.assert_array_equal(got["miss_te"][0][:n], ref["miss_te"])
    assert np.max(np.abs(got["miss_w"][0][:n] - ref["miss_w"]), initial=0) <= G.GATE_TOL


@pytest.mark.parametrize("name,T,rep", [("tiny", 1, 0), ("tiny", 1, 3), ("decode", 1, 0), ("decode", 1, 4),
                                        ("decode", 5, 2), ("decode", 8, 5)])
def test_decode_path_with_resident_mask(name, T, rep):
    """The T <= 8 kernels with a resident mask (one-token kernels at T = 1):
    non-resident picks are skipped in gate/up, down and the combine, and
    listed as misses."""
    w = synth.WORKLOADS[name]
    nw = (w.n_experts + 31) // 32
    bits = np.random.default_rng(100 + rep).random(w.n_experts) < 0.5   # about half resident
    mask = np.zeros(nw, np.uint32)
    for e in np.nonzero(bits)[0]:
        mask[e // 32] |= np.uint32(1) << np.uint32(e % 32)
    w, L, x, T = _layer_case(name, T=T, rep=rep, with_mask=mask)
    print(f"case {name} T={T} masked rep={rep}", flush=True)
    ref = _oracle_layer(w, L, synth.bf16_to_f32(x))
    got = G.run_forward(w, [G.layer_to_dev(L)], G.dev(x), 0, T)
    G.assert_route_equal(got["route"][0], ref)
    G.assert_close(got["y"], ref["out"])
    n = int(got["miss_count"][0])
    assert n == ref["miss_count"]
    np.testing.assert_array_equal(got["miss_te"][0][:n], ref["miss_te"])
    assert np.max(np.abs(got["miss_w"][0][:n] - ref["miss_w"]), initial=0) <= G.GATE_TOL


def test_tiny_miss_list_overflow_keeps_true_count():
    mask = np.array([0b0000_0000_0000_0001], np.uint32)      # only expert 0 resident
    w, L, x, T = _layer_case("tiny", with_mask=mask)
    ref = _oracle_layer(w, L, synth.bf16_to_f32(x))
    got = G.run_forward(w, [G.layer_to_dev(L)], G.dev(x), 0, T, miss_cap=3)
    assert int(got["miss_count"][0]) == ref["miss_count"] > 3
    np.testing.assert_array_equal(got["miss_te"][0][:3], ref["miss_te"][:3])


def test_decode_layer_full_size():
    w, L, x, T = _layer_case("decode")
    print("case decode T=1", flush=True)
    ref = _oracle_layer(w, L, synth.bf16_to_f32(x))
    got = G.run_forward(w, [G.layer_to_dev(L)], G.dev(x), 0, T)
    G.assert_route_equal(got["route"][0], ref)
    r = G.assert_close(got["y"], ref["out"])
    print(f"decode max-abs/RMS {r:.2e}")


def test_verify_batch_five_tokens_and_batch_invariance():
    w = synth.WORKLOADS["decode"]
    L = W.layer_data(w, 0)
    x, _ = W.draw_tokens(w, L["Wr"], None, range(5), rep=3)
    print("case T=5 one layer", flush=True)
    ref = _oracle_layer(w, L, synth.bf16_to_f32(x))
    dl = [G.layer_to_dev(L)]
    got = G.run_forward(w, dl, G.dev(x), 0, 5)
    G.assert_route_equal(got["route"][0], ref)
    G.assert_close(got["y"], ref["out"])
    # the verify batch equals token-by-token evaluation, bit for bit
    for t in range(5):
        one = G.run_forward(w, dl, G.dev(x[t:t + 1]), 0, 1, want_route=False)
        np.testing.assert_array_equal(one["y"][0], got["y"][t])


@pytest.mark.parametrize("T", [2, 6, 8])
def test_full_size_batches_match_oracle_and_single_tokens(T):
    """Other T <= 8 batch sizes on the full-size layer (T = 8: 80 picks):
    routing bit-exact, outputs against the oracle, and each token's row equal
    to its own one-token call bit for bit."""
    w = synth.WORKLOADS["decode"]
    L = W.layer_data(w, 0)
    x, _ = W.draw_tokens(w, L["Wr"], None, range(T), rep=11 + T)
    print(f"case full-size T={T}", flush=True)
    ref = _oracle_layer(w, L, synth.bf16_to_f32(x))
    dl = [G.layer_to_dev(L)]
    got = G.run_forward(w, dl, G.dev(x), 0, T)
    G.assert_route_equal(got["route"][0], ref)
    G.assert_close(got["y"], ref["out"])
    for t in range(T):
        one = G.run_forward(w, dl, G.dev(x[t:t + 1]), 0, 1, want_route=False)
        np.testing.assert_array_equal(one["y"][0], got["y"][t])


def test_decode_repeat_is_bitwise_identical():
    w, L, x, T = _layer_case("decode", rep=5)
    dl = [G.layer_to_dev(L)]
    a = G.run_forward(w, dl, G.dev(x), 0, T)
    b = G.run_forward(w, dl, G.dev(x), 0, T)
    np.testing.assert_array_equal(a["y"], b["y"])


@pytest.mark.parametrize("name,T", [("decode", 1), ("decode", 5), ("tiny", 20)])
def test_prepared_call_equals_forward(name, T):
    """A forward call marshalled once and enqueued several times (the
    binding's PreparedForward, used by the benchmark's timed loop) gives the
    bits of forward() on the same arguments, each time, with a new input
    written into the captured input buffer between calls."""
    import bit_routed_expert_amd as brx
    t = G.torch()
    w = synth.WORKLOADS[name]
    L = W.layer_data(w, 0)
    dl = [G.layer_to_dev(L)]
    sh = G.shape_of(w)
    xs = [W.draw_tokens(w, L["Wr"], None, range(T), rep=60 + i)[0] for i in range(2)]
    nb = brx.workspace_bytes(sh, T, 1)
    ws = t.empty(nb, dtype=t.uint8, device="cuda")
    x_in = G.dev(xs[0]).clone()
    y = t.empty((T, w.d_model), dtype=t.float32, device="cuda")
    resid = t.empty((T, w.d_model), dtype=t.float32, device="cuda")
    print(f"case prepared call {name} T={T}", flush=True)
    call = brx.PreparedForward(sh, dl, x_in, 0, T, y, ws, nb, resid_out=resid)
    for rnd in range(2):
        for x in xs:
            x_in.copy_(G.dev(x))
            brx.forward(sh, dl, x_in, 0, T, y, ws, nb, resid_out=resid)
            t.cuda.synchronize()
            ref = (y.cpu().numpy().copy(), resid.cpu().numpy().copy())
            y.fill_(0.0)
            resid.fill_(0.0)
            call()
            t.cuda.synchronize()
            np.testing.assert_array_equal(y.cpu().numpy(), ref[0])
            np.testing.assert_array_equal(resid.cpu().numpy(), ref[1])


@pytest.mark.parametrize("T", [3, 12, 300])
def test_fp32_input_with_norm_first(T):
    """fp32 residual-stream input, RMS-normalised before routing: the decode
    path (T = 3) and the matrix-core path with hi/lo bf16 activations (T = 12;
    T = 300 spans two 256-token router tiles, the second partial)."""
    w = synth.WORKLOADS["decode"]
    L = W.layer_data(w, 0)
    rng = np.random.default_rng(11 + T)
    # fp32 residual-stream input of a later layer: redraw rows until the margins hold
    xs = []
    while len(xs) < T:
        xr = (7.0 * rng.standard_normal(w.d_model)).astype(np.float32)
        u = oracle.rmsnorm(xr[None])
        if oracle.topk_margin(oracle.logits(u, L["Wr"]), w.top_k)[0] >= W.MARGIN:
            xs.append(xr)
    x = np.stack(xs)
    u = oracle.rmsnorm(x)
    print(f"case fp32 input T={T}", flush=True)
    ref = _oracle_layer(w, L, u)
    got = G.run_forward(w, [G.layer_to_dev(L)], G.dev(x), 1, T, flags=1)
    G.assert_route_equal(got["route"][0], ref)
    G.assert_close(got["y"], ref["out"])
    np.testing.assert_array_equal(got["resid"], (x + got["y"]).astype(np.float32))


def _perturb_scales(scales: np.ndarray, seed: int) -> np.ndarray:
    """Every 10th block (seeded) gets a zero scale (+0 or -0), every other
    10th a negated one."""
    s = scales.copy()
    rng = np.random.default_rng(seed)
    r = rng.random(s.shape)
    s[r < 0.05] = 0x0000
    s[(r >= 0.05) & (r < 0.1)] = 0x8000
    neg = (r >= 0.1) & (r < 0.2)
    s[neg] ^= 0x8000
    return s


@pytest.mark.parametrize("name,bits,T", [("tiny", 3, 3), ("tiny", 2, 3), ("tiny", 3, 20), ("tiny", 2, 20),
                                         ("decode", 3, 1), ("decode", 3, 9)])
def test_zero_and_negative_block_scales(name, bits, T):
    """Blocks with zero (or -0) scales contribute nothing and negative scales
    flip their block, on the decode GEMV path (T <= 8) and on the matrix-core
    path (T > 8), whose scale folding treats zero scales separately."""
    w, L, x, T = _layer_case(name, T=T, rep=5, bits=bits)
    L["scales"] = _perturb_scales(L["scales"], 99 + T + bits)
    print(f"case {name} bits={bits} T={T} perturbed scales", flush=True)
    ref = _oracle_layer(w, L, synth.bf16_to_f32(x))
    got = G.run_forward(w, [G.layer_to_dev(L)], G.dev(x), 0, T)
    G.assert_route_equal(got["route"][0], ref)
    G.assert_close(got["y"], ref["out"])


@pytest.mark.parametrize("bits", [3, 2])
def test_three_layer_stack_on_matrix_core_path(bits):
    """L = 3, T = 20 on the small layer: layers 1 and 2 take the normalised
    fp32 residual stream (hi/lo bf16 activations on the matrix cores).  Ids
    bit-exact against the oracle's chain; gates against the oracle run on the
    GPU's own layer input (chained one-layer calls, equal to the stack
    bitwise); y_2 and x_3 within tolerance."""
    w = synth.WORKLOADS["tiny"]
    if bits != w.bits:
        w = synth.Workload(w.name + f"_b{bits}", w.n_experts, w.top_k, w.d_model, w.d_ff, bits, w.tokens,
                           seed=w.seed + 0x100)
    T, nl = 20, 3
    t = G.torch()
    Ls, refs = [], []
    x0 = None
    xl = None
    for l in range(nl):
        attempt = 0
        while True:
            Lr = W.layer_data(w, l, attempt)
            if l == 0:
                x0, _ = W.draw_tokens(w, Lr["Wr"], None, range(T), rep=21)
                xl = synth.bf16_to_f32(x0)
            u = oracle.layer_input(xl, l)
            if oracle.topk_margin(oracle.logits(u, Lr["Wr"]), w.top_k).min() >= W.MARGIN:
                break
            attempt += 1
        r = oracle.moe_layer(w.bits, w.n_experts, w.top_k, w.d_model, w.d_ff, u, Lr["Wr"], Lr["codes"],
                             Lr["scales"])
        Ls.append(Lr)
        refs.append(r)
        y_last = r["out"]
        xl = oracle.residual_add(xl, r["out"])
    print(f"case 3-layer stack bits={bits} T={T}", flush=True)
    dl = [G.layer_to_dev(L) for L in Ls]
    got = G.run_forward(w, dl, G.dev(x0), 0, T)
    G.assert_close(got["y"], y_last, what="y_2")
    G.assert_close(got["resid"], xl, what="x_3")
    xc, xd = G.dev(x0), 0
    inputs = [synth.bf16_to_f32(x0)]
    for l in range(nl):
        one = G.run_forward(w, [dl[l]], xc, xd, T, flags=(1 if l > 0 else 0))
        np.testing.assert_array_equal(one["route"][0]["topk_idx"], got["route"][l]["topk_idx"])
        np.testing.assert_array_equal(one["route"][0]["topk_w"], got["route"][l]["topk_w"])
        xc, xd = t.from_numpy(one["resid"]).cuda(), 1
        inputs.append(one["resid"])
    np.testing.assert_array_equal(one["resid"], got["resid"])
    for l in range(nl):
        np.testing.assert_array_equal(got["route"][l]["topk_idx"], refs[l]["idx"])
        u_gpu = oracle.layer_input(inputs[l], l)
        _, gate_g = oracle.select(oracle.logits(u_gpu, Ls[l]["Wr"]), w.top_k)
        assert np.max(np.abs(got["route"][l]["topk_w"] - gate_g)) <= G.GATE_TOL, f"layer {l} gates"


@pytest.mark.parametrize("T", [1, 5, 12])
def test_exact_logit_ties_break_by_lower_index(T):
    """Router rows duplicated in pairs (expert 2i+1 has expert 2i's row), so
    every logit occurs exactly twice and each pair is an exact tie that the
    lower index wins; with k = 9 the ninth pick splits a pair.  Tokens keep
    margins >= 1e-3 between distinct logits.  Decode kernels (T = 1, 5) and
    the matrix-core path (T = 12)."""
    base = synth.WORKLOADS["decode"]
    w = synth.Workload("decode_k9", base.n_experts, 9, base.d_model, base.d_ff, base.bits, T, seed=base.seed + 0x79)
    L = W.layer_data(w, 0)
    Wr = L["Wr"].copy()
    Wr[1::2] = Wr[0::2]
    L["Wr"] = Wr
    # margins over the distinct logits: half the experts, top 6 of them (the 9 picks span 5 pairs)
    wd = synth.Workload("decode_k9_distinct", base.n_experts // 2, 6, base.d_model, base.d_ff, base.bits, T,
                        seed=base.seed + 0x7A)
    x, _ = W.draw_tokens(wd, Wr[0::2], None, range(T), rep=29)
    print(f"case paired router rows k=9 T={T}", flush=True)
    ref = _oracle_layer(w, L, synth.bf16_to_f32(x))
    assert np.all(ref["idx"][:, 8] % 2 == 0) and np.all(ref["idx"][:, 0::2] % 2 == 0)   # each pair's lower index first
    got = G.run_forward(w, [G.layer_to_dev(L)], G.dev(x), 0, T)
    G.assert_route_equal(got["route"][0], ref)
    G.assert_close(got["y"], ref["out"])


@pytest.mark.parametrize("T", [1, 12])
def test_zero_router_picks_lowest_indices(T):
    """A zero router: all 512 logits tie, so every token picks experts 0..k-1
    in index order with equal gates (more than 64 keys reach the threshold,
    which exercises the round-by-round selection)."""
    w = synth.WORKLOADS["decode"]
    L = W.layer_data(w, 0)
    L["Wr"] = np.zeros_like(L["Wr"])
    x = synth.x_tokens(w, np.arange(T), np.zeros(T, np.int64), 31)
    print(f"case zero router T={T}", flush=True)
    ref = _oracle_layer(w, L, synth.bf16_to_f32(x))
    np.testing.assert_array_equal(ref["idx"], np.tile(np.arange(w.top_k), (T, 1)))
    got = G.run_forward(w, [G.layer_to_dev(L)], G.dev(x), 0, T)
    G.assert_route_equal(got["route"][0], ref)
    G.assert_close(got["y"], ref["out"])


@pytest.mark.parametrize("name,T,masked,L", [("tiny", 1, True, 1), ("tiny", 4, True, 2), ("tiny", 20, True, 2),
                                             ("decode", 1, False, 2), ("decode", 5, False, 2),
                                             ("decode", 37, False, 1)])
def test_workspace_contents_do_not_matter(name, T, masked, L):
    """A workspace full of 0xFF bytes (NaN as fp32, -1 as int32) gives the
    same results, bit for bit, as a zeroed one: every call writes what it
    reads (one-token, T <= 8 and matrix-core paths, with and without a
    mask, one and two layers)."""
    mask = np.array([0b0110_1011_1001_0111], np.uint32) if masked else None
    w, L0, x, T = _layer_case(name, T=T, with_mask=mask)
    print(f"case workspace fill {name} T={T} masked={masked} L={L}", flush=True)
    layers = [G.layer_to_dev(L0) for _ in range(L)]
    a = G.run_forward(w, layers, G.dev(x), 0, T, flags=0)
    b = G.run_forward(w, layers, G.dev(x), 0, T, flags=0, ws_fill=0xFF)
    for key in ("y", "resid") + (("miss_te", "miss_w", "miss_count") if masked else ()):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    for ra, rb in zip(a["route"], b["route"]):
        for key in ra:
            np.testing.assert_array_equal(ra[key], rb[key], err_msg=key)
    if L == 1:
        G.assert_close(a["y"], _oracle_layer(w, L0, synth.bf16_to_f32(x))["out"])
