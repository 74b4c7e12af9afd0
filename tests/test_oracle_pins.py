"""Pins of the oracle against facts fixed outside the oracle itself.

Each check is chosen so that a plausible mistake in oracle.c fails it:
hand-derived bytes (tests/golden) for the block layout, numpy's own binary16
decoding for the scales, closed forms, brute force on the small layer,
invariants at full size, numpy float64 matmuls for the dense SwiGLU MLP, and
the mask identity y_full = y_masked + sum of missed gate * y_expert.
"""
from __future__ import annotations

import itertools
import math
import os

import numpy as np
import pytest

import oracle
import synth
from tests import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if "=" in line:
            k, v = line.split("=", 1)
            vals[k.strip()] = v.split()
    return vals


def _hexbytes(tokens):
    return np.array([int(t, 16) for t in tokens], dtype=np.uint8)


# ------------------------------------------------------------------ format
def test_half_decoding_matches_numpy_binary16():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_float(int(p)) for p in pats[::7]])
    r = ref[::7]
    fin = np.isfinite(r)
    assert np.array_equal(got[fin], r[fin])
    assert np.array_equal(np.isnan(got), np.isnan(r))


def test_3bit_unit_i_mod_8_golden():
    g = _golden("format_3bit_unit.txt")
    unit = _hexbytes(g["unit_i_mod_8"])
    mat = np.tile(unit, 64)                      # 16 x 128 matrix, every unit alike
    codes = oracle.unpack_codes(3, mat, 16, 128)
    expect = np.tile(np.arange(128) % 8, (16, 1))
    assert np.array_equal(codes, expect)
    # pack is the inverse
    assert np.array_equal(oracle.pack_codes(3, expect), mat)
    # scale 1.0 everywhere -> w = (c % 8) - 3.5
    w = oracle.dequant(3, mat, np.full(8, 0x3C00, np.uint16), 16, 128)
    assert np.array_equal(w, expect - 3.5)


def test_3bit_all_seven_scale_2m4():
    g = _golden("format_3bit_unit.txt")
    mat = np.tile(_hexbytes(g["unit_all_7"]), 64)
    w = oracle.dequant(3, mat, np.full(8, 0x2C00, np.uint16), 16, 128)   # fp16 0x2C00 = 2^-4
    assert np.all(w == 0.21875)


@pytest.mark.parametrize("name,place,value", [("unit_c_bit31", 31, 4), ("unit_a_bit0", 0, 1),
                                              ("unit_b_bit3", 24, 2)])
def test_3bit_single_bits(name, place, value):
    g = _golden("format_3bit_unit.txt")
    unit = _hexbytes(g[name])
    mat = np.zeros(16 * 128 * 3 // 8, np.uint8)
    mat[:12] = unit                             # row 0, columns 0..31
    codes = oracle.unpack_codes(3, mat, 16, 128)
    expect = np.zeros((16, 128), np.uint8)
    expect[0, place] = value
    assert np.array_equal(codes, expect)


def test_3bit_position_golden():
    off, byte, r, c, v = _golden("format_3bit_unit.txt")["position_32x256"]
    mat = np.zeros(32 * 256 * 3 // 8, np.uint8)
    mat[int(off)] = int(byte, 16)
    codes = oracle.unpack_codes(3, mat, 32, 256)
    expect = np.zeros((32, 256), np.uint8)
    expect[int(r), int(c)] = int(v)
    assert np.array_equal(codes, expect)


def test_2bit_goldens():
    g = _golden("format_2bit_unit.txt")
    mat = np.tile(_hexbytes(g["unit_i_mod_4"]), 64)
    codes = oracle.unpack_codes(2, mat, 16, 128)
    expect = np.tile(np.arange(128) % 4, (16, 1))
    assert np.array_equal(codes, expect)
    w = oracle.dequant(2, mat, np.full(8, 0x3C00, np.uint16), 16, 128)
    assert np.array_equal(w, expect - 1.5)
    mat = np.zeros(16 * 128 // 4, np.uint8)
    mat[:8] = _hexbytes(g["unit_a_bits23"])
    e2 = np.zeros((16, 128), np.uint8)
    e2[0, 8] = 3
    assert np.array_equal(oracle.unpack_codes(2, mat, 16, 128), e2)
    off, byte, r, c, v = g["position_32x256"]
    mat = np.zeros(32 * 256 // 4, np.uint8)
    mat[int(off)] = int(byte, 16)
    e3 = np.zeros((32, 256), np.uint8)
    e3[int(r), int(c)] = int(v)
    assert np.array_equal(oracle.unpack_codes(2, mat, 32, 256), e3)


@pytest.mark.parametrize("bits", [3, 2])
def test_pack_unpack_identity_random(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(48, 384)).astype(np.uint8)
    mat = oracle.pack_codes(bits, codes)
    assert mat.size * 8 == codes.size * bits            # dense: exactly `bits` bits per code
    assert np.array_equal(oracle.unpack_codes(bits, mat, 48, 384), codes)
    # uniform random bytes decode to uniform codes (what the generator relies on)
    rb = rng.integers(0, 256, size=mat.size).astype(np.uint8)
    hist = np.bincount(oracle.unpack_codes(bits, rb, 48, 384).ravel(), minlength=1 << bits)
    assert hist.min() > 0.9 * codes.size / (1 << bits)


def test_bits_per_weight():
    # 3-bit codes + one fp16 scale per 256 weights = 3 + 16/256 = 3.0625 bit/weight,
    # the "about 3.06 bit/weight" the pages give for IQ3_XXS (wiselychen.com, technique 1)
    for bits, bpw in ((3, 3.0625), (2, 2.0625)):
        w = synth.Workload("t", 512, 10, 2048, 768, bits, 1)
        total = w.code_bytes_per_expert + 2 * w.blocks_per_expert
        assert total * 8 / (3 * 2048 * 768) == bpw
    assert round(3.0625, 2) == 3.06


def test_scale_index_is_flattened_block():
    # tiny down matrix [256][128]: one 256-block spans two rows
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 8, size=(256, 128)).astype(np.uint8)
    mat = oracle.pack_codes(3, codes)
    scales = (np.arange(128) + 0x3C00).astype(np.uint16)       # distinct per block
    w = oracle.dequant(3, mat, scales, 256, 128)
    sv = scales.view(np.float16).astype(np.float64)
    expect = sv[(np.arange(256 * 128) // 256)].reshape(256, 128) * (codes - 3.5)
    assert np.array_equal(w, expect)


# ------------------------------------------------------------------ router
def test_logits_zero_router_and_one_hot():
    rng = np.random.default_rng(1)
    u = rng.standard_normal((3, 64)).astype(np.float32)
    assert np.all(oracle.logits(u, np.zeros((8, 64), np.float32)) == 0)
    Wr = np.zeros((8, 64), np.float32)
    for e in range(8):
        Wr[e, 7 * e % 64] = 0.5 * (e + 1)
    z = oracle.logits(u, Wr)
    for e in range(8):
        assert np.array_equal(z[:, e], (u[:, 7 * e % 64] * np.float32(0.5 * (e + 1))).astype(np.float32))


def test_logits_match_numpy_float64_matmul():
    rng = np.random.default_rng(2)
    u = rng.standard_normal((5, 2048)).astype(np.float32)
    Wr = (rng.standard_normal((512, 2048)) / math.sqrt(2048)).astype(np.float32)
    b = rng.standard_normal(512).astype(np.float32)
    z = oracle.logits(u, Wr, b)
    ref = u.astype(np.float64) @ Wr.astype(np.float64).T + b
    assert np.max(np.abs(z - ref)) <= 2 ** -22 * np.max(np.abs(ref)) + 1e-9


def test_topk_brute_force_small_layer():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((200, 16)).astype(np.float32)
    z[:20, 5] = z[:20, 9]                    # planted exact ties
    idx, gate = oracle.select(z, 2)
    for t in range(200):
        best = None
        for sub in itertools.combinations(range(16), 2):
            key = (float(z[t, list(sub)].astype(np.float64).sum()), [-s for s in sorted(sub)])
            if best is None or key > best[0]:
                best = (key, sub)
        chosen = sorted(best[1], key=lambda e: (-z[t, e], e))
        assert list(idx[t]) == chosen


def test_topk_zero_router_pins_tie_break_and_gates():
    z = np.zeros((3, 512), np.float32)
    idx, gate = oracle.select(z, 10)
    assert np.array_equal(idx, np.tile(np.arange(10), (3, 1)))
    assert np.all(np.abs(gate - 0.1) <= 1e-7)


def test_gates_closed_form_and_sum():
    rng = np.random.default_rng(4)
    z = (3 * rng.standard_normal((64, 512))).astype(np.float32)
    idx, gate = oracle.select(z, 10)
    zs = np.take_along_axis(z, idx, 1).astype(np.float64)
    ref = np.exp(zs - zs.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    assert np.max(np.abs(gate - ref)) <= 1e-7
    assert np.all(np.abs(gate.astype(np.float64).sum(1) - 1) <= 1e-6)
    # invariants: k distinct ids; every selected logit >= every unselected one; ordered
    for t in range(64):
        assert len(set(idx[t])) == 10
        sel = z[t, idx[t]]
        rest = np.delete(z[t], idx[t])
        assert sel.min() >= rest.max()
        assert np.all(np.diff(sel) <= 0)


# ------------------------------------------------------------------ margins
# The margin of a token is the smallest gap between neighbours in the list
# of its k+1 largest logits, sorted in descending order (all E logits when
# E <= k+1): a margin above the rounding error of any summation order makes
# the ordered top-k and the (k+1)-th exclusion unique.
@pytest.mark.parametrize("z,k,expect", [
    # smallest gap between ranks 1 and 2 (logits stored out of order)
    ([2.0, 5.0, 0.0, 3.5, 4.0, 1.0], 3, 0.5),
    # smallest gap between ranks k and k+1
    ([5.0, 3.0, -1.0, 1.0, 0.875], 3, 0.125),
    # a tiny gap below rank k+1 does not count
    ([0.0, 5.0, 3.0, 1.0, -0.0009765625], 2, 2.0),
    # an exact tie inside the top-(k+1) gives 0, wherever the tied pair sits
    ([1.0, 2.0, 2.0, 0.0], 2, 0.0),
    ([4.0, 1.0, 3.0, 1.0, -2.0], 3, 0.0),
    # a tie exactly at ranks k+1 and k+2 does not count
    ([5.0, 1.0, 3.0, 1.0, -2.0], 2, 2.0),
    # E = k + 1: every logit is in the list
    ([0.0, 1.0, 3.0], 2, 1.0),
    # E = k: the k logits alone
    ([1.0, 2.5], 2, 1.5),
    # negative logits and a single gap
    ([-7.0, -3.0], 1, 4.0),
])
def test_topk_margin_hand_examples(z, k, expect):
    m = oracle.topk_margin(np.array([z], np.float32), k)
    assert m.shape == (1,) and float(m[0]) == expect


def test_topk_margin_against_numpy_sort():
    """Brute force: np.sort of each row, gaps of its k+1 largest."""
    rng = np.random.default_rng(21)
    for E, k in ((16, 2), (16, 5), (64, 10), (512, 10), (11, 10)):
        z = rng.standard_normal((300, E)).astype(np.float32)
        z[:30, 3] = z[:30, 7]                      # planted ties, inside or outside the top
        z[30:60] = np.round(z[30:60] * 8) / 8      # coarse grid: many equal gaps and ties
        s = -np.sort(-z.astype(np.float64), axis=1)[:, : min(k + 1, E)]
        ref = np.min(s[:, :-1] - s[:, 1:], axis=1)
        got = oracle.topk_margin(z, k).astype(np.float64)
        assert np.array_equal(got, ref.astype(np.float32).astype(np.float64)), (E, k)


def test_topk_margin_sees_router_bias():
    """The margin is taken on the biased logits that the top-k uses: a bias
    that brings two experts within 2^-12 of each other must show up, and one
    that separates them must too.  One-hot router rows and integer inputs
    keep every logit exact."""
    E, d, k = 8, 16, 3
    Wr = np.zeros((E, d), np.float32)
    for e in range(E):
        Wr[e, e] = 1.0
    u = np.zeros((1, d), np.float32)
    u[0, :E] = [9, 1, 7, 3, 5, 0, 2, 4]            # unbiased top-4: 9, 7, 5, 4 -> margin 1
    assert float(oracle.topk_margin(oracle.logits(u, Wr), k)[0]) == 1.0
    bias = np.zeros(E, np.float32)
    bias[4] = 2.0 - 2.0 ** -12                     # expert 4: 7 - 2^-12, next to expert 2's 7
    assert float(oracle.topk_margin(oracle.logits(u, Wr, bias), k)[0]) == 2.0 ** -12
    bias[:] = 0.0
    bias[[0, 2, 4, 7]] = [30.0, 20.0, 10.0, 0.0]   # 39, 27, 15, 4 -> margin 11
    assert float(oracle.topk_margin(oracle.logits(u, Wr, bias), k)[0]) == 11.0


def test_generated_tokens_meet_the_margin():
    """The token generator's guarantee, checked on its output with numpy."""
    w = synth.WORKLOADS["decode"]
    L = W.layer_data(w, 0)
    x, attempts = W.draw_tokens(w, L["Wr"], None, range(64), rep=5)
    z = synth.bf16_to_f32(x).astype(np.float64) @ L["Wr"].astype(np.float64).T
    s = -np.sort(-z, axis=1)[:, : w.top_k + 1]
    assert np.min(s[:, :-1] - s[:, 1:]) >= W.MARGIN * (1 - 1e-4)
    assert attempts.max() >= 1                     # some tokens needed a redraw


# ------------------------------------------------------------- permutation
def test_permute_is_stable_sort():
    rng = np.random.default_rng(6)
    T, k, E = 300, 10, 64
    idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)], np.int32)
    counts, offsets, perm, pos = oracle.permute(idx, E)
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts) and offsets[-1] == T * k
    assert np.array_equal(perm, np.argsort(idx.ravel(), kind="stable"))
    assert np.array_equal(np.sort(perm), np.arange(T * k))          # bijection
    assert np.array_equal(pos[perm], np.arange(T * k))              # inverse


def test_misses_are_filtered_routing():
    rng = np.random.default_rng(7)
    T, k, E = 50, 10, 512
    idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)], np.int32)
    gate = rng.random((T, k)).astype(np.float32)
    mask = rng.integers(0, 2 ** 32, size=16, dtype=np.uint64).astype(np.uint32)
    te, w, n = oracle.misses(idx, gate, mask, T * k)
    ref = [(t, int(idx[t, r]), gate[t, r]) for t in range(T) for r in range(k)
           if not (int(mask[idx[t, r] // 32]) >> int(idx[t, r] % 32)) & 1]
    assert n == len(ref)
    assert [(int(a), int(b)) for a, b in te] == [(a, b) for a, b, _ in ref]
    assert np.array_equal(w, np.array([c for _, _, c in ref], np.float32))
    te2, w2, n2 = oracle.misses(idx, gate, mask, 7)                # overflow: true count, first cap
    assert n2 == n and np.array_equal(te2, te[:7])


# ------------------------------------------------------------------ expert
def _silu(v):
    return v / (1 + np.exp(-v))


def test_expert_ffn_matches_dense_numpy_mlp():
    w = synth.WORKLOADS["tiny"]
    codes, scales = synth.expert_codes(w, 0, 3), synth.expert_scales(w, 0, 3)
    d, f, mb, sb = w.d_model, w.d_ff, w.code_bytes_per_matrix, w.d_model * w.d_ff // 256
    Wg = oracle.dequant(3, codes[:mb], scales[:sb], f, d)
    Wu = oracle.dequant(3, codes[mb:2 * mb], scales[sb:2 * sb], f, d)
    Wd = oracle.dequant(3, codes[2 * mb:], scales[2 * sb:], d, f)
    u = np.random.default_rng(8).standard_normal(d)
    ref = Wd @ (_silu(Wg @ u) * (Wu @ u))
    got = oracle.expert_ffn(3, codes, scales, d, f, u)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
    # gate and up are not interchangeable: swapping them must change the result
    swapped = Wd @ (_silu(Wu @ u) * (Wg @ u))
    assert np.max(np.abs(swapped - ref)) > 1e-3 * np.max(np.abs(ref))


def test_expert_ffn_closed_form_constant_codes():
    d, f = 256, 128
    g = _golden("format_3bit_unit.txt")
    mat = np.tile(_hexbytes(g["unit_all_7"]), d * f * 3 // 8 // 12)
    codes = np.concatenate([mat, mat, mat])
    s = 0.0625
    scales = np.full(3 * d * f // 256, 0x2C00, np.uint16)          # 2^-4 everywhere
    a = 0.75
    u = np.full(d, a)
    y = oracle.expert_ffn(3, codes, scales, d, f, u)
    gg = d * 3.5 * s * a
    h = gg / (1 + math.exp(-gg)) * gg
    assert np.allclose(y, f * 3.5 * s * h, rtol=1e-14, atol=0)
    # 2-bit: all codes 0 -> w = -1.5 * s
    codes2 = np.zeros(3 * d * f // 4, np.uint8)
    y2 = oracle.expert_ffn(2, codes2, scales, d, f, u)
    g2 = -d * 1.5 * s * a
    h2 = g2 / (1 + math.exp(-g2)) * g2
    assert np.allclose(y2, -f * 1.5 * s * h2, rtol=1e-14, atol=0)


def test_grouped_equals_per_expert_call():
    w = synth.WORKLOADS["tiny"]
    codes, scales = synth.expert_codes(w, 0, 1), synth.expert_scales(w, 0, 1)
    u = np.random.default_rng(9).standard_normal((6, w.d_model))
    yg = oracle.expert_ffn_grouped(3, codes, scales, w.d_model, w.d_ff, u)
    for t in range(6):
        assert np.array_equal(yg[t], oracle.expert_ffn(3, codes, scales, w.d_model, w.d_ff, u[t]))


# ------------------------------------------------------------------- layer
def _tiny_layer(mask=None):
    w = synth.WORKLOADS["tiny"]
    L = W.layer_data(w, 0)
    x, _ = W.draw_tokens(w, L["Wr"], None, range(w.tokens))
    u = synth.bf16_to_f32(x)
    return w, L, u


def test_tiny_layer_matches_dense_reference():
    w, L, u = _tiny_layer()
    r = oracle.moe_layer(3, w.n_experts, w.top_k, w.d_model, w.d_ff, u, L["Wr"], L["codes"], L["scales"])
    # independent composition: numpy float64 dense MLPs on the oracle-dequantised weights,
    # numpy softmax/top-k on numpy logits
    z = u.astype(np.float64) @ L["Wr"].astype(np.float64).T
    out = np.zeros((w.tokens, w.d_model))
    for t in range(w.tokens):
        order = sorted(range(w.n_experts), key=lambda e: (-z[t, e], e))[: w.top_k]
        assert list(r["idx"][t]) == order
        p = np.exp(z[t, order] - z[t, order].max())
        p /= p.sum()
        assert np.max(np.abs(r["gate"][t] - p)) < 1e-6
        ys = []
        for e in order + [w.n_experts]:
            c = W.expert_slice(w, L["codes"], e, "codes")
            s = W.expert_slice(w, L["scales"], e, "scales")
            mb, sb = w.code_bytes_per_matrix, w.d_model * w.d_ff // 256
            Wg = oracle.dequant(3, c[:mb], s[:sb], w.d_ff, w.d_model)
            Wu = oracle.dequant(3, c[mb:2 * mb], s[sb:2 * sb], w.d_ff, w.d_model)
            Wd = oracle.dequant(3, c[2 * mb:], s[2 * sb:], w.d_model, w.d_ff)
            ut = u[t].astype(np.float64)
            ys.append(Wd @ (_silu(Wg @ ut) * (Wu @ ut)))
        out[t] = ys[-1] + sum(float(r["gate"][t, i]) * ys[i] for i in range(w.top_k))
    rms = np.sqrt(np.mean(out ** 2))
    assert np.max(np.abs(r["out"] - out)) <= 1e-6 * rms


def test_layer_grouped_equals_per_token():
    w, L, u = _tiny_layer()
    a = oracle.moe_layer(3, w.n_experts, w.top_k, w.d_model, w.d_ff, u, L["Wr"], L["codes"], L["scales"],
                         grouped=True)
    b = oracle.moe_layer(3, w.n_experts, w.top_k, w.d_model, w.d_ff, u, L["Wr"], L["codes"], L["scales"],
                         grouped=False)
    assert np.array_equal(a["out"], b["out"])


def test_mask_identity_full_equals_masked_plus_misses():
    w, L, u = _tiny_layer()
    mask = np.array([0b1010_0110_1100_1011], np.uint32)
    full = oracle.moe_layer(3, w.n_experts, w.top_k, w.d_model, w.d_ff, u, L["Wr"], L["codes"], L["scales"])
    part = oracle.moe_layer(3, w.n_experts, w.top_k, w.d_model, w.d_ff, u, L["Wr"], L["codes"], L["scales"],
                            mask=mask)
    assert part["miss_count"] > 0
    recon = part["out"].astype(np.float64)
    for (t, e), g in zip(part["miss_te"], part["miss_w"]):
        c = W.expert_slice(w, L["codes"], e, "codes")
        s = W.expert_slice(w, L["scales"], e, "scales")
        recon[t] += float(g) * oracle.expert_ffn(3, c, s, w.d_model, w.d_ff, u[t].astype(np.float64))
    rms = np.sqrt(np.mean(full["out"].astype(np.float64) ** 2))
    assert np.max(np.abs(recon - full["out"])) <= 1e-6 * rms
    # routing is unaffected by the mask
    assert np.array_equal(full["idx"], part["idx"]) and np.array_equal(full["perm"], part["perm"])


def test_rmsnorm_closed_forms():
    x = np.array([[2.0] * 8, [-3.0, 3.0] * 4], np.float32)
    u = oracle.rmsnorm(x, eps=0.0)
    assert np.allclose(u, np.sign(x), rtol=0, atol=1e-7)
    rng = np.random.default_rng(10)
    x = (5 * rng.standard_normal((4, 2048))).astype(np.float32)
    ref = x / np.sqrt((x.astype(np.float64) ** 2).mean(1, keepdims=True) + 1e-6)
    assert np.max(np.abs(oracle.rmsnorm(x) - ref)) <= 1e-6


def test_zipf_targets_and_generated_popularity():
    w = synth.WORKLOADS["zipf_prefill"]
    t = synth.zipf_targets(512, 10, 1.1)
    assert abs(t.sum() - 10) < 1e-9 and t[0] == 1.0 and np.all(np.diff(t) <= 0)
    # popularity under the calibrated bias, measured with the oracle's router on
    # generated tokens, follows the capped Zipf targets at the head of the ranking
    bias = synth.zipf_bias(w)
    Wr = synth.router_weights(w, 0)
    x = synth.x_tokens(w, range(1024))
    idx, _ = oracle.select(oracle.logits(synth.bf16_to_f32(x), Wr, bias), 10)
    pop = np.bincount(idx.ravel(), minlength=512) / 1024
    ranks = synth.expert_ranks(w)
    assert np.all(np.abs(pop[ranks[:20]] - t[:20]) < 0.12)
    hit = np.isin(idx, ranks[: w.resident]).mean()
    assert 0.6 < hit < 0.99        # the pages' hit-rate band is roughly 67.8-98%


def test_resident_topn_hand_example():
    """Hand-worked resident sets: largest counts first, equal counts to the
    lower index, n = 0 and n = E at the ends."""
    counts = [5, 9, 9, 0, 7, 9, 1, 7]
    # order by (count desc, index asc): 1, 2, 5, 4, 7, 0, 6, 3
    assert list(oracle.resident_topn(counts, 3)) == [(1 << 1) | (1 << 2) | (1 << 5)]
    assert list(oracle.resident_topn(counts, 4)) == [(1 << 1) | (1 << 2) | (1 << 5) | (1 << 4)]
    assert list(oracle.resident_topn(counts, 5)) == [(1 << 1) | (1 << 2) | (1 << 5) | (1 << 4) | (1 << 7)]
    assert list(oracle.resident_topn(counts, 0)) == [0]
    assert list(oracle.resident_topn(counts, 8)) == [0xFF]
    # across words: 40 experts, the top 2 in the second word
    c40 = [0] * 40
    c40[33], c40[38] = 4, 4
    assert list(oracle.resident_topn(c40, 2)) == [0, (1 << 1) | (1 << 6)]
    # all equal: the lowest indices
    assert list(oracle.resident_topn([3] * 40, 35)) == [0xFFFFFFFF, 0x7]
