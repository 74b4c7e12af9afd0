"""Seeded synthetic inputs for the MoE layer forward.

This module is shared by the tests, the oracle checks and the benchmark.  It
holds none of the layer's arithmetic (no routing, no dequantisation, no
matmul): it only draws the inputs the layer consumes, from counter-based
streams (SplitMix64 finaliser over (seed, labels, index), implemented in
``synth.c``) so that any slice can be regenerated on its own.

Workload shapes follow the pages' model description: 512 routed experts per
layer, 10 routed + 1 shared per token, 48 layers (greenbean-ai, "Strata 如何讓
12GB 顯卡跑 Qwen3.8-Flash-Next？", section 一; wiselychen.com, "30 秒定位" fact
table).  Sizes d = 2048, f = 768, the block format and the distributions are
this library's fixed workload definitions (the pages name only the IQ3/Q2
quantisation classes).

Packed expert codes are plain uniform random bytes: every bit layout of
b-bit codes is a bijection on bit strings, so uniform bytes are uniform codes
in 0..2^b-1 whatever the layout, and the generator never needs to know it.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# stream labels
TAG_X, TAG_WR, TAG_CODES, TAG_SCALES, TAG_RANK, TAG_BIAS_MC, TAG_REP = 1, 2, 3, 4, 5, 6, 7


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (OpenMP)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [u64, u64, u64, u64, u64]
        lib.synth_bytes.argtypes = [u64, u64, u64, vp, i32]
        lib.synth_normal_f64.argtypes = [u64, u64, u64, vp, i32]
        lib.synth_normal_f32.argtypes = [u64, u64, u64, dbl, vp, i32]
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, vp, i32]
        lib.synth_uniform_f16.argtypes = [u64, u64, u64, dbl, dbl, dbl, vp, i32]
        lib.synth_uniform_f64.argtypes = [u64, u64, u64, vp, i32]
        lib.synth_words.argtypes = [u64, u64, u64, vp]
        _lib = lib
    return _lib


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except Exception:  # pragma: no cover
        return 4


def key(seed: int, a: int = 0, b: int = 0, c: int = 0, d: int = 0) -> int:
    return int(_load().synth_key(seed & (2**64 - 1), a, b, c, d))


# ---------------------------------------------------------------- primitives
def random_bytes(k: int, n: int, offset: int = 0, out: Optional[np.ndarray] = None) -> np.ndarray:
    if out is None:
        out = np.empty(n, dtype=np.uint8)
    assert out.dtype == np.uint8 and out.size == n and out.flags.c_contiguous
    _load().synth_bytes(k, offset, n, out.ctypes.data, _threads())
    return out


def random_bytes_into(k: int, n: int, ptr: int, offset: int = 0) -> None:
    """Fill n bytes at a raw host address (e.g. a pinned torch buffer)."""
    _load().synth_bytes(k, offset, n, ctypes.c_void_p(ptr), _threads())


def normal_f64(k: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_normal_f64(k, offset, n, out.ctypes.data, _threads())
    return out


def normal_f32(k: int, n: int, stddev: float = 1.0, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal_f32(k, offset, n, float(stddev), out.ctypes.data, _threads())
    return out


def normal_bf16(k: int, n: int, offset: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0,1) deviates, rounded to nearest even."""
    out = np.empty(n, dtype=np.uint16)
    _load().synth_normal_bf16(k, offset, n, out.ctypes.data, _threads())
    return out


def uniform_f16(k: int, n: int, lo: float, hi: float, mult: float, offset: int = 0) -> np.ndarray:
    """fp16 bit patterns (uint16) of U(lo, hi) * mult, rounded to nearest even."""
    out = np.empty(n, dtype=np.uint16)
    _load().synth_uniform_f16(k, offset, n, lo, hi, mult, out.ctypes.data, _threads())
    return out


def uniform_f64(k: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform_f64(k, offset, n, out.ctypes.data, _threads())
    return out


def words(k: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_words(k, offset, n, out.ctypes.data)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- workloads
@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: layer shape, batch, depth and input recipe."""
    name: str
    n_experts: int
    top_k: int
    d_model: int
    d_ff: int
    bits: int            # 3 or 2
    tokens: int          # total tokens
    layers: int = 1
    chunk: int = 0       # tokens per call (0: all at once)
    zipf_s: float = 0.0  # >0: router bias calibrated to capped Zipf popularity
    resident: int = 0    # >0: resident mask = this many most popular experts
    seed: int = 0x5EED0000
    n_shared: int = 1

    @property
    def calls(self) -> int:
        return 1 if not self.chunk else self.tokens // self.chunk

    @property
    def tokens_per_call(self) -> int:
        return self.chunk or self.tokens

    @property
    def code_bytes_per_matrix(self) -> int:
        return self.d_model * self.d_ff * self.bits // 8

    @property
    def code_bytes_per_expert(self) -> int:
        return 3 * self.code_bytes_per_matrix

    @property
    def blocks_per_expert(self) -> int:
        return 3 * self.d_model * self.d_ff // 256

    @property
    def experts_total(self) -> int:
        return self.n_experts + self.n_shared


WORKLOADS = {
    # small layer: 16 routed top-2 + 1 shared, d=256, f=128, T=4, 3-bit
    "tiny": Workload("tiny", 16, 2, 256, 128, 3, 4, seed=0x5EED0001),
    # full-size decode layer, one token, 3-bit
    "decode": Workload("decode", 512, 10, 2048, 768, 3, 1, seed=0x5EED0002),
    # MTP verify: 5 tokens through 48 independent full-size 3-bit layers
    "mtp_verify": Workload("mtp_verify", 512, 10, 2048, 768, 3, 5, layers=48, seed=0x5EED0003),
    # prefill chunk: 4096 tokens, one full-size layer, 2-bit blocks
    "prefill_2bit": Workload("prefill_2bit", 512, 10, 2048, 768, 2, 4096, seed=0x5EED0004),
    # skewed long prefill: 32768 tokens in 4096-token calls, Zipf(1.1) popularity, 165 resident
    "zipf_prefill": Workload("zipf_prefill", 512, 10, 2048, 768, 3, 32768, chunk=4096, zipf_s=1.1,
                             resident=165, seed=0x5EED0005),
}


def x_tokens(w: Workload, token_ids, attempts=None, rep: int = 0) -> np.ndarray:
    """bf16 bit patterns [n][d] of N(0,1) inputs; token t's row is drawn from its own
    stream (token id, redraw attempt, repetition) so one row can be redrawn alone."""
    token_ids = list(token_ids)
    out = np.empty((len(token_ids), w.d_model), dtype=np.uint16)
    for i, t in enumerate(token_ids):
        a = 0 if attempts is None else int(attempts[i])
        out[i] = normal_bf16(key(w.seed, TAG_X, t, a, rep), w.d_model)
    return out


def router_weights(w: Workload, layer: int, attempt: int = 0) -> np.ndarray:
    """fp32 [E][d] with entries N(0, 1/d)."""
    k = key(w.seed, TAG_WR, layer, attempt)
    return normal_f32(k, w.n_experts * w.d_model, 1.0 / math.sqrt(w.d_model)).reshape(w.n_experts, w.d_model)


def expert_codes_key(w: Workload, layer: int, expert: int) -> int:
    return key(w.seed, TAG_CODES, layer, expert)


def expert_codes(w: Workload, layer: int, expert: int) -> np.ndarray:
    """Packed code bytes of one expert (gate, up, down), uniform random."""
    return random_bytes(expert_codes_key(w, layer, expert), w.code_bytes_per_expert)


def expert_scales(w: Workload, layer: int, expert: int) -> np.ndarray:
    """fp16 bit patterns of the expert's per-block scales, U(0.5, 1.5)/sqrt(d)."""
    k = key(w.seed, TAG_SCALES, layer, expert)
    return uniform_f16(k, w.blocks_per_expert, 0.5, 1.5, 1.0 / math.sqrt(w.d_model))


def layer_codes_into(w: Workload, layer: int, ptr: int) -> None:
    """Write all E+1 experts' code bytes of one layer, expert-major, at a host address."""
    nb = w.code_bytes_per_expert
    for e in range(w.experts_total):
        random_bytes_into(expert_codes_key(w, layer, e), nb, ptr + e * nb)


def layer_scales(w: Workload, layer: int) -> np.ndarray:
    return np.concatenate([expert_scales(w, layer, e) for e in range(w.experts_total)])


# ------------------------------------------------------- skewed popularity
def zipf_targets(n: int, k: int, s: float) -> np.ndarray:
    """Capped Zipf popularity per rank: min(1, c * r^-s) with c chosen so the
    targets sum to k (a token picks each expert at most once, so plain Zipf
    is infeasible at the top ranks)."""
    r = np.arange(1, n + 1, dtype=np.float64)
    lo, hi = 0.0, float(k) * 10
    for _ in range(200):
        c = 0.5 * (lo + hi)
        if np.minimum(1.0, c * r ** -s).sum() > k:
            hi = c
        else:
            lo = c
    return np.minimum(1.0, 0.5 * (lo + hi) * r ** -s)


def expert_ranks(w: Workload) -> np.ndarray:
    """rank -> expert id: a seeded permutation of the routed experts."""
    ws = words(key(w.seed, TAG_RANK), w.n_experts)
    return np.argsort(ws, kind="stable").astype(np.int64)


def zipf_bias(w: Workload, samples: int = 4096, iters: int = 80) -> np.ndarray:
    """fp32 per-expert router bias so that expert popularity follows capped
    Zipf(s) over a seeded rank order.

    Calibrated on a model of the logits, not on the layer itself: for random
    router rows N(0, 1/d) and inputs N(0, 1) a token's logits are close to iid
    N(0, 1) across experts, so a fixed sample of iid normal logit vectors is
    drawn once and the bias is moved by a clipped log-ratio step towards the
    target pick rate, for a fixed number of iterations.
    """
    E, k = w.n_experts, w.top_k
    ranks = expert_ranks(w)
    target = np.empty(E)
    target[ranks] = zipf_targets(E, k, w.zipf_s)
    z = normal_f64(key(w.seed, TAG_BIAS_MC), samples * E).reshape(samples, E)
    b = np.zeros(E)
    for _ in range(iters):
        top = np.argpartition(-(z + b), k - 1, axis=1)[:, :k]
        pop = np.bincount(top.ravel(), minlength=E) / samples
        step = np.log(np.clip(target, 1e-4, 1.0)) - np.log(np.clip(pop, 0.5 / samples, 1.0))
        b = b + np.clip(0.7 * step, -0.5, 0.5)
    return b.astype(np.float32)


def resident_mask(w: Workload) -> np.ndarray:
    """uint32 bitset [ceil(E/32)] with the `resident` most popular ranks set."""
    ranks = expert_ranks(w)
    m = np.zeros((w.n_experts + 31) // 32, dtype=np.uint32)
    for e in ranks[: w.resident]:
        m[e // 32] |= np.uint32(1) << np.uint32(e % 32)
    return m
