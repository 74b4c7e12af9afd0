"""ORACLE for the sparse MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library
``bit_routed_expert_amd`` and its binding) never imports, links or runs it,
and it shares no code, header, table or constant generator with that path.

The arithmetic lives in ``oracle.c`` (plain C, double precision, written from
the layer's definition; its header states the definition, the byte layout of
the weight blocks and the passages of the pages it follows).  This module only
marshals numpy arrays into it and chains layers.

Readings of the pages that the oracle fixes (listed with reasons in the design
notes):
  * layer l > 0 consumes rmsnorm(x_l) (no learnt gain, eps 1e-6) of the fp32
    residual stream x_l; layer 0 consumes its input as given;
  * x_{l+1} = x_l + out_l in fp32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

RMS_EPS = 1e-6


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc.  Strict IEEE double (no fast-math, no
    contraction) so the summation order written in oracle.c is the one run."""
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-mavx2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                               "-fno-fast-math", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i32, i64, vp, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        lib.oracle_half_to_double.restype = dbl
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_code_at.restype = i32
        lib.oracle_code_at.argtypes = [i32, vp, i64, i64, i64, i64]
        lib.oracle_unpack_codes.argtypes = [i32, vp, i64, i64, vp]
        lib.oracle_pack_codes.argtypes = [i32, vp, i64, i64, vp]
        lib.oracle_dequant.argtypes = [i32, vp, vp, i64, i64, vp]
        lib.oracle_logits.argtypes = [vp, i32, i32, vp, vp, i32, vp, i32]
        lib.oracle_select.argtypes = [vp, i32, i32, i32, vp, vp]
        lib.oracle_topk_margin.argtypes = [vp, i32, i32, i32, vp]
        lib.oracle_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        lib.oracle_misses.restype = i32
        lib.oracle_misses.argtypes = [vp, vp, i32, i32, vp, vp, vp, i32]
        lib.oracle_expert_ffn.argtypes = [i32, vp, vp, i32, i32, vp, vp]
        lib.oracle_expert_ffn_grouped.argtypes = [i32, vp, vp, i32, i32, i32, vp, vp, i32]
        lib.oracle_moe_layer.restype = i32
        lib.oracle_moe_layer.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                         vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32]
        lib.oracle_rmsnorm.argtypes = [vp, i32, i32, dbl, vp]
        _lib = lib
    return _lib


def _threads() -> int:
    """Threads the oracle uses: every CPU this process may run on, or fewer
    when OMP_NUM_THREADS says so (a machine shared between jobs sets it to
    this job's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        n = os.cpu_count() or 4
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return None if a is None else a.ctypes.data


# ------------------------------------------------------------------ format
def half_to_float(h: int) -> float:
    return float(_load().oracle_half_to_double(int(h) & 0xFFFF))


def unpack_codes(bits: int, mat: np.ndarray, out: int, inn: int) -> np.ndarray:
    mat = _c(mat, np.uint8)
    assert mat.size == out * inn * bits // 8
    codes = np.empty((out, inn), dtype=np.uint8)
    _load().oracle_unpack_codes(bits, _p(mat), out, inn, _p(codes))
    return codes


def pack_codes(bits: int, codes: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.uint8)
    out, inn = codes.shape
    mat = np.empty(out * inn * bits // 8, dtype=np.uint8)
    _load().oracle_pack_codes(bits, _p(codes), out, inn, _p(mat))
    return mat


def dequant(bits: int, mat: np.ndarray, scales: np.ndarray, out: int, inn: int) -> np.ndarray:
    mat, scales = _c(mat, np.uint8), _c(scales, np.uint16)
    w = np.empty((out, inn), dtype=np.float64)
    _load().oracle_dequant(bits, _p(mat), _p(scales), out, inn, _p(w))
    return w


# ------------------------------------------------------------------ router
def logits(u: np.ndarray, Wr: np.ndarray, bias=None) -> np.ndarray:
    u, Wr = _c(u, np.float32), _c(Wr, np.float32)
    T, d = u.shape
    E = Wr.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    z = np.empty((T, E), dtype=np.float32)
    _load().oracle_logits(_p(u), T, d, _p(Wr), _p(b), E, _p(z), _threads())
    return z


def select(z: np.ndarray, k: int):
    z = _c(z, np.float32)
    T, E = z.shape
    assert 1 <= k <= min(E, 64)
    idx = np.empty((T, k), dtype=np.int32)
    gate = np.empty((T, k), dtype=np.float32)
    _load().oracle_select(_p(z), T, E, k, _p(idx), _p(gate))
    return idx, gate


def topk_margin(z: np.ndarray, k: int) -> np.ndarray:
    z = _c(z, np.float32)
    T, E = z.shape
    m = np.empty(T, dtype=np.float32)
    _load().oracle_topk_margin(_p(z), T, E, k, _p(m))
    return m


def permute(idx: np.ndarray, E: int):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(T * k, dtype=np.int32)
    pos = np.empty(T * k, dtype=np.int32)
    _load().oracle_permute(_p(idx), T, k, E, _p(counts), _p(offsets), _p(perm), _p(pos))
    return counts, offsets, perm, pos


def misses(idx: np.ndarray, gate: np.ndarray, mask, cap: int):
    idx, gate = _c(idx, np.int32), _c(gate, np.float32)
    T, k = idx.shape
    m = None if mask is None else _c(mask, np.uint32)
    te = np.zeros((max(cap, 1), 2), dtype=np.int32)
    w = np.zeros(max(cap, 1), dtype=np.float32)
    n = _load().oracle_misses(_p(idx), _p(gate), T, k, _p(m), _p(te), _p(w), cap)
    return te[: min(n, cap)], w[: min(n, cap)], n


# ------------------------------------------------------------------ expert
def expert_ffn(bits: int, codes: np.ndarray, scales: np.ndarray, d: int, f: int, u: np.ndarray) -> np.ndarray:
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint16)
    u = _c(u, np.float64)
    y = np.empty(d, dtype=np.float64)
    _load().oracle_expert_ffn(bits, _p(codes), _p(scales), d, f, _p(u), _p(y))
    return y


def expert_ffn_grouped(bits: int, codes, scales, d: int, f: int, u: np.ndarray) -> np.ndarray:
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint16)
    u = _c(u, np.float64)
    n = u.shape[0]
    y = np.empty((n, d), dtype=np.float64)
    _load().oracle_expert_ffn_grouped(bits, _p(codes), _p(scales), d, f, n, _p(u), _p(y), _threads())
    return y


# ------------------------------------------------------------------- layer
def moe_layer(bits, E, k, d, f, u, Wr, codes, scales, bias=None, mask=None, miss_cap=None, grouped=True,
              threads=None):
    """One layer.  codes: uint8 of (E+1) experts, expert-major; scales: uint16.
    Returns a dict with idx, gate, counts, offsets, perm, pos, out, miss_te,
    miss_w, miss_count.  threads: OpenMP threads (default: _threads())."""
    u = _c(u, np.float32)
    T = u.shape[0]
    Wr = _c(Wr, np.float32)
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint16)
    assert codes.size == (E + 1) * 3 * d * f * bits // 8
    assert scales.size == (E + 1) * 3 * d * f // 256
    b = None if bias is None else _c(bias, np.float32)
    m = None if mask is None else _c(mask, np.uint32)
    cap = T * k if miss_cap is None else miss_cap
    r = dict(idx=np.empty((T, k), np.int32), gate=np.empty((T, k), np.float32),
             counts=np.empty(E, np.int32), offsets=np.empty(E + 1, np.int32),
             perm=np.empty(T * k, np.int32), pos=np.empty(T * k, np.int32),
             out=np.empty((T, d), np.float32), miss_te=np.zeros((max(cap, 1), 2), np.int32),
             miss_w=np.zeros(max(cap, 1), np.float32))
    n = _load().oracle_moe_layer(bits, E, k, d, f, T, _p(u), _p(Wr), _p(b), _p(codes), _p(scales), _p(m),
                                 _p(r["idx"]), _p(r["gate"]), _p(r["counts"]), _p(r["offsets"]), _p(r["perm"]),
                                 _p(r["pos"]), _p(r["out"]), _p(r["miss_te"]), _p(r["miss_w"]), cap,
                                 1 if grouped else 0, _threads() if threads is None else int(threads))
    r["miss_count"] = n
    r["miss_te"] = r["miss_te"][: min(n, cap)]
    r["miss_w"] = r["miss_w"][: min(n, cap)]
    return r


def rmsnorm(x: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    x = _c(x, np.float32)
    T, d = x.shape
    u = np.empty_like(x)
    _load().oracle_rmsnorm(_p(x), T, d, eps, _p(u))
    return u


def layer_input(x_l: np.ndarray, layer: int, norm_first: bool = False) -> np.ndarray:
    """MoE input of layer `layer` from the residual stream x_l."""
    return rmsnorm(x_l) if (layer > 0 or norm_first) else _c(x_l, np.float32)


def residual_add(x_l: np.ndarray, out: np.ndarray) -> np.ndarray:
    """x_{l+1} = x_l + out_l, one fp32 rounding per element."""
    return (_c(x_l, np.float32) + _c(out, np.float32)).astype(np.float32)


def resident_topn(counts, n: int) -> np.ndarray:
    """uint32 bitset [ceil(E/32)] of the n experts with the largest counts,
    ties to the lower index: a stable sort of the experts by descending count
    (the cache keeps the most-used experts: wiselychen.com, technique 2
    "專家快取與 CPU／GPU 分工")."""
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.shape[0]
    order = sorted(range(E), key=lambda e: (-int(counts[e]), e))
    mask = np.zeros((E + 31) // 32, dtype=np.uint32)
    for e in order[:n]:
        mask[e // 32] |= np.uint32(1) << np.uint32(e % 32)
    return mask
