"""Test-side assembly of workload inputs.

Inputs come from ``synth`` (seeded, counter-based).  Token rows whose
router logits have an adjacent gap below MARGIN among the sorted top-(k+1)
are redrawn from their own sub-stream (token, attempt), so the ordered top-k
is unique and robust to fp32 summation order; the margins are measured on the
oracle's logits.  Expected values come only from ``oracle``.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

MARGIN = 1e-3


def layer_data(w: synth.Workload, layer: int, router_attempt: int = 0) -> dict:
    """All inputs of one layer as numpy arrays (fits for one full-size layer)."""
    codes = np.empty(w.experts_total * w.code_bytes_per_expert, dtype=np.uint8)
    synth.layer_codes_into(w, layer, codes.ctypes.data)
    d = dict(codes=codes, scales=synth.layer_scales(w, layer),
             Wr=synth.router_weights(w, layer, router_attempt), bias=None, mask=None)
    if w.zipf_s > 0:
        d["bias"] = synth.zipf_bias(w)
    if w.resident > 0:
        d["mask"] = synth.resident_mask(w)
    return d


def draw_tokens(w: synth.Workload, Wr, bias, token_ids, rep: int = 0, max_attempts: int = 200):
    """bf16 token rows with top-(k+1) margins >= MARGIN on the oracle logits."""
    token_ids = np.asarray(list(token_ids))
    attempts = np.zeros(len(token_ids), dtype=np.int64)
    x = synth.x_tokens(w, token_ids, attempts, rep)
    todo = np.arange(len(token_ids))
    for _ in range(max_attempts):
        z = oracle.logits(synth.bf16_to_f32(x[todo]), Wr, bias)
        bad = todo[oracle.topk_margin(z, w.top_k) < MARGIN]
        if bad.size == 0:
            return x, attempts
        attempts[bad] += 1
        x[bad] = synth.x_tokens(w, token_ids[bad], attempts[bad], rep)
        todo = bad
    raise RuntimeError("could not draw tokens with the required margin")


def expert_slice(w: synth.Workload, arr: np.ndarray, e: int, what: str) -> np.ndarray:
    if what == "codes":
        n = w.code_bytes_per_expert
    else:
        n = w.blocks_per_expert
    return arr[e * n:(e + 1) * n]
