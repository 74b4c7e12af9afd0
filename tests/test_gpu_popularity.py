"""Running expert popularity and the resident set derived from it, through
the C ABI: the n most-picked experts as a mask (count desc, index asc)
against the oracle, the int64 accumulation, and the online resident set on
the Zipf-skewed 32K prompt (each chunk's mask from the counts of the chunks
before it)."""
from __future__ import annotations

import numpy as np
import pytest

import bit_routed_expert_amd as brx
import oracle
import synth
from tests import gpu_util as G
from tests import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("E,n", [(16, 0), (16, 5), (512, 165), (512, 512), (1000, 300), (1024, 1)])
def test_resident_topn_matches_oracle(E, n):
    t = G.torch()
    rng = np.random.default_rng(E + n)
    counts = rng.integers(0, 6, E).astype(np.int64) * 1_000_000_007   # many ties, values past 2^32
    print(f"case resident_topn E={E} n={n}", flush=True)
    acc = t.from_numpy(counts).cuda()
    mask = t.full(((E + 31) // 32,), 0x5A5A5A5A, dtype=t.int32, device="cuda")   # every word is written
    brx.resident_topn(acc, E, n, mask)
    t.cuda.synchronize()
    np.testing.assert_array_equal(mask.cpu().numpy().view(np.uint32), oracle.resident_topn(counts, n))


def test_counts_accumulate_sums_calls():
    t = G.torch()
    E = 512
    rng = np.random.default_rng(3)
    parts = [rng.integers(0, 2**31 - 1, E).astype(np.int32) for _ in range(3)]
    acc = t.zeros(E, dtype=t.int64, device="cuda")
    for p in parts:
        brx.counts_accumulate(acc, t.from_numpy(p).cuda(), E)
    t.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), np.sum([p.astype(np.int64) for p in parts], axis=0))


def test_online_resident_set_on_zipf_chunks():
    t = G.torch()
    w = synth.WORKLOADS["zipf_prefill"]
    T, E, k = w.tokens_per_call, w.n_experts, w.top_k
    L = W.layer_data(w, 0)
    sh = G.shape_of(w)
    ld = brx.LayerData(router_w=G.dev(L["Wr"]), codes=G.dev(np.zeros(16, np.uint8)),
                       scales=G.dev(np.zeros(8, np.uint16)), router_bias=G.dev(L["bias"]))
    nb = brx.workspace_bytes(sh, T)
    ws = t.zeros(nb, dtype=t.uint8, device="cuda")
    acc = t.zeros(E, dtype=t.int64, device="cuda")
    mask = t.zeros((E + 31) // 32, dtype=t.int32, device="cuda")
    static = synth.resident_mask(w)
    sbits = np.unpackbits(static.view(np.uint8), bitorder="little")[:E].astype(bool)
    acc_host = np.zeros(E, np.int64)
    hits_dyn, hits_static = [], []
    for c in range(w.calls):
        x = G.dev(synth.x_tokens(w, range(c * T, (c + 1) * T)))
        out = dict(topk_idx=t.empty((T, k), dtype=t.int32, device="cuda"),
                   counts=t.empty(E, dtype=t.int32, device="cuda"))
        brx.route(sh, ld, x, 0, T, out, ws, nb)
        t.cuda.synchronize()
        idx = out["topk_idx"].cpu().numpy()
        if c > 0:   # this chunk against the mask learnt from the chunks before it
            dbits = np.unpackbits(mask.cpu().numpy().view(np.uint8), bitorder="little")[:E].astype(bool)
            hits_dyn.append(dbits[idx].mean())
            hits_static.append(sbits[idx].mean())
        brx.counts_accumulate(acc, out["counts"], E)
        brx.resident_topn(acc, E, w.resident, mask)
        t.cuda.synchronize()
        acc_host += out["counts"].cpu().numpy()
        np.testing.assert_array_equal(acc.cpu().numpy(), acc_host)
        np.testing.assert_array_equal(mask.cpu().numpy().view(np.uint32), oracle.resident_topn(acc_host, w.resident))
    print(f"hit rate over chunks 1..{w.calls - 1}: online {np.mean(hits_dyn):.4f}, static {np.mean(hits_static):.4f}")
