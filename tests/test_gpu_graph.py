"""Capture of the forward in a HIP graph.

A forward call enqueues only kernel launches on the caller's stream (no
allocation, memset, copy or host synchronisation), so it can be captured in
a graph.  Replays with new inputs written into the captured input buffer
equal eager calls bit for bit, on the one-token kernels, the T = 2..8
kernels and the matrix-core path, with eager calls in between the replays.
"""
from __future__ import annotations

import numpy as np
import pytest

import bit_routed_expert_amd as brx
import synth
from tests import gpu_util as G
from tests import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T", [("decode", 1), ("decode", 5), ("tiny", 20)])
def test_graph_replays_equal_eager_calls(name, T):
    t = G.torch()
    w = synth.WORKLOADS[name]
    L = W.layer_data(w, 0)
    ld = G.layer_to_dev(L)
    sh = G.shape_of(w)
    xs = [W.draw_tokens(w, L["Wr"], None, range(T), rep=40 + i)[0] for i in range(3)]
    nb = brx.workspace_bytes(sh, T, 1)
    ws = t.zeros(nb, dtype=t.uint8, device="cuda")
    x_in = G.dev(xs[0]).clone()
    y = t.empty((T, w.d_model), dtype=t.float32, device="cuda")
    resid = t.empty((T, w.d_model), dtype=t.float32, device="cuda")
    idx = t.empty((T, w.top_k), dtype=t.int32, device="cuda")
    gate = t.empty((T, w.top_k), dtype=t.float32, device="cuda")
    ro = [dict(topk_idx=idx, topk_w=gate)]

    def call():
        brx.forward(sh, [ld], x_in, 0, T, y, ws, nb, resid_out=resid, route_outs=ro)

    def results():
        return [a.cpu().numpy().copy() for a in (y, resid, idx, gate)]

    print(f"case graph {name} T={T}", flush=True)
    eager = []
    for x in xs:
        x_in.copy_(G.dev(x))
        call()
        t.cuda.synchronize()
        eager.append(results())
    # warm-up on a side stream, then capture on the graph's stream
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        call()
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        call()
    for _ in range(2):
        for i, x in enumerate(xs):
            x_in.copy_(G.dev(x))
            g.replay()
            t.cuda.synchronize()
            for got, ref in zip(results(), eager[i]):
                np.testing.assert_array_equal(got, ref)
        x_in.copy_(G.dev(xs[1]))   # an eager call between rounds of replays
        call()
        t.cuda.synchronize()
        for got, ref in zip(results(), eager[1]):
            np.testing.assert_array_equal(got, ref)
