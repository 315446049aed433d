"""HIP-graph capture of the hot path: the sink+window attention (bf16 cache,
and an INT8 cache in both attention modes) and the text cross-attention,
captured once into a graph (torch.cuda.CUDAGraph on the capture stream) and
replayed several times, with the program's own eager work between replays.
Every replay must reproduce the eager result bit for bit: the calls launch
kernels only (no allocation, no memset), so they are capturable as they are.
Method: LongLive: Real-time Interactive Long Video Generation, §3.3 (short
window + frame sink) and §3.1 (text cross-attention)."""

import math

import numpy as np
import pytest
import torch

from sink_short_window_amd import ll, synth
from sink_short_window_amd.synth import Q, K, V, K_TXT, V_TXT
from gpu_util import need_gpu, say, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("kv", ["bf16", "int8", "int8-ink"])
def test_graph_replay_matches_eager(kv):
    T, C, S, W, H, D = 100, 1, 1, 3, 4, 128      # ragged tiles: 100 tokens per chunk
    kvd = ll.LL_BF16 if kv == "bf16" else ll.LL_I8
    cfg = ll.make_config(1, H, D, T, C, S, W, ll.LL_BF16, kvd)
    cache = ll.Cache(cfg, "cuda")
    try:
        if kv == "int8-ink":
            cache.set_int8_dequant(ll.LL_I8_IN_KERNEL)
        g = lambda shape, c, t: dev(synth.normal(shape, "bf16", 170, 0, c, 0, t), "bf16")
        for c in range(3):
            cache.append_chunk(0, g((T, H, D), c, K), g((T, H, D), c, V))
        q, kc, vc = g((T, H, D), 3, Q), g((T, H, D), 3, K), g((T, H, D), 3, V)
        kt, vt = g((77, H, D), 0, K_TXT), g((77, H, D), 0, V_TXT)
        scale = 1.0 / math.sqrt(D)
        out = torch.empty_like(q)
        lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
        xout = torch.empty_like(q)

        def step():
            cache.attn(0, q, kc, vc, scale, out, lse)
            ll.ll_cross_attn(out, kt, vt, scale, xout, ll.LL_BF16)

        step()                                   # eager reference (and warm-up)
        torch.cuda.synchronize()
        want = (out.clone(), lse.clone(), xout.clone())
        say(f"[graph {kv}] capture")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for rep in range(3):
            for t in (out, lse, xout):           # eager work between replays
                t.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for name, got, ref in zip(("out", "lse", "cross"), (out, lse, xout), want):
                assert torch.equal(got, ref), f"replay {rep}: {name} differs from the eager call"
        say(f"[graph {kv}] 3 replays equal the eager call")
        del graph
    finally:
        cache.close()


def test_graph_replay_of_the_allocation_free_backward():
    """The training step's forward and its allocation-free backward (whose
    delta workspace is the library's static device array) captured in one
    graph: three replays equal the eager calls bit for bit.  The first eager
    call looks up the array's address; inside the capture only kernels are
    launched."""
    T, C, S, W, H, D = 100, 1, 1, 3, 4, 128
    cfg = ll.make_config(1, H, D, T, C, S, W, ll.LL_BF16, ll.LL_BF16)
    cache = ll.Cache(cfg, "cuda")
    try:
        g = lambda c, t: dev(synth.normal((T, H, D), "bf16", 171, 0, c, 0, t), "bf16")
        for c in range(3):
            cache.append_chunk(0, g(c, K), g(c, V))
        q, kc, vc, dout = g(3, Q), g(3, K), g(3, V), g(4, Q)
        scale = 1.0 / math.sqrt(D)
        out = torch.empty_like(q)
        lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
        dq, dk, dv = (torch.empty((T, H, D), dtype=torch.float32, device="cuda") for _ in range(3))

        def step():
            cache.attn(0, q, kc, vc, scale, out, lse)
            ll.ll_sink_window_attn_bwd_noalloc(cache.handle, 0, q, kc, vc, scale, out, lse, dout, dq, dk, dv)

        step()
        torch.cuda.synchronize()
        want = [t.clone() for t in (out, lse, dq, dk, dv)]
        say("[graph bwd] capture")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for rep in range(3):
            for t in (out, lse, dq, dk, dv):
                t.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for name, got, ref in zip(("out", "lse", "dq", "dk", "dv"), (out, lse, dq, dk, dv), want):
                assert torch.equal(got, ref), f"replay {rep}: {name} differs from the eager call"
        say("[graph bwd] 3 replays equal the eager calls")
        del graph
    finally:
        cache.close()
