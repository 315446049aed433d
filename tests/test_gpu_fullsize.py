"""GPU parity at full size, in the launch configuration bench.py times.

The 30-layer prompt-switch workload (12 heads x 128, 1560 tokens per frame,
3-frame chunks, sink 3 frames, window 9 frames, 512 text tokens; LongLive:
Real-time Interactive Long Video Generation, §3.1 KV recache, §3.3 short
window + frame sink) runs through bench.Workload, the same driver and inputs
the benchmark times, for all 80 chunks: prompt switches (KV-recache of all 30
layers) come before chunks 20, 30, ..., 70.  For sampled (chunk, pass, layer)
calls -- after the first switch, mid-stream and the last chunk -- the
sink+window attention and the text cross-attention outputs are compared, on
sampled query rows, with the float64 oracle replaying the same layer's
history (appends, then each recache payload over the resident window).
"""

import functools
import math

import numpy as np
import pytest
import torch

import bench
from oracle import (CacheGeometry, LayerHistory, sink_window_attention, cross_attention, frame_mask,
                    masked_attention)
from sink_short_window_amd import synth
from gpu_util import need_gpu, say, check_out

pytestmark = pytest.mark.gpu

# chunk -> (pass, layer) checked there
CHUNKS = {3: (0, 0), 20: (1, 7), 22: (3, 29), 37: (3, 3), 79: (0, 29)}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@functools.lru_cache(maxsize=64)
def _pool_cached(cfg_id, shape, index, tensor):
    x = synth.normal(shape, "bf16", cfg_id, 0, index, 0, tensor)
    x.flags.writeable = False
    return x


def _pool(wl, shape, index, tensor):
    return _pool_cached(wl.cfg_id, shape, index, tensor)


def _replay_history(wl, layer, chunk):
    """The layer's history as the oracle defines it, through chunk-1, with the
    recache of chunk ``chunk`` (if it is a switch) applied."""
    g = CacheGeometry(bench.T, bench.C, bench.S, bench.W)
    hist = LayerHistory(g, int8=wl.kv.startswith("int8"))
    for c in range(chunk + 1):
        if bench.is_switch(c):
            i = bench.recache_index(bench.switches_before(c), layer)
            hist.recache(_pool(wl, (2 * bench.CT, bench.H, bench.D), i, synth.RK),
                         _pool(wl, (2 * bench.CT, bench.H, bench.D), i, synth.RV))
        if c == chunk:
            break
        i = bench.pool_index(layer, c, wl.passes)
        hist.append(_pool(wl, (bench.CT, bench.H, bench.D), i, synth.K),
                    _pool(wl, (bench.CT, bench.H, bench.D), i, synth.V))
    return hist


@pytest.mark.parametrize("kv", ["bf16", "int8", "int8-ink"])
def test_fullsize_switch_workload_sampled(kv):
    """bf16 cache, and the int8 cache read through the staged bf16 copy and
    in the attention kernel (the oracle attends over the exactly dequantised
    stored K/V; the current chunk stays bf16)."""
    wl = bench.Workload("switch", kv)
    last = max(CHUNKS)
    wl.prepare(range(last + 1))
    got = {}
    for c in range(last + 1):
        cap = {CHUNKS[c]} if c in CHUNKS else None
        say(f"[fullsize {kv}] chunk {c}" + (f" capture {CHUNKS[c]}" if cap else ""))
        out = wl.step(cap)
        if cap:
            got[c] = out
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(bench.D)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 4607, 4608, 4679],
                                     rng.choice(bench.CT, 9, replace=False)]))
    for c, (p, layer) in sorted(CHUNKS.items()):
        i = bench.pool_index(layer, c, p)
        q = _pool(wl, (bench.CT, bench.H, bench.D), i, synth.Q)
        kc = _pool(wl, (bench.CT, bench.H, bench.D), i, synth.K)
        vc = _pool(wl, (bench.CT, bench.H, bench.D), i, synth.V)
        hist = _replay_history(wl, layer, c)
        hk, hv = hist.keys(kc, vc)
        say(f"[fullsize {kv}] oracle chunk {c} pass {p} layer {layer}: {hk.shape[0]} history keys")
        want, _ = sink_window_attention(q[rows], hk, hv, c, tokens_per_frame=bench.T,
                                        frames_per_chunk=bench.C, sink_frames=bench.S,
                                        window_frames=bench.W, scale=scale)
        check_out(got[c][(p, layer, "attn")][rows], want, "bf16", f"chunk {c} pass {p} layer {layer}")
        if c == max(CHUNKS):
            # every query row at the last chunk (after all six switches): the
            # oracle attends the keys its frame mask allows in the full history
            mask = frame_mask(hk.shape[0], c, tokens_per_frame=bench.T, frames_per_chunk=bench.C,
                              sink_frames=bench.S, window_frames=bench.W)
            say(f"[fullsize {kv}] all rows at chunk {c}: {int(mask.sum())} allowed keys")
            want_all, _ = masked_attention(q, hk[mask], hv[mask], None, scale)
            check_out(got[c][(p, layer, "attn")], want_all, "bf16", f"chunk {c} all rows")
        j = bench.txt_index(bench.switches_before(c), layer)
        kt = _pool(wl, (bench.N_TXT, bench.H, bench.D), j, synth.K_TXT)
        vt = _pool(wl, (bench.N_TXT, bench.H, bench.D), j, synth.V_TXT)
        want_x, _ = cross_attention(q[rows], kt, vt, scale)
        check_out(got[c][(p, layer, "cross")][rows], want_x, "bf16", f"cross chunk {c} layer {layer}")
        del hist, hk, hv
