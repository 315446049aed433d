#!/usr/bin/env python3
"""Benchmark: streaming 30-layer sink + short-window KV-cache step on one MI355X.

Workload (LongLive: Real-time Interactive Long Video Generation, §3.1 KV
recache, §3.3 short window + frame sink, §4 implementation; shapes of a 1.3B
video DiT): 30 layers with independent caches, 12 heads x 128, 1560 tokens per
latent frame, chunks of 3 latent frames (4680 tokens), sink = the first chunk
(3 frames), window = 9 frames including the current chunk.

One step = one generated chunk:
  * before chunks 20, 30, ..., 70 (prompt switch): KV-recache of all 30
    layers' resident window (fresh seeded N(0,1) bf16 K/V, sink kept) and a
    new prompt's text K/V;
  * 4 denoising passes x 30 layers of sink+window attention (queries of the
    chunk over sink + ring + current chunk) and text cross-attention to 512
    text tokens;
  * one cache-append pass: 30 appends (the oldest window chunk is evicted).
Warmup steps generate chunks 0.. W-1 untimed; the K timed steps continue the
same stream.  ``--workload stream`` drops cross-attention and recache (the
30-layer cache step alone); ``--kv int8`` stores K/V as int8 with per-token,
per-head scales, dequantised to a bf16 staging copy once per attention call.

All inputs are seeded synthetic N(0,1) values (bf16) drawn on the host from
pools and copied to the device once before timing.

Prints ONE JSON line.  ``value`` is latent frames per second over the timed
steps (3 latent frames per step); the attention kernel's roofline figures
are measured live with HIP events around each attention launch.
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s + latent frames/sec (30-layer cache step) on 1 MI355X; % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0

# geometry
L, H, D = 30, 12, 128
T, C, S, W = 1560, 3, 3, 9
CT = C * T                    # 4680 tokens per chunk
N_TXT = 512
PASSES = 4
SWITCH_FIRST, SWITCH_EVERY = 20, 10
POOL = 8                      # Q/K/V pool size
# Inside the timed region HIP events bracket one attention launch in this
# many; 7 is coprime with the 120 launches of a step, so over 7 steps the
# sample covers every (pass, layer).  Bracketing all of them measured ~3%
# slower steps.
ATTN_EVENT_EVERY = 7
TXT_POOL = 16
RECACHE_POOL = 8
CFG_ID = {"switch": 3, "stream": 2}
# window/sink sweep (one layer, steady state): latent frames
SWEEP_WINDOWS = (3, 6, 9, 12, 15, 18, 21, 24, 27)
SWEEP_SINKS = (0, 3)
SWEEP_CFG_ID = 5
KERNEL_SOURCE = os.path.join(ROOT, "sink_short_window_amd", "csrc", "kernels.hip")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "attn_bf16_sink3_win9_hbm_counters.txt")


def pool_index(layer, chunk, pass_):
    """Which pooled Q/K/V tensor a (layer, chunk, pass) uses; pass 4 = append."""
    return (7 * layer + 3 * chunk + pass_) % POOL


def switches_before(chunk):
    """Number of prompt switches that happen at or before ``chunk``."""
    if chunk < SWITCH_FIRST:
        return 0
    return 1 + (chunk - SWITCH_FIRST) // SWITCH_EVERY


def is_switch(chunk):
    return chunk >= SWITCH_FIRST and (chunk - SWITCH_FIRST) % SWITCH_EVERY == 0


def txt_index(prompt, layer):
    return (prompt * L + layer) % TXT_POOL


def recache_index(switch, layer):
    return (3 * layer + switch) % RECACHE_POOL


class Workload:
    """Input pools, the 30-layer cache and the per-chunk step."""

    def __init__(self, workload="switch", kv="bf16", device="cuda", n_chunks=80, passes=PASSES):
        import torch
        from sink_short_window_amd import ll, synth
        self.torch, self.ll, self.synth = torch, ll, synth
        self.workload, self.kv, self.passes = workload, kv, passes
        self.cfg_id = CFG_ID[workload] + (10 if kv.startswith("int8") else 0)
        self.device = device
        self.scale = 1.0 / math.sqrt(D)
        gen = lambda shape, chunk, tensor: synth.to_torch(
            synth.normal(shape, "bf16", self.cfg_id, 0, chunk, 0, tensor), "bf16", device)
        # disjoint pools (different tensor ids) so no query equals a resident key
        self.q = [gen((CT, H, D), i, synth.Q) for i in range(POOL)]
        self.k = [gen((CT, H, D), i, synth.K) for i in range(POOL)]
        self.v = [gen((CT, H, D), i, synth.V) for i in range(POOL)]
        self.with_text = workload == "switch"
        if self.with_text:
            self.ktxt = [gen((N_TXT, H, D), i, synth.K_TXT) for i in range(TXT_POOL)]
            self.vtxt = [gen((N_TXT, H, D), i, synth.V_TXT) for i in range(TXT_POOL)]
            self.rk = [gen((2 * CT, H, D), i, synth.RK) for i in range(RECACHE_POOL)]
            self.rv = [gen((2 * CT, H, D), i, synth.RV) for i in range(RECACHE_POOL)]
        # queries of the re-encoding pass after a recache (the 2 window chunks)
        self.qwin = gen((2 * CT, H, D), POOL, synth.Q)
        self.payload = {}
        kvcode = ll.LL_I8 if kv.startswith("int8") else ll.LL_BF16
        cfg = ll.make_config(L, H, D, T, C, S, W, ll.LL_BF16, kvcode)
        self.cache = ll.Cache(cfg, device)
        if kv == "int8-ink":   # int8 codes read inside the attention kernel
            self.cache.set_int8_dequant(ll.LL_I8_IN_KERNEL)
        self.out = torch.empty((CT, H, D), dtype=torch.bfloat16, device=device)
        self.xout = torch.empty((CT, H, D), dtype=torch.bfloat16, device=device)
        self.xwin = torch.empty((2 * CT, H, D), dtype=torch.bfloat16, device=device)
        self.chunk = 0
        self.timers = None
        self.timed_kinds = ("attn", "cross", "append", "recache")
        self.launches = {}

    def recache_payload(self, switch):
        """[L][2*CT][H][D] K and V for the ``switch``-th prompt switch."""
        if switch not in self.payload:
            t = self.torch
            self.payload[switch] = (
                t.stack([self.rk[recache_index(switch, l)] for l in range(L)]).contiguous(),
                t.stack([self.rv[recache_index(switch, l)] for l in range(L)]).contiguous())
        return self.payload[switch]

    def prepare(self, chunks):
        """Build every recache payload the given chunks need (before timing)."""
        if self.with_text:
            for c in chunks:
                if is_switch(c):
                    self.recache_payload(switches_before(c))

    def _timed(self, kind, fn, work=0.0):
        """Run ``fn``; with timers on for ``kind``, bracket it with HIP events
        recorded on the stream the library launches on (torch's current
        stream).  Attention launches are bracketed one in ATTN_EVENT_EVERY
        (each event pair idles the GPU for a few microseconds between
        kernels); every launch is counted in ``self.launches``."""
        self.launches[kind] = self.launches.get(kind, 0) + 1
        if self.timers is None or kind not in self.timed_kinds:
            return fn()
        if kind == "attn" and self.launches[kind] % ATTN_EVENT_EVERY:
            return fn()
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.timers.setdefault(kind, []).append((a, b, work))

    def step(self, capture=None):
        """Generate one chunk.  ``capture``: set of (pass, layer) whose
        attention (and cross-attention) outputs are copied out and returned."""
        ll, c = self.ll, self.chunk
        cache = self.cache
        got = {}
        prompt = switches_before(c)
        if self.with_text and is_switch(c):
            pk, pv = self.recache_payload(prompt)
            self._timed("recache", lambda: cache.recache(-1, pk, pv, 2 * CT))
        for p in range(self.passes):
            for layer in range(L):
                i = pool_index(layer, c, p)
                self._timed("attn", lambda: cache.attn(layer, self.q[i], self.k[i], self.v[i],
                                                       self.scale, self.out),
                            attn_flops(keys_at(c)))
                if capture and (p, layer) in capture:
                    got[(p, layer, "attn")] = self.out.clone()
                if self.with_text:
                    j = txt_index(prompt, layer)
                    self._timed("cross", lambda: ll.ll_cross_attn(
                        self.q[i], self.ktxt[j], self.vtxt[j], self.scale, self.xout, ll.LL_BF16))
                    if capture and (p, layer) in capture:
                        got[(p, layer, "cross")] = self.xout.clone()
        for layer in range(L):
            i = pool_index(layer, c, self.passes)
            self._timed("append", lambda: cache.append_chunk(layer, self.k[i], self.v[i]))
        self.chunk += 1
        return got


def reencode_flops():
    """Algorithmic flop of one re-encoding call over the 2 resident window
    chunks: window chunk r's C_tok queries attend sink + chunks 0..r."""
    return 4.0 * D * H * CT * sum(CT + (r + 1) * CT for r in range((W - C) // C))


def time_reencode(wl, reps=3):
    """Re-encoding attention of every layer on the cache as the timed steps
    left it (sink + 2 window chunks), HIP events around each launch."""
    t = wl.torch
    ms = []
    for _ in range(reps):
        for layer in range(L):
            a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
            a.record()
            wl.cache.reencode_attn(layer, wl.qwin, wl.scale, wl.xwin)
            b.record()
            ms.append((a, b))
    t.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ms) / len(ms)


def sweep_point(sink, window, reps=20):
    """One layer with sink ``sink`` and window ``window`` (latent frames) at the
    workload's shapes: fill the sink and the ring, evict one chunk, then time
    the attention call of the next chunk (sink + full ring + itself).
    Returns a dict with keys per call, ms per call (median of reps/4 batches
    of 10 calls), TFLOP/s and cache bytes."""
    import torch
    from sink_short_window_amd import ll, synth
    gen = lambda i, tensor: synth.to_torch(
        synth.normal((CT, H, D), "bf16", SWEEP_CFG_ID, 0, i, 0, tensor), "bf16", "cuda")
    ks = [gen(i, synth.K) for i in range(3)]
    vs = [gen(i, synth.V) for i in range(3)]
    q = gen(0, synth.Q)
    out = torch.empty_like(q)
    cfg = ll.make_config(1, H, D, T, C, sink, window, ll.LL_BF16, ll.LL_BF16)
    cache_bytes = ll.ll_cache_required_bytes(cfg)
    cache = ll.Cache(cfg, "cuda")
    ring = (window - C) // C
    for c in range(sink // C + ring + 1):
        cache.append_chunk(0, ks[c % 3], vs[c % 3])
    keys = sink * T + ring * CT + CT
    call = lambda: cache.attn(0, q, ks[0], vs[0], 1.0 / math.sqrt(D), out)

    def batch(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            call()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    # After an idle gap the first ~10 ms of calls run ~15% slower while the
    # clock settles; warm up for 150 ms of GPU time before timing.
    warm = 0.0
    while warm < 150.0:
        warm += batch(10)
    ms = sorted(batch(10) / 10 for _ in range(reps // 4))[reps // 8]
    cache.close()
    return {"sink_frames": sink, "window_frames": window, "keys_per_call": keys,
            "ms_per_call": ms, "tflops": attn_flops(keys) / (ms * 1e-3) / 1e12,
            "cache_bytes_per_layer": cache_bytes, "cache_bytes_30_layers": L * cache_bytes}


def window_sweep():
    """Print one JSON line per (sink, window) point, then a summary comparing
    the paper's short window + sink (9 + 3) with its long window (21) and its
    short window without sink (12)."""
    pts = {}
    for sink in SWEEP_SINKS:
        for window in SWEEP_WINDOWS:
            p = sweep_point(sink, window)
            pts[(sink, window)] = p
            print(json.dumps(p), flush=True)
    short, long_, nosink = pts[(3, 9)], pts[(0, 21)], pts[(0, 12)]
    print(json.dumps({
        "summary": "attention call (4680 queries) and cache bytes per layer, median of 5 batches of 10 calls after a 150 ms warmup",
        "short9_sink3_vs_long21": {"time": short["ms_per_call"] / long_["ms_per_call"],
                                   "cache_bytes": short["cache_bytes_per_layer"] / long_["cache_bytes_per_layer"],
                                   "keys": short["keys_per_call"] / long_["keys_per_call"]},
        "short9_sink3_vs_short12": {"time": short["ms_per_call"] / nosink["ms_per_call"],
                                    "cache_bytes": short["cache_bytes_per_layer"] / nosink["cache_bytes_per_layer"],
                                    "keys": short["keys_per_call"] / nosink["keys_per_call"]}}))


def backward_flops():
    """Algorithmic flop of one backward call at 18720 keys: S, dP and dQ over
    every key, dV and dK over the current chunk's keys:
    2 * D * H * L_q * (3 * L_k + 2 * C_tok)."""
    return 2.0 * D * H * CT * (3 * keys_at(10) + 2 * CT)


def time_backward(wl, reps=10):
    """Backward of layer 0's call (sink + 2 window chunks + the current chunk,
    18720 keys) on the cache as the timed steps left it: forward once for out
    and lse, then HIP events around each backward call (its three kernels)."""
    t = wl.torch
    q, k, v, g = wl.q[0], wl.k[0], wl.v[0], wl.q[1]
    out = t.empty_like(q)
    lse = t.empty((H, CT), dtype=t.float32, device=wl.device)
    wl.cache.attn(0, q, k, v, wl.scale, out, lse)
    delta = t.empty((H, CT), dtype=t.float32, device=wl.device)
    dq, dk, dv = (t.empty((CT, H, D), dtype=t.float32, device=wl.device) for _ in range(3))
    call = lambda: wl.cache.attn_bwd(0, q, k, v, wl.scale, out, lse, g, delta, dq, dk, dv)
    for _ in range(3):
        call()
    ms = []
    for _ in range(reps):
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        ms.append((a, b))
    t.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in ms)[reps // 2]


def linear_bytes():
    """Algorithmic HBM bytes of one linear-attention call at 18720 keys: Q and
    O once, the K/V of every key once (the state and normaliser are a few MB
    of on-chip-sized partials)."""
    return float(H * D * 2 * (2 * CT + 2 * keys_at(10)))


def linear_flops():
    """Algorithmic flop of one linear-attention call: phi(K)^T V and phi(K)^T 1
    over the keys, phi(Q) S and phi(Q) . z over the queries."""
    return 2.0 * H * D * (D + 1) * (keys_at(10) + CT)


def time_linear(wl, reps=10):
    """Linear-attention variant of layer 0's call (same key set as the softmax
    call, 18720 keys): HIP events around each call (its three kernels)."""
    t = wl.torch
    q, k, v = wl.q[0], wl.k[0], wl.v[0]
    out = t.empty_like(q)
    call = lambda: wl.cache.linear_attn(0, q, k, v, out)
    for _ in range(3):
        call()
    ms = []
    for _ in range(reps):
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        ms.append((a, b))
    t.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in ms)[reps // 2]


def linear_only():
    """One layer at the workload's shapes: chunks 0..3 appended (sink = chunk 0,
    window = chunks 2, 3), then the linear-attention variant of chunk 4's call
    (18720 keys) timed after a warmup of ~40 calls (median of 5 batches of
    10), next to the softmax call on the same inputs.  Prints one JSON line."""
    import torch
    from sink_short_window_amd import ll, synth
    gen = lambda i, tensor: synth.to_torch(
        synth.normal((CT, H, D), "bf16", SWEEP_CFG_ID, 2, i, 0, tensor), "bf16", "cuda")
    cfg = ll.make_config(1, H, D, T, C, S, W, ll.LL_BF16, ll.LL_BF16)
    cache = ll.Cache(cfg, "cuda")
    for c in range(4):
        cache.append_chunk(0, gen(c, synth.K), gen(c, synth.V))
    q, k, v = gen(4, synth.Q), gen(4, synth.K), gen(4, synth.V)
    out = torch.empty_like(q)

    def timed(call):
        def batch(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(n):
                call()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b)
        batch(40)
        return sorted(batch(10) / 10 for _ in range(5))[2]

    ms = timed(lambda: cache.linear_attn(0, q, k, v, out))
    sm = timed(lambda: cache.attn(0, q, k, v, 1.0 / math.sqrt(D), out))
    print(json.dumps({"linear_ms_per_call": ms, "keys_per_call": keys_at(10),
                      "bytes_per_call": linear_bytes(), "GBps": linear_bytes() / (ms * 1e-3) / 1e9,
                      "flop_per_call": linear_flops(), "tflops": linear_flops() / (ms * 1e-3) / 1e12,
                      "softmax_ms_per_call": sm, "speedup_vs_softmax": sm / ms}))
    cache.close()


def backward_only():
    """One layer at the workload's shapes: chunks 0..3 appended (sink = chunk 0,
    window = chunks 2, 3), the forward of chunk 4 for out and lse, then the
    backward of that call timed after a warmup of ~40 calls (median of 5
    batches of 10).  Prints one JSON line."""
    import torch
    from sink_short_window_amd import ll, synth
    gen = lambda i, tensor: synth.to_torch(
        synth.normal((CT, H, D), "bf16", SWEEP_CFG_ID, 1, i, 0, tensor), "bf16", "cuda")
    cfg = ll.make_config(1, H, D, T, C, S, W, ll.LL_BF16, ll.LL_BF16)
    cache = ll.Cache(cfg, "cuda")
    for c in range(4):
        cache.append_chunk(0, gen(c, synth.K), gen(c, synth.V))
    q, k, v, g = gen(4, synth.Q), gen(4, synth.K), gen(4, synth.V), gen(5, synth.Q)
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device="cuda")
    out, lse = torch.empty_like(q), f32(H, CT)
    scale = 1.0 / math.sqrt(D)
    cache.attn(0, q, k, v, scale, out, lse)
    delta, dq, dk, dv = f32(H, CT), f32(CT, H, D), f32(CT, H, D), f32(CT, H, D)
    call = lambda: cache.attn_bwd(0, q, k, v, scale, out, lse, g, delta, dq, dk, dv)

    def batch(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            call()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    batch(40)
    ms = sorted(batch(10) / 10 for _ in range(5))[2]
    print(json.dumps({"backward_ms_per_call": ms, "keys_per_call": keys_at(10),
                      "flop_per_call": backward_flops(),
                      "tflops": backward_flops() / (ms * 1e-3) / 1e12}))
    cache.close()


def kernel_stats(timers, kind):
    """(average ms per launch, total work, total ms) of one kernel kind."""
    ev = timers.get(kind, [])
    if not ev:
        return None, 0.0, 0.0
    ms = [a.elapsed_time(b) for a, b, _ in ev]
    return sum(ms) / len(ms), sum(w for _, _, w in ev), sum(ms)


def keys_at(chunk):
    """Keys attended by chunk ``chunk``: sink + resident ring chunks + itself."""
    return CT * min(chunk + 1, 1 + (W - C) // C + 1)


def attn_flops(n_keys):
    """Algorithmic flop of one attention call: 4 * L_q * L_k * D * H."""
    return 4.0 * CT * n_keys * D * H


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _blas():
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        return [{"library": i.get("internal_api"), "version": i.get("version"),
                 "threads": i.get("num_threads"), "file": os.path.basename(i.get("filepath", ""))}
                for i in info], max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        return None, len(os.sched_getaffinity(0))


def tiny_config_run():
    """The tiny fp32 configuration through the oracle: 1 head x 64, 16 tokens
    per frame, chunks of 1 frame, sink 1 frame, window 2 frames, 8 chunks, each
    attending sink + window + itself and then appended.  Returns seconds."""
    import oracle
    from sink_short_window_amd import synth
    t, c, s, w, h, d = 16, 1, 1, 2, 1, 64
    g = oracle.CacheGeometry(t, c, s, w)
    hist = oracle.LayerHistory(g)
    t0 = time.perf_counter()
    for j in range(8):
        q, k, v = (synth.normal((t * c, h, d), "f32", 0, 0, j, 0, x) for x in (synth.Q, synth.K, synth.V))
        hk, hv = hist.keys(k, v)
        oracle.sink_window_attention(q, hk, hv, j, tokens_per_frame=t, frames_per_chunk=c,
                                     sink_frames=s, window_frames=w, scale=1 / math.sqrt(d))
        hist.append(k, v)
    return time.perf_counter() - t0


def cpu_baseline(k_steps, warmup, budget_s=20.0, passes=PASSES):
    """Time the oracle (float64 numpy, as it stands) on a bounded sample of the
    same workload and scale it to latent frames/s.

    Sample: one steady-state attention call (chunk 4: sink + 2 ring chunks +
    current chunk, 18720 allowed keys out of a 23400-key history), whole heads
    at a time with the BLAS library's default threads until ``budget_s`` is
    spent, then one head with one thread; plus the tiny fp32 configuration's
    whole 8-chunk run."""
    import oracle
    from sink_short_window_amd import synth
    blas, cores = _blas()
    g = oracle.CacheGeometry(T, C, S, W)
    hist = oracle.LayerHistory(g)
    ks = [synth.normal((CT, H, D), "bf16", 90, 0, j, 0, synth.K) for j in range(5)]
    vs = [synth.normal((CT, H, D), "bf16", 90, 0, j, 0, synth.V) for j in range(5)]
    for j in range(4):
        hist.append(ks[j], vs[j])
    hk, hv = hist.keys(ks[4], vs[4])
    q = synth.normal((CT, H, D), "bf16", 90, 0, 4, 0, synth.Q)

    def one_head(h):
        hs = slice(h, h + 1)
        oracle.sink_window_attention(q[:, hs], hk[:, hs], hv[:, hs], 4, tokens_per_frame=T,
                                     frames_per_chunk=C, sink_frames=S, window_frames=W,
                                     scale=1 / math.sqrt(D))

    heads, spent = 0, 0.0
    t0 = time.perf_counter()
    while heads < H and spent < budget_s:
        one_head(heads)
        heads += 1
        spent = time.perf_counter() - t0
    per_call = spent / heads * H             # one full call at a 5-chunk history
    one_thread = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            one_head(0)
            one_thread = (time.perf_counter() - t1) * H
    except Exception:
        pass
    # The oracle masks the whole history, so its cost grows with the chunk
    # index; scale each timed chunk's calls by its history length.
    scale_steps = lambda call_s: sum(passes * L * call_s * (c + 1) / 5.0 for c in range(warmup, warmup + k_steps))
    total = scale_steps(per_call)
    flop = attn_flops(keys_at(4))
    res = {"value": 3.0 * k_steps / total, "unit": "latent frames/s", "cores": int(cores),
           "kind": "oracle",
           "sample": f"oracle sink+window attention, {heads} of {H} heads x {CT} queries of one "
                     f"call at chunk 4 (23400-key history, 18720 allowed) in {spent:.1f} s "
                     f"({per_call:.1f} s per call); extrapolated to {passes}x{L} calls per chunk "
                     f"for chunks {warmup}..{warmup + k_steps - 1} with cost scaled by history "
                     f"length; cross-attention, append and recache not counted",
           "cpu_model": _cpu_model(), "host_cpus": len(os.sched_getaffinity(0)), "blas": blas,
           "s_per_call": per_call, "gflops_per_call": flop / per_call / 1e9,
           "tiny_fp32_8_chunks_s": tiny_config_run()}
    if one_thread:
        res["one_thread"] = {"s_per_call": one_thread, "gflops_per_call": flop / one_thread / 1e9,
                             "latent_frames_per_s": 3.0 * k_steps / scale_steps(one_thread),
                             "sample": "1 head of the same call with BLAS limited to 1 thread, x12 heads"}
    return res


def kernel_source_digest():
    """sha256 of the kernel source with comments and whitespace removed, so
    that the counter record survives edits that cannot change the code."""
    src = open(KERNEL_SOURCE).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return hashlib.sha256(re.sub(r"\s+", "", src).encode()).hexdigest()


def recorded_traffic():
    """HBM bytes per attention launch from the committed FETCH_SIZE/WRITE_SIZE
    record, or None when the kernel source changed since it was taken."""
    try:
        rec = dict(line.split(":", 1) for line in open(TRAFFIC_RECORD)
                   if line.startswith(("kernel_source_sha256:", "traffic_bytes_per_launch:")))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256", "").strip() != kernel_source_digest():
        return None
    return int(rec["traffic_bytes_per_launch"].strip())


def copy_calibration():
    """A plain device copy of a known size (2 GiB read + 2 GiB written), run
    three times: the FETCH_SIZE / WRITE_SIZE counters of its kernel give the
    factor that turns those counters into bytes on this chip."""
    import torch
    n = 1 << 29
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": 4 * n, "bytes_written": 4 * n,
                                           "launches": 3}}))


def gemm_ceiling():
    """Reference point for the MFMA roofline: the vendor bf16 GEMM (torch.matmul,
    8192^3) on N(0,1) operands and on all-zero operands.  MI355X holds a lower
    clock under MFMA load with real data, so the first figure is the practical
    ceiling a bf16 contraction reaches on this chip."""
    import torch
    n = 8192
    g = torch.Generator(device="cuda").manual_seed(7)
    res = {}
    for name in ("normal", "zeros"):
        if name == "normal":
            a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
            b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
        else:
            a = torch.zeros(n, n, device="cuda", dtype=torch.bfloat16)
            b = torch.zeros(n, n, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            c = a @ b
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record()
        for _ in range(reps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)
        del c
    print(json.dumps({"gemm_ceiling_tflops": res, "shape": [n, n, n], "dtype": "bf16"}))


def run_timed(wl, warmup, steps):
    """Warmup steps (cross-attention and append launches timed there: same
    kernels and shapes as in the timed steps), then the timed region of K
    whole steps between HIP events.  Inside it events bracket one attention
    launch in ATTN_EVENT_EVERY (and every rare recache) on the launch stream,
    so the attention kernel's duration comes from the same run; events around
    every launch would cost ~3% of the step."""
    torch = wl.torch
    wl.prepare(range(wl.chunk, wl.chunk + warmup + steps))
    wl.timers, wl.timed_kinds = {}, ("cross", "append")
    for _ in range(warmup):
        wl.step()
    torch.cuda.synchronize()
    warm_timers, wl.timers = wl.timers, None
    wl.timers, wl.timed_kinds = {}, ("attn", "recache")
    wl.launches = {}
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    first = wl.chunk
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    marks = [start]  # one event per step boundary: switch-step vs steady-step latency
    for _ in range(steps):
        wl.step()
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        marks.append(e)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timers, wl.timers = wl.timers, None
    return {"gpu_ms": start.elapsed_time(stop), "timers": timers, "warm_timers": warm_timers,
            "marks": marks, "first": first, "wall": wall}


def append_bytes(kv):
    """Algorithmic HBM bytes of one layer's append: the chunk's K/V read
    (bf16) and written in the cache's dtype (plus the int8 scales)."""
    i8 = kv.startswith("int8")
    return CT * H * D * 2 * 2 + CT * H * D * (1 if i8 else 2) * 2 + (CT * H * 4 * 2 if i8 else 0)


def int8_subrun(warmup, steps, passes, kv="int8"):
    """The same prompt-switch workload over an INT8 KV cache (per-token,
    per-head scales), reported beside the bf16-cache line: latent frames/s,
    the attention call (events around the whole call: the staging launch and
    the attention for kv "int8", the attention that reads the codes itself for
    "int8-ink") and the append rate."""
    wl = Workload("switch", kv, passes=passes)
    run = run_timed(wl, warmup, steps)
    attn_ms, attn_work, attn_total = kernel_stats(run["timers"], "attn")
    app_ms, _, _ = kernel_stats(run["warm_timers"], "append")
    res = {"latent_frames_per_s": 3.0 * steps / (run["gpu_ms"] / 1e3),
           "ms_per_step": run["gpu_ms"] / steps, "steps": steps, "warmup": warmup,
           "attention_ms_per_call": attn_ms,
           "attention_tflops": attn_work / (attn_total * 1e-3) / 1e12 if attn_ms else None,
           "append_ms": app_ms,
           "append_GBps": append_bytes("int8") / (app_ms * 1e-3) / 1e9 if app_ms else None}
    wl.cache.close()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=76)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", choices=["switch", "stream"], default="switch")
    ap.add_argument("--kv", choices=["bf16", "int8", "int8-ink"], default="bf16",
                    help="KV cache: bf16, or int8 read through a staged bf16 copy (int8) or inside "
                         "the attention kernel (int8-ink)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-int8-subrun", action="store_true",
                    help="skip the INT8-cache run of the same workload that the bf16 line reports in extra")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--passes", type=int, default=PASSES,
                    help="attention passes per chunk (4 denoising; 5 adds the append pass's own attention)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 2 GiB device copy (HBM counter calibration) and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="only time one layer's attention call for windows of 3..27 frames with and "
                         "without the 3-frame sink (JSON line per point) and exit")
    ap.add_argument("--backward", action="store_true",
                    help="only time the backward of one layer's call (training step) and exit")
    ap.add_argument("--linear", action="store_true",
                    help="only time the linear-attention variant of one layer's call and exit")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="only time the vendor bf16 GEMM on random and on zero operands and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this path has no multi-GPU mode "
              "(each interactive stream is independent and runs on one GPU).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gemm_ceiling:
        gemm_ceiling()
        return
    if args.sweep:
        window_sweep()
        return
    if args.backward:
        backward_only()
        return
    if args.linear:
        linear_only()
        return
    if args.passes < 1:
        print("--passes must be >= 1", file=sys.stderr)
        sys.exit(2)
    if args.warmup + args.steps > 80:
        print("warmup + steps must be <= 80 chunks (240 latent frames)", file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.init()
    wl = Workload(args.workload, args.kv, passes=args.passes)
    run = run_timed(wl, args.warmup, args.steps)
    gpu_ms, timers, warm_timers, marks, first, wall = (
        run["gpu_ms"], run["timers"], run["warm_timers"], run["marks"], run["first"], run["wall"])
    ms_per_step = gpu_ms / args.steps
    frames_per_s = 3.0 * args.steps / (gpu_ms / 1e3)

    attn_ms, attn_work, attn_total_ms = kernel_stats(timers, "attn")
    tflops = attn_work / (attn_total_ms * 1e-3) / 1e12 if attn_ms else None
    keys = keys_at(first)
    extra = {"attention_ms_per_call": attn_ms, "attention_tflops": tflops,
             "attention_flop_per_call_steady": attn_flops(keys_at(10)),
             "attention_calls": wl.launches.get("attn", 0),
             "attention_calls_timed": len(timers.get("attn", [])),
             "attention_share_of_step": (attn_ms or 0.0) * wl.launches.get("attn", 0) / gpu_ms,
             "timed_chunks": [first, first + args.steps - 1], "wall_s": wall}
    app_ms, _, _ = kernel_stats(warm_timers, "append")
    if app_ms:
        extra["append_ms"] = app_ms
        extra["append_GBps"] = append_bytes(args.kv) / (app_ms * 1e-3) / 1e9
    x_ms, _, _ = kernel_stats(warm_timers, "cross")
    if x_ms:
        xf = 4.0 * CT * N_TXT * D * H
        extra["cross_attn_ms"] = x_ms
        extra["cross_attn_tflops"] = xf / (x_ms * 1e-3) / 1e12
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    sw = [m for i, m in enumerate(step_ms) if is_switch(first + i)]
    steady = [m for i, m in enumerate(step_ms) if not is_switch(first + i) and first + i >= 3]
    if steady:
        extra["steady_step_ms"] = sum(steady) / len(steady)
    if sw and args.workload == "switch":
        extra["switch_step_ms"] = sum(sw) / len(sw)
        extra["switch_steps"] = len(sw)
    rc_ms, _, _ = kernel_stats(timers, "recache")
    if rc_ms:
        i8 = args.kv.startswith("int8")
        rc_bytes = L * 2 * (2 * CT * H * D) * (3 if i8 else 4) + (L * 2 * 2 * CT * H * 4 if i8 else 0)
        extra["recache_ms"] = rc_ms
        extra["recache_GBps"] = rc_bytes / (rc_ms * 1e-3) / 1e9

    # After the timed region: the re-encoding attention of a recache
    # (window queries over sink + window, causal across chunks).
    re_ms = time_reencode(wl)
    extra["reencode_ms_per_call"] = re_ms
    extra["reencode_flop_per_call"] = reencode_flops()
    extra["reencode_tflops"] = reencode_flops() / (re_ms * 1e-3) / 1e12
    # The training step's backward of one call (bf16 cache only).
    if args.kv == "bf16":
        bw_ms = time_backward(wl)
        extra["backward_ms_per_call"] = bw_ms
        extra["backward_flop_per_call"] = backward_flops()
        extra["backward_tflops"] = backward_flops() / (bw_ms * 1e-3) / 1e12
    # The linear-attention variant of the same call (same cache, same key set).
    li_ms = time_linear(wl)
    extra["linear_ms_per_call"] = li_ms
    extra["linear_GBps"] = linear_bytes() / (li_ms * 1e-3) / 1e9
    extra["linear_tflops"] = linear_flops() / (li_ms * 1e-3) / 1e12

    # The INT8-cache run of the same workload, reported beside this line.
    if args.kv == "bf16" and not args.no_int8_subrun:
        extra["int8_cache"] = int8_subrun(args.warmup, args.steps, args.passes, "int8")
        extra["int8_cache_in_kernel"] = int8_subrun(args.warmup, args.steps, args.passes, "int8-ink")
        # The staged call is the staging launch plus the bf16 kernel, inside one C
        # call; its extra time over this line's bf16 call estimates the staging.
        st = extra["int8_cache"].get("attention_ms_per_call")
        if st and extra.get("attention_ms_per_call"):
            extra["int8_cache"]["staging_ms_vs_bf16_call"] = st - extra["attention_ms_per_call"]

    roofline = None
    if tflops:
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                    "traffic": recorded_traffic() if args.kv == "bf16" else None}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.steps, args.warmup, args.cpu_budget, args.passes)

    name = {"switch": "30-layer streaming step with prompt switches (KV-recache) and text cross-attention",
            "stream": "30-layer streaming cache step"}[args.workload]
    line = {
        "metric": METRIC,
        "value": round(frames_per_s, 3),
        "unit": "latent frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name + {"bf16": "", "int8": " (int8 KV cache, staged bf16 copy)",
                                       "int8-ink": " (int8 KV cache read in the attention kernel)"}[args.kv],
                   "layers": L, "heads": H, "head_dim": D, "tokens_per_frame": T,
                   "chunk_frames": C, "sink_frames": S, "window_frames": W,
                   "chunk_tokens": CT, "keys_per_call": keys, "attention_passes": args.passes,
                   "text_tokens": N_TXT if args.workload == "switch" else 0,
                   "kv_cache": args.kv, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
