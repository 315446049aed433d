"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
the same seeded inputs.

Cache bytes (indexing, eviction order, recache placement, int8 codes and
scales) must be bit-exact; outputs must be within 1e-4 max-abs (fp32) or
2e-2 max-abs / 5e-3 mean-abs (bf16), plus the diagnostic relative-L2 and LSE
gates.  Paper: LongLive: Real-time Interactive Long Video Generation, §3.1
(KV recache), §3.3 (short window + frame sink).
"""

import math

import numpy as np
import pytest
import torch

from oracle import (CacheGeometry, DequeCacheModel, LayerHistory, sink_window_attention,
                    window_reencode_attention, resident_window_chunks,
                    masked_attention, cross_attention, quantize_int8)
from sink_short_window_amd import ll, synth
from sink_short_window_amd.synth import Q, K, V, K_TXT, V_TXT, RK, RV
from gpu_util import (need_gpu, say, dev, host, check_out, check_lse, act_code)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _expected_rows(chunks, payloads, ct):
    """[H][n*ct][D] expected cache rows from token-major payloads."""
    return np.concatenate([payloads[j].transpose(1, 0, 2) for j in chunks], axis=1)


def _check_cache_bytes(cache, layer, g, sim, payloads, dtype, int8):
    """Sink and ring rows equal the payloads the FIFO model says they hold."""
    ct = g.chunk_tokens
    segs = [(ll.LL_SEG_SINK, list(sim.sink))]
    if g.ring_slots:
        segs.append((ll.LL_SEG_RING, list(sim.slot_chunk)))
    for which, tensor_payloads in ((ll.LL_WHICH_K, payloads[0]), (ll.LL_WHICH_V, payloads[1])):
        for seg, chunks in segs:
            got = cache.rows(layer, which, seg)
            if which == ll.LL_WHICH_V and cache.v_tiled():
                _check_v_padding(cache, layer, seg, chunks)
            for i, j in enumerate(chunks):
                if j < 0:
                    continue
                rows = slice(i * ct, (i + 1) * ct)
                x = tensor_payloads[j].transpose(1, 0, 2)          # [H][ct][D]
                if int8:
                    qw, sw = quantize_int8(np.ascontiguousarray(x, dtype=np.float32))
                    gq = got[:, rows, :].cpu().numpy()
                    assert np.array_equal(gq, qw), f"int8 codes differ (seg {seg}, chunk {j})"
                    sc = cache.tensor(layer, ll.LL_WHICH_KSCALE if which == ll.LL_WHICH_K
                                      else ll.LL_WHICH_VSCALE, seg)
                    gs = sc[:, rows, 0].cpu().numpy()
                    assert np.array_equal(gs.view(np.uint32), sw.view(np.uint32)), "scales differ"
                elif dtype == "bf16":
                    gb = got[:, rows, :].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                    assert np.array_equal(gb, synth.bf16_bits(x)), f"bytes differ (seg {seg}, chunk {j})"
                else:
                    gf = got[:, rows, :].cpu().numpy()
                    assert np.array_equal(gf.view(np.uint32), x.astype(np.float32).view(np.uint32))


def _check_v_padding(cache, layer, seg, chunks):
    """The transposed V tiles hold exact zeros after each stored chunk's last key."""
    pad = cache.v_padding(layer, seg)                     # [H][slots][D][pad columns]
    for i, j in enumerate(chunks):
        if j >= 0 and pad.shape[-1]:
            assert int(torch.count_nonzero(pad[:, i])) == 0, f"V padding not zero (seg {seg}, slot {i})"


def run_stream(cfg_id, T, C, S, W, H, D, dtype, n_chunks, int8=False, check_bytes=True,
               n_cur_zero_at=(), i8_mode=ll.LL_I8_STAGED):
    """Generate ``n_chunks`` chunks through the ABI and compare every attention
    output with the oracle; check the cache bytes after every append.  An int8
    cache is read as ``i8_mode`` selects (staged bf16 copy or in the kernel)."""
    kv = ll.LL_I8 if int8 else act_code(dtype)
    cfg = ll.make_config(1, H, D, T, C, S, W, act_code(dtype), kv)
    cache = ll.Cache(cfg)
    if int8:
        cache.set_int8_dequant(i8_mode)
    g = CacheGeometry(T, C, S, W)
    hist = LayerHistory(g, int8=int8)
    sim = DequeCacheModel(g)
    ct = g.chunk_tokens
    scale = 1.0 / math.sqrt(D)
    payloads = ({}, {})
    for c in range(n_chunks):
        q = synth.normal((ct, H, D), dtype, cfg_id, 0, c, 0, Q)
        k = synth.normal((ct, H, D), dtype, cfg_id, 0, c, 0, K)
        v = synth.normal((ct, H, D), dtype, cfg_id, 0, c, 0, V)
        dq, dk, dv = dev(q, dtype), dev(k, dtype), dev(v, dtype)
        out = torch.empty_like(dq)
        lse = torch.empty((H, ct), dtype=torch.float32, device="cuda")
        use_cur = c not in n_cur_zero_at
        if not use_cur and c == 0:
            use_cur = True
        say(f"[stream cfg={cfg_id} T={T} C={C} S={S} W={W} H={H} D={D} {dtype}{' i8' if int8 else ''}] chunk {c}")
        cache.attn(0, dq, dk if use_cur else None, dv if use_cur else None, scale, out, lse)
        torch.cuda.synchronize()
        hk, hv = hist.keys(k, v) if use_cur else hist.keys()
        want, wlse = sink_window_attention(q, hk, hv, c, tokens_per_frame=T, frames_per_chunk=C,
                                           sink_frames=S, window_frames=W, scale=scale)
        check_out(out, want, dtype, f"chunk {c}")
        check_lse(lse, wlse, dtype, f"chunk {c}")
        cache.append_chunk(0, dk, dv)
        hist.append(k, v)
        sim.append()
        payloads[0][c], payloads[1][c] = k, v
        if check_bytes:
            torch.cuda.synchronize()
            _check_cache_bytes(cache, 0, g, sim, payloads, dtype, int8)
        q_state = cache.query(0)
        assert q_state["chunks_appended"] == c + 1
        assert q_state["slot_chunk"] == sim.slot_chunk
    return cache


def test_tiny_fp32_stream():
    """Tiny fp32 workload: 1 head x 64, 16 tokens/frame, chunk = 1 frame,
    sink 1 frame, window 2 frames, 8 chunks with append + evict."""
    run_stream(0, 16, 1, 1, 2, 1, 64, "f32", 8)


def test_fp32_d128_ragged():
    run_stream(101, 37, 2, 2, 6, 2, 128, "f32", 6)


@pytest.mark.parametrize("D", [128, 64])
def test_bf16_stream_ragged_tiles(D):
    """Several key tiles with ragged tails (chunk of 100 tokens, 400 keys
    at steady state) and a ragged query tile."""
    run_stream(102 + D, 50, 2, 2, 6, 2, D, "bf16", 7)


def test_bf16_stream_two_sink_chunks_no_sink():
    run_stream(110, 24, 1, 2, 3, 3, 128, "bf16", 7)      # sink = 2 chunks
    run_stream(111, 24, 1, 0, 3, 3, 128, "bf16", 6)      # no sink (window only)


def test_bf16_sink_only_cache_only():
    """W = C (no ring) and n_cur = 0: a query chunk attends the sink alone."""
    run_stream(112, 40, 2, 2, 2, 2, 128, "bf16", 5, n_cur_zero_at=(2, 3, 4))


def test_bf16_max_ring_slots():
    """The largest window: 30 ring slots (32 key runs per call)."""
    run_stream(113, 8, 1, 1, 31, 2, 128, "bf16", 34, check_bytes=False)


def test_bf16_max_key_runs():
    """8 sink chunks + 30 ring slots + the current chunk: 39 key runs, the
    most a BF16 cache walks (each sink chunk is a run of its own)."""
    run_stream(114, 8, 1, 8, 31, 2, 64, "bf16", 40, check_bytes=False)


I8_MODES = pytest.mark.parametrize("i8_mode", [ll.LL_I8_STAGED, ll.LL_I8_IN_KERNEL],
                                   ids=["staged", "in_kernel"])


@I8_MODES
def test_int8_stream_bitexact_and_parity(i8_mode):
    """INT8 KV: codes and scales bit-exact vs the oracle quantiser; attention
    vs the oracle on the identically dequantised values, both ways of reading
    the codes."""
    run_stream(120, 50, 2, 2, 6, 2, 128, "bf16", 6, int8=True, i8_mode=i8_mode)
    run_stream(121, 33, 1, 1, 3, 3, 64, "bf16", 5, int8=True, i8_mode=i8_mode)


def _config1_inputs(c, tensor):
    return synth.normal((4680, 12, 128), "bf16", 1, 0, c, 0, tensor)


def test_config1_snapshot_full():
    """Single layer at full size: 12 heads x 128, 1560 tokens/frame, chunk = 3
    frames (4680 tokens), sink 3 frames, window 9 frames.  Chunks 0..3 are
    appended, then chunk 4 attends sink (chunk 0) + ring (chunks 3, 2) +
    itself: 18720 keys.  Every query row of every head, and the log-sum-exp,
    is checked against the oracle; the cache bytes are checked in full."""
    T, C, S, W, H, D = 1560, 3, 3, 9, 12, 128
    cfg = ll.make_config(1, H, D, T, C, S, W, ll.LL_BF16, ll.LL_BF16)
    cache = ll.Cache(cfg)
    ks, vs = {}, {}
    for c in range(4):
        ks[c], vs[c] = _config1_inputs(c, K), _config1_inputs(c, V)
        cache.append_chunk(0, dev(ks[c], "bf16"), dev(vs[c], "bf16"))
    q = _config1_inputs(4, Q)
    k4, v4 = _config1_inputs(4, K), _config1_inputs(4, V)
    out = torch.empty((4680, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, 4680), dtype=torch.float32, device="cuda")
    say("[config1 snapshot] attention chunk 4 (18720 keys)")
    cache.attn(0, dev(q, "bf16"), dev(k4, "bf16"), dev(v4, "bf16"), 1 / math.sqrt(D), out, lse)
    torch.cuda.synchronize()
    st = cache.query(0)
    assert st["slot_chunk"] == [3, 2] and st["ring_valid"] == 2
    hk = np.concatenate([ks[0], ks[2], ks[3], k4])
    hv = np.concatenate([vs[0], vs[2], vs[3], v4])
    say("[config1 snapshot] oracle over all 4680 x 12 query rows")
    want, wlse = masked_attention(q, hk, hv, None, 1 / math.sqrt(D))
    check_out(out, want, "bf16", "config1 all rows")
    check_lse(lse, wlse, "bf16", "config1 all rows")
    assert torch.isfinite(out.float()).all()
    _check_v_padding(cache, 0, ll.LL_SEG_SINK, [0])
    _check_v_padding(cache, 0, ll.LL_SEG_RING, [3, 2])
    # cache bytes: sink = chunk 0, slot 0 = chunk 3, slot 1 = chunk 2
    for which, src in ((ll.LL_WHICH_K, ks), (ll.LL_WHICH_V, vs)):
        sink = cache.rows(0, which, ll.LL_SEG_SINK).contiguous().view(torch.int16).cpu().numpy()
        ring = cache.rows(0, which, ll.LL_SEG_RING).contiguous().view(torch.int16).cpu().numpy()
        assert np.array_equal(sink.view(np.uint16), synth.bf16_bits(src[0].transpose(1, 0, 2)))
        want_ring = np.concatenate([src[3], src[2]]).transpose(1, 0, 2)
        assert np.array_equal(ring.view(np.uint16), synth.bf16_bits(want_ring))


def test_recache_all_layers_and_order_invariance():
    """KV-recache of every layer (layer = -1): resident window chunks are
    rewritten oldest first, bit-exact, the sink is kept, and attention equals
    the oracle on the recached history.  Two caches holding the same logical
    window in different physical slot orders give the same output (P7)."""
    T, C, S, W, H, D, L = 40, 2, 2, 6, 2, 128, 3
    g = CacheGeometry(T, C, S, W)
    ct = g.chunk_tokens
    scale = 1 / math.sqrt(D)
    outs = []
    for n_pre in (4, 5):                       # ring rotations differ
        cfg = ll.make_config(L, H, D, T, C, S, W, ll.LL_BF16, ll.LL_BF16)
        cache = ll.Cache(cfg)
        hists = [LayerHistory(g) for _ in range(L)]
        sims = [DequeCacheModel(g) for _ in range(L)]
        for c in range(n_pre):
            for layer in range(L):
                k = synth.normal((ct, H, D), "bf16", 130, layer, c, 0, K)
                v = synth.normal((ct, H, D), "bf16", 130, layer, c, 0, V)
                cache.append_chunk(layer, dev(k, "bf16"), dev(v, "bf16"))
                hists[layer].append(k, v)
                sims[layer].append()
        n = 2 * ct
        pk = synth.normal((L, n, H, D), "bf16", 130, 0, 99, 0, RK)
        pv = synth.normal((L, n, H, D), "bf16", 130, 0, 99, 0, RV)
        say(f"[recache] n_pre={n_pre} layer=-1")
        cache.recache(-1, dev(pk, "bf16"), dev(pv, "bf16"), n)
        torch.cuda.synchronize()
        q = synth.normal((ct, H, D), "bf16", 130, 0, 50, 0, Q)
        kc = synth.normal((ct, H, D), "bf16", 130, 0, 50, 0, K)
        vc = synth.normal((ct, H, D), "bf16", 130, 0, 50, 0, V)
        for layer in range(L):
            hists[layer].recache(pk[layer], pv[layer])
            # bytes: oldest resident chunk's slot holds the payload's first chunk
            sim = sims[layer]
            for which, p in ((ll.LL_WHICH_K, pk[layer]), (ll.LL_WHICH_V, pv[layer])):
                ring = cache.rows(layer, which, ll.LL_SEG_RING)
                for i, ch in enumerate(sim.resident_ring_chunks()):
                    s = sim.slot_chunk.index(ch)
                    got = ring[:, s * ct:(s + 1) * ct].contiguous().view(torch.int16).cpu().numpy()
                    want = synth.bf16_bits(p[i * ct:(i + 1) * ct].transpose(1, 0, 2))
                    assert np.array_equal(got.view(np.uint16), want)
            out = torch.empty((ct, H, D), dtype=torch.bfloat16, device="cuda")
            cache.attn(layer, dev(q, "bf16"), dev(kc, "bf16"), dev(vc, "bf16"), scale, out)
            torch.cuda.synchronize()
            hk, hv = hists[layer].keys(kc, vc)
            want, _ = sink_window_attention(q, hk, hv, n_pre, tokens_per_frame=T, frames_per_chunk=C,
                                            sink_frames=S, window_frames=W, scale=scale)
            check_out(out, want, "bf16", f"recache n_pre={n_pre} layer {layer}")
            if layer == 0:
                outs.append(host(out))
    # Same logical key set {sink = chunk 0, payload chunks, current} in both.
    assert np.abs(outs[0] - outs[1]).max() <= 2e-2


@pytest.mark.parametrize("segment", ["sink", "ring_old", "ring_new", "current"])
@pytest.mark.parametrize("strength", [40.0, 300.0])
def test_planted_key_per_segment(segment, strength):
    """A key aligned with query i (k = strength * q_i/|q_i|) in each key run
    in turn: the output row i is that key's value (detects a dropped run).
    Strength 300 puts the score ~430 (log2 units) above the others, past the
    fp32 range of 2^s: the softmax must move its reference."""
    T, C, S, W, H, D = 64, 1, 1, 3, 2, 128
    ct = T
    cfg = ll.make_config(1, H, D, T, C, S, W, ll.LL_BF16, ll.LL_BF16)
    cache = ll.Cache(cfg)
    c_now = 6
    frame = {"sink": 0, "ring_old": 4, "ring_new": 5, "current": 6}[segment]
    i, j = 9, 17
    q = synth.normal((ct, H, D), "bf16", 140, 0, c_now, 0, Q)
    plant = strength * q[i] / np.linalg.norm(q[i], axis=-1, keepdims=True)
    plant = synth.bf16_to_f32(synth.bf16_bits(plant.astype(np.float32)))
    vals = {}
    for c in range(c_now + 1):
        k = synth.normal((ct, H, D), "bf16", 140, 0, c, 0, K) * np.float32(0.0625)
        v = synth.normal((ct, H, D), "bf16", 140, 0, c, 0, V)
        if c == frame:
            k[j] = plant
        vals[c] = (k, v)
        if c < c_now:
            cache.append_chunk(0, dev(k, "bf16"), dev(v, "bf16"))
    k, v = vals[c_now]
    out = torch.empty((ct, H, D), dtype=torch.bfloat16, device="cuda")
    cache.attn(0, dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), 1 / math.sqrt(D), out)
    torch.cuda.synchronize()
    got = host(out)[i]
    want = vals[frame][1][j]
    say(f"[planted {segment} {strength}] max diff {np.abs(got - want).max():.3e}")
    assert np.abs(got - want).max() <= 2e-2


@pytest.mark.parametrize("order", ["rising", "falling"])
def test_extreme_score_ranges(order):
    """Key magnitudes that grow (or shrink) by 2^6 per chunk: logits from
    ~1e-2 to ~1e4.  Rising scores overflow 2^s against the first tile's
    reference several times; falling ones underflow to zero.  The output must
    still equal the float64 softmax."""
    T, C, S, W, H, D = 64, 1, 1, 4, 2, 128
    g = CacheGeometry(T, C, S, W)
    cfg = ll.make_config(1, H, D, T, C, S, W, ll.LL_BF16, ll.LL_BF16)
    cache = ll.Cache(cfg)
    hist = LayerHistory(g)
    n = 6
    factors = [2.0 ** (6 * c - 8) for c in range(n)]
    if order == "falling":
        factors = factors[::-1]
    q = synth.normal((T, H, D), "bf16", 160, 0, n - 1, 0, Q)
    for c in range(n):
        k = synth.normal((T, H, D), "bf16", 160, 0, c, 0, K) * np.float32(factors[c])
        v = synth.normal((T, H, D), "bf16", 160, 0, c, 0, V)
        if c < n - 1:
            cache.append_chunk(0, dev(k, "bf16"), dev(v, "bf16"))
            hist.append(k, v)
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    cache.attn(0, dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), 1 / math.sqrt(D), out, lse)
    torch.cuda.synchronize()
    hk, hv = hist.keys(k, v)
    want, wlse = sink_window_attention(q, hk, hv, n - 1, tokens_per_frame=T, frames_per_chunk=C,
                                       sink_frames=S, window_frames=W, scale=1 / math.sqrt(D))
    assert torch.isfinite(out.float()).all()
    check_out(out, want, "bf16", f"extreme scores {order}")
    # lse reaches ~1e7 here; the scores carry the bf16 rounding of the scaled
    # queries (relative 2^-9), so compare relative to the size
    gl = host(lse)
    assert np.all(np.abs(gl - wlse) <= 1e-2 + 4e-3 * np.abs(wlse))


def test_single_query_and_zero_queries():
    T, C, S, W, H, D = 30, 1, 1, 2, 2, 128
    cfg = ll.make_config(1, H, D, T, C, S, W, ll.LL_BF16, ll.LL_BF16)
    cache = ll.Cache(cfg)
    k = synth.normal((T, H, D), "bf16", 150, 0, 0, 0, K)
    v = synth.normal((T, H, D), "bf16", 150, 0, 0, 0, V)
    q = synth.normal((1, H, D), "bf16", 150, 0, 0, 0, Q)
    out = torch.empty((1, H, D), dtype=torch.bfloat16, device="cuda")
    cache.attn(0, dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), 0.1, out)
    torch.cuda.synchronize()
    want, _ = masked_attention(q, k, v, None, 0.1)
    check_out(out, want, "bf16", "single query")
    empty = torch.empty((0, H, D), dtype=torch.bfloat16, device="cuda")
    cache.attn(0, empty, dev(k, "bf16"), dev(v, "bf16"), 0.1, empty)


@pytest.mark.parametrize("dtype,D,n_q,n_txt", [("bf16", 128, 300, 512), ("bf16", 128, 4680, 512),
                                               ("bf16", 64, 77, 33), ("f32", 64, 50, 77),
                                               ("f32", 128, 20, 1)])
def test_cross_attention(dtype, D, n_q, n_txt):
    H = 12 if D == 128 and dtype == "bf16" else 3
    q = synth.normal((n_q, H, D), dtype, 160, 0, n_q, 0, Q)
    kt = synth.normal((n_txt, H, D), dtype, 160, 0, n_txt, 0, K_TXT)
    vt = synth.normal((n_txt, H, D), dtype, 160, 0, n_txt, 0, V_TXT)
    out = torch.empty((n_q, H, D), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                      device="cuda")
    lse = torch.empty((H, n_q), dtype=torch.float32, device="cuda")
    say(f"[cross-attn {dtype} D={D} n_q={n_q} n_txt={n_txt}]")
    ll.ll_cross_attn(dev(q, dtype), dev(kt, dtype), dev(vt, dtype), 1 / math.sqrt(D), out,
                     act_code(dtype), lse)
    torch.cuda.synchronize()
    rows = np.arange(n_q) if n_q <= 512 else np.unique(np.r_[0, 127, 128, n_q - 1,
                                                              np.random.default_rng(0).choice(n_q, 200)])
    want, wlse = cross_attention(q[rows], kt, vt, 1 / math.sqrt(D))
    check_out(out[rows], want, dtype, "cross")
    check_lse(lse[:, rows], wlse, dtype, "cross")
    if n_txt == 1:
        assert np.abs(host(out) - vt[0][None]).max() <= (1e-6 if dtype == "f32" else 1e-2)


# --------------------------------------------------------------------------
# re-encoding attention after a KV-recache
# --------------------------------------------------------------------------

def run_reencode(cfg_id, T, C, S, W, H, D, dtype, n_chunks, check_at, int8=False, i8_mode=ll.LL_I8_STAGED):
    """Append ``n_chunks`` chunks; after each chunk in ``check_at`` recache the
    resident window with a fresh payload and run the re-encoding attention of
    the window chunks through the ABI, against the oracle on the same history
    (the int8 cache: on the exactly dequantised stored K/V)."""
    kv = ll.LL_I8 if int8 else act_code(dtype)
    cfg = ll.make_config(1, H, D, T, C, S, W, act_code(dtype), kv)
    cache = ll.Cache(cfg)
    if int8:
        cache.set_int8_dequant(i8_mode)
    g = CacheGeometry(T, C, S, W)
    hist = LayerHistory(g, int8=int8)
    ct = g.chunk_tokens
    scale = 1.0 / math.sqrt(D)
    for c in range(n_chunks):
        k = synth.normal((ct, H, D), dtype, cfg_id, 0, c, 0, K)
        v = synth.normal((ct, H, D), dtype, cfg_id, 0, c, 0, V)
        cache.append_chunk(0, dev(k, dtype), dev(v, dtype))
        hist.append(k, v)
        if c not in check_at:
            continue
        win = resident_window_chunks(c + 1, g)
        n = len(win) * ct
        rk = synth.normal((n, H, D), dtype, cfg_id, 1, c, 0, RK)
        rv = synth.normal((n, H, D), dtype, cfg_id, 1, c, 0, RV)
        q = synth.normal((n, H, D), dtype, cfg_id, 1, c, 0, Q)
        say(f"[reencode cfg={cfg_id} T={T} C={C} S={S} W={W} H={H} D={D} {dtype}"
            f"{' i8' if int8 else ''}] after chunk {c}: window chunks {win}")
        cache.recache(0, dev(rk, dtype), dev(rv, dtype), n)
        hist.recache(rk, rv)
        dq = dev(q, dtype)
        out = torch.empty_like(dq)
        lse = torch.empty((H, n), dtype=torch.float32, device="cuda")
        cache.reencode_attn(0, dq, scale, out, lse)
        torch.cuda.synchronize()
        hk, hv = hist.keys()
        want, wlse = window_reencode_attention(q, hk, hv, win, tokens_per_frame=T,
                                               frames_per_chunk=C, sink_frames=S,
                                               window_frames=W, scale=scale)
        check_out(out, want, dtype, f"re-encode after chunk {c}")
        check_lse(lse, wlse, dtype, f"re-encode after chunk {c}")


def test_reencode_bf16_ragged_partial_and_full_window():
    """100-token chunks (ragged key and query tiles), sink = 1 chunk, 3 ring
    slots: a window of 1, 2, then 3 chunks after evictions."""
    run_reencode(140, 50, 2, 2, 8, 2, 128, "bf16", 7, (1, 2, 5))


def test_reencode_bf16_d64_no_sink_two_query_tiles_per_chunk():
    """No sink; 300-token chunks span two query tiles, the second ragged."""
    run_reencode(141, 150, 2, 0, 6, 3, 64, "bf16", 5, (0, 1, 4))


def test_reencode_bf16_two_sink_chunks():
    run_reencode(142, 24, 1, 2, 4, 3, 128, "bf16", 7, (2, 6))


@I8_MODES
def test_reencode_int8_cache(i8_mode):
    run_reencode(143, 50, 2, 2, 6, 2, 128, "bf16", 5, (1, 4), int8=True, i8_mode=i8_mode)


def test_reencode_fp32():
    run_reencode(144, 37, 2, 2, 6, 2, 128, "f32", 5, (1, 4))


def test_reencode_config1_sampled():
    """Full size: 12 heads x 128, 4680-token chunks, sink 1 chunk, 2 ring
    slots.  Chunks 0..3 appended, the window (chunks 2, 3) recached, then the
    9360 window queries re-encoded; sampled rows of both chunks vs the oracle."""
    T, C, S, W, H, D = 1560, 3, 3, 9, 12, 128
    g = CacheGeometry(T, C, S, W)
    cfg = ll.make_config(1, H, D, T, C, S, W, ll.LL_BF16, ll.LL_BF16)
    cache = ll.Cache(cfg)
    hist = LayerHistory(g)
    for c in range(4):
        k, v = _config1_inputs(c, K), _config1_inputs(c, V)
        cache.append_chunk(0, dev(k, "bf16"), dev(v, "bf16"))
        hist.append(k, v)
    win = resident_window_chunks(4, g)
    assert win == [2, 3]
    pay = [synth.normal((9360, H, D), "bf16", 1, 1, 4, 0, t) for t in (RK, RV, Q)]
    cache.recache(0, dev(pay[0], "bf16"), dev(pay[1], "bf16"), 9360)
    hist.recache(pay[0], pay[1])
    out = torch.empty((9360, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, 9360), dtype=torch.float32, device="cuda")
    say("[reencode config1] 9360 window queries over sink + window (9360 / 14040 keys)")
    cache.reencode_attn(0, dev(pay[2], "bf16"), 1 / math.sqrt(D), out, lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 255, 256, 4607, 4608, 4679, 4680, 4681, 4935, 4936,
                                      9287, 9288, 9359], rng.choice(9360, 120, replace=False)]))
    hk, hv = hist.keys()
    want, wlse = window_reencode_attention(pay[2], hk, hv, win, tokens_per_frame=T,
                                           frames_per_chunk=C, sink_frames=S, window_frames=W,
                                           scale=1 / math.sqrt(D), rows=rows)
    check_out(out[rows], want, "bf16", "config1 re-encode sampled rows")
    check_lse(lse[:, rows], wlse, "bf16", "config1 re-encode sampled rows")


# --------------------------------------------------------------------------
# window/sink sweep shapes at full size
# --------------------------------------------------------------------------

@pytest.mark.parametrize("S,W", [(0, 21), (3, 27), (0, 3), (3, 3), (0, 12)])
def test_window_sweep_shapes_sampled(S, W):
    """The sweep's extreme shapes at full size (12 heads x 128, 4680-token
    chunks): the paper's long window (21 frames, no sink), the longest window
    with sink, a window of the current chunk alone with and without sink, and
    the short window without sink.  The sink and ring are filled and one
    chunk evicted; sampled rows of the next chunk's call vs the oracle."""
    T, C, H, D = 1560, 3, 12, 128
    g = CacheGeometry(T, C, S, W)
    cfg = ll.make_config(1, H, D, T, C, S, W, ll.LL_BF16, ll.LL_BF16)
    cache = ll.Cache(cfg)
    hist = LayerHistory(g)
    n = S // C + (W - C) // C + 1
    for c in range(n):
        k = synth.normal((4680, H, D), "bf16", 150, S, c, W, K)
        v = synth.normal((4680, H, D), "bf16", 150, S, c, W, V)
        cache.append_chunk(0, dev(k, "bf16"), dev(v, "bf16"))
        hist.append(k, v)
    q, k, v = (synth.normal((4680, H, D), "bf16", 150, S, n, W, t) for t in (Q, K, V))
    out = torch.empty((4680, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, 4680), dtype=torch.float32, device="cuda")
    say(f"[sweep S={S} W={W}] chunk {n}: {S * T + W * T} keys")
    cache.attn(0, dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), 1 / math.sqrt(D), out, lse)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 255, 256, 4607, 4608, 4679],
                                     np.random.default_rng(S + W).choice(4680, 40, replace=False)]))
    hk, hv = hist.keys(k, v)
    want, wlse = sink_window_attention(q[rows], hk, hv, n, tokens_per_frame=T, frames_per_chunk=C,
                                       sink_frames=S, window_frames=W, scale=1 / math.sqrt(D))
    check_out(out[rows], want, "bf16", f"sweep S={S} W={W}")
    check_lse(lse[:, rows], wlse, "bf16", f"sweep S={S} W={W}")


# --------------------------------------------------------------------------
# random small geometries (fixed draw)
# --------------------------------------------------------------------------

def _random_geometries(n=24, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        C = int(rng.integers(1, 4))
        T = int(rng.integers(3, 70))
        nsc = int(rng.integers(0, 3))
        R = int(rng.integers(0, 6))
        H = int(rng.integers(1, 4))
        D = int(rng.choice([64, 128]))
        kind = ["bf16", "f32", "int8"][i % 3]
        out.append((200 + i, T, C, nsc * C, (R + 1) * C, H, D, kind, nsc + R + 2))
    return out


@pytest.mark.parametrize("geom", _random_geometries(), ids=lambda g: f"cfg{g[0]}-{g[7]}")
def test_random_geometry_stream(geom):
    """A fixed draw of small geometries (tokens per frame, frames per chunk,
    sink chunks, ring slots, heads, head dim, bf16 / fp32 / int8 cache),
    streamed past the first eviction: every attention output against the
    oracle and the cache bytes after every append."""
    cfg_id, T, C, S, W, H, D, kind, n = geom
    # the int8 geometries alternate between the two ways of reading the codes
    mode = ll.LL_I8_IN_KERNEL if (cfg_id // 3) % 2 else ll.LL_I8_STAGED
    run_stream(cfg_id, T, C, S, W, H, D, "f32" if kind == "f32" else "bf16", n, int8=kind == "int8",
               i8_mode=mode)
