"""GPU parity of the linear-attention variant (ll_sink_window_linear_attn)
against the float64 oracle (oracle/linear_attention.py) on the same seeded
inputs: streams with ragged tiles, no sink, an int8 cache, cache-only calls,
a closed form, and the full-size snapshot sampled.  Reading (the pages give no
formulation; LongLive: Real-time Interactive Long Video Generation, §4
"Implementation"): the softmax call's key set, weights max(q,0).max(k,0),
normalised weighted sum of V.
"""

import numpy as np
import pytest
import torch

from oracle import CacheGeometry, LayerHistory, linear_sink_window_attention, linear_masked_attention, frame_mask
from sink_short_window_amd import ll, synth
from sink_short_window_amd.synth import Q, K, V
from gpu_util import need_gpu, say, dev, check_out

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run_linear_stream(cfg_id, T, C, S, W, H, D, n_chunks, int8=False, n_cur_zero_at=()):
    cfg = ll.make_config(1, H, D, T, C, S, W, ll.LL_BF16, ll.LL_I8 if int8 else ll.LL_BF16)
    cache = ll.Cache(cfg)
    g = CacheGeometry(T, C, S, W)
    hist = LayerHistory(g, int8=int8)
    ct = g.chunk_tokens
    for c in range(n_chunks):
        q = synth.normal((ct, H, D), "bf16", cfg_id, 0, c, 0, Q)
        k = synth.normal((ct, H, D), "bf16", cfg_id, 0, c, 0, K)
        v = synth.normal((ct, H, D), "bf16", cfg_id, 0, c, 0, V)
        dq, dk, dv = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
        out = torch.empty_like(dq)
        use_cur = c == 0 or c not in n_cur_zero_at
        say(f"[linear cfg={cfg_id} T={T} C={C} S={S} W={W} H={H} D={D}{' i8' if int8 else ''}] chunk {c}")
        cache.linear_attn(0, dq, dk if use_cur else None, dv if use_cur else None, out)
        torch.cuda.synchronize()
        hk, hv = hist.keys(k, v) if use_cur else hist.keys()
        want = linear_sink_window_attention(q, hk, hv, c, tokens_per_frame=T, frames_per_chunk=C,
                                            sink_frames=S, window_frames=W)
        check_out(out, want, "bf16", f"chunk {c}")
        cache.append_chunk(0, dk, dv)
        hist.append(k, v)
    return cache


@pytest.mark.parametrize("D", [128, 64])
def test_linear_stream_ragged_tiles(D):
    """Chunks of 100 tokens (ragged key and query tiles), sink 1 chunk, 2 ring
    slots, 7 chunks with eviction."""
    run_linear_stream(301 + D, 50, 2, 2, 6, 2, D, 7)


def test_linear_stream_no_sink_cache_only_calls():
    run_linear_stream(311, 24, 2, 0, 8, 3, 128, 6, n_cur_zero_at=(2, 4))


def test_linear_stream_int8_cache():
    run_linear_stream(312, 40, 2, 2, 6, 2, 128, 5, int8=True)


@pytest.mark.parametrize("H,D", [(2, 128), (32, 128), (40, 64)])
def test_linear_many_tiles_several_splits(H, D):
    """700-token chunks, 2 sink chunks and 3 ring slots: 55 ragged 64-key tiles
    in 5 runs at the last chunk.  The key splits (min(32, tiles, 256 / H) of
    them, split s taking tiles s, s + n_split, ...) hold 1 or 2 tiles at H = 2
    and 7 to 10 at H = 32 and 40, so the state kernel's 4-stage LDS ring wraps
    and one split crosses runs and V layouts (the cache's transposed tiles,
    the current chunk's rows)."""
    run_linear_stream(313 + H, 350, 2, 4, 8, H, D, 5)


def test_linear_closed_forms_on_gpu():
    """Queries with no positive entry have all weights 0: output exactly 0.
    Constant V: output V * den / (den + eps) (~V)."""
    T, C, S, W, H, D = 32, 2, 2, 4, 2, 128
    cfg = ll.make_config(1, H, D, T, C, S, W, ll.LL_BF16, ll.LL_BF16)
    cache = ll.Cache(cfg)
    ct = T * C
    rng = np.random.default_rng(9)
    vconst = np.broadcast_to(rng.standard_normal((1, H, D)).astype(np.float32), (ct, H, D)).copy()
    for c in range(3):
        k = synth.normal((ct, H, D), "bf16", 320, 0, c, 0, K)
        cache.append_chunk(0, dev(k, "bf16"), dev(vconst, "bf16"))
    k = synth.normal((ct, H, D), "bf16", 320, 0, 3, 0, K)
    q = synth.normal((ct, H, D), "bf16", 320, 0, 3, 0, Q)
    out = torch.empty((ct, H, D), dtype=torch.bfloat16, device="cuda")
    cache.linear_attn(0, dev(-np.abs(q), "bf16"), dev(k, "bf16"), dev(vconst, "bf16"), out)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out)) == 0
    cache.linear_attn(0, dev(q, "bf16"), dev(k, "bf16"), dev(vconst, "bf16"), out)
    torch.cuda.synchronize()
    want = np.broadcast_to(synth.to_torch(vconst, "bf16", "cpu").double().numpy()[:1], (ct, H, D))
    check_out(out, want, "bf16", "constant V")


def test_linear_config1_snapshot_sampled():
    """Full size: 12 heads x 128, 4680 queries of chunk 4 over sink (chunk 0),
    ring (chunks 2, 3) and the current chunk, 18720 keys; sampled queries."""
    T, C, S, W, H, D = 1560, 3, 3, 9, 12, 128
    ct = C * T
    cfg = ll.make_config(1, H, D, T, C, S, W, ll.LL_BF16, ll.LL_BF16)
    cache = ll.Cache(cfg)
    g = CacheGeometry(T, C, S, W)
    hist = LayerHistory(g)
    for c in range(4):
        k = synth.normal((ct, H, D), "bf16", 1, 0, c, 0, K)
        v = synth.normal((ct, H, D), "bf16", 1, 0, c, 0, V)
        cache.append_chunk(0, dev(k, "bf16"), dev(v, "bf16"))
        hist.append(k, v)
    q = synth.normal((ct, H, D), "bf16", 1, 0, 4, 0, Q)
    k = synth.normal((ct, H, D), "bf16", 1, 0, 4, 0, K)
    v = synth.normal((ct, H, D), "bf16", 1, 0, 4, 0, V)
    out = torch.empty((ct, H, D), dtype=torch.bfloat16, device="cuda")
    say("[linear config1 snapshot] launch")
    cache.linear_attn(0, dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), out)
    torch.cuda.synchronize()
    hk, hv = hist.keys(k, v)
    rows = np.sort(np.random.default_rng(5).choice(ct, 96, replace=False))
    mask = frame_mask(hk.shape[0], 4, tokens_per_frame=T, frames_per_chunk=C, sink_frames=S, window_frames=W)
    assert int(mask.sum()) == 4 * ct
    want = linear_masked_attention(q[rows], hk, hv, mask)
    check_out(out[torch.as_tensor(rows, device="cuda")], want, "bf16", "sampled queries")
