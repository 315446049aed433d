"""The allocation-free backward (ll_sink_window_attn_bwd_noalloc, static delta
workspace) against the backward with a caller workspace
(ll_sink_window_attn_bwd): identical gradients on two calls in a row, the
second smaller, through the C ABI."""

import math

import pytest
import torch

from sink_short_window_amd import ll, synth
from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

Q, K, V = synth.Q, synth.K, synth.V


def _case(cache, cfg_id, n_q, ct, H, D, with_cur, chunk):
    dev = lambda x: synth.to_torch(x, "bf16", "cuda")
    scale = 1.0 / math.sqrt(D)
    q = dev(synth.normal((n_q, H, D), "bf16", cfg_id, 0, chunk, 0, Q))
    g = dev(synth.normal((n_q, H, D), "bf16", cfg_id, 0, chunk, 1, Q))
    kc = dev(synth.normal((ct, H, D), "bf16", cfg_id, 0, chunk, 0, K)) if with_cur else None
    vc = dev(synth.normal((ct, H, D), "bf16", cfg_id, 0, chunk, 0, V)) if with_cur else None
    out = torch.empty_like(q)
    lse = torch.empty((H, n_q), dtype=torch.float32, device="cuda")
    cache.attn(0, q, kc, vc, scale, out, lse)
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
    delta = f32(H, n_q)
    ref = [f32(n_q, H, D)] + ([f32(ct, H, D), f32(ct, H, D)] if with_cur else [None, None])
    got = [f32(n_q, H, D)] + ([f32(ct, H, D), f32(ct, H, D)] if with_cur else [None, None])
    for t in got:
        if t is not None:
            t.fill_(float("nan"))
    cache.attn_bwd(0, q, kc, vc, scale, out, lse, g, delta, *ref)
    ll.ll_sink_window_attn_bwd_noalloc(cache.handle, 0, q, kc, vc, scale, out, lse, g, *got)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        if a is None:
            continue
        say(f"  {name}: max |diff| = {float((a - b).abs().max()):.3e}")
        assert torch.equal(a, b), name


def test_noalloc_backward_matches_workspace_backward():
    need_gpu()
    T, C, S, W, H, D = 50, 2, 2, 6, 3, 128
    ct = C * T
    cache = ll.Cache(ll.make_config(1, H, D, T, C, S, W, ll.LL_BF16, ll.LL_BF16))
    dev = lambda x: synth.to_torch(x, "bf16", "cuda")
    for c in range(3):
        cache.append_chunk(0, dev(synth.normal((ct, H, D), "bf16", 170, 0, c, 0, K)),
                           dev(synth.normal((ct, H, D), "bf16", 170, 0, c, 0, V)))
    say("[noalloc] call 1: 100 queries with the current chunk")
    _case(cache, 170, ct, ct, H, D, True, 3)
    say("[noalloc] call 2: 37 queries, cache only")
    _case(cache, 170, 37, ct, H, D, False, 4)
    # a smaller geometry on another cache: the static workspace is shared
    cache2 = ll.Cache(ll.make_config(1, 1, 64, 24, 1, 1, 3, ll.LL_BF16, ll.LL_BF16))
    for c in range(2):
        cache2.append_chunk(0, dev(synth.normal((24, 1, 64), "bf16", 171, 0, c, 0, K)),
                            dev(synth.normal((24, 1, 64), "bf16", 171, 0, c, 0, V)))
    say("[noalloc] call 3: another cache, 1 head x 64, 24 queries")
    _case(cache2, 171, 24, 24, 1, 64, True, 2)
