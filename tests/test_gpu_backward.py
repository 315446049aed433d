"""GPU parity of the backward of the sink+window call (training step).

LongLive: Real-time Interactive Long Video Generation, §3.2 (gradients flow
through the current clip only; earlier frames are detached) and §3.3 (the
window's K/V without gradient, the current clip's with gradient, the sink
concatenated).  The forward runs through ll_sink_window_attn (which also gives
the lse the backward needs); the backward's dQ, dK_cur and dV_cur are
compared with the float64 oracle on the same bf16 inputs.

Tolerance: the kernel rounds Q*scale*log2(e), P and dS to bf16 (relative
2^-9 each) and forms delta from the bf16 forward output, with fp32
accumulation; the gradients are checked per tensor by relative L2 error
(<= 2e-2) and max-abs error relative to the tensor's largest value (<= 3e-2).
"""

import math

import numpy as np
import pytest
import torch

from oracle import CacheGeometry, LayerHistory, sink_window_attention_grad
from sink_short_window_amd import ll, synth
from sink_short_window_amd.synth import Q, K, V
from gpu_util import need_gpu, say, dev, host

pytestmark = pytest.mark.gpu

GRAD_REL_L2 = 2e-2
GRAD_MAX_REL = 3e-2
DOUT = 20     # synth tensor id of the upstream gradient


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def check_grad(got, want, what):
    g = host(got)
    assert np.isfinite(g).all(), f"{what}: non-finite gradient"
    err = np.abs(g - want)
    scale = max(float(np.abs(want).max()), 1e-30)
    rel = float(np.linalg.norm(g - want) / max(np.linalg.norm(want), 1e-30))
    say(f"  {what}: rel_l2={rel:.3e} max_abs={float(err.max()):.3e} (max |want| {scale:.3e})")
    assert rel <= GRAD_REL_L2, f"{what}: rel L2 {rel}"
    assert float(err.max()) <= GRAD_MAX_REL * scale, f"{what}: max abs {float(err.max())}"


def run_bwd(cfg_id, T, C, S, W, H, D, n_pre, with_cur=True, rows=None, int8=False):
    cfg = ll.make_config(1, H, D, T, C, S, W, ll.LL_BF16, ll.LL_I8 if int8 else ll.LL_BF16)
    cache = ll.Cache(cfg)
    g = CacheGeometry(T, C, S, W)
    hist = LayerHistory(g, int8=int8)
    ct = g.chunk_tokens
    scale = 1.0 / math.sqrt(D)
    for c in range(n_pre):
        k = synth.normal((ct, H, D), "bf16", cfg_id, 0, c, 0, K)
        v = synth.normal((ct, H, D), "bf16", cfg_id, 0, c, 0, V)
        cache.append_chunk(0, dev(k, "bf16"), dev(v, "bf16"))
        hist.append(k, v)
    c = n_pre
    q, k, v, do = (synth.normal((ct, H, D), "bf16", cfg_id, 0, c, 0, t) for t in (Q, K, V, DOUT))
    dq_, dk_, dv_, ddo = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(do, "bf16")
    out = torch.empty_like(dq_)
    lse = torch.empty((H, ct), dtype=torch.float32, device="cuda")
    say(f"[bwd cfg={cfg_id} T={T} C={C} S={S} W={W} H={H} D={D}{' i8' if int8 else ''}] chunk {c}"
        f"{'' if with_cur else ' (cache only)'}")
    kc, vc = (dk_, dv_) if with_cur else (None, None)
    cache.attn(0, dq_, kc, vc, scale, out, lse)
    # The workspace and the gradient buffers start as NaN: every element the
    # call must write is checked finite, and the Q' copy the call keeps in dq
    # before the dQ kernel overwrites it must not survive anywhere.
    nan = lambda *shape: torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    delta = nan(H, ct)
    gq = nan(ct, H, D)
    gk = nan(ct, H, D) if with_cur else None
    gv = nan(ct, H, D) if with_cur else None
    cache.attn_bwd(0, dq_, kc, vc, scale, out, lse, ddo, delta, gq, gk, gv)
    torch.cuda.synchronize()
    hk, hv = hist.keys(k, v) if with_cur else hist.keys()
    n_grad = ct if with_cur else 0
    wq, wk, wv = sink_window_attention_grad(q, hk, hv, c, do, n_grad, tokens_per_frame=T,
                                            frames_per_chunk=C, sink_frames=S, window_frames=W,
                                            scale=scale)
    sel = slice(None) if rows is None else rows
    check_grad(gq[sel], wq[sel], "dq")
    if with_cur:
        check_grad(gk[sel], wk[sel], "dk_cur")
        check_grad(gv[sel], wv[sel], "dv_cur")


def test_bwd_ragged_tiles_d128():
    """100-token chunks: ragged key tiles in every run, one ragged query tile
    and one ragged key block of the current chunk; sink + full ring."""
    run_bwd(160, 50, 2, 2, 6, 2, 128, 4)


def test_bwd_d64_no_sink_several_tiles():
    """300-token chunks: three query tiles and three key blocks, no sink."""
    run_bwd(161, 150, 2, 0, 6, 3, 64, 3)


def test_bwd_cache_only_dq():
    """n_cur = 0: the key set is the cached context alone; only dQ."""
    run_bwd(162, 40, 2, 2, 6, 2, 128, 3, with_cur=False)


def test_bwd_two_sink_chunks_first_chunk():
    """Early chunk (window not full yet) and a sink of two chunks."""
    run_bwd(163, 24, 1, 2, 4, 3, 128, 1)
    run_bwd(164, 24, 1, 2, 4, 3, 128, 5)


def test_bwd_config1_full():
    """Full size: 12 heads x 128, 4680 queries over sink + 2 window chunks +
    the current chunk (18720 keys); every row of dQ, dK_cur and dV_cur
    checked against the full float64 oracle."""
    run_bwd(165, 1560, 3, 3, 9, 12, 128, 4)


def test_bwd_int8_cache():
    """INT8 cache: the detached context is the exactly dequantised stored K/V
    (the oracle's int8 history); the current chunk stays bf16."""
    run_bwd(166, 50, 2, 2, 6, 2, 128, 4, int8=True)


def _random_bwd_geometries(n=12, seed=2027):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        C = int(rng.integers(1, 4))
        T = int(rng.integers(3, 90))
        nsc = int(rng.integers(0, 3))
        R = int(rng.integers(0, 4))
        H = int(rng.integers(1, 4))
        D = int(rng.choice([64, 128]))
        n_pre = int(rng.integers(0, nsc + R + 3))
        with_cur = bool(n_pre == 0 or i % 4 != 3)  # every fourth: cache-only (dQ alone)
        out.append((300 + i, T, C, nsc * C, (R + 1) * C, H, D, n_pre, with_cur, i % 3 == 2))
    return out


@pytest.mark.parametrize("geom", _random_bwd_geometries(),
                         ids=lambda g: f"cfg{g[0]}-D{g[6]}{'-i8' if g[9] else ''}{'' if g[8] else '-dq'}")
def test_bwd_random_geometries(geom):
    """A fixed draw of small geometries (tokens per frame, frames per chunk,
    sink chunks, ring slots, heads, head dim, chunks already cached, bf16 or
    int8 cache, with or without the current chunk): every row of every
    gradient against the float64 oracle."""
    cfg_id, T, C, S, W, H, D, n_pre, with_cur, int8 = geom
    run_bwd(cfg_id, T, C, S, W, H, D, n_pre, with_cur=with_cur, int8=int8)
