"""Pins for the linear-attention variant of the oracle (oracle/linear_attention.py),
checked against things other than the oracle itself: a pure-Python streaming
simulation, a hand-worked example, closed forms and invariants.

Reading (the pages give no formulation; LongLive: Real-time Interactive Long
Video Generation, §4 "Implementation", only says the method was also built on a
linear-attention model): the softmax call's key set, weights
w_ij = max(q_i, 0) . max(k_j, 0), o_i = sum_j w_ij v_j / (sum_j w_ij + eps).
"""

from collections import deque

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

from oracle import (CacheGeometry, LayerHistory, LINEAR_EPS, linear_masked_attention,
                    linear_sink_window_attention)


def _bf_linear(qrow, keys, vals, eps):
    """Pure-Python linear attention of one query row over lists of rows."""
    fq = [x if x > 0 else 0.0 for x in qrow]
    w = [sum(a * (b if b > 0 else 0.0) for a, b in zip(fq, k)) for k in keys]
    den = sum(w)
    return [sum(w[j] * vals[j][d] for j in range(len(keys))) / (den + eps) for d in range(len(vals[0]))]


def _streaming_bruteforce(qs, ks, vs, T, C, S, W, eps):
    """Streaming generation with an explicit cache (sink list + FIFO of window
    chunks, oldest evicted); every query of chunk c attends sink + cached window
    + chunk c."""
    ct = C * T
    R = (W - C) // C
    sink_k, sink_v, fifo = [], [], deque()
    H = qs[0].shape[1]
    res = []
    for c in range(len(qs)):
        out = np.zeros(qs[c].shape)
        for h in range(H):
            keys = [r[h].tolist() for r in sink_k]
            vals = [r[h].tolist() for r in sink_v]
            for ck, cv in fifo:
                keys += [r[h].tolist() for r in ck]
                vals += [r[h].tolist() for r in cv]
            keys += [r[h].tolist() for r in ks[c]]
            vals += [r[h].tolist() for r in vs[c]]
            for i in range(ct):
                out[i, h] = _bf_linear(qs[c][i, h].tolist(), keys, vals, eps)
        res.append(out)
        if len(sink_k) < S * T:
            sink_k += list(ks[c])
            sink_v += list(vs[c])
        elif R > 0:
            if len(fifo) == R:
                fifo.popleft()
            fifo.append((ks[c], vs[c]))
    return res


geom_strategy = st.tuples(
    st.integers(1, 4),            # T
    st.integers(1, 3),            # C
    st.integers(0, 2),            # sink chunks
    st.integers(0, 3),            # ring slots
    st.integers(1, 2),            # H
    st.sampled_from([4, 8]),      # D
    st.integers(0, 2 ** 31 - 1),  # seed
)


@settings(max_examples=30, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(geom_strategy)
def test_linear_bruteforce_streaming(params):
    """The oracle (explicit frame mask over the full history) equals a
    pure-Python streaming simulation with explicit loops for the weights."""
    T, C, nsc, R, H, D, seed = params
    S, W = nsc * C, (R + 1) * C
    g = CacheGeometry(T, C, S, W)
    rng = np.random.default_rng(seed)
    n_chunks = nsc + R + 3
    f = lambda: [rng.standard_normal((C * T, H, D)) for _ in range(n_chunks)]
    qs, ks, vs = f(), f(), f()
    want = _streaming_bruteforce(qs, ks, vs, T, C, S, W, LINEAR_EPS)
    hist = LayerHistory(g)
    for c in range(n_chunks):
        hk, hv = hist.keys(ks[c], vs[c])
        got = linear_sink_window_attention(qs[c], hk, hv, c, tokens_per_frame=T, frames_per_chunk=C,
                                           sink_frames=S, window_frames=W)
        np.testing.assert_allclose(got, want[c], rtol=0, atol=1e-12)
        hist.append(ks[c], vs[c])


def test_linear_hand_worked_example():
    """q = (1, -1) so phi(q) = (1, 0); keys (2, 3), (-1, 5), (0.5, -2) give
    weights 2, 0, 0.5; values (1, 0), (7, 7), (0, 4): numerator (2, 2),
    denominator 2.5, output (2, 2) / (2.5 + 1e-6)."""
    q = np.array([[[1.0, -1.0]]])
    k = np.array([[[2.0, 3.0]], [[-1.0, 5.0]], [[0.5, -2.0]]])
    v = np.array([[[1.0, 0.0]], [[7.0, 7.0]], [[0.0, 4.0]]])
    got = linear_masked_attention(q, k, v, None)
    np.testing.assert_allclose(got[0, 0], [2.0 / 2.500001, 2.0 / 2.500001], rtol=0, atol=1e-15)
    # masking the first key leaves weight 0.5 on the third: (0, 2) / 0.500001
    got = linear_masked_attention(q, k, v, np.array([False, True, True]))
    np.testing.assert_allclose(got[0, 0], [0.0, 2.0 / 0.500001], rtol=0, atol=1e-15)


def test_linear_closed_forms():
    """Constant V gives V * den / (den + eps); a query with no positive entry
    has all weights 0 and output exactly 0; one allowed key gives its V scaled
    by w / (w + eps)."""
    rng = np.random.default_rng(3)
    n_k, H, D = 30, 2, 8
    q = rng.standard_normal((5, H, D))
    k = rng.standard_normal((n_k, H, D))
    vconst = np.broadcast_to(rng.standard_normal((1, H, D)), (n_k, H, D)).copy()
    mask = rng.random(n_k) < 0.7
    got = linear_masked_attention(q, k, vconst, mask)
    fq, fk = np.maximum(q, 0), np.maximum(k, 0)
    den = np.einsum("qhd,khd->qhk", fq, fk)[:, :, mask].sum(-1)
    np.testing.assert_allclose(got, vconst[:1] * (den / (den + LINEAR_EPS))[..., None], rtol=1e-13, atol=0)

    got = linear_masked_attention(-np.abs(q), k, rng.standard_normal((n_k, H, D)), mask)
    assert (got == 0).all()

    v = rng.standard_normal((n_k, H, D))
    one = np.zeros(n_k, dtype=bool)
    one[7] = True
    got = linear_masked_attention(q, k, v, one)
    w = np.einsum("qhd,hd->qh", fq, fk[7])
    np.testing.assert_allclose(got, v[7][None] * (w / (w + LINEAR_EPS))[..., None], rtol=1e-13, atol=0)


def test_linear_mask_and_order_invariance():
    """Keys outside the allowed set do not affect the output, and the physical
    order of the keys does not matter."""
    rng = np.random.default_rng(4)
    n_k, H, D = 40, 2, 8
    q = rng.standard_normal((6, H, D))
    k = rng.standard_normal((n_k, H, D))
    v = rng.standard_normal((n_k, H, D))
    mask = rng.random(n_k) < 0.5
    a = linear_masked_attention(q, k, v, mask)
    k2, v2 = k.copy(), v.copy()
    k2[~mask] = rng.standard_normal(k2[~mask].shape) * 100
    v2[~mask] = rng.standard_normal(v2[~mask].shape) * 100
    np.testing.assert_allclose(linear_masked_attention(q, k2, v2, mask), a, rtol=0, atol=1e-13)
    perm = rng.permutation(n_k)
    np.testing.assert_allclose(linear_masked_attention(q, k[perm], v[perm], mask[perm]), a, rtol=0, atol=1e-13)


def test_linear_empty_key_set_is_rejected():
    with pytest.raises(ValueError):
        linear_masked_attention(np.zeros((1, 1, 2)), np.zeros((3, 1, 2)), np.zeros((3, 1, 2)),
                                np.zeros(3, dtype=bool))
