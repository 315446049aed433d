"""Oracle linear-attention variant of the sink + short-window attention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages say that the method carries over to any model that rolls out
autoregressively over a KV cache, and that it was also built on a
linear-attention video generator for further speed (LongLive: Real-time
Interactive Long Video Generation, §4 "Implementation", last sentence; the same
point in the conclusion).  They give no formulation.  The reading taken here
(the plainest one the rest of the method supports):

* the key set is the softmax call's: the frame sink, the resident window and
  the current chunk (:func:`oracle.attention.frame_mask`);
* softmax is replaced by the linear-attention kernel
  ``w_ij = phi(q_i) . phi(k_j)`` with the feature map ``phi(x) = max(x, 0)``
  applied elementwise (non-negative, so every weight is >= 0);
* ``o_i = sum_j w_ij v_j / (sum_j w_ij + eps)``, ``eps = 1e-6`` keeping a row
  whose weights are all zero finite (its output is 0); no logit scale.

This module computes the pairwise (explicit) form in float64: every weight is
formed and masked, then the weighted sum and the normaliser.
"""

import numpy as np

from .attention import frame_mask

LINEAR_EPS = 1e-6


def feature_map(x):
    """phi(x) = max(x, 0), elementwise, in float64."""
    return np.maximum(np.asarray(x, dtype=np.float64), 0.0)


def linear_masked_attention(q, k, v, key_mask, eps=LINEAR_EPS, query_block=512):
    """Linear attention with an explicit key mask, in float64.

    q: [n_q, H, D]; k: [n_k, H, D]; v: [n_k, H, Dv]; key_mask: bool [n_k]
    (None = all keys).  Returns out [n_q, H, Dv] float64 with
    ``out_i = sum_j w_ij v_j / (sum_j w_ij + eps)``, ``w_ij = phi(q_i).phi(k_j)``
    over the allowed keys (masked keys get weight exactly 0).
    """
    fq = feature_map(q)
    fk = feature_map(k)
    v = np.asarray(v, dtype=np.float64)
    n_q, H, _ = fq.shape
    n_k = fk.shape[0]
    if key_mask is None:
        key_mask = np.ones(n_k, dtype=bool)
    if not key_mask.any():
        raise ValueError("attention over an empty key set is undefined")
    out = np.empty((n_q, H, v.shape[2]), dtype=np.float64)
    for h in range(H):
        kh = fk[:, h, :]
        vh = v[:, h, :]
        for q0 in range(0, n_q, query_block):
            w = fq[q0:q0 + query_block, h, :] @ kh.T     # [b, n_k] pairwise weights
            w[:, ~key_mask] = 0.0
            out[q0:q0 + query_block, h, :] = (w @ vh) / (w.sum(axis=1, keepdims=True) + eps)
    return out


def linear_sink_window_attention(q, hist_k, hist_v, chunk, *, tokens_per_frame,
                                 frames_per_chunk, sink_frames, window_frames,
                                 eps=LINEAR_EPS, query_block=512):
    """Linear-attention counterpart of :func:`oracle.attention.sink_window_attention`:
    chunk ``chunk``'s queries over the same frame sink + window key set of the
    layer's token history ``hist_k``/``hist_v`` [n_hist, H, D]."""
    mask = frame_mask(hist_k.shape[0], chunk, tokens_per_frame=tokens_per_frame,
                      frames_per_chunk=frames_per_chunk, sink_frames=sink_frames,
                      window_frames=window_frames)
    return linear_masked_attention(q, hist_k, hist_v, mask, eps, query_block)
