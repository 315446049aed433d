"""Oracle attention: explicit frame masks and float64 softmax.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Notation (per layer): T tokens per latent frame, C frames per chunk, S sink
frames, W window frames (the window includes the chunk being generated),
H heads, D head dimension.  Token t of the generation history belongs to frame
``t // T``; chunk c covers frames ``[c*C, (c+1)*C)``.

What is computed, and where it is stated:

* Frame-level autoregression with a KV cache: each chunk of latent frames is
  generated conditioned on the cached keys/values of earlier chunks
  (LongLive: Real-time Interactive Long Video Generation, Abstract and §3.2
  "Streaming long tuning").  Causality is across chunks only: every query of a
  chunk sees the same key set, which includes the whole current chunk.
* Short-window attention: attention is restricted to a fixed window of the most
  recent frames (same paper, §3.3 "Efficient long inference", short window
  attention; Fig. 5 caption: window 9 latent frames + sink 3).
* Frame sink: the tokens of the first frame chunk stay in the cache for good and
  are concatenated to every layer's keys and values, so they are always
  attendable; they share one softmax with the window (same paper, §3.3, frame
  sink; §4 "Implementation": all tokens of the first frame chunk are the sink).
* Text cross-attention: the prompt is injected by cross-attention layers that
  alternate with self-attention in each DiT block (same paper, §3.1
  "KV recache").  It is plain unmasked softmax attention to the text K/V.
* Re-encoding at a KV-recache: at a prompt switch the cache is rebuilt by
  encoding the frames already generated again, paired with the new prompt
  (same paper, §3.1 "KV recache"; Fig. 2, right).  The self-attention of that
  pass is :func:`window_reencode_attention`.
* Training side (streaming long tuning): each step keeps the last W frames'
  K/V of the earlier context without gradient, the current supervised clip's
  K/V with gradient, and the sink tokens concatenated to every layer (same
  paper, §3.3 "Consistency between training and inference"; §3.2: generated
  frames are detached, gradients flow through the current clip only).  The
  backward of the attention call is :func:`sink_window_attention_grad`.
"""

import numpy as np


def allowed_frames(chunk, *, frames_per_chunk, sink_frames, window_frames):
    """Set of frame indices the queries of chunk ``chunk`` may attend.

    The sink is frames ``[0, S)``; the window is the W most recent frames
    ending with the last frame of the current chunk, ``[(c+1)C - W, (c+1)C)``
    clipped at 0.  The union is taken, so a frame in both is counted once
    (LongLive paper, §3.3: sink tokens concatenated to the windowed K/V).
    """
    C, S, W = frames_per_chunk, sink_frames, window_frames
    end = (chunk + 1) * C
    start = max(0, end - W)
    return set(range(0, min(S, end))) | set(range(start, end))


def frame_mask(n_keys, chunk, *, tokens_per_frame, frames_per_chunk,
               sink_frames, window_frames):
    """Boolean key mask of length ``n_keys`` over the token history.

    Key j is allowed iff its frame ``j // T`` is in :func:`allowed_frames`.
    The mask is the same for every query of the chunk (no causal mask inside a
    chunk: causality is across chunks).
    """
    frames = np.arange(n_keys) // tokens_per_frame
    ok = allowed_frames(chunk, frames_per_chunk=frames_per_chunk,
                        sink_frames=sink_frames, window_frames=window_frames)
    return np.isin(frames, np.fromiter(ok, dtype=np.int64, count=len(ok)))


def masked_attention(q, k, v, key_mask, scale, query_block=512):
    """Softmax attention with an explicit key mask, in float64.

    q: [n_q, H, D]; k: [n_k, H, D]; v: [n_k, H, Dv]; key_mask: bool [n_k]
    (None = all keys).
    Returns (out [n_q, H, Dv] float64, lse [H, n_q] float64), where
    ``lse = log(sum_j exp(scale * q.k_j))`` over the allowed keys.

    Logits are formed for every key and the masked ones set to -inf before the
    softmax, so masked keys get probability exactly 0.  Queries are processed in
    blocks only to bound memory; each block is the same plain formula.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, H, D = q.shape
    n_k = k.shape[0]
    if key_mask is None:
        key_mask = np.ones(n_k, dtype=bool)
    if not key_mask.any():
        raise ValueError("attention over an empty key set is undefined")
    out = np.empty((n_q, H, v.shape[2]), dtype=np.float64)
    lse = np.empty((H, n_q), dtype=np.float64)
    for h in range(H):
        kh = k[:, h, :]
        vh = v[:, h, :]
        for q0 in range(0, n_q, query_block):
            qb = q[q0:q0 + query_block, h, :]
            logits = scale * (qb @ kh.T)                  # [b, n_k]
            logits[:, ~key_mask] = -np.inf
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            s = e.sum(axis=1, keepdims=True)
            p = e / s
            out[q0:q0 + query_block, h, :] = p @ vh
            lse[h, q0:q0 + query_block] = (m + np.log(s))[:, 0]
    return out, lse


def sink_window_attention(q, hist_k, hist_v, chunk, *, tokens_per_frame,
                          frames_per_chunk, sink_frames, window_frames, scale,
                          query_block=512):
    """Attention of chunk ``chunk``'s queries over the frame sink + window.

    ``hist_k``/``hist_v`` hold the layer's whole token history in generation
    order, [n_hist, H, D]: every earlier chunk as it was appended (or as a
    KV-recache rewrote it), followed by the current chunk's keys/values when
    the call includes them.  Nothing is dropped from the history; the frame
    mask alone decides which keys take part.
    """
    mask = frame_mask(hist_k.shape[0], chunk, tokens_per_frame=tokens_per_frame,
                      frames_per_chunk=frames_per_chunk, sink_frames=sink_frames,
                      window_frames=window_frames)
    return masked_attention(q, hist_k, hist_v, mask, scale, query_block)


def cross_attention(q, k_txt, v_txt, scale, query_block=512):
    """Unmasked softmax attention of the chunk's queries to the prompt's text
    K/V (LongLive paper, §3.1: cross-attention layers inject the prompt)."""
    return masked_attention(q, k_txt, v_txt, None, scale, query_block)


def window_reencode_attention(q_win, hist_k, hist_v, window_chunks, *, tokens_per_frame,
                              frames_per_chunk, sink_frames, window_frames, scale,
                              rows=None, query_block=512):
    """Self-attention of the re-encoding pass of a KV-recache.

    At a prompt switch the resident window chunks ``window_chunks``
    (j_0 < ... < j_{n-1}, as :func:`oracle.resident_window_chunks` gives them)
    are encoded again with the new prompt, and their keys/values replace the
    cached ones (LongLive paper, §3.1 "KV recache"; §3.3: the cache holds the
    sink and the short window only).  Reading taken here: each chunk j_r is
    encoded as in generation, under the frame rule of its own chunk
    (:func:`allowed_frames`), over what the rebuilt cache holds: the sink frames
    and the frames of the window chunks j_0 .. j_r.  Frames before chunk j_0
    that are not sink frames have left the cache and take no part, and no
    chunk sees a later one (causal across chunks, none inside a chunk).

    q_win: [n * C_tok, H, D], chunk j_0's queries first; hist_k/hist_v: the
    layer's token history (with the recache payload applied), covering at
    least every frame of chunk j_{n-1}.  Returns (out [n*C_tok, H, D],
    lse [H, n*C_tok]) in float64; with ``rows`` (sorted query indices) only
    those queries are computed and returned, in that order.
    """
    T, C, S = tokens_per_frame, frames_per_chunk, sink_frames
    ct = C * T
    chunks = list(window_chunks)
    if not chunks or q_win.shape[0] != len(chunks) * ct:
        raise ValueError("one chunk of queries per window chunk is required")
    rows = np.arange(q_win.shape[0]) if rows is None else np.asarray(rows)
    frames = np.arange(hist_k.shape[0]) // T
    first = chunks[0] * C
    out = np.empty((len(rows), q_win.shape[1], hist_v.shape[2]), dtype=np.float64)
    lse = np.empty((q_win.shape[1], len(rows)), dtype=np.float64)
    for r, j in enumerate(chunks):
        ok = allowed_frames(j, frames_per_chunk=C, sink_frames=S, window_frames=window_frames)
        ok = [f for f in ok if f < S or f >= first]
        mask = np.isin(frames, np.asarray(ok, dtype=np.int64))
        sel = np.nonzero((rows >= r * ct) & (rows < (r + 1) * ct))[0]
        if len(sel):
            out[sel], lse[:, sel] = masked_attention(q_win[rows[sel]], hist_k, hist_v, mask,
                                                     scale, query_block)
    return out, lse


def sink_window_attention_grad(q, hist_k, hist_v, chunk, dout, n_grad, *, tokens_per_frame,
                               frames_per_chunk, sink_frames, window_frames, scale,
                               query_block=512):
    """Gradients of :func:`sink_window_attention` for the training step.

    The last ``n_grad`` tokens of the history (the current clip's K/V) carry
    gradient; the earlier ones (sink and window context) are detached (LongLive
    paper, §3.2 and §3.3).  With P = softmax(S) over the allowed keys,
    S = scale * q.k, O = P V and upstream gradient dO:

        dV = P^T dO,   dP = dO V^T,   dS = P * (dP - rowsum(P * dP)),
        dQ = scale * dS K,   dK = scale * dS^T Q,

    the textbook derivative of softmax attention, in float64.  Returns
    (dq [n_q, H, D], dk [n_grad, H, D], dv [n_grad, H, Dv]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(hist_k, dtype=np.float64)
    v = np.asarray(hist_v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    n_q, H, D = q.shape
    n_k = k.shape[0]
    mask = frame_mask(n_k, chunk, tokens_per_frame=tokens_per_frame,
                      frames_per_chunk=frames_per_chunk, sink_frames=sink_frames,
                      window_frames=window_frames)
    if not mask.any():
        raise ValueError("attention over an empty key set is undefined")
    g0 = n_k - n_grad
    dq = np.zeros_like(q)
    dk = np.zeros((n_grad, H, D), dtype=np.float64)
    dv = np.zeros((n_grad, H, v.shape[2]), dtype=np.float64)
    for h in range(H):
        kh, vh = k[:, h, :], v[:, h, :]
        for q0 in range(0, n_q, query_block):
            qb = q[q0:q0 + query_block, h, :]
            dob = do[q0:q0 + query_block, h, :]
            logits = scale * (qb @ kh.T)
            logits[:, ~mask] = -np.inf
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            p = e / e.sum(axis=1, keepdims=True)
            dp = dob @ vh.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[q0:q0 + query_block, h, :] = scale * (ds @ kh)
            dk[:, h, :] += scale * (ds[:, g0:].T @ qb)
            dv[:, h, :] += p[:, g0:].T @ dob
    return dq, dk, dv
