"""Oracle cache model: where each chunk lives, what a recache rewrites, and the
full token history one layer has seen.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The paper states the cache policy in words (LongLive: Real-time Interactive
Long Video Generation, §3.3 "Efficient long inference"): the first frame chunk
is kept for good as the frame sink; the rest of the KV cache is a short rolling
window whose oldest entries are evicted in the usual way.  A KV-recache at a
prompt switch recomputes the cache from the most recently generated frames
(§3.1 "KV recache"; §3.3 last paragraph: only the most recent W frames are
rebuilt); the sink is kept.

Readings taken where the text is silent:

* eviction is first-in first-out by whole chunks (the window minus the current
  chunk holds R = (W - C) / C chunks);
* the sink is the first S / C chunks, S a multiple of C (the paper's setting
  has S = C: one chunk of three latent frames);
* a recache rewrites every resident non-sink window chunk, oldest to newest,
  and leaves the sink alone.
"""

from collections import deque
from dataclasses import dataclass

import numpy as np

from .attention import allowed_frames
from .quant import quantize_int8, dequantize_int8


@dataclass(frozen=True)
class CacheGeometry:
    """Frame-level cache geometry of one layer (T, C, S, W as in attention.py)."""
    tokens_per_frame: int
    frames_per_chunk: int
    sink_frames: int
    window_frames: int

    def __post_init__(self):
        T, C, S, W = (self.tokens_per_frame, self.frames_per_chunk,
                      self.sink_frames, self.window_frames)
        if T < 1 or C < 1 or S < 0 or W < C:
            raise ValueError("need T >= 1, C >= 1, S >= 0, W >= C")
        if S % C or (W - C) % C:
            raise ValueError("S and W - C must be whole numbers of chunks")

    @property
    def chunk_tokens(self):
        return self.tokens_per_frame * self.frames_per_chunk

    @property
    def sink_chunks(self):
        return self.sink_frames // self.frames_per_chunk

    @property
    def ring_slots(self):
        return (self.window_frames - self.frames_per_chunk) // self.frames_per_chunk


def slot_of_chunk(j, g):
    """Closed form: where appended chunk ``j`` is stored.

    Returns ("sink", i) for the i-th sink chunk, ("ring", s) for ring slot s, or
    ("none", None) when the window has no ring (W == C) and the chunk is not
    part of the sink.
    """
    if j < g.sink_chunks:
        return ("sink", j)
    if g.ring_slots == 0:
        return ("none", None)
    return ("ring", (j - g.sink_chunks) % g.ring_slots)


class DequeCacheModel:
    """Step-by-step simulation of the cache's contents, independent of the
    closed form: the sink takes chunks until it is full; after that a FIFO of R
    physical slots takes each chunk, the newest chunk reusing the slot of the
    one it evicts (or the lowest free slot while the ring is filling)."""

    def __init__(self, g):
        self.g = g
        self.sink = []                      # chunk ids in the sink, in order
        self.fifo = deque()                 # resident ring chunk ids, oldest first
        self.slot_chunk = [-1] * g.ring_slots
        self.appended = 0

    def append(self):
        j = self.appended
        self.appended += 1
        if len(self.sink) < self.g.sink_chunks:
            self.sink.append(j)
            return ("sink", len(self.sink) - 1)
        if self.g.ring_slots == 0:
            return ("none", None)
        if len(self.fifo) == self.g.ring_slots:
            oldest = self.fifo.popleft()
            slot = self.slot_chunk.index(oldest)
        else:
            slot = self.slot_chunk.index(-1)
        self.slot_chunk[slot] = j
        self.fifo.append(j)
        return ("ring", slot)

    def resident_ring_chunks(self):
        """Resident ring chunks, oldest first."""
        return list(self.fifo)


def resident_window_chunks(next_chunk, g):
    """Chunks a recache before chunk ``next_chunk`` rewrites, oldest first.

    From the definitions alone: the already generated chunks j < next_chunk
    that are not sink chunks and whose frames lie in the window of the next
    query chunk.
    """
    ok = allowed_frames(next_chunk, frames_per_chunk=g.frames_per_chunk,
                        sink_frames=g.sink_frames, window_frames=g.window_frames)
    C = g.frames_per_chunk
    out = []
    for j in range(g.sink_chunks, next_chunk):
        if all(f in ok for f in range(j * C, (j + 1) * C)):
            out.append(j)
    return out


class LayerHistory:
    """The full token history one layer has seen, in generation order.

    Each generated chunk keeps the keys/values it was appended with, unless a
    KV-recache rewrote it.  With ``int8=True`` the stored K/V are what the INT8
    cache holds, dequantised exactly (float64), while the current chunk passed
    to :meth:`keys` stays at full precision: only stored K/V are quantised.
    """

    def __init__(self, g, int8=False):
        self.g = g
        self.int8 = int8
        self.k = []   # per chunk: float64 [C_tok, H, D]
        self.v = []

    @property
    def chunks(self):
        return len(self.k)

    def _stored(self, x):
        x = np.asarray(x, dtype=np.float64)
        if self.int8:
            q, s = quantize_int8(x.astype(np.float32))
            return dequantize_int8(q, s)
        return x

    def append(self, k, v):
        assert k.shape[0] == self.g.chunk_tokens and v.shape == k.shape
        self.k.append(self._stored(k))
        self.v.append(self._stored(v))

    def recache(self, k, v):
        """Rewrite the resident window chunks (oldest first) with ``k``/``v``
        of shape [n_chunks * C_tok, H, D]."""
        chunks = resident_window_chunks(self.chunks, self.g)
        ct = self.g.chunk_tokens
        if not chunks or k.shape[0] != len(chunks) * ct:
            raise ValueError("recache payload must cover exactly the resident window")
        for i, j in enumerate(chunks):
            self.k[j] = self._stored(k[i * ct:(i + 1) * ct])
            self.v[j] = self._stored(v[i * ct:(i + 1) * ct])

    def keys(self, k_cur=None, v_cur=None):
        """History K/V, followed by the current chunk's K/V when given."""
        ks = list(self.k)
        vs = list(self.v)
        if k_cur is not None:
            ks.append(np.asarray(k_cur, dtype=np.float64))
            vs.append(np.asarray(v_cur, dtype=np.float64))
        return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)
