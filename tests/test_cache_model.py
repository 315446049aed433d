"""Pins for the oracle's cache model: the closed-form slot formula, the
step-by-step FIFO simulation and the definition-based resident window agree
(P6).  Paper: LongLive: Real-time Interactive Long Video Generation, §3.3
(sink kept, rolling window evicted in the usual way), §3.1 (KV recache)."""

import itertools

import pytest

from oracle import CacheGeometry, slot_of_chunk, DequeCacheModel, resident_window_chunks


GEOMS = [CacheGeometry(T, C, S, W)
         for T, C in [(1, 1), (16, 1), (1560, 3), (2, 2)]
         for S in (0, C, 2 * C)
         for W in (C, 2 * C, 3 * C, 5 * C)]


@pytest.mark.parametrize("g", GEOMS, ids=lambda g: f"C{g.frames_per_chunk}S{g.sink_frames}W{g.window_frames}")
def test_closed_form_equals_fifo_simulation(g):
    sim = DequeCacheModel(g)
    for j in range(60):
        assert sim.append() == slot_of_chunk(j, g)


@pytest.mark.parametrize("g", GEOMS, ids=lambda g: f"C{g.frames_per_chunk}S{g.sink_frames}W{g.window_frames}")
def test_resident_window_equals_fifo_contents(g):
    """The chunks a recache rewrites (window chunks from the frame definition,
    minus sink and current) are exactly the chunks the FIFO holds."""
    sim = DequeCacheModel(g)
    for c in range(40):
        assert resident_window_chunks(c, g) == sim.resident_ring_chunks()
        sim.append()


def test_paper_setting_snapshot():
    """Sink 3 frames + window 9 frames, 3-frame chunks: after chunks 0..3 are
    appended the sink holds chunk 0, ring slot 0 holds chunk 3 and slot 1
    holds chunk 2 (chunk 1 was evicted)."""
    g = CacheGeometry(1560, 3, 3, 9)
    sim = DequeCacheModel(g)
    for _ in range(4):
        sim.append()
    assert sim.sink == [0]
    assert sim.slot_chunk == [3, 2]
    assert sim.resident_ring_chunks() == [2, 3]
    assert g.chunk_tokens == 4680 and g.ring_slots == 2 and g.sink_chunks == 1


@pytest.mark.parametrize("T,C,S,W", [(4, 2, 3, 6), (4, 2, 2, 5), (4, 2, 2, 1), (0, 1, 0, 1)])
def test_geometry_rejects_partial_chunks(T, C, S, W):
    with pytest.raises(ValueError):
        CacheGeometry(T, C, S, W)
