"""CPU tests of the C ABI (no GPU).

* libll.so loads and exports every function include/ll.h declares.
* The real ABI layer and bookkeeping (ll_api.cpp + cache_state.cpp), linked
  against a launch stub that records launches, are driven through their error
  paths and state machine, and checked against the oracle's cache model:
  slot assignment after every append (P6), recache destination order, and the
  key-run table an attention call would launch with.
"""

import ctypes
import os
import re

import pytest

from oracle import CacheGeometry, DequeCacheModel, slot_of_chunk, resident_window_chunks, allowed_frames
from sink_short_window_amd import ll, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ll.h")

FAKE_BUF = 1 << 20          # never dereferenced by the stub
FAKE_ACT = 1 << 30


@pytest.fixture(scope="module")
def libs():
    if not (os.path.exists(build.LIB_LL) and os.path.exists(build.LIB_HOSTSTUB)):
        build.build_all()
    # LL_HOSTSTUB selects another build of the stub (the sanitizer build)
    stub = ctypes.CDLL(os.environ.get("LL_HOSTSTUB", build.LIB_HOSTSTUB))
    ll.bind(stub)
    stub.llh_last_attn.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    stub.llh_last_copy.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    stub.llh_last_copy_vt.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    stub.llh_last_attn_chunks.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    stub.llh_last_bwd.argtypes = [ctypes.POINTER(ctypes.c_int64)]
    stub.llh_last_stage.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                    ctypes.POINTER(ctypes.c_int64)]
    stub.llh_last_lin.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]
    return stub


RUN_FIELDS = 11  # llh_last_attn: k, v, head_stride, row_stride, key_start, len, v_head_stride, v_tiled,
                 # ks, vs, i8
VT_KEYS = 64


def tiles_per_slot(ct):
    return (ct + VT_KEYS - 1) // VT_KEYS


def header_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:ll_status|const char\s*\*)\s*(ll_\w+)\s*\(", txt, re.M)))


def test_header_and_binding_agree():
    assert header_functions() == sorted(ll.EXPORTS)


def test_libll_loads_and_exports_every_declared_symbol():
    if not os.path.exists(build.LIB_LL):
        build.build_ll()
    lib = ctypes.CDLL(build.LIB_LL)
    for name in header_functions():
        assert hasattr(lib, name), name


def cfg(L=2, H=3, D=64, T=4, C=2, S=2, W=6, act=ll.LL_BF16, kv=ll.LL_BF16):
    return ll.make_config(L, H, D, T, C, S, W, act, kv)


def create(stub, c, nbytes=None):
    need = ll.ll_cache_required_bytes(c, lib=stub)
    h = ctypes.c_void_p()
    st = stub.ll_cache_create(ctypes.byref(c), FAKE_BUF, need if nbytes is None else nbytes, ctypes.byref(h))
    assert st == 0, stub.ll_last_error()
    return h.value


def status(stub, st):
    return ll.STATUS[st]


@pytest.mark.parametrize("bad,code", [
    (dict(D=96), "LL_ERR_UNSUPPORTED"),
    (dict(S=3), "LL_ERR_UNSUPPORTED"),
    (dict(W=5), "LL_ERR_UNSUPPORTED"),
    (dict(W=1), "LL_ERR_UNSUPPORTED"),
    (dict(C=1, W=40), "LL_ERR_UNSUPPORTED"),
    (dict(L=0), "LL_ERR_INVALID_ARG"),
    (dict(H=0), "LL_ERR_INVALID_ARG"),
    (dict(T=0), "LL_ERR_INVALID_ARG"),
    (dict(S=-2), "LL_ERR_INVALID_ARG"),
    (dict(act=ll.LL_F32, kv=ll.LL_BF16), "LL_ERR_UNSUPPORTED"),
    (dict(act=ll.LL_I8, kv=ll.LL_I8), "LL_ERR_UNSUPPORTED"),
    (dict(act=ll.LL_F32, kv=ll.LL_I8), "LL_ERR_UNSUPPORTED"),
    (dict(C=1, S=10, W=31), "LL_ERR_UNSUPPORTED"),   # bf16: 10 sink chunks + 30 slots + current > 40 runs
    (dict(C=1, S=10, W=31, kv=ll.LL_I8), "LL_ERR_UNSUPPORTED"),  # int8 is attended through a bf16 copy
])
def test_config_rejected(libs, bad, code):
    n = ctypes.c_size_t(123)
    st = libs.ll_cache_required_bytes(ctypes.byref(cfg(**bad)), ctypes.byref(n))
    assert status(libs, st) == code
    assert libs.ll_last_error()
    assert n.value == 123


def test_many_runs_fine_for_fp32_cache(libs):
    """BF16 and I8 caches walk each sink chunk as its own run; F32 keeps the
    sink as one run."""
    n = ctypes.c_size_t(0)
    assert libs.ll_cache_required_bytes(ctypes.byref(cfg(C=1, S=10, W=31, act=ll.LL_F32, kv=ll.LL_F32)),
                                        ctypes.byref(n)) == 0
    for kv in (ll.LL_BF16, ll.LL_I8):
        assert libs.ll_cache_required_bytes(ctypes.byref(cfg(C=1, S=9, W=31, kv=kv)), ctypes.byref(n)) == 0


def _align(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("kw", [dict(), dict(kv=ll.LL_I8), dict(act=ll.LL_F32, kv=ll.LL_F32, D=128),
                                dict(S=0, W=2), dict(T=1560, C=3, S=3, W=9, H=12, D=128, L=30)])
def test_required_bytes_matches_layout(libs, kw):
    c = cfg(**kw)
    L, H, D, T, C, S, W = (c.num_layers, c.num_heads, c.head_dim, c.tokens_per_frame,
                           c.frames_per_chunk, c.sink_frames, c.window_frames)
    rows = S * T + (W - C) // C * C * T
    esz = {ll.LL_F32: 4, ll.LL_BF16: 2, ll.LL_I8: 1}[c.kv_dtype]
    kb = _align(H * rows * D * esz)
    if c.kv_dtype != ll.LL_F32:      # V transposed in whole 64-key tiles per chunk slot
        slots = S // C + (W - C) // C
        vb = _align(H * slots * tiles_per_slot(C * T) * VT_KEYS * D * esz)
    else:
        vb = kb
    scb = _align(H * rows * 4) if c.kv_dtype == ll.LL_I8 else 0
    stage = 0
    if c.kv_dtype == ll.LL_I8:        # one layer's bf16 staging copy: K rows + V tiles
        slots = S // C + (W - C) // C
        stage = _align(H * rows * D * 2) + _align(H * slots * tiles_per_slot(C * T) * VT_KEYS * D * 2)
    assert ll.ll_cache_required_bytes(c, lib=libs) == L * max(kb + vb + 2 * scb, 256) + stage
    if kw.get("L") == 30:     # the paper-shaped 30-layer bf16 cache: 3 slots of 74 tiles for V
        assert ll.ll_cache_required_bytes(c, lib=libs) == 30 * (12 * 14040 * 128 * 2 + 12 * 3 * 74 * 64 * 128 * 2)


def test_create_errors(libs):
    c = cfg()
    need = ll.ll_cache_required_bytes(c, lib=libs)
    h = ctypes.c_void_p()
    assert status(libs, libs.ll_cache_create(ctypes.byref(c), None, need, ctypes.byref(h))) == "LL_ERR_INVALID_ARG"
    assert status(libs, libs.ll_cache_create(ctypes.byref(c), FAKE_BUF + 16, need, ctypes.byref(h))) == "LL_ERR_INVALID_ARG"
    assert status(libs, libs.ll_cache_create(ctypes.byref(c), FAKE_BUF, need - 1, ctypes.byref(h))) == "LL_ERR_BUFFER_TOO_SMALL"
    assert status(libs, libs.ll_cache_create(ctypes.byref(c), FAKE_BUF, need, None)) == "LL_ERR_INVALID_ARG"
    assert libs.ll_cache_destroy(None) == 0
    for s in range(7):
        assert libs.ll_status_str(s).decode() == ll.STATUS[s]


def query(stub, h, layer, R):
    return ll.ll_cache_query(h, layer, R, lib=stub)


def test_append_state_matches_fifo_model(libs):
    """P6 on the C++ bookkeeping: after every append, ll_cache_query and the
    destination row of the launched copy equal the oracle's FIFO model."""
    for (T, C, S, W) in [(4, 2, 2, 6), (4, 1, 0, 3), (2, 2, 4, 2), (1560, 3, 3, 9), (3, 1, 2, 5)]:
        c = cfg(T=T, C=C, S=S, W=W)
        g = CacheGeometry(T, C, S, W)
        h = create(libs, c)
        sim = DequeCacheModel(g)
        R = g.ring_slots
        for j in range(3 * (g.sink_chunks + R) + 5):
            calls = libs.llh_copy_calls()
            assert libs.ll_cache_append_chunk(h, 1, FAKE_ACT, FAKE_ACT, None) == 0
            where = sim.append()
            assert where == slot_of_chunk(j, g)
            if where[0] == "none":
                assert libs.llh_copy_calls() == calls          # counted, not stored
            else:
                nl = ctypes.c_int32()
                rows = (ctypes.c_int32 * 40)()
                assert libs.llh_last_copy(ctypes.byref(nl), rows) == 1
                want = where[1] * g.chunk_tokens if where[0] == "sink" else \
                    g.sink_frames * T + where[1] * g.chunk_tokens
                assert rows[0] == want
                tps, slot = ctypes.c_int32(), (ctypes.c_int32 * 40)()
                assert libs.llh_last_copy_vt(ctypes.byref(tps), slot) == 1      # bf16 cache: tiled V
                assert tps.value == tiles_per_slot(g.chunk_tokens)
                assert slot[0] == (where[1] if where[0] == "sink" else g.sink_chunks + where[1])
            qd = query(libs, h, 1, R)
            assert qd["chunks_appended"] == j + 1
            assert qd["slot_chunk"] == sim.slot_chunk
            assert qd["ring_valid"] == len(sim.fifo)
            assert query(libs, h, 0, R)["chunks_appended"] == 0   # layers independent
        libs.ll_cache_destroy(h)


def test_append_errors_leave_state_unchanged(libs):
    c = cfg()
    h = create(libs, c)
    R = 2
    before = query(libs, h, 0, R)
    assert status(libs, libs.ll_cache_append_chunk(h, 2, FAKE_ACT, FAKE_ACT, None)) == "LL_ERR_INVALID_ARG"
    assert status(libs, libs.ll_cache_append_chunk(h, -1, FAKE_ACT, FAKE_ACT, None)) == "LL_ERR_INVALID_ARG"
    assert status(libs, libs.ll_cache_append_chunk(h, 0, None, FAKE_ACT, None)) == "LL_ERR_INVALID_ARG"
    assert status(libs, libs.ll_cache_append_chunk(h, 0, FAKE_ACT + 8, FAKE_ACT, None)) == "LL_ERR_INVALID_ARG"
    assert status(libs, libs.ll_cache_append_chunk(None, 0, FAKE_ACT, FAKE_ACT, None)) == "LL_ERR_INVALID_ARG"
    libs.llh_fail_next_launch()
    assert status(libs, libs.ll_cache_append_chunk(h, 0, FAKE_ACT, FAKE_ACT, None)) == "LL_ERR_HIP"
    assert "stub" in libs.ll_last_error().decode()
    assert query(libs, h, 0, R) == before
    assert libs.ll_cache_append_chunk(h, 0, FAKE_ACT, FAKE_ACT, None) == 0
    assert libs.ll_last_error().decode() == ""
    assert query(libs, h, 0, R)["chunks_appended"] == 1
    assert libs.ll_cache_reset(h) == 0
    assert query(libs, h, 0, R) == before
    libs.ll_cache_destroy(h)


def test_recache_targets_resident_window_oldest_first(libs):
    T, C, S, W = 2, 1, 1, 4          # R = 3
    c = cfg(L=3, T=T, C=C, S=S, W=W)
    g = CacheGeometry(T, C, S, W)
    h = create(libs, c)
    ct = g.chunk_tokens
    assert status(libs, libs.ll_cache_recache(h, 0, FAKE_ACT, FAKE_ACT, 0, None)) == "LL_ERR_BAD_STATE"
    sim = DequeCacheModel(g)
    for j in range(7):
        for layer in range(3):
            assert libs.ll_cache_append_chunk(h, layer, FAKE_ACT, FAKE_ACT, None) == 0
        sim.append()
        chunks = resident_window_chunks(j + 1, g)
        if not chunks:
            assert status(libs, libs.ll_cache_recache(h, 0, FAKE_ACT, FAKE_ACT, 0, None)) == "LL_ERR_BAD_STATE"
            continue
        n = len(chunks) * ct
        assert status(libs, libs.ll_cache_recache(h, 0, FAKE_ACT, FAKE_ACT, n + ct, None)) == "LL_ERR_INVALID_ARG"
        assert status(libs, libs.ll_cache_recache(h, 5, FAKE_ACT, FAKE_ACT, n, None)) == "LL_ERR_INVALID_ARG"
        for layer in (1, -1):
            assert libs.ll_cache_recache(h, layer, FAKE_ACT, FAKE_ACT, n, None) == 0
            nl = ctypes.c_int32()
            rows = (ctypes.c_int32 * 40)()
            k = libs.llh_last_copy(ctypes.byref(nl), rows)
            assert nl.value == (3 if layer == -1 else 1)
            want = [S * T + sim.slot_chunk.index(ch) * ct for ch in chunks]
            assert list(rows[:k]) == want
            tps, slot = ctypes.c_int32(), (ctypes.c_int32 * 40)()
            assert libs.llh_last_copy_vt(ctypes.byref(tps), slot) == 1
            assert list(slot[:k]) == [g.sink_chunks + sim.slot_chunk.index(ch) for ch in chunks]
    # layers out of step: layer -1 refused
    assert libs.ll_cache_append_chunk(h, 0, FAKE_ACT, FAKE_ACT, None) == 0
    n = len(resident_window_chunks(8, g)) * ct
    assert status(libs, libs.ll_cache_recache(h, -1, FAKE_ACT, FAKE_ACT, n, None)) == "LL_ERR_BAD_STATE"
    libs.ll_cache_destroy(h)


def _layout(stub, h, layer, which, seg):
    return ll.ll_cache_layout(h, layer, which, seg, lib=stub)


def test_attention_key_runs_cover_exactly_the_allowed_chunks(libs):
    """The run table an attention call launches with covers exactly the sink
    chunks and window chunks the frame definition allows (each once), points
    at their rows, and ends with the current chunk."""
    for (T, C, S, W) in [(4, 2, 2, 6), (4, 1, 0, 3), (2, 2, 4, 2), (1560, 3, 3, 9), (3, 1, 2, 5)]:
        c = cfg(L=2, T=T, C=C, S=S, W=W, H=3, D=64)
        g = CacheGeometry(T, C, S, W)
        h = create(libs, c)
        sim = DequeCacheModel(g)
        ct = g.chunk_tokens
        H, D = 3, 64
        k_sink_off, st_sink, _ = _layout(libs, h, 1, ll.LL_WHICH_K, ll.LL_SEG_SINK)
        k_ring_off, st_ring, _ = _layout(libs, h, 1, ll.LL_WHICH_K, ll.LL_SEG_RING)
        v_sink_off, st_v, _ = _layout(libs, h, 1, ll.LL_WHICH_V, ll.LL_SEG_SINK)
        slot_bytes = tiles_per_slot(ct) * VT_KEYS * D * 2
        for chunk in range(3 * (g.sink_chunks + g.ring_slots) + 3):
            for n_cur in (ct, 0):
                st = libs.ll_sink_window_attn(h, 1, FAKE_ACT, 5, FAKE_ACT, FAKE_ACT, n_cur, 0.125,
                                              FAKE_ACT, None, None)
                if chunk == 0 and n_cur == 0:
                    assert status(libs, st) == "LL_ERR_BAD_STATE"
                    continue
                assert st == 0, libs.ll_last_error()
                nk = ctypes.c_int64()
                runs = (ctypes.c_int64 * (RUN_FIELDS * 40))()
                n_seg = libs.llh_last_attn(ctypes.byref(nk), runs)
                covered = []
                start = 0
                for i in range(n_seg):
                    kp, vp, hs, rs, ks, ln, vhs, vtl = runs[RUN_FIELDS * i:RUN_FIELDS * i + 8]
                    assert ks == start and ln > 0
                    start += ln
                    if kp == FAKE_ACT:                 # current chunk, token-major
                        assert i == n_seg - 1 and ln == ct and vp == FAKE_ACT
                        assert (hs, rs, vtl) == (D, H * D, 0)
                        covered.append(chunk)
                        continue
                    assert (hs, rs) == (st_sink[0], D)
                    row = (kp - FAKE_BUF - k_sink_off) // (2 * D)
                    # one chunk slot per run; V in the slot's transposed tiles
                    assert ln == ct and row % ct == 0 or row >= S * T and (row - S * T) % ct == 0
                    assert ln == ct and vtl == 1 and vhs == st_v[0]
                    slot = row // ct if row < S * T else S // C + (row - S * T) // ct
                    assert vp - FAKE_BUF - v_sink_off == slot * slot_bytes
                    if row < S * T:
                        covered.append(row // ct)                  # sink chunk index
                    else:
                        covered.append(sim.slot_chunk[(row - S * T) // ct])
                assert nk.value == start
                ok = allowed_frames(chunk, frames_per_chunk=C, sink_frames=S, window_frames=W)
                want = sorted({f // C for f in ok if n_cur or f // C != chunk})
                assert sorted(covered) == want
                assert len(covered) == len(set(covered))
            assert libs.ll_cache_append_chunk(h, 1, FAKE_ACT, FAKE_ACT, None) == 0
            sim.append()
        libs.ll_cache_destroy(h)


def test_int8_dequant_mode_setter(libs):
    h = create(libs, cfg(kv=ll.LL_I8))
    for bad in (-1, 2, 7):
        assert status(libs, libs.ll_cache_set_int8_dequant(h, bad)) == "LL_ERR_INVALID_ARG"
    assert libs.ll_cache_set_int8_dequant(h, ll.LL_I8_IN_KERNEL) == 0
    assert libs.ll_cache_set_int8_dequant(h, ll.LL_I8_STAGED) == 0
    assert status(libs, libs.ll_cache_set_int8_dequant(None, 0)) == "LL_ERR_INVALID_ARG"
    h2 = create(libs, cfg())
    assert status(libs, libs.ll_cache_set_int8_dequant(h2, ll.LL_I8_IN_KERNEL)) == "LL_ERR_INVALID_ARG"
    libs.ll_cache_destroy(h)
    libs.ll_cache_destroy(h2)


def test_int8_attention_staged_by_default(libs):
    """By default an I8 cache's attention launches the bf16 staging of the
    layer's resident chunks first, and its cache runs read the staging copy
    (bf16 K rows, bf16 V tiles), not the codes."""
    T, C, S, W, H, D = 40, 2, 2, 8, 3, 64
    c = cfg(L=2, T=T, C=C, S=S, W=W, H=H, D=D, kv=ll.LL_I8)
    h = create(libs, c)
    for _ in range(4):
        assert libs.ll_cache_append_chunk(h, 1, FAKE_ACT, FAKE_ACT, None) == 0
    stages = libs.llh_stage_calls()
    assert libs.ll_sink_window_attn(h, 1, FAKE_ACT, 5, FAKE_ACT, FAKE_ACT, C * T, 0.125,
                                    FAKE_ACT, None, None) == 0, libs.ll_last_error()
    assert libs.llh_stage_calls() == stages + 1
    row0 = (ctypes.c_int32 * 40)()
    slot = (ctypes.c_int32 * 40)()
    bases = (ctypes.c_int64 * 3)()
    n_st = libs.llh_last_stage(row0, slot, bases)
    nk = ctypes.c_int64()
    runs = (ctypes.c_int64 * (RUN_FIELDS * 40))()
    n_seg = libs.llh_last_attn(ctypes.byref(nk), runs)
    assert n_st == n_seg - 1                                   # every cache run is staged
    for i in range(n_seg - 1):
        kp, vp, _, _, _, ln, _, vtl, ksp, vsp, i8 = runs[RUN_FIELDS * i:RUN_FIELDS * (i + 1)]
        assert (i8, vtl, ksp, vsp) == (0, 1, 0, 0)
        assert kp == bases[1] + 2 * row0[i] * D and vp >= bases[2]
    libs.ll_cache_destroy(h)


def test_int8_attention_reads_codes_in_place(libs):
    """With LL_I8_IN_KERNEL an I8 cache is attended in place: every cache run
    is an int8 run whose K points at the chunk's code rows, V at its slot of
    int8 V tiles and the scale pointers at the same rows of the K and V scale
    arrays; the current chunk stays a bf16 run; no staging launch is
    enqueued."""
    T, C, S, W, H, D = 40, 2, 2, 8, 3, 64
    c = cfg(L=2, T=T, C=C, S=S, W=W, H=H, D=D, kv=ll.LL_I8)
    g = CacheGeometry(T, C, S, W)
    h = create(libs, c)
    assert libs.ll_cache_set_int8_dequant(h, ll.LL_I8_IN_KERNEL) == 0
    sim = DequeCacheModel(g)
    ct = g.chunk_tokens
    tps = tiles_per_slot(ct)
    k_off, _, _ = _layout(libs, h, 1, ll.LL_WHICH_K, ll.LL_SEG_SINK)
    v_off, st_v, _ = _layout(libs, h, 1, ll.LL_WHICH_V, ll.LL_SEG_SINK)
    ks_off, _, _ = _layout(libs, h, 1, ll.LL_WHICH_KSCALE, ll.LL_SEG_SINK)
    vs_off, _, _ = _layout(libs, h, 1, ll.LL_WHICH_VSCALE, ll.LL_SEG_SINK)
    stages = libs.llh_stage_calls()
    for chunk in range(6):
        assert libs.ll_sink_window_attn(h, 1, FAKE_ACT, 5, FAKE_ACT, FAKE_ACT, ct, 0.125,
                                        FAKE_ACT, None, None) == 0, libs.ll_last_error()
        nk = ctypes.c_int64()
        runs = (ctypes.c_int64 * (RUN_FIELDS * 40))()
        n_seg = libs.llh_last_attn(ctypes.byref(nk), runs)
        for i in range(n_seg - 1):
            kp, vp, hs, rs, _, ln, vhs, vtl, ksp, vsp, i8 = runs[RUN_FIELDS * i:RUN_FIELDS * (i + 1)]
            row = kp - FAKE_BUF - k_off                     # int8: one byte per element
            assert row % D == 0
            row //= D
            assert (i8, vtl, hs, rs, vhs, ln) == (1, 1, (S * T + g.ring_slots * ct) * D, D, st_v[0], ct)
            slot = row // ct if row < S * T else S // C + (row - S * T) // ct
            assert vp - FAKE_BUF - v_off == slot * tps * VT_KEYS * D
            assert ksp - FAKE_BUF - ks_off == 4 * row and vsp - FAKE_BUF - vs_off == 4 * row
        last = runs[RUN_FIELDS * (n_seg - 1):RUN_FIELDS * n_seg]
        assert last[0] == FAKE_ACT and last[10] == 0 and last[8] == 0
        assert libs.ll_cache_append_chunk(h, 1, FAKE_ACT, FAKE_ACT, None) == 0
        sim.append()
    assert libs.llh_stage_calls() == stages
    libs.ll_cache_destroy(h)


@pytest.mark.parametrize("T,C,S,W,act,kv", [
    (4, 2, 2, 6, ll.LL_BF16, ll.LL_BF16), (4, 1, 0, 3, ll.LL_BF16, ll.LL_BF16),
    (3, 1, 2, 5, ll.LL_BF16, ll.LL_BF16), (4, 2, 2, 8, ll.LL_BF16, ll.LL_I8),
    (2, 2, 4, 8, ll.LL_F32, ll.LL_F32)])
def test_reencode_runs_are_sink_then_window_oldest_first(libs, T, C, S, W, act, kv):
    """The re-encoding call walks the sink, then the resident window chunks
    oldest first, with the chunk-causal split recorded: window chunk r attends
    the first n_seg0 + r runs, i.e. exactly the sink chunks and the window
    chunks 0..r the oracle's reading names."""
    c = cfg(L=2, T=T, C=C, S=S, W=W, H=3, D=64, act=act, kv=kv)
    g = CacheGeometry(T, C, S, W)
    h = create(libs, c)
    if kv == ll.LL_I8:
        assert libs.ll_cache_set_int8_dequant(h, ll.LL_I8_IN_KERNEL) == 0
    sim = DequeCacheModel(g)
    ct, D = g.chunk_tokens, 64
    elt = {ll.LL_BF16: 2, ll.LL_I8: 1, ll.LL_F32: 4}[kv]
    k_sink_off, _, _ = _layout(libs, h, 1, ll.LL_WHICH_K, ll.LL_SEG_SINK)
    A = FAKE_ACT
    stage_calls = libs.llh_stage_calls()
    for chunk in range(g.sink_chunks + 2 * g.ring_slots + 2):
        win = resident_window_chunks(chunk, g) if chunk > g.sink_chunks else []
        n_q = len(win) * ct
        st = libs.ll_window_reencode_attn(h, 1, A, n_q, 0.125, A, None, None)
        if not win:
            assert status(libs, st) == "LL_ERR_BAD_STATE"
        else:
            assert st == 0, libs.ll_last_error()
            nk = ctypes.c_int64()
            runs = (ctypes.c_int64 * (RUN_FIELDS * 40))()
            n_seg = libs.llh_last_attn(ctypes.byref(nk), runs)
            n_seg0 = ctypes.c_int32()
            assert libs.llh_last_attn_chunks(ctypes.byref(n_seg0)) == ct
            chunks_of_run = []
            k0, esz = FAKE_BUF + k_sink_off, elt
            # in-kernel mode: an I8 cache is attended in place (int8 runs), no staging launch
            assert libs.llh_stage_calls() == stage_calls
            for i in range(n_seg):
                assert runs[RUN_FIELDS * i + 10] == (kv == ll.LL_I8)
                kp, ln = runs[RUN_FIELDS * i], runs[RUN_FIELDS * i + 5]
                row = (kp - k0) // (esz * D)
                if row < S * T:
                    chunks_of_run.append(list(range(row // ct, (row + ln) // ct)))
                else:
                    assert ln == ct
                    chunks_of_run.append([sim.slot_chunk[(row - S * T) // ct]])
            n_sink = n_seg0.value - 1
            assert n_seg == n_sink + len(win)
            for r in range(len(win)):
                seen = [j for run in chunks_of_run[:n_sink + r + 1] for j in run]
                assert seen == list(range(g.sink_chunks)) + win[:r + 1]
            bad = libs.ll_window_reencode_attn(h, 1, A, n_q - 1, 0.125, A, None, None)
            assert status(libs, bad) == "LL_ERR_INVALID_ARG"
            bad = libs.ll_window_reencode_attn(h, 1, A, n_q, float("inf"), A, None, None)
            assert status(libs, bad) == "LL_ERR_INVALID_ARG"
            bad = libs.ll_window_reencode_attn(h, 1, A, n_q, 0.125, A + 2, None, None)
            assert status(libs, bad) == "LL_ERR_INVALID_ARG"
            bad = libs.ll_window_reencode_attn(h, 2, A, n_q, 0.125, A, None, None)
            assert status(libs, bad) == "LL_ERR_INVALID_ARG"
        assert libs.ll_cache_append_chunk(h, 1, A, A, None) == 0
        sim.append()
    libs.ll_cache_destroy(h)


def test_backward_validation_and_launch(libs):
    """The backward takes the forward's run table; only the current chunk
    carries dK/dV; bf16 only; every pointer is checked before launching."""
    c = cfg(L=2, T=4, C=2, S=2, W=6, H=3, D=64)
    h = create(libs, c)
    ct = 8
    A, F = FAKE_ACT, FAKE_ACT + (1 << 24)
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("layer", 1), ("q", A), ("n_q", 5), ("k", A), ("v", A), ("n_cur", ct), ("scale", 0.1),
        ("out", A), ("lse", F), ("dout", A), ("delta", F), ("dq", F), ("dk", F), ("dv", F))] + [None]
    call = lambda **kw: status(libs, libs.ll_sink_window_attn_bwd(h, *args(**kw)))
    for _ in range(3):
        assert libs.ll_cache_append_chunk(h, 1, A, A, None) == 0
    assert call() == "LL_OK"
    nk = ctypes.c_int64()
    runs = (ctypes.c_int64 * (RUN_FIELDS * 40))()
    n_seg = libs.llh_last_attn(ctypes.byref(nk), runs)
    libs.ll_sink_window_attn(h, 1, A, 5, A, A, ct, 0.1, A, None, None)
    nk2 = ctypes.c_int64()
    runs2 = (ctypes.c_int64 * (RUN_FIELDS * 40))()
    assert libs.llh_last_attn(ctypes.byref(nk2), runs2) == n_seg and nk.value == nk2.value
    assert list(runs[:RUN_FIELDS * n_seg]) == list(runs2[:RUN_FIELDS * n_seg])
    assert runs[RUN_FIELDS * (n_seg - 1)] == A                     # the current chunk is last
    ptrs = (ctypes.c_int64 * 7)()
    assert libs.llh_last_bwd(ptrs) == 1 and list(ptrs[:4]) == [F, F, F, F]
    assert call(n_cur=0, dk=None, dv=None, k=None, v=None) == "LL_OK"
    assert libs.llh_last_bwd(ptrs) == 0 and ptrs[2] == 0 and ptrs[3] == 0
    for bad in (dict(n_q=0), dict(n_cur=ct - 1), dict(scale=0.0), dict(lse=None), dict(delta=None),
                dict(dq=None), dict(dq=F + 4), dict(dk=None), dict(dv=F + 8), dict(dout=None),
                dict(out=A + 2), dict(q=None), dict(layer=2)):
        calls = libs.llh_bwd_calls()
        assert call(**bad) == "LL_ERR_INVALID_ARG", bad
        assert libs.llh_bwd_calls() == calls
    # the dK/dV kernel's 32-bit offsets: (n_q + 64) * H * D * 2 < 2^32 (H=3, D=64: 384 bytes a query)
    n_max = (1 << 32) // 384 - 64
    assert call(n_q=n_max) == "LL_OK"
    calls = libs.llh_bwd_calls()
    assert call(n_q=n_max + 1) == "LL_ERR_UNSUPPORTED" and b"4 GiB" in libs.ll_last_error()
    assert libs.llh_bwd_calls() == calls
    assert call(n_q=n_max + 1, n_cur=0, dk=None, dv=None, k=None, v=None) == "LL_OK"  # dQ alone
    libs.llh_fail_next_launch()
    assert call() == "LL_ERR_HIP"
    libs.ll_cache_destroy(h)
    h2 = create(libs, cfg(act=ll.LL_F32, kv=ll.LL_F32))
    assert status(libs, libs.ll_sink_window_attn_bwd(h2, *args(layer=0))) == "LL_ERR_UNSUPPORTED"
    libs.ll_cache_destroy(h2)
    h2 = create(libs, cfg(kv=ll.LL_I8))            # int8 context: staged, then the bf16 backward
    stages = libs.llh_stage_calls()
    assert libs.ll_cache_append_chunk(h2, 0, A, A, None) == 0
    assert status(libs, libs.ll_sink_window_attn_bwd(h2, *args(layer=0))) == "LL_OK"
    assert libs.llh_stage_calls() == stages + 1
    libs.ll_cache_destroy(h2)
    h3 = create(libs, cfg())
    assert status(libs, libs.ll_sink_window_attn_bwd(h3, *args(layer=0, n_cur=0, k=None, v=None))) \
        == "LL_ERR_BAD_STATE"
    libs.ll_cache_destroy(h3)


def test_linear_attention_validation_and_launch(libs):
    """The linear-attention variant takes the softmax call's run table, splits
    the key tiles into at most 32 ranges covering every tile once, carves its
    workspace as documented, is bf16-only and checks every argument before
    launching."""
    c = cfg(L=2, T=4, C=2, S=2, W=6, H=3, D=64)
    h = create(libs, c)
    ct = 8
    A = FAKE_ACT
    need = ll.ll_linear_attn_workspace_bytes(h, lib=libs)
    H, D, up = 3, 64, lambda x: (x + 255) // 256 * 256
    parts = [up(32 * H * D * D * 4), up(32 * H * D * 4), up(H * D * D * 2), up(H * D * D * 2), up(H * D * 4)]
    assert need == sum(parts)
    W0 = FAKE_ACT + (1 << 26)
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("layer", 1), ("q", A), ("n_q", 5), ("k", A), ("v", A), ("n_cur", ct), ("out", A),
        ("work", W0), ("work_bytes", need))] + [None]
    call = lambda **kw: status(libs, libs.ll_sink_window_linear_attn(h, *args(**kw)))
    for _ in range(3):
        assert libs.ll_cache_append_chunk(h, 1, A, A, None) == 0
    calls = libs.llh_lin_calls()
    assert call() == "LL_OK" and libs.llh_lin_calls() == calls + 1
    nk = ctypes.c_int64()
    runs = (ctypes.c_int64 * (RUN_FIELDS * 40))()
    n_seg = libs.llh_last_attn(ctypes.byref(nk), runs)
    tps = ctypes.c_int32()
    ptrs = (ctypes.c_int64 * 5)()
    n_split = libs.llh_last_lin(ctypes.byref(tps), ptrs)
    n_tiles = sum((runs[RUN_FIELDS * i + 5] + 63) // 64 for i in range(n_seg))
    # splits: one state workgroup per CU over the heads (256 / H), at most 32
    # and at most one per tile; split s sums tiles s, s + n_split, ...
    assert n_split == min(32, n_tiles, max(1, 256 // H)) and tps.value == -(-n_tiles // n_split)
    offs = [W0]
    for b in parts[:-1]:
        offs.append(offs[-1] + b)
    assert list(ptrs) == offs
    libs.ll_sink_window_attn(h, 1, A, 5, A, A, ct, 0.1, A, None, None)   # same key set as softmax
    nk2 = ctypes.c_int64()
    runs2 = (ctypes.c_int64 * (RUN_FIELDS * 40))()
    assert libs.llh_last_attn(ctypes.byref(nk2), runs2) == n_seg and nk.value == nk2.value
    assert list(runs[:RUN_FIELDS * n_seg]) == list(runs2[:RUN_FIELDS * n_seg])
    assert call(n_cur=0, k=None, v=None) == "LL_OK"
    assert call(n_q=0) == "LL_OK"
    for bad, code in ((dict(n_cur=ct - 1), "LL_ERR_INVALID_ARG"), (dict(q=None), "LL_ERR_INVALID_ARG"),
                      (dict(out=A + 2), "LL_ERR_INVALID_ARG"), (dict(k=None), "LL_ERR_INVALID_ARG"),
                      (dict(work=None), "LL_ERR_INVALID_ARG"), (dict(work=W0 + 64), "LL_ERR_INVALID_ARG"),
                      (dict(work_bytes=need - 1), "LL_ERR_BUFFER_TOO_SMALL"), (dict(layer=2), "LL_ERR_INVALID_ARG"),
                      (dict(n_q=-1), "LL_ERR_INVALID_ARG")):
        calls = libs.llh_lin_calls()
        assert call(**bad) == code, bad
        assert libs.llh_lin_calls() == calls
    libs.llh_fail_next_launch()
    assert call() == "LL_ERR_HIP"
    libs.ll_cache_destroy(h)
    h2 = create(libs, cfg(act=ll.LL_F32, kv=ll.LL_F32))
    assert status(libs, libs.ll_sink_window_linear_attn(h2, *args(layer=0))) == "LL_ERR_UNSUPPORTED"
    libs.ll_cache_destroy(h2)
    h2 = create(libs, cfg(kv=ll.LL_I8))            # int8 cache: staged, then the bf16 kernels
    stages = libs.llh_stage_calls()
    assert libs.ll_cache_append_chunk(h2, 0, A, A, None) == 0
    assert status(libs, libs.ll_sink_window_linear_attn(h2, *args(layer=0))) == "LL_OK"
    assert libs.llh_stage_calls() == stages + 1
    libs.ll_cache_destroy(h2)
    h3 = create(libs, cfg())
    assert status(libs, libs.ll_sink_window_linear_attn(h3, *args(layer=0, n_cur=0, k=None, v=None))) \
        == "LL_ERR_BAD_STATE"
    libs.ll_cache_destroy(h3)


def test_attention_and_cross_attention_errors(libs):
    c = cfg()
    h = create(libs, c)
    ct = 8
    A = FAKE_ACT
    ok = lambda st: status(libs, st)
    assert ok(libs.ll_sink_window_attn(h, 0, A, 5, A, A, ct - 1, 0.1, A, None, None)) == "LL_ERR_INVALID_ARG"
    assert ok(libs.ll_sink_window_attn(h, 0, A, 5, A, A, ct, 0.0, A, None, None)) == "LL_ERR_INVALID_ARG"
    assert ok(libs.ll_sink_window_attn(h, 0, A, 5, A, A, ct, float("nan"), A, None, None)) == "LL_ERR_INVALID_ARG"
    assert ok(libs.ll_sink_window_attn(h, 0, A, 5, A, A, ct, -1.0, A, None, None)) == "LL_ERR_INVALID_ARG"
    assert ok(libs.ll_sink_window_attn(h, 0, None, 5, A, A, ct, 0.1, A, None, None)) == "LL_ERR_INVALID_ARG"
    assert ok(libs.ll_sink_window_attn(h, 0, A, 5, A, A, ct, 0.1, A + 4, None, None)) == "LL_ERR_INVALID_ARG"
    assert ok(libs.ll_sink_window_attn(h, 0, A, 5, None, A, ct, 0.1, A, None, None)) == "LL_ERR_INVALID_ARG"
    assert ok(libs.ll_sink_window_attn(h, 0, A, 5, A, A, 0, 0.1, A, None, None)) == "LL_ERR_BAD_STATE"
    assert ok(libs.ll_sink_window_attn(h, 7, A, 5, A, A, ct, 0.1, A, None, None)) == "LL_ERR_INVALID_ARG"
    assert ok(libs.ll_sink_window_attn(h, 0, A, -1, A, A, ct, 0.1, A, None, None)) == "LL_ERR_INVALID_ARG"
    calls = libs.llh_attn_calls()
    assert libs.ll_sink_window_attn(h, 0, None, 0, A, A, ct, 0.1, None, None, None) == 0   # n_q = 0: no-op
    assert libs.llh_attn_calls() == calls
    libs.llh_fail_next_launch()
    assert ok(libs.ll_sink_window_attn(h, 0, A, 5, A, A, ct, 0.1, A, None, None)) == "LL_ERR_HIP"
    x = ok(libs.ll_cross_attn(A, 5, A, A, 0, 2, 64, ll.LL_BF16, 0.1, A, None, None))
    assert x == "LL_ERR_INVALID_ARG"
    assert ok(libs.ll_cross_attn(A, 5, A, A, 3, 2, 80, ll.LL_BF16, 0.1, A, None, None)) == "LL_ERR_UNSUPPORTED"
    assert ok(libs.ll_cross_attn(A, 5, A, A, 3, 2, 64, ll.LL_I8, 0.1, A, None, None)) == "LL_ERR_UNSUPPORTED"
    assert ok(libs.ll_cross_attn(A, 5, A, A, 3, 0, 64, ll.LL_BF16, 0.1, A, None, None)) == "LL_ERR_INVALID_ARG"
    # text K/V rows are addressed in whole 64-key tiles with 32-bit byte offsets: (n_txt + 64) * 256 < 2^32
    n_max = (1 << 24) - 65
    assert libs.ll_cross_attn(A, 5, A, A, n_max, 2, 64, ll.LL_BF16, 0.1, A, None, None) == 0
    assert ok(libs.ll_cross_attn(A, 5, A, A, n_max + 1, 2, 64, ll.LL_BF16, 0.1, A, None, None)) == "LL_ERR_UNSUPPORTED"
    assert b"4 GiB" in libs.ll_last_error()
    assert libs.ll_cross_attn(A, 5, A, A, 3, 2, 64, ll.LL_BF16, 0.1, A, A, None) == 0
    nk = ctypes.c_int64()
    runs = (ctypes.c_int64 * (RUN_FIELDS * 40))()
    assert libs.llh_last_attn(ctypes.byref(nk), runs) == 1 and nk.value == 3
    assert tuple(runs[2:4]) == (64, 128) and runs[7] == 0
    libs.ll_cache_destroy(h)


def test_layout_queries(libs):
    c = cfg(kv=ll.LL_I8, T=4, C=2, S=2, W=6, H=3, D=64)
    h = create(libs, c)
    rows = 2 * 4 + 2 * 8
    off_k, st_k, sh_k = _layout(libs, h, 1, ll.LL_WHICH_K, ll.LL_SEG_SINK)
    off_kr, st_kr, sh_kr = _layout(libs, h, 1, ll.LL_WHICH_K, ll.LL_SEG_RING)
    off_s, st_s, sh_s = _layout(libs, h, 1, ll.LL_WHICH_VSCALE, ll.LL_SEG_RING)
    assert st_k == (rows * 64, 64, 1, 1) and sh_k == (3, 8, 64, 1)
    assert sh_kr == (3, 16, 64, 1) and off_kr == off_k + 8 * 64
    off_v, st_v, sh_v = _layout(libs, h, 1, ll.LL_WHICH_V, ll.LL_SEG_SINK)
    off_vr8, st_vr8, sh_vr8 = _layout(libs, h, 1, ll.LL_WHICH_V, ll.LL_SEG_RING)
    # int8 V: transposed 64-key tiles like the bf16 cache, 1 sink + 2 ring slots of 1 tile
    assert st_v == st_vr8 == (3 * 64 * 64, 64 * 64, 64, 1)
    assert sh_v == (3, 1, 64, 64) and sh_vr8 == (3, 2, 64, 64) and off_vr8 == off_v + 64 * 64
    assert st_s == (rows, 1, 1, 1) and sh_s == (3, 16, 1, 1)
    assert off_k % 256 == 0
    assert status(libs, libs.ll_cache_layout(h, 0, 9, 0, ctypes.byref(ctypes.c_size_t()),
                                             (ctypes.c_int64 * 4)(), None)) == "LL_ERR_INVALID_ARG"
    h2 = create(libs, cfg(T=40, C=2, S=2, W=6, H=3, D=64))   # bf16: chunk of 80 keys = 2 tiles
    with pytest.raises(ll.LLError):
        _layout(libs, h2, 0, ll.LL_WHICH_KSCALE, ll.LL_SEG_SINK)
    vhe = 3 * 2 * 64 * 64                                      # 3 slots x 2 tiles x [64][64]
    off_vs, st_vs, sh_vs = _layout(libs, h2, 1, ll.LL_WHICH_V, ll.LL_SEG_SINK)
    off_vr, st_vr, sh_vr = _layout(libs, h2, 1, ll.LL_WHICH_V, ll.LL_SEG_RING)
    assert st_vs == st_vr == (vhe, 64 * 64, 64, 1)
    assert sh_vs == (3, 2, 64, 64) and sh_vr == (3, 4, 64, 64)
    assert off_vr == off_vs + 2 * 64 * 64 * 2 and off_vs % 256 == 0
    libs.ll_cache_destroy(h)
    libs.ll_cache_destroy(h2)


def test_get_config_round_trips(libs):
    c = cfg(L=3, H=5, D=128, T=7, C=2, S=4, W=8, kv=ll.LL_I8)
    h = create(libs, c)
    got = ll.ll_cache_get_config(h, lib=libs)
    for f, _ in ll.ll_cache_config._fields_:
        assert getattr(got, f) == getattr(c, f), f
    assert status(libs, libs.ll_cache_get_config(None, ctypes.byref(got))) == "LL_ERR_INVALID_ARG"
    assert status(libs, libs.ll_cache_get_config(h, None)) == "LL_ERR_INVALID_ARG"
    libs.ll_cache_destroy(h)


def test_binding_rejects_mismatched_shapes_before_the_library(libs):
    """Every wrapper checks tensor shapes against the cache geometry before it
    touches the library (the C ABI cannot see buffer sizes).  A wrong shape
    raises 'must have shape'; the right shapes get as far as the device check
    (these are CPU tensors)."""
    import torch
    L, H, D, T, C, S, W = 2, 3, 64, 4, 2, 2, 6
    ct = C * T
    h = create(libs, cfg(L, H, D, T, C, S, W))
    bf = lambda *sh: torch.zeros(sh, dtype=torch.bfloat16)
    f32 = lambda *sh: torch.zeros(sh, dtype=torch.float32)

    def shape_error(fn, *a, **kw):
        with pytest.raises(ValueError, match="shape|3-D|both"):
            fn(*a, **kw)

    def device_error(fn, *a, **kw):
        with pytest.raises(ValueError, match="device tensor"):
            fn(*a, **kw)

    A = ll.LL_BF16
    # append: k, v [C_tok, H, D]
    device_error(ll.ll_cache_append_chunk, h, 0, bf(ct, H, D), bf(ct, H, D), A, lib=libs)
    shape_error(ll.ll_cache_append_chunk, h, 0, bf(ct - 1, H, D), bf(ct, H, D), A, lib=libs)
    shape_error(ll.ll_cache_append_chunk, h, 0, bf(ct, H, D), bf(ct, H + 1, D), A, lib=libs)
    # recache: [n, H, D] for one layer, [L, n, H, D] for all
    device_error(ll.ll_cache_recache, h, 0, bf(2 * ct, H, D), bf(2 * ct, H, D), 2 * ct, A, lib=libs)
    shape_error(ll.ll_cache_recache, h, 0, bf(ct, H, D), bf(2 * ct, H, D), 2 * ct, A, lib=libs)
    device_error(ll.ll_cache_recache, h, -1, bf(L, ct, H, D), bf(L, ct, H, D), ct, A, lib=libs)
    shape_error(ll.ll_cache_recache, h, -1, bf(ct, H, D), bf(ct, H, D), ct, A, lib=libs)
    # attention: q/out [n_q, H, D], k_cur/v_cur [C_tok, H, D], lse [H, n_q]
    n = 5
    ok = dict(q=bf(n, H, D), k_cur=bf(ct, H, D), v_cur=bf(ct, H, D), out=bf(n, H, D), lse=f32(H, n))

    def attn(**kw):
        a = dict(ok, **kw)
        return ll.ll_sink_window_attn(h, 0, a["q"], a["k_cur"], a["v_cur"], 0.125, a["out"], A,
                                      lse=a["lse"], lib=libs)

    device_error(attn)
    device_error(attn, k_cur=None, v_cur=None)
    for bad in (dict(q=bf(n, H, D + 1)), dict(q=bf(n * H * D)), dict(out=bf(n - 1, H, D)),
                dict(k_cur=bf(ct + 1, H, D)), dict(v_cur=bf(ct, H, 2 * D)), dict(v_cur=None),
                dict(lse=f32(H, n + 1)), dict(lse=f32(n, H))):
        shape_error(attn, **bad)
    # re-encoding attention, linear variant and backward share the checks
    device_error(ll.ll_window_reencode_attn, h, 0, bf(n, H, D), 0.1, bf(n, H, D), A, lib=libs)
    shape_error(ll.ll_window_reencode_attn, h, 0, bf(n, H, D), 0.1, bf(n + 1, H, D), A, lib=libs)
    shape_error(ll.ll_sink_window_linear_attn, h, 0, bf(n, H, D), bf(ct, H, D), bf(ct, H, D),
                bf(n, 1, D), torch.zeros(16, dtype=torch.uint8), lib=libs)

    def bwd(**kw):
        a = dict(q=bf(n, H, D), k=bf(ct, H, D), v=bf(ct, H, D), out=bf(n, H, D), lse=f32(H, n),
                 dout=bf(n, H, D), delta=f32(H, n), dq=f32(n, H, D), dk=f32(ct, H, D), dv=f32(ct, H, D))
        a.update(kw)
        return ll.ll_sink_window_attn_bwd(h, 0, a["q"], a["k"], a["v"], 0.1, a["out"], a["lse"],
                                          a["dout"], a["delta"], a["dq"], a["dk"], a["dv"], lib=libs)

    device_error(bwd)
    for bad in (dict(dout=bf(n, H, D - 1)), dict(delta=f32(H, n - 1)), dict(dq=f32(n, H, 1)),
                dict(dk=f32(ct - 1, H, D)), dict(dv=f32(ct, H, D + 1))):
        shape_error(bwd, **bad)
    # cross-attention: q [n_q, H, D]; k_txt, v_txt [n_txt, H, D]
    device_error(ll.ll_cross_attn, bf(n, H, D), bf(7, H, D), bf(7, H, D), 0.1, bf(n, H, D), A, lib=libs)
    for q_, k_, v_, o_ in ((bf(n, H, D), bf(7, H + 1, D), bf(7, H, D), bf(n, H, D)),
                           (bf(n, H, D), bf(7, H, D), bf(6, H, D), bf(n, H, D)),
                           (bf(n, H, D), bf(7, H, D), bf(7, H, D), bf(n + 1, H, D)),
                           (bf(n * H * D), bf(7, H, D), bf(7, H, D), bf(n, H, D))):
        shape_error(ll.ll_cross_attn, q_, k_, v_, 0.1, o_, A, lib=libs)
    libs.ll_cache_destroy(h)


# The kernels index chunk elements, cache rows and transposed V tiles with
# 32-bit integers; the geometry check bounds each product by 2^30 - 1.  Each
# pair sits on one side of one bound.
LIM = 2 ** 30 - 1


@pytest.mark.parametrize("kw,ok", [
    # C_tok * H * D: T=1024, C=1, D=128 -> H * 2^17
    (dict(T=1024, C=1, S=0, W=2, H=8191, D=128), True),
    (dict(T=1024, C=1, S=0, W=2, H=8192, D=128), False),
    # rows * D with 30 ring slots: 30 * T * 128
    (dict(T=279620, C=1, S=0, W=31, H=1, D=128, act=ll.LL_F32, kv=ll.LL_F32), True),
    (dict(T=279621, C=1, S=0, W=31, H=1, D=128, act=ll.LL_F32, kv=ll.LL_F32), False),
    # transposed V tiles (BF16 cache): 30 slots * ceil(T/64) * 64 * 128; T = 64k + 1
    # pads each slot, so this bound bites before rows * D does
    (dict(T=64 * 4368 + 1, C=1, S=0, W=31, H=1, D=128), True),
    (dict(T=64 * 4369 + 1, C=1, S=0, W=31, H=1, D=128), False),
    (dict(T=64 * 4369 + 1, C=1, S=0, W=31, H=1, D=128, kv=ll.LL_I8), False),
    (dict(T=64 * 4369 + 1, C=1, S=0, W=31, H=1, D=128, act=ll.LL_F32, kv=ll.LL_F32), True),
])
def test_geometry_32bit_bounds(libs, kw, ok):
    c = cfg(**{"L": 1, **kw})
    n = ctypes.c_size_t(0)
    st = libs.ll_cache_required_bytes(ctypes.byref(c), ctypes.byref(n))
    T, C, H, D = kw["T"], kw["C"], kw["H"], kw["D"]
    ct = T * C
    rows = (kw["S"] + kw["W"] - C) * T
    vt = (kw["S"] // C + (kw["W"] - C) // C) * -(-ct // 64) * 64 * D
    tiled = kw.get("kv", ll.LL_BF16) != ll.LL_F32
    assert (ct * H * D <= LIM and rows * D <= LIM and (not tiled or vt <= LIM)) == ok
    if ok:
        assert st == 0, libs.ll_last_error()
    else:
        assert status(libs, st) == "LL_ERR_UNSUPPORTED"
        assert b"32-bit" in libs.ll_last_error()


@pytest.mark.parametrize("H,ok", [(258111, True), (258112, False)])
def test_chunk_tile_range_bound(libs, H, ok):
    """A chunk of activations is addressed in whole 64-token tiles with 32-bit
    byte offsets: (C_tok + 64) * H * D * 2 must stay below 4 GiB (C_tok = 1,
    D = 128: 65 * 256 bytes a head)."""
    c = cfg(L=1, T=1, C=1, S=0, W=2, H=H, D=128)
    n = ctypes.c_size_t(0)
    st = libs.ll_cache_required_bytes(ctypes.byref(c), ctypes.byref(n))
    assert (65 * H * 256 < 1 << 32) == ok
    if ok:
        assert st == 0, libs.ll_last_error()
    else:
        assert status(libs, st) == "LL_ERR_UNSUPPORTED" and b"4 GiB" in libs.ll_last_error()


def test_noalloc_backward_validation_and_launch(libs):
    """The allocation-free backward takes the library's static delta
    workspace (the stub's stand-in address), bounds num_heads * n_q by its
    size and otherwise checks and launches as the backward does."""
    c = cfg(L=2, T=4, C=2, S=2, W=6, H=3, D=64)
    h = create(libs, c)
    ct = 8
    A, F = FAKE_ACT, FAKE_ACT + (1 << 24)
    call = lambda n_q, n_cur=ct, dq=F: status(libs, libs.ll_sink_window_attn_bwd_noalloc(
        h, 1, A, n_q, A, A, n_cur, 0.1, A, F, A, dq, F, F, None))
    assert call(5) == "LL_OK"
    ptrs = (ctypes.c_int64 * 7)()
    assert libs.llh_last_bwd(ptrs) == 1
    assert ptrs[0] == 0x5C0000000 and ptrs[1] == F
    assert call((1 << 20) // 3) == "LL_OK"
    assert call((1 << 20) // 3 + 1) == "LL_ERR_UNSUPPORTED"
    assert b"static workspace" in libs.ll_last_error()
    assert call(0) == "LL_ERR_INVALID_ARG"
    assert call(5, dq=None) == "LL_ERR_INVALID_ARG"
    assert call(5, n_cur=ct - 1) == "LL_ERR_INVALID_ARG"
    libs.ll_cache_destroy(h)


# --------------------------------------------------------------------------
# random operation sequences against the oracle's cache model
# --------------------------------------------------------------------------

from hypothesis import HealthCheck, given, settings, strategies as hst  # noqa: E402

# appends dominate, so that sequences run well past the first evictions
_OPS = hst.lists(hst.tuples(hst.sampled_from(["append"] * 8 + ["recache", "recache_all", "attn",
                                                               "attn_cache_only", "reset"]),
                            hst.integers(0, 1)), min_size=1, max_size=60)


@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(T=hst.integers(1, 9), C=hst.integers(1, 3), nsc=hst.integers(0, 3), R=hst.integers(0, 4), ops=_OPS)
def test_state_machine_matches_the_cache_model_under_random_operations(libs, T, C, nsc, R, ops):
    """Any interleaving of appends (two layers, out of step), recaches of one
    or all layers (all layers only when their rings hold the same slots in
    the same order), attention calls with and without the current chunk and
    resets: after every operation ll_cache_query equals the oracle's FIFO
    model, a recache rewrites exactly the resident window chunks oldest
    first, and an attention call's run table covers exactly the chunks the
    frame rule allows, each once, ending with the current chunk."""
    S, W = nsc * C, (R + 1) * C
    L, H, D = 2, 2, 64
    g = CacheGeometry(T, C, S, W)
    h = create(libs, cfg(L=L, T=T, C=C, S=S, W=W, H=H, D=D))
    ct = g.chunk_tokens
    sims = [DequeCacheModel(g) for _ in range(L)]
    k_sink_off = _layout(libs, h, 0, ll.LL_WHICH_K, ll.LL_SEG_SINK)[0]
    layer_bytes = _layout(libs, h, 1, ll.LL_WHICH_K, ll.LL_SEG_SINK)[0] - k_sink_off
    try:
        for op, layer in ops:
            n = sims[layer].appended
            if op == "append":
                assert libs.ll_cache_append_chunk(h, layer, FAKE_ACT, FAKE_ACT, None) == 0
                sims[layer].append()
            elif op == "reset":
                assert libs.ll_cache_reset(h) == 0
                sims = [DequeCacheModel(g) for _ in range(L)]
            elif op in ("recache", "recache_all"):
                target = -1 if op == "recache_all" else layer
                chunks = resident_window_chunks(n, g)

                def slots(sim):
                    return [sim.slot_chunk.index(ch) for ch in resident_window_chunks(sim.appended, g)]

                # all layers at once needs one ring arrangement: the same slots, oldest first
                same_ring = all(slots(s) == slots(sims[layer]) for s in sims)
                st = libs.ll_cache_recache(h, target, FAKE_ACT, FAKE_ACT, len(chunks) * ct, None)
                if not chunks or (target == -1 and not same_ring):
                    assert status(libs, st) == "LL_ERR_BAD_STATE"
                else:
                    assert st == 0, libs.ll_last_error()
                    nl = ctypes.c_int32()
                    rows = (ctypes.c_int32 * 40)()
                    k = libs.llh_last_copy(ctypes.byref(nl), rows)
                    assert nl.value == (L if target == -1 else 1)
                    assert list(rows[:k]) == [S * T + sims[layer].slot_chunk.index(ch) * ct for ch in chunks]
            else:
                n_cur = ct if op == "attn" else 0
                st = libs.ll_sink_window_attn(h, layer, FAKE_ACT, 3, FAKE_ACT, FAKE_ACT, n_cur, 0.125,
                                              FAKE_ACT, None, None)
                ok = allowed_frames(n, frames_per_chunk=C, sink_frames=S, window_frames=W)
                want = {f // C for f in ok if n_cur or f // C != n}
                if not want:
                    assert status(libs, st) == "LL_ERR_BAD_STATE"
                    continue
                assert st == 0, libs.ll_last_error()
                nk = ctypes.c_int64()
                runs = (ctypes.c_int64 * (RUN_FIELDS * 40))()
                n_seg = libs.llh_last_attn(ctypes.byref(nk), runs)
                covered, start = [], 0
                for i in range(n_seg):
                    kp, _vp, _hs, _rs, ks, ln = runs[RUN_FIELDS * i:RUN_FIELDS * i + 6]
                    assert ks == start and ln == ct
                    start += ln
                    if kp == FAKE_ACT:
                        assert i == n_seg - 1
                        covered.append(n)
                        continue
                    row = (kp - FAKE_BUF - k_sink_off - layer * layer_bytes) // (2 * D)
                    covered.append(row // ct if row < S * T else sims[layer].slot_chunk[(row - S * T) // ct])
                assert nk.value == start
                assert sorted(covered) == sorted(want)
                assert len(covered) == len(set(covered))
            for lay in range(L):
                q = query(libs, h, lay, g.ring_slots)
                assert q["chunks_appended"] == sims[lay].appended
                assert q["slot_chunk"] == sims[lay].slot_chunk
                assert q["ring_valid"] == len(sims[lay].fifo)
    finally:
        libs.ll_cache_destroy(h)
