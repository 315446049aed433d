"""ctypes binding of libll.so (include/ll.h), one Python function per C entry
point with the same name.  Argument marshalling only: every step of the path
runs in the library's HIP kernels; torch supplies device memory and streams.

Tensors are passed as torch tensors.  Their shapes are checked against the
cache's geometry (ll_cache_get_config) before their device, dtype and
contiguity, and before anything reaches the library, whose C ABI sees only
pointers and so cannot bound a buffer; the stream defaults to torch's current stream on the tensor's
device.  A non-OK status raises :class:`LLError` with the library's message.
If the library has not been built, loading raises instead of falling back to
anything else.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libll.so")

LL_F32, LL_BF16, LL_I8 = 0, 1, 2
LL_WHICH_K, LL_WHICH_V, LL_WHICH_KSCALE, LL_WHICH_VSCALE = 0, 1, 2, 3
LL_SEG_SINK, LL_SEG_RING = 0, 1
LL_I8_STAGED, LL_I8_IN_KERNEL = 0, 1
LL_MAX_RING_SLOTS = 30

STATUS = {0: "LL_OK", 1: "LL_ERR_INVALID_ARG", 2: "LL_ERR_BAD_STATE", 3: "LL_ERR_UNSUPPORTED",
          4: "LL_ERR_BUFFER_TOO_SMALL", 5: "LL_ERR_HIP", 6: "LL_ERR_INTERNAL"}

# Every function include/ll.h declares (checked against the header by the tests).
EXPORTS = ("ll_cache_required_bytes", "ll_cache_create", "ll_cache_get_config", "ll_cache_destroy",
           "ll_cache_reset", "ll_cache_set_int8_dequant",
           "ll_cache_append_chunk", "ll_cache_recache", "ll_sink_window_attn",
           "ll_window_reencode_attn", "ll_sink_window_attn_bwd", "ll_sink_window_attn_bwd_noalloc",
           "ll_sink_window_linear_attn",
           "ll_linear_attn_workspace_bytes", "ll_cross_attn", "ll_cache_query", "ll_cache_layout",
           "ll_status_str", "ll_last_error")


class ll_cache_config(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("tokens_per_frame", ctypes.c_int32),
                ("frames_per_chunk", ctypes.c_int32), ("sink_frames", ctypes.c_int32),
                ("window_frames", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32)]


class LLError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {message}")


_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_P = ctypes.POINTER

_SIGS = {
    "ll_cache_required_bytes": (_i32, [_P(ll_cache_config), _P(_sz)]),
    "ll_cache_create": (_i32, [_P(ll_cache_config), _vp, _sz, _P(_vp)]),
    "ll_cache_get_config": (_i32, [_vp, _P(ll_cache_config)]),
    "ll_cache_destroy": (_i32, [_vp]),
    "ll_cache_reset": (_i32, [_vp]),
    "ll_cache_set_int8_dequant": (_i32, [_vp, _i32]),
    "ll_cache_append_chunk": (_i32, [_vp, _i32, _vp, _vp, _vp]),
    "ll_cache_recache": (_i32, [_vp, _i32, _vp, _vp, _i64, _vp]),
    "ll_sink_window_attn": (_i32, [_vp, _i32, _vp, _i64, _vp, _vp, _i64, _f32, _vp, _vp, _vp]),
    "ll_window_reencode_attn": (_i32, [_vp, _i32, _vp, _i64, _f32, _vp, _vp, _vp]),
    "ll_sink_window_attn_bwd": (_i32, [_vp, _i32, _vp, _i64, _vp, _vp, _i64, _f32, _vp, _vp, _vp,
                                       _vp, _vp, _vp, _vp, _vp]),
    "ll_sink_window_attn_bwd_noalloc": (_i32, [_vp, _i32, _vp, _i64, _vp, _vp, _i64, _f32, _vp, _vp, _vp,
                                               _vp, _vp, _vp, _vp]),
    "ll_sink_window_linear_attn": (_i32, [_vp, _i32, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "ll_linear_attn_workspace_bytes": (_i32, [_vp, _P(_sz)]),
    "ll_cross_attn": (_i32, [_vp, _i64, _vp, _vp, _i64, _i32, _i32, _i32, _f32, _vp, _vp, _vp]),
    "ll_cache_query": (_i32, [_vp, _i32, _P(_i64), _P(_i32), _P(_i32), _P(_i64)]),
    "ll_cache_layout": (_i32, [_vp, _i32, _i32, _i32, _P(_sz), _P(_i64), _P(_i64)]),
    "ll_status_str": (ctypes.c_char_p, [_i32]),
    "ll_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load(path=None):
    """Load (once) and return the library; raises if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} is missing: build it first (python -m sink_short_window_amd.build)")
    lib = ctypes.CDLL(p)
    bind(lib)
    if path is None:
        _lib = lib
    return lib


def bind(lib):
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def _check(lib, st):
    if st != 0:
        raise LLError(st, lib.ll_last_error().decode())


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


_ACT = {LL_F32: "float32", LL_BF16: "bfloat16"}


def _dev_ptr(t, name, dtype=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and str(t.dtype) != "torch." + dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream, like):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    torch = _torch()
    return torch.cuda.current_stream(like.device).cuda_stream


def _shape(t, name, shape):
    """Raise unless tensor ``t`` (if given) has exactly ``shape``.  Checked
    before anything reaches the library: the C ABI sees only pointers, so an
    undersized buffer would be read or written out of bounds on the device."""
    if t is None:
        return
    got = tuple(t.shape)
    if got != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {got}")


def _chunk_tokens(cfg):
    return cfg.tokens_per_frame * cfg.frames_per_chunk


def make_config(num_layers, num_heads, head_dim, tokens_per_frame, frames_per_chunk,
                sink_frames, window_frames, act_dtype=LL_BF16, kv_dtype=LL_BF16):
    return ll_cache_config(num_layers, num_heads, head_dim, tokens_per_frame, frames_per_chunk,
                           sink_frames, window_frames, act_dtype, kv_dtype)


# ---------------------------------------------------------------------------
# the C entry points
# ---------------------------------------------------------------------------

def ll_cache_required_bytes(cfg, lib=None):
    lib = lib or load()
    n = _sz()
    _check(lib, lib.ll_cache_required_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def ll_cache_create(cfg, dev_buf, lib=None):
    """dev_buf: a uint8 device tensor of at least ll_cache_required_bytes.
    Returns the opaque handle (int)."""
    lib = lib or load()
    if dev_buf is None or dev_buf.dim() != 1:
        raise ValueError("dev_buf must be a 1-D uint8 tensor")
    ptr = _dev_ptr(dev_buf, "dev_buf", "uint8")
    h = _vp()
    _check(lib, lib.ll_cache_create(ctypes.byref(cfg), ptr, dev_buf.numel(), ctypes.byref(h)))
    return h.value


def ll_cache_get_config(handle, lib=None):
    """The ll_cache_config the handle was created with."""
    lib = lib or load()
    cfg = ll_cache_config()
    _check(lib, lib.ll_cache_get_config(handle, ctypes.byref(cfg)))
    return cfg


def ll_cache_destroy(handle, lib=None):
    lib = lib or load()
    _check(lib, lib.ll_cache_destroy(handle))


def ll_cache_set_int8_dequant(handle, mode, lib=None):
    """LL_I8_STAGED (default) or LL_I8_IN_KERNEL for an I8 cache."""
    lib = lib or load()
    _check(lib, lib.ll_cache_set_int8_dequant(handle, int(mode)))


def ll_cache_reset(handle, lib=None):
    lib = lib or load()
    _check(lib, lib.ll_cache_reset(handle))


def ll_cache_append_chunk(handle, layer, k, v, act_dtype, stream=None, lib=None):
    lib = lib or load()
    g = ll_cache_get_config(handle, lib)
    shape = (_chunk_tokens(g), g.num_heads, g.head_dim)
    _shape(k, "k", shape)
    _shape(v, "v", shape)
    dt = _ACT[act_dtype]
    _check(lib, lib.ll_cache_append_chunk(handle, layer, _dev_ptr(k, "k", dt), _dev_ptr(v, "v", dt),
                                          _stream(stream, k)))


def ll_cache_recache(handle, layer, k, v, n_tokens, act_dtype, stream=None, lib=None):
    lib = lib or load()
    g = ll_cache_get_config(handle, lib)
    lead = (g.num_layers,) if layer == -1 else ()
    shape = lead + (int(n_tokens), g.num_heads, g.head_dim)
    _shape(k, "k", shape)
    _shape(v, "v", shape)
    dt = _ACT[act_dtype]
    _check(lib, lib.ll_cache_recache(handle, layer, _dev_ptr(k, "k", dt), _dev_ptr(v, "v", dt),
                                     int(n_tokens), _stream(stream, k)))


def _check_attn_shapes(g, q, k_cur, v_cur, out, lse=None):
    """q, out: [n_q, H, D]; k_cur, v_cur: both [C_tok, H, D] or both None;
    lse: [H, n_q]."""
    if q is None or q.dim() != 3:
        raise ValueError("q must be a 3-D tensor [n_q, H, D]")
    n_q = q.shape[0]
    H, D = g.num_heads, g.head_dim
    _shape(q, "q", (n_q, H, D))
    _shape(out, "out", (n_q, H, D))
    _shape(lse, "lse", (H, n_q))
    if (k_cur is None) != (v_cur is None):
        raise ValueError("k_cur and v_cur must both be given or both be None")
    _shape(k_cur, "k_cur", (_chunk_tokens(g), H, D))
    _shape(v_cur, "v_cur", (_chunk_tokens(g), H, D))


def ll_sink_window_attn(handle, layer, q, k_cur, v_cur, scale, out, act_dtype, lse=None,
                        stream=None, lib=None):
    """q, out: [n_q, H, D]; k_cur/v_cur: [C_tok, H, D] or None (cache only)."""
    lib = lib or load()
    g = ll_cache_get_config(handle, lib)
    _check_attn_shapes(g, q, k_cur, v_cur, out, lse)
    dt = _ACT[act_dtype]
    n_cur = 0 if k_cur is None else k_cur.shape[0]
    _check(lib, lib.ll_sink_window_attn(
        handle, layer, _dev_ptr(q, "q", dt), q.shape[0],
        _dev_ptr(k_cur, "k_cur", dt, True), _dev_ptr(v_cur, "v_cur", dt, True), n_cur,
        float(scale), _dev_ptr(out, "out", dt), _dev_ptr(lse, "lse", "float32", True),
        _stream(stream, q)))


def ll_window_reencode_attn(handle, layer, q, scale, out, act_dtype, lse=None, stream=None,
                            lib=None):
    """q, out: [resident window chunks * C_tok, H, D], oldest chunk first."""
    lib = lib or load()
    g = ll_cache_get_config(handle, lib)
    _check_attn_shapes(g, q, None, None, out, lse)
    dt = _ACT[act_dtype]
    _check(lib, lib.ll_window_reencode_attn(
        handle, layer, _dev_ptr(q, "q", dt), q.shape[0], float(scale), _dev_ptr(out, "out", dt),
        _dev_ptr(lse, "lse", "float32", True), _stream(stream, q)))


def ll_linear_attn_workspace_bytes(handle, lib=None):
    lib = lib or load()
    n = _sz(0)
    _check(lib, lib.ll_linear_attn_workspace_bytes(handle, ctypes.byref(n)))
    return n.value


def ll_sink_window_linear_attn(handle, layer, q, k_cur, v_cur, out, work, stream=None, lib=None):
    """Linear-attention variant (bf16).  q, out: [n_q, H, D]; k_cur/v_cur:
    [C_tok, H, D] or None; work: a uint8 device tensor of at least
    ll_linear_attn_workspace_bytes."""
    lib = lib or load()
    g = ll_cache_get_config(handle, lib)
    _check_attn_shapes(g, q, k_cur, v_cur, out)
    n_cur = 0 if k_cur is None else k_cur.shape[0]
    _check(lib, lib.ll_sink_window_linear_attn(
        handle, layer, _dev_ptr(q, "q", "bfloat16"), q.shape[0],
        _dev_ptr(k_cur, "k_cur", "bfloat16", True), _dev_ptr(v_cur, "v_cur", "bfloat16", True), n_cur,
        _dev_ptr(out, "out", "bfloat16"), _dev_ptr(work, "work", "uint8"), work.numel(), _stream(stream, q)))


def ll_sink_window_attn_bwd(handle, layer, q, k_cur, v_cur, scale, out, lse, dout, delta, dq,
                            dk_cur=None, dv_cur=None, stream=None, lib=None):
    """Backward of ll_sink_window_attn (bf16).  q, out, dout: [n_q, H, D] bf16;
    lse, delta: float32 [H, n_q]; dq: float32 [n_q, H, D]; k_cur/v_cur: bf16
    [C_tok, H, D] or None; dk_cur/dv_cur: float32 [C_tok, H, D] with them."""
    lib = lib or load()
    g = ll_cache_get_config(handle, lib)
    _check_attn_shapes(g, q, k_cur, v_cur, out, lse)
    n_q = q.shape[0]
    _shape(dout, "dout", tuple(q.shape))
    _shape(delta, "delta", (g.num_heads, n_q))
    _shape(dq, "dq", tuple(q.shape))
    if k_cur is not None:
        _shape(dk_cur, "dk_cur", tuple(k_cur.shape))
        _shape(dv_cur, "dv_cur", tuple(k_cur.shape))
    n_cur = 0 if k_cur is None else k_cur.shape[0]
    _check(lib, lib.ll_sink_window_attn_bwd(
        handle, layer, _dev_ptr(q, "q", "bfloat16"), q.shape[0],
        _dev_ptr(k_cur, "k_cur", "bfloat16", True), _dev_ptr(v_cur, "v_cur", "bfloat16", True), n_cur,
        float(scale), _dev_ptr(out, "out", "bfloat16"), _dev_ptr(lse, "lse", "float32"),
        _dev_ptr(dout, "dout", "bfloat16"), _dev_ptr(delta, "delta", "float32"),
        _dev_ptr(dq, "dq", "float32"), _dev_ptr(dk_cur, "dk_cur", "float32", n_cur == 0),
        _dev_ptr(dv_cur, "dv_cur", "float32", n_cur == 0), _stream(stream, q)))


def ll_sink_window_attn_bwd_noalloc(handle, layer, q, k_cur, v_cur, scale, out, lse, dout, dq,
                                    dk_cur=None, dv_cur=None, stream=None, lib=None):
    """ll_sink_window_attn_bwd with the library's static delta workspace
    (allocates nothing; num_heads * n_q <= 2^20)."""
    lib = lib or load()
    g = ll_cache_get_config(handle, lib)
    _check_attn_shapes(g, q, k_cur, v_cur, out, lse)
    _shape(dout, "dout", tuple(q.shape))
    _shape(dq, "dq", tuple(q.shape))
    if k_cur is not None:
        _shape(dk_cur, "dk_cur", tuple(k_cur.shape))
        _shape(dv_cur, "dv_cur", tuple(k_cur.shape))
    n_cur = 0 if k_cur is None else k_cur.shape[0]
    _check(lib, lib.ll_sink_window_attn_bwd_noalloc(
        handle, layer, _dev_ptr(q, "q", "bfloat16"), q.shape[0],
        _dev_ptr(k_cur, "k_cur", "bfloat16", True), _dev_ptr(v_cur, "v_cur", "bfloat16", True), n_cur,
        float(scale), _dev_ptr(out, "out", "bfloat16"), _dev_ptr(lse, "lse", "float32"),
        _dev_ptr(dout, "dout", "bfloat16"), _dev_ptr(dq, "dq", "float32"),
        _dev_ptr(dk_cur, "dk_cur", "float32", n_cur == 0), _dev_ptr(dv_cur, "dv_cur", "float32", n_cur == 0),
        _stream(stream, q)))


def ll_cross_attn(q, k_txt, v_txt, scale, out, act_dtype, lse=None, stream=None, lib=None):
    """q, out: [n_q, H, D]; k_txt, v_txt: [n_txt, H, D]."""
    lib = lib or load()
    if q is None or q.dim() != 3:
        raise ValueError("q must be a 3-D tensor [n_q, H, D]")
    n_q, H, D = q.shape
    if k_txt is None or k_txt.dim() != 3:
        raise ValueError("k_txt must be a 3-D tensor [n_txt, H, D]")
    _shape(k_txt, "k_txt", (k_txt.shape[0], H, D))
    _shape(v_txt, "v_txt", tuple(k_txt.shape))
    _shape(out, "out", (n_q, H, D))
    _shape(lse, "lse", (H, n_q))
    dt = _ACT[act_dtype]
    _check(lib, lib.ll_cross_attn(
        _dev_ptr(q, "q", dt), n_q, _dev_ptr(k_txt, "k_txt", dt), _dev_ptr(v_txt, "v_txt", dt),
        k_txt.shape[0], H, D, act_dtype, float(scale), _dev_ptr(out, "out", dt),
        _dev_ptr(lse, "lse", "float32", True), _stream(stream, q)))


def ll_cache_query(handle, layer, ring_slots, lib=None):
    lib = lib or load()
    ca, rv, rn = _i64(), _i32(), _i32()
    sc = (_i64 * max(ring_slots, 1))()
    _check(lib, lib.ll_cache_query(handle, layer, ctypes.byref(ca), ctypes.byref(rv),
                                   ctypes.byref(rn), sc))
    return {"chunks_appended": ca.value, "ring_valid": rv.value, "ring_next": rn.value,
            "slot_chunk": list(sc)[:ring_slots]}


def ll_cache_layout(handle, layer, which, segment, lib=None):
    """(byte offset, strides[4], shape[4]) of a cached tensor (see ll.h)."""
    lib = lib or load()
    off = _sz()
    strides = (_i64 * 4)()
    shape = (_i64 * 4)()
    _check(lib, lib.ll_cache_layout(handle, layer, which, segment, ctypes.byref(off), strides, shape))
    return off.value, tuple(strides), tuple(shape)


# key held by physical column p of a transposed V tile (bits 2 and 3 of p swapped)
def vt_column_key(p):
    return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1)


VT_TILE_KEYS = 64


def ll_status_str(status, lib=None):
    lib = lib or load()
    return lib.ll_status_str(status).decode()


def ll_last_error(lib=None):
    lib = lib or load()
    return lib.ll_last_error().decode()


# ---------------------------------------------------------------------------
# convenience: a cache object owning its device buffer and handle
# ---------------------------------------------------------------------------

class Cache:
    """Allocates the cache's device buffer with torch and wraps the handle."""

    def __init__(self, cfg, device="cuda"):
        torch = _torch()
        self.cfg = cfg
        self.nbytes = ll_cache_required_bytes(cfg)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        self.handle = ll_cache_create(cfg, self.buf)

    def close(self):
        if getattr(self, "handle", None):
            ll_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def ring_slots(self):
        return (self.cfg.window_frames - self.cfg.frames_per_chunk) // self.cfg.frames_per_chunk

    def append_chunk(self, layer, k, v, stream=None):
        ll_cache_append_chunk(self.handle, layer, k, v, self.cfg.act_dtype, stream)

    def recache(self, layer, k, v, n_tokens, stream=None):
        ll_cache_recache(self.handle, layer, k, v, n_tokens, self.cfg.act_dtype, stream)

    def attn(self, layer, q, k_cur, v_cur, scale, out, lse=None, stream=None):
        ll_sink_window_attn(self.handle, layer, q, k_cur, v_cur, scale, out, self.cfg.act_dtype,
                            lse, stream)

    def attn_bwd(self, layer, q, k_cur, v_cur, scale, out, lse, dout, delta, dq, dk_cur=None,
                 dv_cur=None, stream=None):
        ll_sink_window_attn_bwd(self.handle, layer, q, k_cur, v_cur, scale, out, lse, dout, delta,
                                dq, dk_cur, dv_cur, stream)

    def reencode_attn(self, layer, q, scale, out, lse=None, stream=None):
        ll_window_reencode_attn(self.handle, layer, q, scale, out, self.cfg.act_dtype, lse, stream)

    def linear_attn(self, layer, q, k_cur, v_cur, out, stream=None):
        """Linear-attention variant; allocates (once) and reuses a workspace."""
        if getattr(self, "_lin_work", None) is None:
            n = ll_linear_attn_workspace_bytes(self.handle)
            self._lin_work = _torch().empty(n, dtype=_torch().uint8, device=self.buf.device)
        ll_sink_window_linear_attn(self.handle, layer, q, k_cur, v_cur, out, self._lin_work, stream)

    def reset(self):
        ll_cache_reset(self.handle)

    def set_int8_dequant(self, mode):
        ll_cache_set_int8_dequant(self.handle, mode)

    def query(self, layer):
        return ll_cache_query(self.handle, layer, self.ring_slots)

    @property
    def chunk_tokens(self):
        return self.cfg.tokens_per_frame * self.cfg.frames_per_chunk

    def v_tiled(self):
        """True when V is stored transposed in 64-key tiles (BF16 and I8 caches)."""
        return self.cfg.kv_dtype != LL_F32

    def tensor(self, layer, which, segment):
        """A strided view of a cached tensor inside the device buffer:
        [H][rows][cols], or [H][tiles][D][64] for the tiled V of a BF16 or I8
        cache."""
        torch = _torch()
        off, strides, shape = ll_cache_layout(self.handle, layer, which, segment)
        if which in (LL_WHICH_KSCALE, LL_WHICH_VSCALE):
            dt, esz = torch.float32, 4
        else:
            dt, esz = {LL_F32: (torch.float32, 4), LL_BF16: (torch.bfloat16, 2),
                       LL_I8: (torch.int8, 1)}[self.cfg.kv_dtype]
        assert off % esz == 0
        flat = self.buf.view(dt) if esz > 1 else self.buf.view(torch.int8)
        view = flat.as_strided(shape, strides, off // esz)
        return view if (which == LL_WHICH_V and self.v_tiled()) else view[..., 0]

    def rows(self, layer, which, segment):
        """A cached tensor in logical order [H][rows][cols] (a copy for tiled V):
        row r of the segment is token r % C_tok of its chunk slot r // C_tok."""
        torch = _torch()
        t = self.tensor(layer, which, segment)
        if not (which == LL_WHICH_V and self.v_tiled()):
            return t
        ct = self.chunk_tokens
        tps = (ct + VT_TILE_KEYS - 1) // VT_TILE_KEYS
        nslots = t.shape[1] // tps
        i = torch.arange(ct, device=t.device)
        col = torch.tensor([vt_column_key(p) for p in range(VT_TILE_KEYS)], device=t.device)
        tiles = (torch.arange(nslots, device=t.device)[:, None] * tps + (i // VT_TILE_KEYS)[None, :]).reshape(-1)
        cols = col[i % VT_TILE_KEYS].repeat(nslots)
        # advanced indices in dims 1 and 3 (separated by a slice) come out first: [R][H][D]
        return t[:, tiles, :, cols].permute(1, 0, 2)

    def v_padding(self, layer, segment):
        """The zero padding after each chunk slot's last key in the tiled V."""
        t = self.tensor(layer, LL_WHICH_V, segment)
        ct = self.chunk_tokens
        tps = (ct + VT_TILE_KEYS - 1) // VT_TILE_KEYS
        last = t[:, tps - 1::tps]
        keys = [vt_column_key(p) for p in range(VT_TILE_KEYS)]
        pad_cols = [p for p, k in enumerate(keys) if (tps - 1) * VT_TILE_KEYS + k >= ct]
        return last[..., pad_cols]
