// The C ABI declared in include/ll.h: validation, host state, launches.
//
// Every entry point validates its arguments and the cache state first and
// returns before enqueuing anything on error (no state change).  Host state
// advances only after a successful launch.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <new>
#include <string>

#include "cache_state.hpp"
#include "launch.hpp"
#include "ll.h"

using ll::fail;

static_assert(ll::kMaxSeg == ll::kMaxKeyRuns, "run table size");

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

ll_status check_layer(const ll_cache* c, int32_t layer, bool allow_all) {
  if (!c) return fail(LL_ERR_INVALID_ARG, "cache handle is NULL");
  const int L = c->state.geom().L;
  if (layer == -1 && allow_all) return LL_OK;
  if (layer < 0 || layer >= L)
    return fail(LL_ERR_INVALID_ARG, "layer " + std::to_string(layer) + " out of range [0, " +
                                        std::to_string(L) + ")");
  return LL_OK;
}

ll_status check_act_ptr(const void* p, const char* name) {
  if (!p) return fail(LL_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned(p, 16)) return fail(LL_ERR_INVALID_ARG, std::string(name) + " is not 16-byte aligned");
  return LL_OK;
}

ll_status launched(int err, const char* what) {
  if (err != 0)
    return fail(LL_ERR_HIP, std::string(what) + ": " + ll::hip_error_string(err));
  return LL_OK;
}

// Key runs of a layer's cache, in the order the attention kernels walk them:
// the sink (for a BF16 or I8 cache one run per sink chunk, each with its own
// slot of V tiles; for F32 one run), then the resident ring chunks, oldest
// first.  An I8 cache's runs are int8 codes with their scales, or, with
// `staged`, point into its bf16 staging area (see stage_int8).  Appends to
// a.seg and keys; returns the number of sink runs.
int add_cache_runs(const ll::CacheState& cs, int32_t layer, ll::AttnArgs& a, int32_t& keys,
                   bool staged = false) {
  const ll::Geometry& g = cs.geom();
  const ll::Layout& lay = cs.layout();
  const char* buf = static_cast<const char*>(cs.buffer());
  const char* base = buf + lay.layer_bytes * size_t(layer);
  const size_t kelt = ll::dtype_bytes(g.kv);
  auto add_cache_run = [&](int64_t row0, int64_t len) {
    ll::KvSeg& s = a.seg[a.n_seg++];
    s.head_stride = g.rows * g.D;
    s.row_stride = g.D;
    s.ks = s.vs = nullptr;
    s.s_head_stride = 0;
    s.i8 = 0;
    const int64_t slot = ll::slot_of_row(g, row0);
    if (staged && g.staged) {  // bf16 staging copy in the BF16 layout
      s.k = buf + lay.stage_k_off + size_t(row0 * g.D) * 2;
      s.v = buf + lay.stage_v_off + size_t(slot * g.tps * ll::kVtTileKeys * g.D) * 2;
      s.v_head_stride = g.vt_head_elems;
      s.v_tiled = 1;
    } else if (g.vt) {  // one chunk slot of the transposed tile layout
      s.k = base + lay.k_off + size_t(row0 * g.D) * kelt;
      s.v = base + lay.v_off + size_t(slot * g.tps * ll::kVtTileKeys * g.D) * kelt;
      s.v_head_stride = g.vt_head_elems;
      s.v_tiled = 1;
      if (g.kv == LL_I8) {
        s.ks = reinterpret_cast<const float*>(base + lay.ks_off) + row0;
        s.vs = reinterpret_cast<const float*>(base + lay.vs_off) + row0;
        s.s_head_stride = g.rows;
        s.i8 = 1;
      }
    } else {
      s.k = base + lay.k_off + size_t(row0 * g.D) * kelt;
      s.v = base + lay.v_off + size_t(row0 * g.D) * kelt;
      s.v_head_stride = 0;
      s.v_tiled = 0;
    }
    s.key_start = keys;
    s.len = int32_t(len);
    keys += int32_t(len);
  };
  const int64_t sink_rows = cs.sink_valid_rows(layer);
  if (g.vt) {
    for (int64_t r0 = 0; r0 < sink_rows; r0 += g.ctok) add_cache_run(r0, g.ctok);
  } else if (sink_rows > 0) {
    add_cache_run(0, sink_rows);
  }
  const int n_sink = a.n_seg;
  for (int32_t slot : cs.resident_slots(layer)) add_cache_run(g.sink_rows + int64_t(slot) * g.ctok, g.ctok);
  return n_sink;
}

// The staged attention mode (the default), the backward and the
// linear-attention variant read an I8 cache through a bf16 copy of the
// layer's resident chunks (sink chunks and resident ring slots) in the
// staging area, dequantised to bf16(q * s) by one launch per call.  No-op for
// other caches.
int stage_int8(const ll::CacheState& cs, int32_t layer, void* stream) {
  const ll::Geometry& g = cs.geom();
  if (!g.staged) return 0;
  const ll::Layout& lay = cs.layout();
  char* buf = static_cast<char*>(cs.buffer());
  ll::StageArgs s;
  s.layer = buf + lay.layer_bytes * size_t(layer);
  s.k_off = int64_t(lay.k_off);
  s.v_off = int64_t(lay.v_off);
  s.ks_off = int64_t(lay.ks_off);
  s.vs_off = int64_t(lay.vs_off);
  s.dst_k = buf + lay.stage_k_off;
  s.dst_v = buf + lay.stage_v_off;
  s.rows = g.rows;
  s.vt_head_elems = g.vt_head_elems;
  s.tps = g.tps;
  s.ctok = int32_t(g.ctok);
  s.H = g.H;
  s.D = g.D;
  auto add = [&](int64_t row0) {
    s.row0[s.n_chunks] = int32_t(row0);
    s.slot[s.n_chunks] = ll::slot_of_row(g, row0);
    ++s.n_chunks;
  };
  for (int64_t r0 = 0; r0 < cs.sink_valid_rows(layer); r0 += g.ctok) add(r0);
  for (int32_t slot : cs.resident_slots(layer)) add(g.sink_rows + int64_t(slot) * g.ctok);
  return ll::launch_stage_int8(s, stream);
}

// The caller's current chunk (token-major [n_cur][H][D]) as the last run.
void add_current_run(const ll::Geometry& g, const void* k_cur, const void* v_cur, int64_t n_cur,
                     ll::AttnArgs& a, int32_t& keys) {
  ll::KvSeg& s = a.seg[a.n_seg++];
  s.k = k_cur;
  s.v = v_cur;
  s.ks = s.vs = nullptr;
  s.head_stride = g.D;
  s.row_stride = int64_t(g.H) * g.D;
  s.v_head_stride = 0;
  s.s_head_stride = 0;
  s.v_tiled = 0;
  s.i8 = 0;
  s.key_start = keys;
  s.len = int32_t(n_cur);
  keys += int32_t(n_cur);
}

// The backward of one call with its delta workspace (caller-provided or the
// library's static one); `static_delta` replaces the caller checks of delta
// by the size bound of the static workspace.
ll_status attn_bwd_impl(const ll_cache* cache, int32_t layer, const void* q, int64_t n_q,
                        const void* k_cur, const void* v_cur, int64_t n_cur, float scale,
                        const void* out, const float* lse, const void* dout, float* delta,
                        bool static_delta, float* dq, float* dk_cur, float* dv_cur, ll_stream_t stream) {
  ll_status st = check_layer(cache, layer, false);
  if (st != LL_OK) return st;
  const ll::CacheState& cs = cache->state;
  const ll::Geometry& g = cs.geom();
  if (g.act != LL_BF16) return fail(LL_ERR_UNSUPPORTED, "the backward supports BF16 activations");
  if (n_q < 1 || n_q > INT32_MAX / 2) return fail(LL_ERR_INVALID_ARG, "n_q must be in [1, 2^30)");
  if (n_cur != 0 && n_cur != g.ctok)
    return fail(LL_ERR_INVALID_ARG, "n_cur must be 0 or the chunk's token count " + std::to_string(g.ctok));
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(LL_ERR_INVALID_ARG, "scale must be finite and > 0");
  if ((st = check_act_ptr(q, "q")) != LL_OK || (st = check_act_ptr(out, "out")) != LL_OK ||
      (st = check_act_ptr(dout, "dout")) != LL_OK || (st = check_act_ptr(dq, "dq")) != LL_OK)
    return st;
  if (!lse || !aligned(lse, 4)) return fail(LL_ERR_INVALID_ARG, "lse is NULL or not 4-byte aligned");
  if (static_delta) {
    if (int64_t(g.H) * n_q > ll::kBwdScratchFloats)
      return fail(LL_ERR_UNSUPPORTED, "num_heads * n_q = " + std::to_string(int64_t(g.H) * n_q) +
                                          " exceeds the static workspace of " +
                                          std::to_string(ll::kBwdScratchFloats) + " floats");
  } else if (!delta || !aligned(delta, 4)) {
    return fail(LL_ERR_INVALID_ARG, "delta is NULL or not 4-byte aligned");
  }
  if (n_cur > 0) {
    if ((st = check_act_ptr(k_cur, "k_cur")) != LL_OK || (st = check_act_ptr(v_cur, "v_cur")) != LL_OK ||
        (st = check_act_ptr(dk_cur, "dk_cur")) != LL_OK || (st = check_act_ptr(dv_cur, "dv_cur")) != LL_OK)
      return st;
    // The dK/dV kernel addresses the bf16 queries and dout with 32-bit byte
    // offsets, rounded up to whole 64-query tiles.
    if ((n_q + 64) * int64_t(g.H) * g.D * 2 >= (int64_t(1) << 32))
      return fail(LL_ERR_UNSUPPORTED, "with dk_cur/dv_cur, (n_q + 64) * num_heads * head_dim * 2 bytes must be "
                                      "below 4 GiB");
  }
  ll::AttnBwdArgs b;
  int32_t keys = 0;
  add_cache_runs(cs, layer, b.a, keys, /*staged=*/true);
  if (n_cur > 0) add_current_run(g, k_cur, v_cur, n_cur, b.a, keys);
  if (keys == 0) return fail(LL_ERR_BAD_STATE, "empty key set: nothing cached and n_cur == 0");
  if (static_delta && (st = launched(ll::bwd_scratch(&delta), "static workspace lookup")) != LL_OK) return st;
  b.a.n_keys = keys;
  b.a.q = q;
  b.a.out = nullptr;
  b.a.lse = nullptr;
  b.a.n_q = int32_t(n_q);
  b.a.H = g.H;
  b.a.D = g.D;
  b.a.act = g.act;
  b.a.scale = scale;
  b.out = out;
  b.dout = dout;
  b.lse = lse;
  b.delta = delta;
  b.dq = dq;
  b.dk = n_cur > 0 ? dk_cur : nullptr;
  b.dv = n_cur > 0 ? dv_cur : nullptr;
  if ((st = launched(stage_int8(cs, layer, stream), "int8 staging launch")) != LL_OK) return st;
  return launched(ll::launch_attention_bwd(b, stream), "attention backward launch");
}

}  // namespace

extern "C" {

const char* ll_status_str(ll_status s) {
  switch (s) {
    case LL_OK: return "LL_OK";
    case LL_ERR_INVALID_ARG: return "LL_ERR_INVALID_ARG";
    case LL_ERR_BAD_STATE: return "LL_ERR_BAD_STATE";
    case LL_ERR_UNSUPPORTED: return "LL_ERR_UNSUPPORTED";
    case LL_ERR_BUFFER_TOO_SMALL: return "LL_ERR_BUFFER_TOO_SMALL";
    case LL_ERR_HIP: return "LL_ERR_HIP";
    case LL_ERR_INTERNAL: return "LL_ERR_INTERNAL";
  }
  return "unknown ll_status";
}

const char* ll_last_error(void) { return ll::last_error(); }

ll_status ll_cache_required_bytes(const ll_cache_config* cfg, size_t* bytes) {
  ll::clear_error();
  if (!bytes) return fail(LL_ERR_INVALID_ARG, "bytes is NULL");
  ll::Geometry g;
  ll_status st = ll::make_geometry(cfg, &g);
  if (st != LL_OK) return st;
  *bytes = ll::make_layout(g).total_bytes;
  return LL_OK;
}

ll_status ll_cache_create(const ll_cache_config* cfg, void* dev_buf, size_t dev_bytes,
                          ll_cache** out) {
  ll::clear_error();
  if (!out) return fail(LL_ERR_INVALID_ARG, "out is NULL");
  ll::Geometry g;
  ll_status st = ll::make_geometry(cfg, &g);
  if (st != LL_OK) return st;
  if (!dev_buf) return fail(LL_ERR_INVALID_ARG, "dev_buf is NULL");
  if (!aligned(dev_buf, 256)) return fail(LL_ERR_INVALID_ARG, "dev_buf is not 256-byte aligned");
  const size_t need = ll::make_layout(g).total_bytes;
  if (dev_bytes < need)
    return fail(LL_ERR_BUFFER_TOO_SMALL, "device buffer has " + std::to_string(dev_bytes) +
                                             " bytes, needs " + std::to_string(need));
  ll_cache* c = new (std::nothrow) ll_cache{ll::CacheState(g, dev_buf)};
  if (!c) return fail(LL_ERR_INTERNAL, "out of host memory");
  *out = c;
  return LL_OK;
}

ll_status ll_cache_get_config(const ll_cache* cache, ll_cache_config* cfg) {
  ll::clear_error();
  if (!cache) return fail(LL_ERR_INVALID_ARG, "cache handle is NULL");
  if (!cfg) return fail(LL_ERR_INVALID_ARG, "cfg is NULL");
  const ll::Geometry& g = cache->state.geom();
  *cfg = ll_cache_config{g.L, g.H, g.D, g.T, g.C, g.S, g.W, g.act, g.kv};
  return LL_OK;
}

ll_status ll_cache_set_int8_dequant(ll_cache* cache, int32_t mode) {
  ll::clear_error();
  if (!cache) return fail(LL_ERR_INVALID_ARG, "cache handle is NULL");
  if (mode != LL_I8_STAGED && mode != LL_I8_IN_KERNEL)
    return fail(LL_ERR_INVALID_ARG, "mode must be LL_I8_STAGED or LL_I8_IN_KERNEL");
  if (cache->state.geom().kv != LL_I8) return fail(LL_ERR_INVALID_ARG, "the cache's kv_dtype is not I8");
  cache->state.set_int8_dequant(mode);
  return LL_OK;
}

ll_status ll_cache_destroy(ll_cache* cache) {
  ll::clear_error();
  delete cache;
  return LL_OK;
}

ll_status ll_cache_reset(ll_cache* cache) {
  ll::clear_error();
  if (!cache) return fail(LL_ERR_INVALID_ARG, "cache handle is NULL");
  cache->state.reset();
  return LL_OK;
}

ll_status ll_cache_query(const ll_cache* cache, int32_t layer, int64_t* chunks_appended,
                         int32_t* ring_valid, int32_t* ring_next, int64_t* slot_chunk) {
  ll::clear_error();
  ll_status st = check_layer(cache, layer, false);
  if (st != LL_OK) return st;
  const ll::LayerState& L = cache->state.layer(layer);
  if (chunks_appended) *chunks_appended = L.appended;
  if (ring_valid) *ring_valid = L.ring_valid;
  if (ring_next) *ring_next = L.ring_next;
  if (slot_chunk)
    for (size_t s = 0; s < L.slot_chunk.size(); ++s) slot_chunk[s] = L.slot_chunk[s];
  return LL_OK;
}

ll_status ll_cache_layout(const ll_cache* cache, int32_t layer, int32_t which, int32_t segment,
                          size_t* byte_offset, int64_t* strides, int64_t* shape) {
  ll::clear_error();
  ll_status st = check_layer(cache, layer, false);
  if (st != LL_OK) return st;
  if (!byte_offset || !strides) return fail(LL_ERR_INVALID_ARG, "byte_offset and strides must be non-NULL");
  if (which < LL_WHICH_K || which > LL_WHICH_VSCALE)
    return fail(LL_ERR_INVALID_ARG, "which must be K, V, KSCALE or VSCALE");
  if (segment != LL_SEG_SINK && segment != LL_SEG_RING)
    return fail(LL_ERR_INVALID_ARG, "segment must be SINK or RING");
  const ll::Geometry& g = cache->state.geom();
  const ll::Layout& lay = cache->state.layout();
  const bool scale = which >= LL_WHICH_KSCALE;
  if (scale && g.kv != LL_I8) return fail(LL_ERR_INVALID_ARG, "scales exist only for an I8 cache");
  size_t base = lay.layer_bytes * size_t(layer);
  size_t region = which == LL_WHICH_K ? lay.k_off : which == LL_WHICH_V ? lay.v_off
                : which == LL_WHICH_KSCALE ? lay.ks_off : lay.vs_off;
  const size_t elt = scale ? sizeof(float) : ll::dtype_bytes(g.kv);
  if (which == LL_WHICH_V && g.vt) {
    // [H][tiles][D][64]: the segment's chunk slots, tps tiles each
    const int64_t slot0 = segment == LL_SEG_SINK ? 0 : g.nsc;
    const int64_t nslot = segment == LL_SEG_SINK ? g.nsc : g.R;
    const int64_t tile = int64_t(ll::kVtTileKeys) * g.D;
    *byte_offset = base + region + size_t(slot0 * g.tps * tile) * elt;
    strides[0] = g.vt_head_elems;
    strides[1] = tile;
    strides[2] = ll::kVtTileKeys;
    strides[3] = 1;
    if (shape) {
      shape[0] = g.H;
      shape[1] = nslot * g.tps;
      shape[2] = g.D;
      shape[3] = ll::kVtTileKeys;
    }
    return LL_OK;
  }
  const int64_t cols = scale ? 1 : g.D;
  const int64_t row0 = segment == LL_SEG_SINK ? 0 : g.sink_rows;
  const int64_t nrows = segment == LL_SEG_SINK ? g.sink_rows : g.ring_rows;
  *byte_offset = base + region + size_t(row0 * cols) * elt;
  strides[0] = g.rows * cols;
  strides[1] = cols;
  strides[2] = 1;
  strides[3] = 1;
  if (shape) {
    shape[0] = g.H;
    shape[1] = nrows;
    shape[2] = cols;
    shape[3] = 1;
  }
  return LL_OK;
}

ll_status ll_cache_append_chunk(ll_cache* cache, int32_t layer, const void* k, const void* v,
                                ll_stream_t stream) {
  ll::clear_error();
  ll_status st = check_layer(cache, layer, false);
  if (st != LL_OK) return st;
  if ((st = check_act_ptr(k, "k")) != LL_OK || (st = check_act_ptr(v, "v")) != LL_OK) return st;
  ll::CacheState& cs = cache->state;
  const ll::Geometry& g = cs.geom();
  const ll::AppendPlan p = cs.plan_append(layer);
  if (p.store) {
    ll::CopyArgs a;
    a.src_k = k;
    a.src_v = v;
    a.src_layer_elems = 0;
    a.dst = static_cast<char*>(cs.buffer()) + cs.layout().layer_bytes * size_t(layer);
    a.dst_layer_bytes = int64_t(cs.layout().layer_bytes);
    a.k_off = cs.layout().k_off; a.v_off = cs.layout().v_off;
    a.ks_off = cs.layout().ks_off; a.vs_off = cs.layout().vs_off;
    a.rows = g.rows;
    a.n_chunks = 1;
    a.n_layers = 1;
    a.dst_row0[0] = int32_t(p.row0);
    a.dst_slot[0] = ll::slot_of_row(g, p.row0);
    a.vt = g.vt ? 1 : 0;
    a.tps = g.tps;
    a.vt_head_elems = g.vt_head_elems;
    a.ctok = int32_t(g.ctok);
    a.H = g.H; a.D = g.D; a.act = g.act; a.kv = g.kv;
    st = launched(ll::launch_copy_chunks(a, stream), "append launch");
    if (st != LL_OK) return st;
  }
  cs.commit_append(layer, p);
  return LL_OK;
}

ll_status ll_cache_recache(ll_cache* cache, int32_t layer, const void* k, const void* v,
                           int64_t n_tokens, ll_stream_t stream) {
  ll::clear_error();
  ll_status st = check_layer(cache, layer, true);
  if (st != LL_OK) return st;
  if ((st = check_act_ptr(k, "k")) != LL_OK || (st = check_act_ptr(v, "v")) != LL_OK) return st;
  ll::CacheState& cs = cache->state;
  const ll::Geometry& g = cs.geom();
  const int l0 = layer == -1 ? 0 : layer;
  const int nl = layer == -1 ? g.L : 1;
  const std::vector<int32_t> slots = cs.resident_slots(l0);
  if (slots.empty()) return fail(LL_ERR_BAD_STATE, "no window chunk is resident: nothing to recache");
  for (int l = l0 + 1; l < l0 + nl; ++l)
    if (cs.resident_slots(l) != slots)
      return fail(LL_ERR_BAD_STATE, "layer -1 needs every layer to hold the same ring state");
  const int64_t want = int64_t(slots.size()) * g.ctok;
  if (n_tokens != want)
    return fail(LL_ERR_INVALID_ARG, "n_tokens " + std::to_string(n_tokens) + " != resident window tokens " +
                                        std::to_string(want));
  ll::CopyArgs a;
  a.src_k = k;
  a.src_v = v;
  a.src_layer_elems = want * g.H * g.D;
  a.dst = static_cast<char*>(cs.buffer()) + cs.layout().layer_bytes * size_t(l0);
  a.dst_layer_bytes = int64_t(cs.layout().layer_bytes);
  a.k_off = cs.layout().k_off; a.v_off = cs.layout().v_off;
  a.ks_off = cs.layout().ks_off; a.vs_off = cs.layout().vs_off;
  a.rows = g.rows;
  a.n_chunks = int32_t(slots.size());
  a.n_layers = nl;
  for (size_t i = 0; i < slots.size(); ++i) {
    a.dst_row0[i] = int32_t(g.sink_rows + slots[i] * g.ctok);
    a.dst_slot[i] = g.nsc + slots[i];
  }
  a.vt = g.vt ? 1 : 0;
  a.tps = g.tps;
  a.vt_head_elems = g.vt_head_elems;
  a.ctok = int32_t(g.ctok);
  a.H = g.H; a.D = g.D; a.act = g.act; a.kv = g.kv;
  return launched(ll::launch_copy_chunks(a, stream), "recache launch");
}

ll_status ll_sink_window_attn(const ll_cache* cache, int32_t layer, const void* q, int64_t n_q,
                              const void* k_cur, const void* v_cur, int64_t n_cur, float scale,
                              void* out, float* lse, ll_stream_t stream) {
  ll::clear_error();
  ll_status st = check_layer(cache, layer, false);
  if (st != LL_OK) return st;
  const ll::CacheState& cs = cache->state;
  const ll::Geometry& g = cs.geom();
  if (n_q < 0 || n_q > INT32_MAX / 2) return fail(LL_ERR_INVALID_ARG, "n_q out of range");
  if (n_cur != 0 && n_cur != g.ctok)
    return fail(LL_ERR_INVALID_ARG, "n_cur must be 0 or the chunk's token count " + std::to_string(g.ctok));
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(LL_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (n_q > 0) {
    if ((st = check_act_ptr(q, "q")) != LL_OK || (st = check_act_ptr(out, "out")) != LL_OK) return st;
    if (lse && !aligned(lse, 4)) return fail(LL_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  }
  if (n_cur > 0) {
    if ((st = check_act_ptr(k_cur, "k_cur")) != LL_OK || (st = check_act_ptr(v_cur, "v_cur")) != LL_OK)
      return st;
  }
  ll::AttnArgs a;
  int32_t keys = 0;
  const bool staged = cs.int8_dequant() == LL_I8_STAGED;
  add_cache_runs(cs, layer, a, keys, staged);
  if (n_cur > 0) add_current_run(g, k_cur, v_cur, n_cur, a, keys);
  if (keys == 0) return fail(LL_ERR_BAD_STATE, "empty key set: nothing cached and n_cur == 0");
  if (n_q == 0) return LL_OK;
  a.n_keys = keys;
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.n_q = int32_t(n_q);
  a.H = g.H;
  a.D = g.D;
  a.act = g.act;
  a.scale = scale;
  if (staged && (st = launched(stage_int8(cs, layer, stream), "int8 staging launch")) != LL_OK) return st;
  return launched(ll::launch_attention(a, stream), "attention launch");
}

ll_status ll_sink_window_attn_bwd(const ll_cache* cache, int32_t layer, const void* q, int64_t n_q,
                                  const void* k_cur, const void* v_cur, int64_t n_cur, float scale,
                                  const void* out, const float* lse, const void* dout, float* delta,
                                  float* dq, float* dk_cur, float* dv_cur, ll_stream_t stream) {
  ll::clear_error();
  return attn_bwd_impl(cache, layer, q, n_q, k_cur, v_cur, n_cur, scale, out, lse, dout, delta, false, dq,
                       dk_cur, dv_cur, stream);
}

ll_status ll_sink_window_attn_bwd_noalloc(const ll_cache* cache, int32_t layer, const void* q, int64_t n_q,
                                          const void* k_cur, const void* v_cur, int64_t n_cur, float scale,
                                          const void* out, const float* lse, const void* dout, float* dq,
                                          float* dk_cur, float* dv_cur, ll_stream_t stream) {
  ll::clear_error();
  return attn_bwd_impl(cache, layer, q, n_q, k_cur, v_cur, n_cur, scale, out, lse, dout, nullptr, true, dq,
                       dk_cur, dv_cur, stream);
}

ll_status ll_window_reencode_attn(const ll_cache* cache, int32_t layer, const void* q,
                                  int64_t n_q, float scale, void* out, float* lse,
                                  ll_stream_t stream) {
  ll::clear_error();
  ll_status st = check_layer(cache, layer, false);
  if (st != LL_OK) return st;
  const ll::CacheState& cs = cache->state;
  const ll::Geometry& g = cs.geom();
  const int64_t resident = cs.layer(layer).ring_valid;
  if (resident == 0) return fail(LL_ERR_BAD_STATE, "no window chunk is resident");
  if (n_q != resident * g.ctok)
    return fail(LL_ERR_INVALID_ARG, "n_q must be (resident window chunks) * C_tok = " +
                                        std::to_string(resident * g.ctok));
  if (n_q > INT32_MAX / 2) return fail(LL_ERR_INVALID_ARG, "n_q out of range");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(LL_ERR_INVALID_ARG, "scale must be finite and > 0");
  if ((st = check_act_ptr(q, "q")) != LL_OK || (st = check_act_ptr(out, "out")) != LL_OK) return st;
  if (lse && !aligned(lse, 4)) return fail(LL_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  ll::AttnArgs a;
  int32_t keys = 0;
  const bool staged = cs.int8_dequant() == LL_I8_STAGED;
  const int n_sink = add_cache_runs(cs, layer, a, keys, staged);
  a.n_keys = keys;
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.n_q = int32_t(n_q);
  a.H = g.H;
  a.D = g.D;
  a.act = g.act;
  a.scale = scale;
  a.q_chunk = int32_t(g.ctok);
  a.n_seg0 = n_sink + 1;
  if (staged && (st = launched(stage_int8(cs, layer, stream), "int8 staging launch")) != LL_OK) return st;
  return launched(ll::launch_attention(a, stream), "re-encoding attention launch");
}

ll_status ll_linear_attn_workspace_bytes(const ll_cache* cache, size_t* bytes) {
  ll::clear_error();
  if (!cache) return fail(LL_ERR_INVALID_ARG, "cache handle is NULL");
  if (!bytes) return fail(LL_ERR_INVALID_ARG, "bytes is NULL");
  const ll::Geometry& g = cache->state.geom();
  *bytes = ll::linear_workspace_layout(g.H, g.D).total;
  return LL_OK;
}

ll_status ll_sink_window_linear_attn(const ll_cache* cache, int32_t layer, const void* q, int64_t n_q,
                                     const void* k_cur, const void* v_cur, int64_t n_cur, void* out,
                                     void* work, size_t work_bytes, ll_stream_t stream) {
  ll::clear_error();
  ll_status st = check_layer(cache, layer, false);
  if (st != LL_OK) return st;
  const ll::CacheState& cs = cache->state;
  const ll::Geometry& g = cs.geom();
  if (g.act != LL_BF16) return fail(LL_ERR_UNSUPPORTED, "the linear-attention variant supports BF16 activations");
  if (n_q < 0 || n_q > INT32_MAX / 2) return fail(LL_ERR_INVALID_ARG, "n_q out of range");
  if (n_cur != 0 && n_cur != g.ctok)
    return fail(LL_ERR_INVALID_ARG, "n_cur must be 0 or the chunk's token count " + std::to_string(g.ctok));
  if (n_q > 0 && ((st = check_act_ptr(q, "q")) != LL_OK || (st = check_act_ptr(out, "out")) != LL_OK)) return st;
  if (n_cur > 0 && ((st = check_act_ptr(k_cur, "k_cur")) != LL_OK || (st = check_act_ptr(v_cur, "v_cur")) != LL_OK))
    return st;
  const ll::LinLayout wl = ll::linear_workspace_layout(g.H, g.D);
  if (!work || !aligned(work, 256)) return fail(LL_ERR_INVALID_ARG, "work is NULL or not 256-byte aligned");
  if (work_bytes < wl.total)
    return fail(LL_ERR_BUFFER_TOO_SMALL, "work needs " + std::to_string(wl.total) + " bytes");
  ll::LinArgs p;
  ll::AttnArgs& a = p.a;
  int32_t keys = 0;
  add_cache_runs(cs, layer, a, keys, /*staged=*/true);
  if (n_cur > 0) add_current_run(g, k_cur, v_cur, n_cur, a, keys);
  if (keys == 0) return fail(LL_ERR_BAD_STATE, "empty key set: nothing cached and n_cur == 0");
  if (n_q == 0) return LL_OK;
  a.n_keys = keys;
  a.q = q;
  a.out = out;
  a.n_q = int32_t(n_q);
  a.H = g.H;
  a.D = g.D;
  a.act = g.act;
  // Key splits: one state workgroup per compute unit over all heads (its
  // 128 KB LDS ring holds one per CU), at most kLinMaxSplits and n_tiles.
  int32_t n_tiles = 0;
  for (int r = 0; r < a.n_seg; ++r) n_tiles += (a.seg[r].len + 63) / 64;
  // Split s sums tiles s, s + n_split, ... (at most tiles_per_split of them).
  p.n_split = std::min<int32_t>({ll::kLinMaxSplits, n_tiles, std::max<int32_t>(1, ll::kComputeUnits / g.H)});
  p.tiles_per_split = (n_tiles + p.n_split - 1) / p.n_split;
  char* w = static_cast<char*>(work);
  p.part_s = reinterpret_cast<float*>(w + wl.part_s);
  p.part_z = reinterpret_cast<float*>(w + wl.part_z);
  p.st_hi = w + wl.st_hi;
  p.st_lo = w + wl.st_lo;
  p.z = reinterpret_cast<float*>(w + wl.z);
  if ((st = launched(stage_int8(cs, layer, stream), "int8 staging launch")) != LL_OK) return st;
  return launched(ll::launch_linear_attention(p, stream), "linear attention launch");
}

ll_status ll_cross_attn(const void* q, int64_t n_q, const void* k_txt, const void* v_txt,
                        int64_t n_txt, int32_t num_heads, int32_t head_dim, int32_t dtype,
                        float scale, void* out, float* lse, ll_stream_t stream) {
  ll::clear_error();
  if (num_heads < 1) return fail(LL_ERR_INVALID_ARG, "num_heads must be >= 1");
  if (head_dim != 64 && head_dim != 128) return fail(LL_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (dtype != LL_F32 && dtype != LL_BF16) return fail(LL_ERR_UNSUPPORTED, "dtype must be F32 or BF16");
  if (n_txt < 1 || n_txt > INT32_MAX / 2) return fail(LL_ERR_INVALID_ARG, "n_txt must be in [1, 2^30)");
  // 32-bit byte offsets are formed for whole 64-key tiles: rows past the end
  // must not wrap around into the buffer range.
  if ((n_txt + 64) * num_heads * int64_t(head_dim) * ll::dtype_bytes(dtype) >= (int64_t(1) << 32))
    return fail(LL_ERR_UNSUPPORTED, "text K/V, rounded up to whole 64-key tiles, must be smaller than 4 GiB each");
  if (n_q < 0 || n_q > INT32_MAX / 2) return fail(LL_ERR_INVALID_ARG, "n_q out of range");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(LL_ERR_INVALID_ARG, "scale must be finite and > 0");
  ll_status st;
  if ((st = check_act_ptr(k_txt, "k_txt")) != LL_OK || (st = check_act_ptr(v_txt, "v_txt")) != LL_OK)
    return st;
  if (n_q == 0) return LL_OK;
  if ((st = check_act_ptr(q, "q")) != LL_OK || (st = check_act_ptr(out, "out")) != LL_OK) return st;
  if (lse && !aligned(lse, 4)) return fail(LL_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  ll::AttnArgs a;
  ll::KvSeg& s = a.seg[0];
  s.k = k_txt;
  s.v = v_txt;
  s.ks = s.vs = nullptr;
  s.head_stride = head_dim;
  s.row_stride = int64_t(num_heads) * head_dim;
  s.v_head_stride = 0;
  s.s_head_stride = 0;
  s.v_tiled = 0;
  s.i8 = 0;
  s.key_start = 0;
  s.len = int32_t(n_txt);
  a.n_seg = 1;
  a.n_keys = int32_t(n_txt);
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.n_q = int32_t(n_q);
  a.H = num_heads;
  a.D = head_dim;
  a.act = dtype;
  a.scale = scale;
  return launched(ll::launch_attention(a, stream), "cross-attention launch");
}

}  // extern "C"
