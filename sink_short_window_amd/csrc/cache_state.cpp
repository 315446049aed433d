// Host-side cache bookkeeping (no HIP).  See cache_state.hpp.
#include "cache_state.hpp"

#include <algorithm>
#include <limits>

namespace ll {

namespace {
thread_local std::string g_last_error;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
}  // namespace

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }
const char* last_error() { return g_last_error.c_str(); }
ll_status fail(ll_status st, const std::string& msg) {
  set_error(msg);
  return st;
}

size_t dtype_bytes(int32_t dt) {
  switch (dt) {
    case LL_F32: return 4;
    case LL_BF16: return 2;
    case LL_I8: return 1;
    default: return 0;
  }
}

ll_status make_geometry(const ll_cache_config* cfg, Geometry* g) {
  if (!cfg || !g) return fail(LL_ERR_INVALID_ARG, "config and output must be non-NULL");
  const ll_cache_config& c = *cfg;
  if (c.num_layers < 1 || c.num_heads < 1 || c.tokens_per_frame < 1 || c.frames_per_chunk < 1)
    return fail(LL_ERR_INVALID_ARG, "num_layers, num_heads, tokens_per_frame and frames_per_chunk must be >= 1");
  if (c.sink_frames < 0) return fail(LL_ERR_INVALID_ARG, "sink_frames must be >= 0");
  if (c.head_dim != 64 && c.head_dim != 128)
    return fail(LL_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c.window_frames < c.frames_per_chunk)
    return fail(LL_ERR_UNSUPPORTED, "window_frames must be >= frames_per_chunk (the window counts the current chunk)");
  if (c.sink_frames % c.frames_per_chunk)
    return fail(LL_ERR_UNSUPPORTED, "sink_frames must be a whole number of chunks");
  if ((c.window_frames - c.frames_per_chunk) % c.frames_per_chunk)
    return fail(LL_ERR_UNSUPPORTED, "window_frames - frames_per_chunk must be a whole number of chunks");
  const bool ok_dt = (c.act_dtype == LL_F32 && c.kv_dtype == LL_F32) ||
                     (c.act_dtype == LL_BF16 && c.kv_dtype == LL_BF16) ||
                     (c.act_dtype == LL_BF16 && c.kv_dtype == LL_I8);
  if (!ok_dt) return fail(LL_ERR_UNSUPPORTED, "(act_dtype, kv_dtype) must be (F32,F32), (BF16,BF16) or (BF16,I8)");
  Geometry r;
  r.L = c.num_layers; r.H = c.num_heads; r.D = c.head_dim; r.T = c.tokens_per_frame;
  r.C = c.frames_per_chunk; r.S = c.sink_frames; r.W = c.window_frames;
  r.act = c.act_dtype; r.kv = c.kv_dtype;
  r.ctok = int64_t(r.C) * r.T;
  r.nsc = r.S / r.C;
  r.R = (r.W - r.C) / r.C;
  if (r.R > LL_MAX_RING_SLOTS) return fail(LL_ERR_UNSUPPORTED, "too many ring slots (window too long)");
  r.sink_rows = int64_t(r.S) * r.T;
  r.ring_rows = int64_t(r.R) * r.ctok;
  r.rows = r.sink_rows + r.ring_rows;
  // Kernels index rows and chunk tokens with 32-bit integers.
  const int64_t lim = std::numeric_limits<int32_t>::max() / 2;
  if (r.ctok > lim || r.rows > lim || r.rows * r.D > lim || r.ctok * r.H * r.D > lim)
    return fail(LL_ERR_UNSUPPORTED, "cache too large for 32-bit row indexing");
  r.vt = r.kv != LL_F32;
  r.staged = r.kv == LL_I8;
  r.nslots = r.nsc + r.R;
  r.tps = int32_t((r.ctok + kVtTileKeys - 1) / kVtTileKeys);
  r.vt_head_elems = int64_t(r.nslots) * r.tps * kVtTileKeys * r.D;
  if (r.vt && r.nslots + 1 > kMaxKeyRuns)
    return fail(LL_ERR_UNSUPPORTED, "BF16 and I8 caches walk each sink chunk and ring slot as its own key run: "
                                    "sink chunks + ring slots must be <= " + std::to_string(kMaxKeyRuns - 1));
  if (r.vt && r.vt_head_elems > lim) return fail(LL_ERR_UNSUPPORTED, "cache too large for 32-bit indexing");
  // The kernels address a token-major chunk ([ctok][H][D] activations) with
  // one 32-bit buffer range, whose byte offsets they form for whole 64-token
  // tiles: rows past the chunk's end must not wrap around into the range.
  if ((r.ctok + kVtTileKeys) * r.H * r.D * int64_t(dtype_bytes(r.act)) >= (int64_t(1) << 32))
    return fail(LL_ERR_UNSUPPORTED, "a chunk of activations, rounded up to whole 64-token tiles, must be smaller "
                                    "than 4 GiB");
  *g = r;
  return LL_OK;
}

Layout make_layout(const Geometry& g) {
  Layout l;
  const size_t kv_bytes = size_t(g.H) * g.rows * g.D * dtype_bytes(g.kv);
  const size_t v_bytes = g.vt ? size_t(g.H) * size_t(g.vt_head_elems) * dtype_bytes(g.kv) : kv_bytes;
  const size_t sc_bytes = (g.kv == LL_I8) ? size_t(g.H) * g.rows * sizeof(float) : 0;
  size_t off = 0;
  l.k_off = off; off = align256(off + kv_bytes);
  l.v_off = off; off = align256(off + v_bytes);
  l.ks_off = off; off = align256(off + sc_bytes);
  l.vs_off = off; off = align256(off + sc_bytes);
  l.layer_bytes = std::max<size_t>(off, 256);
  l.total_bytes = l.layer_bytes * size_t(g.L);
  if (g.staged) {
    l.stage_k_off = l.total_bytes;
    l.stage_v_off = align256(l.stage_k_off + size_t(g.H) * g.rows * g.D * 2);
    l.total_bytes = align256(l.stage_v_off + size_t(g.H) * size_t(g.vt_head_elems) * 2);
  }
  return l;
}

void CacheState::reset() {
  for (auto& L : layers_) {
    L.appended = 0;
    L.ring_valid = 0;
    L.ring_next = 0;
    L.slot_chunk.assign(g_.R, -1);
  }
}

AppendPlan CacheState::plan_append(int layer) const {
  const LayerState& L = layers_[layer];
  AppendPlan p;
  p.chunk = L.appended;
  if (L.appended < g_.nsc) {
    p.store = true;
    p.sink = true;
    p.row0 = L.appended * g_.ctok;
  } else if (g_.R > 0) {
    p.store = true;
    p.slot = L.ring_next;
    p.row0 = g_.sink_rows + int64_t(p.slot) * g_.ctok;
  }
  return p;
}

void CacheState::commit_append(int layer, const AppendPlan& p) {
  LayerState& L = layers_[layer];
  L.appended += 1;
  if (p.store && !p.sink) {
    L.slot_chunk[p.slot] = p.chunk;
    L.ring_next = (L.ring_next + 1) % g_.R;
    L.ring_valid = std::min(L.ring_valid + 1, g_.R);
  }
}

std::vector<int32_t> CacheState::resident_slots(int layer) const {
  const LayerState& L = layers_[layer];
  std::vector<int32_t> slots;
  for (int s = 0; s < g_.R; ++s)
    if (L.slot_chunk[s] >= 0) slots.push_back(s);
  std::sort(slots.begin(), slots.end(),
            [&](int a, int b) { return L.slot_chunk[a] < L.slot_chunk[b]; });
  return slots;
}

int32_t slot_of_row(const Geometry& g, int64_t row0) {
  if (row0 < g.sink_rows) return int32_t(row0 / g.ctok);
  return g.nsc + int32_t((row0 - g.sink_rows) / g.ctok);
}

int64_t CacheState::sink_valid_rows(int layer) const {
  return std::min<int64_t>(layers_[layer].appended, g_.nsc) * g_.ctok;
}

}  // namespace ll
