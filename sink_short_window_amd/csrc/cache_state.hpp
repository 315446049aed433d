// Host-side cache bookkeeping for the frame-sink + short-window KV cache.
// No HIP in this translation unit: it is built into libll.so and, for CPU
// tests, into a host-only shim.
//
// Policy (LongLive: Real-time Interactive Long Video Generation, §3.3
// "Efficient long inference"): the first sink chunks are kept for good; the
// remaining chunks go to a rolling window of R one-chunk slots, first in first
// out.  A KV-recache (§3.1) rewrites the resident window chunks.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "ll.h"

namespace ll {

// Thread-local error text behind ll_last_error().
void set_error(const std::string& msg);
void clear_error();
const char* last_error();
ll_status fail(ll_status st, const std::string& msg);

size_t dtype_bytes(int32_t dt);

// Validated geometry with the derived sizes.
struct Geometry {
  int32_t L = 0, H = 0, D = 0, T = 0, C = 0, S = 0, W = 0;
  int32_t act = 0, kv = 0;
  int64_t ctok = 0;       // tokens per chunk, C*T
  int32_t nsc = 0;        // sink chunks, S/C
  int32_t R = 0;          // ring slots, (W-C)/C
  int64_t sink_rows = 0;  // S*T
  int64_t ring_rows = 0;  // R*ctok
  int64_t rows = 0;       // sink_rows + ring_rows, per head
  // BF16 and I8 caches keep V transposed in 64-key tiles (the layout the
  // attention kernel's PV operand wants): per head, nslots chunk slots (sink
  // chunks, then ring slots) of tps tiles, each tile [D][64] with zero
  // padding after the chunk's last key.
  bool vt = false;
  // An I8 cache also holds a bf16 staging area for one layer's resident sink
  // + ring in the BF16 layout (K rows, V tiles), which the backward and the
  // linear-attention variant read; the attention reads the int8 codes.
  bool staged = false;
  int32_t tps = 0;            // tiles per chunk slot, ceil(ctok / 64)
  int32_t nslots = 0;         // nsc + R
  int64_t vt_head_elems = 0;  // nslots * tps * 64 * D
};

// Key runs an attention call may walk (sink chunks, ring slots, current chunk).
constexpr int kMaxKeyRuns = 40;
constexpr int kVtTileKeys = 64;

ll_status make_geometry(const ll_cache_config* cfg, Geometry* g);

// Byte layout of the device buffer.  Per layer, in order, each region
// 256-byte aligned: K [H][rows][D], V [H][rows][D] (kv dtype; for BF16 and
// I8 caches V is [H][nslots*tps][D][64] instead, see Geometry), and with I8
// K scales [H][rows], V scales [H][rows] (fp32).  Rows [0, sink_rows) are the
// sink; ring slot s is rows sink_rows + [s*ctok, (s+1)*ctok).  An I8 cache
// ends with the bf16 staging area: K [H][rows][D], V [H][nslots*tps][D][64].
struct Layout {
  size_t k_off = 0, v_off = 0, ks_off = 0, vs_off = 0;  // within a layer
  size_t layer_bytes = 0;
  size_t stage_k_off = 0, stage_v_off = 0;  // from the buffer base (I8 only)
  size_t total_bytes = 0;
};
Layout make_layout(const Geometry& g);

struct LayerState {
  int64_t appended = 0;
  int32_t ring_valid = 0;
  int32_t ring_next = 0;
  std::vector<int64_t> slot_chunk;  // R entries, -1 = empty
};

// Where the next append of a layer goes.
struct AppendPlan {
  bool store = false;  // false: non-sink chunk with R == 0 (counted only)
  bool sink = false;
  int64_t row0 = 0;    // first row inside the per-head [rows] range
  int32_t slot = -1;
  int64_t chunk = 0;
};

// Chunk slot (sink chunks first, then ring slots) of the chunk stored at row0.
int32_t slot_of_row(const Geometry& g, int64_t row0);

class CacheState {
 public:
  CacheState(const Geometry& g, void* buf) : g_(g), lay_(make_layout(g)), buf_(buf), layers_(g.L) {
    reset();
  }
  const Geometry& geom() const { return g_; }
  const Layout& layout() const { return lay_; }
  void* buffer() const { return buf_; }
  const LayerState& layer(int l) const { return layers_[l]; }

  void reset();
  // How the attention reads an I8 cache (ll_int8_dequant).
  int32_t int8_dequant() const { return i8_mode_; }
  void set_int8_dequant(int32_t m) { i8_mode_ = m; }
  AppendPlan plan_append(int layer) const;
  void commit_append(int layer, const AppendPlan& p);
  // Ring slots of the resident window chunks, oldest chunk first.
  std::vector<int32_t> resident_slots(int layer) const;
  // Valid sink rows of a layer (the sink fills one chunk at a time).
  int64_t sink_valid_rows(int layer) const;

 private:
  Geometry g_;
  Layout lay_;
  void* buf_;
  std::vector<LayerState> layers_;
  int32_t i8_mode_ = LL_I8_STAGED;
};

}  // namespace ll

struct ll_cache {
  ll::CacheState state;
};
