// Launch interface between the C ABI layer (ll_api.cpp) and the HIP kernels
// (kernels.hip).  Plain structs, no HIP types: a stream is passed as void*.
#pragma once

#include <cstdint>

#include "ll.h"

namespace ll {

// One contiguous run of keys, addressed in place.  Element (head h, key i of
// the run, dim d) of K lives at k + (h*head_stride + i*row_stride + d)
// elements, and likewise V unless v_tiled.  A v_tiled run (bf16 and int8
// caches) keeps V transposed in 64-key tiles: element (h, i, d) at
// v + h*v_head_stride + (i/64)*64*D + d*64 + p, where p is i%64 with bits 2
// and 3 swapped (the key order of the PV operand).  Elements are bf16 (or fp32
// for fp32 activations), except in an i8 run: int8 codes of an INT8 cache
// whose key i of head h has the fp32 scales ks[h*s_head_stride + i] (K) and
// vs[h*s_head_stride + i] (V); the value it stands for is code * scale.
struct KvSeg {
  const void* k;
  const void* v;
  const float* ks;         // i8 runs
  const float* vs;         // i8 runs
  int64_t head_stride;     // elements
  int64_t row_stride;      // elements
  int64_t v_head_stride;   // elements, v_tiled runs
  int64_t s_head_stride;   // scales per head, i8 runs
  int32_t key_start;       // first key index of the run in the joint key space
  int32_t len;             // keys in the run
  int32_t v_tiled;         // 1: V in transposed 64-key tiles (see above)
  int32_t i8;              // 1: int8 codes with per-key scales (see above)
};

constexpr int kMaxSeg = 40;

struct AttnArgs {
  KvSeg seg[kMaxSeg];
  int32_t n_seg = 0;
  int32_t n_keys = 0;
  const void* q = nullptr;  // [n_q][H][D]
  void* out = nullptr;      // [n_q][H][D]
  float* lse = nullptr;     // [H][n_q] or null
  int32_t n_q = 0;
  int32_t H = 0;
  int32_t D = 0;
  int32_t act = LL_BF16;    // dtype of q/out and of every run
  float scale = 1.f;
  // Chunk-causal queries (re-encoding pass of a KV-recache): with q_chunk > 0
  // the n_q queries are chunks of q_chunk tokens and chunk r attends only the
  // first n_seg0 + r runs.  q_tiles (query tiles per chunk) is set by the
  // launcher for the kernel's tile height.
  int32_t q_chunk = 0;
  int32_t n_seg0 = 0;
  int32_t q_tiles = 0;
};

// Backward of one sink+window call (training step): the runs of `a` as the
// forward walked them, the last of which (the caller's current chunk,
// token-major) carries gradient.
struct AttnBwdArgs {
  AttnArgs a;
  const void* out = nullptr;   // [n_q][H][D] forward output
  const void* dout = nullptr;  // [n_q][H][D] upstream gradient
  const float* lse = nullptr;  // [H][n_q] forward log-sum-exp (natural log)
  float* delta = nullptr;      // [H][n_q] workspace: rowsum(dout * out)
  float* dq = nullptr;         // [n_q][H][D]
  float* dk = nullptr;         // [len of the last run][H][D], null when it carries none
  float* dv = nullptr;
};

// Copy (or quantise) whole chunks of token-major K/V into cache rows.
// Source chunk i of layer z is src + (z*src_layer_stride + i*ctok*H*D) elements
// (token-major [ctok][H][D]); it goes to rows dst_row0[i] .. + ctok of every
// head in the destination layer z (cache base + z*dst_layer_bytes).  With vt,
// V goes instead to chunk slot dst_slot[i] of the transposed tile layout
// (tps tiles of [D][64] per slot, vt_head_elems per head, zero padding).  An
// I8 cache also gets each token's K and V scales at the same rows of its
// [H][rows] fp32 scale arrays.
constexpr int kMaxCopyChunks = LL_MAX_RING_SLOTS + 1;
struct CopyArgs {
  const void* src_k = nullptr;
  const void* src_v = nullptr;
  int64_t src_layer_elems = 0;  // elements between layers of the source
  char* dst = nullptr;          // cache buffer base of layer 0
  int64_t dst_layer_bytes = 0;
  int64_t k_off = 0, v_off = 0, ks_off = 0, vs_off = 0;  // bytes within a layer
  int64_t rows = 0;             // rows per head in the cache
  int32_t n_chunks = 0;
  int32_t n_layers = 1;
  int32_t dst_row0[kMaxCopyChunks];
  int32_t dst_slot[kMaxCopyChunks];
  int32_t vt = 0;
  int32_t tps = 0;
  int64_t vt_head_elems = 0;
  int32_t ctok = 0;
  int32_t H = 0;
  int32_t D = 0;
  int32_t act = LL_BF16;
  int32_t kv = LL_BF16;
};

// Each returns 0 on success or the hipError_t code of the failed launch.
// bf16 staging copy of an I8 layer's resident chunks for the backward and the
// linear-attention variant: each listed chunk (rows row0[i] .. + ctok of every
// head; V tiles of chunk slot slot[i]) is dequantised to bf16(q * s) into K
// rows [H][rows][D] at dst_k (same row index) and V tiles of the same slot at
// dst_v ([H][nslots*tps][D][64], key order and zero padding as the cache).
struct StageArgs {
  const char* layer = nullptr;  // I8 layer base
  int64_t k_off = 0, v_off = 0, ks_off = 0, vs_off = 0;
  char* dst_k = nullptr;
  char* dst_v = nullptr;
  int64_t rows = 0;
  int64_t vt_head_elems = 0;
  int32_t n_chunks = 0;
  int32_t row0[kMaxSeg];
  int32_t slot[kMaxSeg];
  int32_t tps = 0;
  int32_t ctok = 0;
  int32_t H = 0;
  int32_t D = 0;
};

// Linear-attention variant (ll_sink_window_linear_attn): per head the state
// S = sum_j phi(k_j) v_j^T ([D][D]) and z = sum_j phi(k_j) over the runs of
// `a` are summed in n_split partial sums (split s: the 64-key tiles s,
// s + n_split, ...; at most tiles_per_split of them), reduced, then applied:
// out_i = phi(q_i)^T S / (phi(q_i) . z + eps), phi(x) = max(x, 0).  The
// workspace pointers are parts of the caller's buffer (linear_workspace_layout).
constexpr int kLinMaxSplits = 32;
constexpr int kComputeUnits = 256;  // MI355X (gfx950): 8 XCDs x 32 CUs
struct LinArgs {
  AttnArgs a;                 // runs, q, out, n_q, H, D (scale and lse unused)
  float* part_s = nullptr;    // [n_split][H][D][D] fp32, transposed: [d2][d1]
  float* part_z = nullptr;    // [n_split][H][D] fp32
  void* st_hi = nullptr;      // [H][D][D] bf16: S transposed ([d2][d1]), high part
  void* st_lo = nullptr;      // [H][D][D] bf16: S - hi, rounded
  float* z = nullptr;         // [H][D] fp32
  int32_t n_split = 0;
  int32_t tiles_per_split = 0;
  float eps = 1e-6f;
};

// Byte offsets of the parts of the linear-attention workspace for H heads of
// dimension D, each 256-byte aligned; returns the total size.
struct LinLayout {
  size_t part_s, part_z, st_hi, st_lo, z, total;
};
inline LinLayout linear_workspace_layout(int H, int D) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  LinLayout l{};
  size_t o = 0;
  l.part_s = o; o += up(size_t(kLinMaxSplits) * H * D * D * 4);
  l.part_z = o; o += up(size_t(kLinMaxSplits) * H * D * 4);
  l.st_hi = o;  o += up(size_t(H) * D * D * 2);
  l.st_lo = o;  o += up(size_t(H) * D * D * 2);
  l.z = o;      o += up(size_t(H) * D * 4);
  l.total = o;
  return l;
}

// The allocation-free backward's delta workspace: a file-scope device array
// of this many floats (4 MiB) per GPU; bwd_scratch returns the current
// device's address of it (0 on success, else the hipError_t code).
constexpr int64_t kBwdScratchFloats = int64_t(1) << 20;
int bwd_scratch(float** ptr);

int launch_attention(const AttnArgs& a, void* stream);
int launch_linear_attention(const LinArgs& a, void* stream);
int launch_stage_int8(const StageArgs& a, void* stream);
int launch_attention_bwd(const AttnBwdArgs& a, void* stream);
int launch_copy_chunks(const CopyArgs& a, void* stream);
const char* hip_error_string(int err);

}  // namespace ll
