// Host-only stand-in for the kernel launchers, linked with the real C ABI
// layer (ll_api.cpp) and bookkeeping (cache_state.cpp) into a CPU test
// library.  It records what would have been launched instead of launching,
// and can fail the next launch on request, so the ABI's validation, state
// machine, segment tables and error guarantees run on a machine without a GPU.
// Never part of libll.so.
#include <cstring>

#include "launch.hpp"

namespace ll {
namespace {
AttnArgs g_attn;
AttnBwdArgs g_bwd;
StageArgs g_stage;
CopyArgs g_copy;
LinArgs g_lin;
int g_lin_calls = 0;
int g_attn_calls = 0;
int g_bwd_calls = 0;
int g_stage_calls = 0;
int g_copy_calls = 0;
int g_fail_next = 0;
}  // namespace

int launch_attention(const AttnArgs& a, void*) {
  if (g_fail_next) {
    g_fail_next = 0;
    return 1;
  }
  g_attn = a;
  ++g_attn_calls;
  return 0;
}

int launch_linear_attention(const LinArgs& a, void*) {
  if (g_fail_next) {
    g_fail_next = 0;
    return 1;
  }
  g_lin = a;
  g_attn = a.a;  // the run table, readable through llh_last_attn
  ++g_lin_calls;
  return 0;
}

int launch_attention_bwd(const AttnBwdArgs& a, void*) {
  if (g_fail_next) {
    g_fail_next = 0;
    return 1;
  }
  g_bwd = a;
  g_attn = a.a;  // the run table, readable through llh_last_attn
  ++g_bwd_calls;
  return 0;
}

int launch_stage_int8(const StageArgs& a, void*) {
  if (g_fail_next) {
    g_fail_next = 0;
    return 1;
  }
  g_stage = a;
  ++g_stage_calls;
  return 0;
}

int launch_copy_chunks(const CopyArgs& a, void*) {
  if (g_fail_next) {
    g_fail_next = 0;
    return 1;
  }
  g_copy = a;
  ++g_copy_calls;
  return 0;
}

// A stand-in device address for the allocation-free backward's workspace.
int bwd_scratch(float** ptr) {
  *ptr = reinterpret_cast<float*>(uintptr_t(0x5C0000000ull));
  return 0;
}

const char* hip_error_string(int) { return "launch failure injected by the host test stub"; }

}  // namespace ll

extern "C" {

void llh_fail_next_launch(void) { ll::g_fail_next = 1; }
int llh_attn_calls(void) { return ll::g_attn_calls; }
int llh_copy_calls(void) { return ll::g_copy_calls; }

// Last attention launch: n_seg, n_keys, and per run [k, v, head_stride,
// row_stride, key_start, len, v_head_stride, v_tiled, ks, vs, i8] (pointers
// as integers).
int llh_last_attn(int64_t* n_keys, int64_t* runs /* [n_seg][11] */) {
  const ll::AttnArgs& a = ll::g_attn;
  *n_keys = a.n_keys;
  for (int i = 0; i < a.n_seg; ++i) {
    const ll::KvSeg& s = a.seg[i];
    int64_t* r = runs + 11 * i;
    r[0] = int64_t(reinterpret_cast<intptr_t>(s.k));
    r[1] = int64_t(reinterpret_cast<intptr_t>(s.v));
    r[2] = s.head_stride;
    r[3] = s.row_stride;
    r[4] = s.key_start;
    r[5] = s.len;
    r[6] = s.v_head_stride;
    r[7] = s.v_tiled;
    r[8] = int64_t(reinterpret_cast<intptr_t>(s.ks));
    r[9] = int64_t(reinterpret_cast<intptr_t>(s.vs));
    r[10] = s.i8;
  }
  return a.n_seg;
}

// Last attention launch, chunk-causal fields: returns q_chunk (0 = one key set
// for all queries); n_seg0 receives the runs the first query chunk attends.
int llh_last_attn_chunks(int32_t* n_seg0) {
  *n_seg0 = ll::g_attn.n_seg0;
  return ll::g_attn.q_chunk;
}

int llh_bwd_calls(void) { return ll::g_bwd_calls; }

// Last backward launch: whether dK/dV are produced (the last run carries
// gradient) and the workspace / gradient pointers as integers.
int llh_last_bwd(int64_t* ptrs /* [delta, dq, dk, dv, out, dout, lse] */) {
  const ll::AttnBwdArgs& b = ll::g_bwd;
  ptrs[0] = int64_t(reinterpret_cast<intptr_t>(b.delta));
  ptrs[1] = int64_t(reinterpret_cast<intptr_t>(b.dq));
  ptrs[2] = int64_t(reinterpret_cast<intptr_t>(b.dk));
  ptrs[3] = int64_t(reinterpret_cast<intptr_t>(b.dv));
  ptrs[4] = int64_t(reinterpret_cast<intptr_t>(b.out));
  ptrs[5] = int64_t(reinterpret_cast<intptr_t>(b.dout));
  ptrs[6] = int64_t(reinterpret_cast<intptr_t>(b.lse));
  return b.dk != nullptr;
}

int llh_lin_calls(void) { return ll::g_lin_calls; }

// Last linear-attention launch: returns n_split; tps receives the tiles per
// split and ptrs [part_s, part_z, st_hi, st_lo, z] as integers.
int llh_last_lin(int32_t* tps, int64_t* ptrs) {
  const ll::LinArgs& p = ll::g_lin;
  *tps = p.tiles_per_split;
  ptrs[0] = int64_t(reinterpret_cast<intptr_t>(p.part_s));
  ptrs[1] = int64_t(reinterpret_cast<intptr_t>(p.part_z));
  ptrs[2] = int64_t(reinterpret_cast<intptr_t>(p.st_hi));
  ptrs[3] = int64_t(reinterpret_cast<intptr_t>(p.st_lo));
  ptrs[4] = int64_t(reinterpret_cast<intptr_t>(p.z));
  return p.n_split;
}

int llh_stage_calls(void) { return ll::g_stage_calls; }

// Last int8 staging launch: n_chunks; row0/slot receive each chunk's first
// row and chunk slot; bases receive [layer, dst_k, dst_v] as integers.
int llh_last_stage(int32_t* row0, int32_t* slot, int64_t* bases) {
  const ll::StageArgs& s = ll::g_stage;
  for (int i = 0; i < s.n_chunks; ++i) {
    row0[i] = s.row0[i];
    slot[i] = s.slot[i];
  }
  bases[0] = int64_t(reinterpret_cast<intptr_t>(s.layer));
  bases[1] = int64_t(reinterpret_cast<intptr_t>(s.dst_k));
  bases[2] = int64_t(reinterpret_cast<intptr_t>(s.dst_v));
  return s.n_chunks;
}

// Last copy launch: n_chunks, n_layers and the destination row of each chunk.
int llh_last_copy(int32_t* n_layers, int32_t* dst_row0 /* [n_chunks] */) {
  const ll::CopyArgs& c = ll::g_copy;
  *n_layers = c.n_layers;
  for (int i = 0; i < c.n_chunks; ++i) dst_row0[i] = c.dst_row0[i];
  return c.n_chunks;
}

// Last copy launch, transposed-V part: returns vt; dst_slot receives the
// chunk slot of each chunk, tps the tiles per slot.
int llh_last_copy_vt(int32_t* tps, int32_t* dst_slot /* [n_chunks] */) {
  const ll::CopyArgs& c = ll::g_copy;
  *tps = c.tps;
  for (int i = 0; i < c.n_chunks; ++i) dst_slot[i] = c.dst_slot[i];
  return c.vt;
}

}  // extern "C"
