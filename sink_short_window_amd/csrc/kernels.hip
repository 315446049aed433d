// HIP kernels for gfx950 (MI355X): sink + short-window attention (also used
// for text cross-attention and the re-encoding pass of a recache), the cache
// chunk writers (append / recache, copy or int8 quantise) and the bf16
// staging of an int8 cache for the attention.
//
// Attention (LongLive: Real-time Interactive Long Video Generation, §3.3):
// one softmax over the union of the frame-sink tokens, the resident window
// chunks and the current chunk, with no mask inside the set.  The key set
// arrives as a table of runs (KvSeg) that point into the cache or into the
// caller's buffers, so nothing is concatenated.  The key loop walks the runs
// in order and each run in tiles of 64 keys (a tile never straddles runs; the
// last tile of a run is masked), so every tile is addressed by one uniform
// buffer resource plus a per-lane 32-bit offset, and rows past the run's end
// read as zero.
//
// bf16 kernel (attn_pp_kernel), per workgroup: 8 waves x 32 queries of one
// head, each wave's queries in two blocks of 16.  Per 64-key tile:
//   S^T[key][q] = K Q^T      bf16 MFMA 16x16x32, A = K rows from LDS (each
//                            read serves both query blocks), B = the wave's Q
//                            fragments kept in registers.  Each lane owns two
//                            queries and 16 of the 64 keys of each, so row
//                            max / row sum are lane-local plus two swaps.
//   online softmax in the log2 domain against a reference that the first
//   tile sets to its max and that moves only when a tile's P would leave the
//   safe fp32/bf16 range (exact: any reference gives the same softmax).
//   O^T[d][q] += V^T P^T     bf16 MFMA 16x16x32; B = P straight from the S^T
//                            accumulators; A = V^T: for the bf16 cache, whose
//                            V is stored transposed in 64-key tiles, a plain
//                            16-byte LDS read; for row-major V (the caller's
//                            current chunk, text K/V) the gfx950 transpose
//                            read (ds_read_b64_tr_b16).
// The 16x16x32 shape moves half the accumulator data per flop of the
// 32x32x16 one; under the chip's power limit that buys more MFMA throughput.
// The two halves of the workgroup alternate between an MFMA phase and a
// softmax phase (details above attn_pp_kernel); K/V tiles reach LDS by
// direct-to-LDS buffer loads.  An int8 cache is read either through a bf16
// staging copy in the bf16 cache's layout (stage_int8_kernel, one launch per
// call: every code becomes bf16(q * s) once, not once per query tile), or by
// attn_i8_kernel, which converts the codes to bf16 on chip and applies the
// scales to the scores and to P (details above it).
// fp32 activations use a plainer kernel with the fp32 MFMA 32x32x2.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "launch.hpp"

namespace ll {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x8 __attribute__((__vector_size__(8 * sizeof(float))));
typedef float f32x2 __attribute__((__vector_size__(2 * sizeof(float))));
typedef unsigned int u32x4 __attribute__((__vector_size__(4 * sizeof(unsigned))));
typedef unsigned int u32x2 __attribute__((__vector_size__(2 * sizeof(unsigned))));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // queries per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;   // fp32 kernel: rescale when the max grows by more than 2^8
// bf16 kernel: a tile's sum of P above this (some score more than ~2^60
// above the reference, or inf) makes the softmax raise its reference.
constexpr float kTileSumLimit = 0x1p60f;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr bf16x8 kOnes8 = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                           (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

// Value held by lane l^32 (the other half of the wave, which owns the same
// query column), via v_permlane32_swap: with operands (x, x) the first result
// holds, in lanes 32..63, lanes 0..31 of x and the second result holds, in
// lanes 0..31, lanes 32..63 of x.  Picking "second" in the low half and
// "first" in the high half gives the partner's value whether or not both
// operands share a register.
__device__ __forceinline__ float partner_half(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  const unsigned lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  return __builtin_bit_cast(float, lane < 32 ? p[1] : p[0]);
}
// Value held by lane l^16, via v_permlane16_swap: with operands (x, x) the
// first result holds, in every lane, the value of the lane with bit 4 clear
// and the second the value of the lane with bit 4 set.
__device__ __forceinline__ float partner_row(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  const unsigned lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  return __builtin_bit_cast(float, (lane & 16) ? p[0] : p[1]);
}
__device__ __forceinline__ float swap_halves_max(float x) { return fmaxf(x, partner_half(x)); }
__device__ __forceinline__ float swap_halves_sum(float x) { return x + partner_half(x); }

// gfx950 LDS transpose read of 4 bf16.  Within each group of 16 lanes, lane
// i receives element (i & 3) of the 8 bytes addressed by lane 4*e + (i >> 2),
// for e = 0..3.
__device__ __forceinline__ bf16x4 tr_read(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// Walks the tiles of the key runs in order.
struct TileCursor {
  int run;   // current run
  int tile;  // tile index inside the run
  __device__ void advance(const AttnArgs& a) {
    ++tile;
    if (tile * kBN >= a.seg[run].len) {
      ++run;
      tile = 0;
    }
  }
};

__device__ __forceinline__ int count_tiles(const AttnArgs& a, int n_seg) {
  int n = 0;
  for (int r = 0; r < n_seg; ++r) n += (a.seg[r].len + kBN - 1) / kBN;
  return n;
}

// Queries [q0, q_end) of query tile `qtile` (tile height bm) and the number of
// leading runs they attend.  With chunk-causal queries, chunk r of q_chunk
// tokens is cut into q_tiles tiles and attends runs [0, n_seg0 + r).
struct QueryTile {
  int q0, q_end, n_seg;
};
__device__ __forceinline__ QueryTile query_tile(const AttnArgs& a, int qtile, int bm) {
  if (a.q_chunk == 0) return {qtile * bm, a.n_q, a.n_seg};
  const int r = qtile / a.q_tiles;
  return {r * a.q_chunk + (qtile - r * a.q_tiles) * bm, (r + 1) * a.q_chunk, a.n_seg0 + r};
}

// ---------------------------------------------------------------------------
// bf16 activations
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// bf16 ping-pong kernel: 8 waves per workgroup in two groups of 4 (wave i and
// wave i+4 share a SIMD), each wave owning 32 queries of one head, 256 queries
// per workgroup.  Per key tile t a group runs
//   M(t): S(t) = K(t) Q^T and O += V(t-1) P(t-1)^T   (MFMA phase)
//   V(t): online softmax of S(t) -> P(t)             (VALU phase)
// separated by workgroup barriers, with group B one barrier interval behind
// group A: while one wave of a SIMD issues MFMAs the other runs its softmax.
//
// K/V tiles live in a 4-stage LDS ring, rows unpadded, with the 16-byte
// granules of each row XOR-swizzled by a function of the row so that the
// rows one MFMA operand read touches spread over the banks.  bf16 tiles are
// loaded straight from memory into LDS (buffer_load ... lds): at the start of
// its softmax phase t group A loads K(t+3) and group B V(t+3), three tiles
// ahead.
// ---------------------------------------------------------------------------
constexpr int kPPWaves = 8;
constexpr int kPPThreads = 64 * kPPWaves;
constexpr int kPPBM = 32 * kPPWaves;  // queries per workgroup
constexpr int kPPStages = 4;

template <int D>
struct SwzStage {
  static constexpr int kRowB = D * 2;                // bytes per row
  static constexpr int kGran = kRowB / 16;           // 16-byte granules per row
  static constexpr int kRowsPerLoad = 1024 / kRowB;  // rows one 64-lane 16-byte load covers
  __bf16 k[kBN * D];
  __bf16 v[kBN * D];
};

// Byte offset of logical granule g of row r inside a swizzled tile.  The two
// operands are read differently, so they get different swizzles (both
// measured bank-conflict-free on gfx950): K rows are read 16 bytes per lane
// down 32 consecutive rows (XOR the granule with r mod G); V rows are read by
// ds_read_b64_tr_b16, 4 rows x 32 bytes per 16 lanes (XOR with 2 (r mod G/2)).
template <int D>
__device__ __forceinline__ int k_swz_gran(int r, int g) {
  return g ^ (r & (SwzStage<D>::kGran - 1));
}
template <int D>
__device__ __forceinline__ int v_swz_gran(int r, int g) {
  return g ^ ((r & (SwzStage<D>::kGran / 2 - 1)) << 1);
}
template <int D>
__device__ __forceinline__ int k_swz(int r, int g) {
  return r * SwzStage<D>::kRowB + (k_swz_gran<D>(r, g) << 4);
}
template <int D>
__device__ __forceinline__ int v_swz(int r, int g) {
  return r * SwzStage<D>::kRowB + (v_swz_gran<D>(r, g) << 4);
}

// Swizzles of the bf16 kernel's tiles, whose operands are read for the MFMA
// 16x16x32 (granule g of row r is stored at g ^ mask(r)).  K: the 16 rows
// that one 16-lane group reads together differ in bits 0-2 and 4 of the row
// (see mfma_phase16); their masks are distinct (D = 128: 16 granules per
// row) or distinct per row parity (D = 64: two rows per bank line).  V, read
// by ds_read_b64_tr_b16: the 8 rows that 32 lanes read together differ in
// bits 0-2 and get distinct masks on the granule pair.  Neither mask looks
// at bits 3 and 5, which the key blocks and key steps add.
template <int D>
__device__ __forceinline__ int k16_mask(int r) {
  static_assert(D == 64 || D == 128, "head dim");
  if constexpr (D == 128) return (r & 7) | (((r >> 4) & 1) << 3);
  else return ((r >> 1) & 3) | (((r >> 4) & 1) << 2);
}
template <int D>
__device__ __forceinline__ int v16_mask(int r) {
  static_assert(D == 64 || D == 128, "head dim");
  if constexpr (D == 128) return (r & 7) << 1;
  else return ((r >> 1) & 3) << 1;
}

// Workgroup barrier that waits only for this wave's LDS operations; global
// and LDS-DMA loads stay in flight (callers wait for them explicitly).
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// s_waitcnt vmcnt(N) (N <= 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 15, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
  __asm__ __volatile__("" ::: "memory");
}

// Walks the 64-key tiles of the key runs, keeping the current run's buffer
// resources (for one head) in scalar registers; the run table is read only
// when the run changes.
struct RunCursor {
  int run;
  int tile;
  int len;
  int vt;       // V of this run in transposed 64-key tiles
  int i8;       // int8 codes with per-key scales (rks, rvs)
  uint32_t rs;  // row stride in bytes
  __amdgpu_buffer_rsrc_t rk, rv, rks, rvs;

  // Every field is uniform across the workgroup; readfirstlane says so to the
  // compiler, which keeps the descriptors in scalar registers (a descriptor
  // it believed divergent would turn each buffer load into a loop).
  static __device__ __forceinline__ const char* uni(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    return reinterpret_cast<const char*>((uint64_t(hi) << 32) | lo);
  }
  __device__ void open(const AttnArgs& a, int head, int r) {
    r = __builtin_amdgcn_readfirstlane(r);
    run = r;
    tile = 0;
    if (r >= a.n_seg) return;
    const KvSeg& s = a.seg[r];
    len = __builtin_amdgcn_readfirstlane(s.len);
    i8 = __builtin_amdgcn_readfirstlane(s.i8);
    const int elt = i8 ? 1 : 2;  // int8 codes or bf16
    rs = __builtin_amdgcn_readfirstlane(uint32_t(s.row_stride) * elt);
    const int64_t hoff = int64_t(head) * s.head_stride * elt;
    rk = make_rsrc(uni(static_cast<const char*>(s.k) + hoff), uint32_t(len) * rs);
    if (i8) {
      const int64_t soff = int64_t(head) * s.s_head_stride;
      rks = make_rsrc(uni(s.ks + soff), uint32_t(len) * 4);
      rvs = make_rsrc(uni(s.vs + soff), uint32_t(len) * 4);
    }
    vt = __builtin_amdgcn_readfirstlane(s.v_tiled);
    if (vt) {
      // whole zero-padded tiles; a tile is 64 rows of the cache's K row size
      const uint32_t tiles = uint32_t(len + kBN - 1) / kBN;
      rv = make_rsrc(uni(static_cast<const char*>(s.v) + int64_t(head) * s.v_head_stride * elt), tiles * kBN * rs);
    } else {
      rv = make_rsrc(uni(static_cast<const char*>(s.v) + hoff), uint32_t(len) * rs);
    }
  }
  __device__ void advance(const AttnArgs& a, int head) {
    ++tile;
    if (tile * kBN >= len) open(a, head, run + 1);
  }
};

// LDS-DMA load of rows [row_lo, row_lo + 16) of a tile (bf16 runs), in the
// swizzle of the kernel that reads it: kMfma16 for the bf16 kernel's
// 16x16x32 operand reads (k16_mask / v16_mask), else the int8 kernel's.
template <int D, bool kMfma16 = false>
__device__ __forceinline__ void dma_rows(const RunCursor& c, bool v_side, __bf16* tile_base, int row_lo,
                                         int lane) {
  using S = SwzStage<D>;
  const int row0 = c.tile * kBN;
#pragma unroll
  for (int r0 = 0; r0 < 16; r0 += S::kRowsPerLoad) {
    const int row = row_lo + r0 + lane / S::kGran;
    const int pg = lane % S::kGran;
    // XOR swizzles are their own inverse
    const int lg = kMfma16 ? pg ^ (v_side ? v16_mask<D>(row) : k16_mask<D>(row))
                           : (v_side ? v_swz_gran<D>(row, pg) : k_swz_gran<D>(row, pg));
    // row stride is a multiple of the (power-of-two) row size, so OR-ing in
    // the granule offset is exact and keeps the address a 32-bit value
    const uint32_t voff = (uint32_t(row0 + row) * c.rs) | (uint32_t(lg) << 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(v_side ? c.rv : c.rk,
                                             (__attribute__((address_space(3))) void*)(tile_base + (row_lo + r0) * D),
                                             16, voff, 0, 0, 0);
  }
}

// LDS-DMA load of this wave's quarter of a transposed V tile ([D][64] bf16,
// 128-byte rows).  LDS granule g of row d holds logical granule
// g ^ ((d >> 1) & 7), which keeps the PV operand reads (32 rows, one granule
// each per 16 lanes) free of bank conflicts.
template <int D>
__device__ __forceinline__ void dma_vt(const RunCursor& c, __bf16* tile_base, int wq, int lane) {
  constexpr int kPer = D / 32;  // 1 KB loads per wave: D rows x 128 B over 4 waves
  const uint32_t tile0 = uint32_t(c.tile) * uint32_t(kBN * D * 2);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int ins = wq * kPer + i;
    const int d = ins * 8 + (lane >> 3);
    const int lg = (lane & 7) ^ ((d >> 1) & 7);
    const uint32_t voff = tile0 + uint32_t(d * 128 + lg * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        c.rv, (__attribute__((address_space(3))) void*)(reinterpret_cast<char*>(tile_base) + ins * 1024), 16, voff,
        0, 0, 0);
  }
}

// 8 int8 codes q (two words) -> 8 bf16 of q * s.  Each byte is read as the
// unsigned u = q + 128 (sign bit flipped), so (u - 128) * s is one fma.
__device__ __forceinline__ u32x4 int8x8_dequant_bf16x8(u32x2 w, float s) {
  const float ms = -128.f * s;  // exact: a power-of-two multiple
  u32x4 o;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t u = w[h] ^ 0x80808080u;
    const f32x2 lo = {fmaf(float(u & 0xff), s, ms), fmaf(float((u >> 8) & 0xff), s, ms)};
    const f32x2 hi = {fmaf(float((u >> 16) & 0xff), s, ms), fmaf(float(u >> 24), s, ms)};
    o[2 * h] = __builtin_bit_cast(unsigned, __builtin_convertvector(lo, bf16x2));
    o[2 * h + 1] = __builtin_bit_cast(unsigned, __builtin_convertvector(hi, bf16x2));
  }
  return o;
}

// Workgroups are dispatched to the 8 XCDs round-robin by linear id, and each
// XCD has its own L2.  Give XCD x a contiguous range of (head, query-tile)
// units, head-major, so the query tiles that share a head's K/V run on the
// same XCD at the same time and fetch each K/V tile from memory once.
constexpr int kXcds = 8;
__device__ __forceinline__ void xcd_unit(int& head, int& qtile) {
  const int nq = gridDim.x;
  const int total = nq * gridDim.y;
  const int lin = blockIdx.y * nq + blockIdx.x;
  const int xcd = lin % kXcds;
  const int slot = lin / kXcds;
  const int per = total / kXcds, extra = total % kXcds;  // XCDs < extra get per + 1
  const int unit = xcd * per + min(xcd, extra) + slot;
  head = unit / nq;
  qtile = unit % nq;
}

// Chunk-causal query tiles (the re-encoding call): the tiles of window chunk
// r attend one chunk more than those of chunk r-1, so their work grows with
// r.  The workgroups are numbered chunk-major, latest chunk first, head-major
// inside a chunk, and keep the hardware's round-robin dealing of linear ids
// to the XCDs: every XCD then gets the same mix of sizes and starts its
// largest units first, so no CU runs two of the largest back to back while
// others idle.  (The K/V of a head are then read on every XCD, which the
// prefetch three tiles ahead hides; the call stays MFMA-bound.)
__device__ __forceinline__ void chunk_major_unit(const AttnArgs& a, int& head, int& qtile) {
  const int lin = blockIdx.y * gridDim.x + blockIdx.x;
  const int per_chunk = gridDim.y * a.q_tiles;  // heads x query tiles of one chunk
  const int n_chunks = gridDim.x / a.q_tiles;
  const int rem = lin % per_chunk;
  head = rem / a.q_tiles;
  qtile = (n_chunks - 1 - lin / per_chunk) * a.q_tiles + rem % a.q_tiles;
}

// One MFMA phase of a wave of the int8 kernel: S(t) = K(t) Q^T (kQK) and
// O += V(t-1)^T P(t-1)^T (kPV), as 16 + 16 MFMAs 32x32x16 (the bf16 kernel's
// 16x16x32 phase, mfma_phase16, is built the same way).  The operand reads
// are software pipelined by hand: kAhead LDS reads are in flight ahead of the
// MFMA that consumes them, and sched_barrier keeps the compiler from
// regrouping them (left alone it waits for every pair of reads before each
// pair of MFMAs).
// Five reads ahead measured as fast as six with fewer registers spilled.
constexpr int kAhead = 5;

struct NoExtra {
  __device__ __forceinline__ void operator()(int) const {}
};

// extra(i) runs right after MFMA i is issued: other work of the same wave
// (the int8 kernel's tile conversion) placed in the shadow of the MFMAs.
template <int D, bool kQK, bool kPV, bool kVT, typename Extra = NoExtra>
__device__ __forceinline__ void mfma_phase(const char* kt, const char* vt, int k_row, int k_x,
                                           const int (&voff)[2][D / 32], const int (&vb)[4],
                                           const bf16x8 (&qf)[D / 16], const f32x16& cinit, f32x16 (&s)[2],
                                           f32x16 (&o)[D / 32], const bf16x8 (&pb)[4],
                                           const Extra& extra = Extra()) {
  using S = SwzStage<D>;
  constexpr int NK = kQK ? D / 8 : 0;          // K operand reads / QK MFMAs
  constexpr int NV = kPV ? 4 * (D / 32) : 0;   // V^T operand reads / PV MFMAs
  constexpr int N = NK + NV;
  static_assert(N >= kAhead, "phase shorter than the read-ahead");
  // operand i: K rows (j = i/2, 32-key block kb = i%2), then V^T for the
  // 16-key step and 32-dim block of the PV MFMA
  auto rd = [&](int i) -> bf16x8 {
    if (i < NK) {
      const int j = i >> 1, kb = i & 1;
      return *reinterpret_cast<const bf16x8*>(kt + k_row + (((2 * j) ^ k_x) << 4) + kb * 32 * S::kRowB);
    }
    const int ii = i - NK;
    const int step = ii / (D / 32), db = ii % (D / 32);
    if constexpr (kVT) {  // transposed tile: one 16-byte read of row 32*db + r32
      return *reinterpret_cast<const bf16x8*>(vt + vb[step] + db * 32 * 128);
    } else {
      const char* base = vt + 16 * step * S::kRowB;
      const bf16x4 lo = tr_read(reinterpret_cast<const __bf16*>(base + voff[0][db]));
      const bf16x4 hi = tr_read(reinterpret_cast<const __bf16*>(base + voff[1][db]));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  bf16x8 rb[kAhead];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) rb[i] = rd(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    if (i < NK) {
      const int j = i >> 1, kb = i & 1;
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rb[i % kAhead], qf[j], j == 0 ? cinit : s[kb], 0, 0, 0);
    } else {
      const int ii = i - NK;
      const int step = ii / (D / 32), db = ii % (D / 32);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rb[i % kAhead], pb[step], o[db], 0, 0, 0);
    }
    extra(i);
    if (i + kAhead < N) rb[i % kAhead] = rd(i + kAhead);
  }
  __builtin_amdgcn_sched_barrier(0);
}

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

// One MFMA phase of a wave of the bf16 kernel: S(t) = K(t) Q'^T (kQK) and
// O += V(t-1)^T P(t-1)^T (kPV) as MFMA 16x16x32 bf16, two per operand read:
// the wave's two 16-query blocks share every K and V^T operand.  Operand i:
// K (d-step kd = i/4, key block kb = i%4), then V^T (key step ks, 16-dim
// block db).  A-row 4m + i of key block kb is the key
//   32 (kb >> 1) + 16 (m >> 1) + 8 (kb & 1) + 4 (m & 1) + i,
// so lane group g holds, in the S^T accumulators of blocks 2ks and 2ks + 1,
// the keys 32 ks + swap23(8g + j), j = 0..7 (swap23 exchanges bits 2 and 3):
// the keys of granule g of key step ks in a cached V^T tile, whose column p
// holds key swap23(p).  That is the B operand of the PV MFMA as it stands.
template <int D, bool kQK, bool kPV, bool kVT>
__device__ __forceinline__ void mfma_phase16(const char* kt, const char* vt, const int (&koff)[D / 32],
                                             const int (&voff)[D / 16], const int (&vb)[2],
                                             const bf16x8 (&qf)[2][D / 32], const f32x4 (&cinit)[2],
                                             f32x4 (&s)[2][4], f32x4 (&o)[2][D / 16], const bf16x8 (&pb)[2][2]) {
  constexpr int kRowB = D * 2;
  constexpr int NK = kQK ? 4 * (D / 32) : 0;
  constexpr int NV = kPV ? 2 * (D / 16) : 0;
  constexpr int N = NK + NV;
  static_assert(N >= kAhead, "phase shorter than the read-ahead");
  auto rd = [&](int i) -> bf16x8 {
    if (i < NK) {
      const int kd = i >> 2, kb = i & 3;
      return *reinterpret_cast<const bf16x8*>(kt + koff[kd] + (32 * (kb >> 1) + 8 * (kb & 1)) * kRowB);
    }
    const int ii = i - NK;
    const int ks = ii / (D / 16), db = ii % (D / 16);
    if constexpr (kVT) {  // transposed tile: one 16-byte read of row 16 db + lane % 16
      return *reinterpret_cast<const bf16x8*>(vt + vb[ks] + db * 16 * 128);
    } else {  // row-major: the lane's keys 0..3 and 4..7 (8 rows apart), by two transpose reads
      const char* base = vt + 32 * ks * kRowB + voff[db];
      const bf16x4 lo = tr_read(reinterpret_cast<const __bf16*>(base));
      const bf16x4 hi = tr_read(reinterpret_cast<const __bf16*>(base + 8 * kRowB));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  bf16x8 rb[kAhead];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) rb[i] = rd(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    if (i < NK) {
      const int kd = i >> 2, kb = i & 3;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        s[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rb[i % kAhead], qf[qb][kd],
                                                            kd == 0 ? cinit[qb] : s[qb][kb], 0, 0, 0);
    } else {
      const int ii = i - NK;
      const int ks = ii / (D / 16), db = ii % (D / 16);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rb[i % kAhead], pb[qb][ks], o[qb][db], 0, 0, 0);
    }
    if (i + kAhead < N) rb[i % kAhead] = rd(i + kAhead);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, bool kOneRun>
__global__ __launch_bounds__(kPPThreads) void attn_pp_kernel(AttnArgs a) {
  using S = SwzStage<D>;
  constexpr int kLoads = 16 / S::kRowsPerLoad;  // DMA loads per wave per tile side
  __shared__ __attribute__((aligned(16))) S stage[kPPStages];

  int head, qtile;
  if (a.q_chunk == 0) xcd_unit(head, qtile);
  else chunk_major_unit(a, head, qtile);
  const int lane = threadIdx.x & 63;
  // wave-uniform by construction; readfirstlane lets the compiler keep the
  // group's branches and the buffer descriptors scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = wave >> 2;
  const int wq = wave & 3;
  // MFMA 16x16x32 lane roles: r16 = lane % 16 is the query column of each
  // 16-query block, g = lane / 16 the 8-wide slice of the contraction and the
  // 4-row slice of the result.
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const QueryTile qt = query_tile(a, qtile, kPPBM);
  const int n_seg = __builtin_amdgcn_readfirstlane(qt.n_seg);
  // A wave whose 32 queries all lie past the tile's end (the ragged last
  // query tile of a head) skips its MFMAs and softmax arithmetic, but still
  // loads its share of every K/V tile and meets every wait and barrier: the
  // power it does not draw goes to the other waves' clock.
  const bool idle = __builtin_amdgcn_readfirstlane(qt.q0 + wave * 32) >= qt.q_end;
  int qi[2];
  bool q_ok[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    qi[qb] = qt.q0 + wave * 32 + qb * 16 + r16;
    q_ok[qb] = qi[qb] < qt.q_end;
  }
  const float c = a.scale * kLog2e;

  // The lane's slices of its two queries, raw; converted to the MFMA
  // fragment once the first K/V tiles' loads are in flight, so the two
  // memory latencies overlap.  (They are issued before any LDS-DMA load, so
  // every vmcnt wait below that covers a tile also covers them.)
  u32x4 qw[2][D / 32];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const u32x4* q = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(a.q) +
                                                    (int64_t(qi[qb]) * a.H + head) * D);
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd) qw[qb][kd] = q_ok[qb] ? q[4 * kd + g] : u32x4{0, 0, 0, 0};
  }

  f32x4 o[2][D / 16];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[qb][db][r] = 0.f;
  // Running reference max per query in log2 units; the S accumulators start
  // at -m_run (cinit), so the MFMA output is already c*q.k - m_run.
  float m_run[2] = {0.f, 0.f};
  f32x4 cinit[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int r = 0; r < 4; ++r) cinit[qb][r] = 0.f;
  float l_run[2] = {0.f, 0.f};
  bf16x8 pb[2][2];  // P of the last softmaxed tile per query block and 32-key step

  // Byte offsets of this lane's operand reads.
  // K (A of S^T): key row 16 (m >> 1) + 4 (m & 1) + i, m = r16 >> 2,
  // i = r16 & 3, of block 0 (the other blocks add 8 or 32 rows, which keep
  // the mask), granule 4 kd + g.
  int koff[D / 32];
  {
    const int row = 16 * ((r16 >> 3) & 1) + 4 * ((r16 >> 2) & 1) + (r16 & 3);
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd) koff[kd] = row * S::kRowB + (((4 * kd + g) ^ k16_mask<D>(row)) << 4);
  }
  // Row-major V (transpose reads): lane r16 of group g addresses row
  // 16 (g >> 1) + 4 (g & 1) + (r16 >> 2) (+8 for the upper four keys, +32
  // per key step; neither changes the mask) at column 16 db + 4 (r16 & 3);
  // after the transpose it holds column 16 db + r16 of four consecutive rows.
  int voff[D / 16];
  {
    const int row = 16 * (g >> 1) + 4 * (g & 1) + (r16 >> 2);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const int col = 16 * db + 4 * (r16 & 3);
      voff[db] = row * S::kRowB + (((col >> 3) ^ v16_mask<D>(row)) << 4) + ((col & 7) << 1);
    }
  }
  // V^T tiles (128-byte rows, see dma_vt): row 16 db + r16, logical granule
  // 4 ks + g, stored at granule (4 ks + g) ^ ((r16 >> 1) & 7).
  int vb[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) vb[ks] = r16 * 128 + (((4 * ks + g) ^ ((r16 >> 1) & 7)) << 4);

  // Tiles in the key set; the host never launches an empty one.
  const int n = kOneRun ? (a.seg[0].len + kBN - 1) / kBN : count_tiles(a, n_seg);
  if (n == 0) return;
  // tiles of the leading runs whose V is in transposed tiles
  int n_vt = 0;
  for (int r = 0; r < n_seg && a.seg[r].v_tiled; ++r) n_vt += (a.seg[r].len + kBN - 1) / kBN;
  n_vt = __builtin_amdgcn_readfirstlane(n_vt);
  RunCursor cu;  // tile being softmaxed (masking)
  cu.open(a, head, 0);
  RunCursor ld;  // next K tile (group A) / V tile (group B) to load
  ld.open(a, head, 0);

  // Prologue: group A loads K(0..2), group B V(0..2); A waits for K(0) (B
  // waits for V(0) after its first MFMA phase).
  {
    const int pre = min(n, 3);
    for (int j = 0; j < pre; ++j) {
      if (group == 0) dma_rows<D, true>(ld, false, stage[j].k, 16 * wq, lane);
      else if (ld.vt) dma_vt<D>(ld, stage[j].v, wq, lane);
      else dma_rows<D, true>(ld, true, stage[j].v, 16 * wq, lane);
      ld.advance(a, head);
    }
    if (group == 0) {
      if (pre == 3) wait_vmcnt<2 * kLoads>();
      else if (pre == 2) wait_vmcnt<kLoads>();
      else wait_vmcnt<0>();
    }
  }
  // Q fragments with the logit scale folded in: Q' = bf16(Q * scale * log2 e),
  // so the MFMA yields scores in log2 units.
  bf16x8 qf[2][D / 32];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd) {
      f32x8 f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __builtin_bit_cast(float, qw[qb][kd][i] << 16) * c;
        f[2 * i + 1] = __builtin_bit_cast(float, qw[qb][kd][i] & 0xffff0000u) * c;
      }
      qf[qb][kd] = __builtin_convertvector(f, bf16x8);
    }
  wg_barrier();
  if (group == 1) wg_barrier();  // group B runs one interval behind

  // S^T accumulators: block kb of query block qb; element i of lane (r16, g)
  // is key 32 (kb >> 1) + 16 (g >> 1) + 8 (kb & 1) + 4 (g & 1) + i against
  // query 16 qb + r16.
  f32x4 s[2][4];

  // Each group keeps three tiles of its side (A: K, B: V) in flight, issuing
  // tile t+3 at the start of its softmax phase t.  Group B makes sure V(t)
  // has landed at the end of its MFMA phase t, before group A's MFMA phase
  // t+1 multiplies with it.  (A wave's LDS reads wait behind its own
  // outstanding LDS-DMA loads, and the compiler puts a full wait before each
  // transpose read, so loads issued any earlier would only stall the reads.)
  auto after_mfma = [&](int t) {
    if (group == 1) {
      if (t + 2 < n) wait_vmcnt<2 * kLoads>();
      else if (t + 1 < n) wait_vmcnt<kLoads>();
      else wait_vmcnt<0>();
    }
  };

  // Softmax phase t: online softmax of S(t) -> P(t).
  auto softmax_phase = [&](int t) {
    if (t + 3 < n) {  // A: K(t+3), B: V(t+3), straight into LDS
      if (group == 0) dma_rows<D, true>(ld, false, stage[(t + 3) % kPPStages].k, 16 * wq, lane);
      else if (ld.vt) dma_vt<D>(ld, stage[(t + 3) % kPPStages].v, wq, lane);
      else dma_rows<D, true>(ld, true, stage[(t + 3) % kPPStages].v, 16 * wq, lane);
      ld.advance(a, head);
    }
    const int valid = min(kBN, cu.len - cu.tile * kBN);
    cu.advance(a, head);
    if (!idle) {  // the loads and the cursor above, and group A's wait below, run in every wave
      if (valid < kBN) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = 32 * (kb >> 1) + 16 * (g >> 1) + 8 * (kb & 1) + 4 * (g & 1) + i;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              if (key >= valid) s[qb][kb][i] = -INFINITY;
          }
      }
      // Scores are relative to the reference m_run (cinit).  The first tile
      // sets the reference to its max.  Later tiles skip the max: P = 2^s is
      // formed and summed first, and only a tile whose sum leaves the safe range
      // (a score more than ~2^60 above the reference, or an overflow to inf)
      // takes the slow path that raises the reference and redoes P.  Any
      // reference gives the same softmax; the bound keeps P, the row sum and O
      // finite in fp32 and bf16.  A query's keys are spread over the four
      // lanes r16 + 16g, which reduce with two swaps.
      auto tile_max = [&](float (&mx)[2]) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          float mp[4];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) mp[kb] = fmaxf(fmaxf(s[qb][kb][0], s[qb][kb][1]), fmaxf(s[qb][kb][2], s[qb][kb][3]));
          const float m4 = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
          mx[qb] = swap_halves_max(fmaxf(m4, partner_row(m4)));
        }
      };
      // Move the reference of query block qb up by sh[qb] (sh = 0 leaves it).
      auto shift_reference = [&](const float (&sh)[2], bool rescale) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          if (rescale) {
            const float alpha = __builtin_amdgcn_exp2f(-sh[qb]);
            l_run[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < D / 16; ++db)
#pragma unroll
              for (int r = 0; r < 4; ++r) o[qb][db][r] *= alpha;
          }
          m_run[qb] += sh[qb];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) s[qb][kb][r] -= sh[qb];
#pragma unroll
          for (int r = 0; r < 4; ++r) cinit[qb][r] = -m_run[qb];
        }
      };
      // P = 2^s as bf16 pairs (one 32-bit word each) for the PV operand: key
      // step ks takes blocks 2ks (keys 0..3 of the lane's eight) and 2ks + 1
      // (keys 4..7).  s is kept.  The tile's row sums of exactly these rounded
      // values come from two MFMAs per query block with an all-ones A operand
      // (every result row is the sum over the 64 keys), not from VALU adds:
      // while the other wave of the SIMD streams MFMAs this wave gets about one
      // VALU issue per MFMA, so the softmax phase is priced in VALU
      // instructions.  Each lane then holds its queries' full tile sums.
      auto form_p = [&](float (&lt)[2]) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            u32x4 pw;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const f32x4& src = s[qb][2 * ks + (w >> 1)];
              const int i0 = 2 * (w & 1);
              const f32x2 f = {__builtin_amdgcn_exp2f(src[i0]), __builtin_amdgcn_exp2f(src[i0 + 1])};
              pw[w] = __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
            }
            pb[qb][ks] = __builtin_bit_cast(bf16x8, pw);
          }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          f32x4 sum = {0.f, 0.f, 0.f, 0.f};
          sum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kOnes8, pb[qb][0], sum, 0, 0, 0);
          sum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kOnes8, pb[qb][1], sum, 0, 0, 0);
          lt[qb] = sum[0];
        }
      };
      if (t == 0) {
        float mx[2];
        tile_max(mx);
        shift_reference(mx, false);
      }
      float lt[2];
      form_p(lt);
      if (__builtin_amdgcn_ballot_w64(!(lt[0] <= kTileSumLimit) || !(lt[1] <= kTileSumLimit))) {
        float mx[2];
        tile_max(mx);
        mx[0] = fmaxf(mx[0], 0.f);
        mx[1] = fmaxf(mx[1], 0.f);
        shift_reference(mx, true);
        form_p(lt);
      }
      l_run[0] += lt[0];
      l_run[1] += lt[1];
    }
    // group A: K(t+1) must be in LDS before M(t+1); K(t+2), K(t+3) may fly on
    if (group == 0) {
      if (t + 3 < n) wait_vmcnt<2 * kLoads>();
      else if (t + 2 < n) wait_vmcnt<kLoads>();
      else wait_vmcnt<0>();
    }
  };

  auto kt = [&](int t) { return reinterpret_cast<const char*>(stage[t % kPPStages].k); };
  auto vt = [&](int t) { return reinterpret_cast<const char*>(stage[t % kPPStages].v); };

  // Per key tile t a group runs MFMA phase t (QK of tile t, PV of tile t-1)
  // and softmax phase t, each closed by a workgroup barrier; the first and
  // last MFMA phases are peeled so the steady one is one straight-line block.
  __builtin_amdgcn_s_setprio(1);
  if (!idle) mfma_phase16<D, true, false, false>(kt(0), vt(0), koff, voff, vb, qf, cinit, s, o, pb);
  __builtin_amdgcn_s_setprio(0);
  after_mfma(0);
  wg_barrier();
  softmax_phase(0);
  wg_barrier();
  // Runs with transposed V tiles (cache runs) come before the others (the
  // caller's current chunk), so the steady loop splits in two, each with one
  // straight-line MFMA phase (one loop holding both variants spills the
  // accumulators).
  const int t1 = min(n_vt + 1, n);
  for (int t = 1; t < t1; ++t) {  // PV of tile t-1 < n_vt: transposed V
    __builtin_amdgcn_s_setprio(1);
    if (!idle) mfma_phase16<D, true, true, true>(kt(t), vt(t - 1), koff, voff, vb, qf, cinit, s, o, pb);
    __builtin_amdgcn_s_setprio(0);
    after_mfma(t);
    wg_barrier();
    softmax_phase(t);
    wg_barrier();
  }
  for (int t = t1; t < n; ++t) {  // row-major V: transpose reads
    __builtin_amdgcn_s_setprio(1);
    if (!idle) mfma_phase16<D, true, true, false>(kt(t), vt(t - 1), koff, voff, vb, qf, cinit, s, o, pb);
    __builtin_amdgcn_s_setprio(0);
    after_mfma(t);
    wg_barrier();
    softmax_phase(t);
    wg_barrier();
  }
  __builtin_amdgcn_s_setprio(1);
  if (!idle) {
    if (n - 1 < n_vt) mfma_phase16<D, false, true, true>(kt(n), vt(n - 1), koff, voff, vb, qf, cinit, s, o, pb);
    else mfma_phase16<D, false, true, false>(kt(n), vt(n - 1), koff, voff, vb, qf, cinit, s, o, pb);
  }
  __builtin_amdgcn_s_setprio(0);
  after_mfma(n);
  wg_barrier();
  wg_barrier();  // the softmax phase n does not exist; keep the two groups' barrier counts equal
  if (group == 0) wg_barrier();

  // O^T accumulators: element i of lane (r16, g) in block (qb, db) is
  // dimension 16 db + 4g + i of query 16 qb + r16.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = l_run[qb];  // already summed over the 4 lanes of the query
    if (!q_ok[qb]) continue;
    const float inv = 1.f / l_tot;
    __bf16* orow = static_cast<__bf16*>(a.out) + (int64_t(qi[qb]) * a.H + head) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const f32x4 f = o[qb][db] * inv;
      *reinterpret_cast<bf16x4*>(orow + 16 * db + 4 * g) = __builtin_convertvector(f, bf16x4);
    }
    if (a.lse && g == 0) a.lse[int64_t(head) * a.n_q + qi[qb]] = (m_run[qb] + __log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// INT8 cache, dequantised inside the attention.  The cache runs hold int8
// codes c with fp32 scales per key: K = c_k * ks, V = c_v * vs (V stored
// transposed in 64-key tiles like the bf16 cache).  Every code is an integer
// in [-127, 127], exact in bf16, so
//   S^T[key][q] = ks[key] * sum_d c_k[key][d] Q'[q][d]
//     MFMA over the exact codes, then the K scale on each score column;
//   O^T[d][q] += sum_key c_v[key][d] * (P[q][key] * vs[key])
//     the V scale folded into P before its bf16 rounding;
// and the row sum takes P itself.  The values attended are the exact q * s.
//
// Same 8-wave ping-pong as attn_pp_kernel (group A runs MFMA phase t in
// interval 2t and softmax phase t in 2t+1, group B one interval later), with
// this staging:
//   * int8 tiles (K rows and V^T, 64 * D bytes each) go straight into a
//     3-slot int8 ring (buffer_load ... lds) three tiles ahead, issued in the
//     softmax phase: group A loads the K side and both scale vectors (into a
//     4-slot scale ring), group B the V side;
//   * the conversion to bf16 runs inside MFMA phases, between the MFMAs,
//     where a wave's own VALU work hides behind its MFMAs: group A converts
//     K(t+1) in its MFMA phase t, group B converts V(t) in its MFMA phase t.
//     Each lane converts exactly the 16-byte pieces its own loads fetched,
//     so a wave only waits for its own loads (vmcnt);
//   * the caller's current chunk (bf16, row-major) goes straight into the
//     3-stage bf16 ring two tiles ahead, as in the bf16 kernel.
// Lifetimes: K(j) in bf16 stage j%3 is written in interval 2j-2 (converted)
// or loaded from 2j-3 (bf16) and read in 2j, 2j+1; V(j) is written in 2j+1
// (converted) or loaded from 2j-2 and read in 2j+2, 2j+3; int8 K(j) / V(j)
// are loaded in 2j-5 / 2j-4 and converted in 2j-2 / 2j+1; the scales of tile
// j are loaded in 2j-5 and read in 2j+1, 2j+2.  No write lands in a slot
// whose previous reader runs in the same or a later interval, and every
// interval ends with a workgroup barrier.
// ---------------------------------------------------------------------------
constexpr int kI8Stages = 3;
constexpr int kScaleStages = 4;

template <int D>
struct I8Slot {
  char k8[kBN * D];  // K rows, int8
  char v8[kBN * D];  // V^T [D][64], int8
};
struct ScaleSlot {
  float ks[kBN];
  float vs[kBN];
};

// 8 int8 codes (two words) -> 8 bf16 holding the same integers (exact).
__device__ __forceinline__ bf16x8 i8x8_bf16(uint32_t w0, uint32_t w1) {
  f32x8 f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = float(int8_t(w0 >> (8 * i)));
    f[4 + i] = float(int8_t(w1 >> (8 * i)));
  }
  return __builtin_convertvector(f, bf16x8);
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 8].
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    default: wait_vmcnt<8>(); break;
  }
}

template <int D>
__global__ __launch_bounds__(kPPThreads) void attn_i8_kernel(AttnArgs a) {
  using S = SwzStage<D>;
  constexpr int kLoads = 16 / S::kRowsPerLoad;       // bf16 loads per wave per tile side
  constexpr int kI8Loads = kBN * D / (16 * 256);     // int8 loads per wave per tile side
  static_assert(kI8Loads >= 1 && kI8Loads <= 2, "int8 tile pieces per lane");
  __shared__ __attribute__((aligned(16))) S stage[kI8Stages];
  __shared__ __attribute__((aligned(16))) I8Slot<D> ring[kI8Stages];
  __shared__ __attribute__((aligned(16))) ScaleSlot sring[kScaleStages];

  int head, qtile;
  if (a.q_chunk == 0) xcd_unit(head, qtile);
  else chunk_major_unit(a, head, qtile);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = wave >> 2;
  const int wq = wave & 3;
  const int r32 = lane & 31;
  const int half = lane >> 5;
  const QueryTile qt = query_tile(a, qtile, kPPBM);
  const int n_seg = __builtin_amdgcn_readfirstlane(qt.n_seg);
  const int qi = qt.q0 + wave * 32 + r32;
  const bool q_ok = qi < qt.q_end;
  const float c = a.scale * kLog2e;
  const int64_t qrow = (int64_t(qi) * a.H + head) * D;

  u32x4 qw[D / 16];
  {
    const u32x4* q = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(a.q) + qrow);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) qw[j] = q_ok ? q[2 * j + half] : u32x4{0, 0, 0, 0};
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  // Scores leave the MFMA raw (accumulators start at zero); the softmax
  // forms s = raw * ks - m_run (log2 units) itself.
  float m_run = 0.f;
  f32x16 zero;
#pragma unroll
  for (int r = 0; r < 16; ++r) zero[r] = 0.f;
  float l_run = 0.f;
  bf16x8 pb[4];

  const int k_row = r32 * S::kRowB + ((half ^ (r32 & 1)) << 4);
  const int k_x = r32 & (S::kGran - 2);
  const int g16 = lane >> 4, j16 = lane & 15;
  int voff[2][D / 32];
#pragma unroll
  for (int aa = 0; aa < 2; ++aa)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int row = 8 * aa + 4 * (g16 >> 1) + (j16 >> 2);
      const int col = 32 * db + 16 * (g16 & 1) + 4 * (j16 & 3);
      voff[aa][db] = v_swz<D>(row, col >> 3) + ((col & 7) << 1);
    }
  int vb[4];
  {
    const int f = (r32 >> 1) & 7;
#pragma unroll
    for (int step = 0; step < 4; ++step)
      vb[step] = r32 * 128 + ((((2 * step) ^ (f & 6)) | (half ^ (f & 1))) << 4);
  }

  const int n = count_tiles(a, n_seg);
  if (n == 0) return;
  // tiles of the leading int8 runs (the cache; the current chunk follows)
  int n8 = 0;
  for (int r = 0; r < n_seg && a.seg[r].i8; ++r) n8 += (a.seg[r].len + kBN - 1) / kBN;
  n8 = __builtin_amdgcn_readfirstlane(n8);
  RunCursor cu;  // tile being softmaxed (masking)
  cu.open(a, head, 0);
  RunCursor ld;  // next tile to load (A: its K side and the scales, B: its V side)
  ld.open(a, head, 0);

  // Loads this wave issued in its last issuing phase (c1) and the one before
  // (c2): what may still be in flight behind an older tile.
  int c1 = 0, c2 = 0;
  // Issuing phase p (softmax phase p; the prologue runs p = -3, -2, -1): the
  // int8 tile p+3, or the bf16 tile p+2, of this group's side.  kMayI8: an
  // int8 tile can be due.
  auto issue_phase = [&](int p, auto may_i8_tag) {
    constexpr bool kMayI8 = decltype(may_i8_tag)::value;
    int cnt = 0;
    if (kMayI8 && p + 3 < n8) {
      const int j = p + 3;
      char* dst = group == 0 ? ring[j % kI8Stages].k8 : ring[j % kI8Stages].v8;
      const uint32_t base = uint32_t(ld.tile) * uint32_t(kBN * D);
#pragma unroll
      for (int i = 0; i < kI8Loads; ++i) {
        const int idx = i * 256 + wq * 64;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(group == 0 ? ld.rk : ld.rv,
                                                 (__attribute__((address_space(3))) void*)(dst + idx * 16), 16,
                                                 base + uint32_t(idx + lane) * 16, 0, 0, 0);
      }
      cnt = kI8Loads;
      if (group == 0 && wq < 2) {
        float* sd = wq == 0 ? sring[j % kScaleStages].ks : sring[j % kScaleStages].vs;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wq == 0 ? ld.rks : ld.rvs,
                                                 (__attribute__((address_space(3))) void*)(sd), 4,
                                                 uint32_t(ld.tile * kBN + lane) * 4, 0, 0, 0);
        ++cnt;
      }
      ld.advance(a, head);
    } else if (p + 2 >= n8 && p + 2 < n) {
      const int j = p + 2;
      if (group == 0) dma_rows<D>(ld, false, stage[j % kI8Stages].k, 16 * wq, lane);
      else dma_rows<D>(ld, true, stage[j % kI8Stages].v, 16 * wq, lane);
      cnt = kLoads;
      ld.advance(a, head);
    }
    c2 = c1;
    c1 = cnt;
  };

  // Conversion of this group's side of int8 tile j (A: K rows into bf16
  // stage j%3 in the swizzled row layout; B: V^T rows of 64 keys, 128 bytes,
  // in the layout dma_vt gives), in pieces run between MFMAs: at i == 1 wait
  // for the wave's own loads of the tile (vmcnt(behind): loads issued after
  // them) and read its int8 pieces, then convert and store piece p at
  // i == 4 + 4p.
  struct Conv {
    u32x4 w[2];
  };
  auto conv_step = [&](int i, int j, int behind, Conv& cv) {
    const I8Slot<D>& rg = ring[j % kI8Stages];
    if (i == 1) {
      wait_vmcnt_dyn(behind);
#pragma unroll
      for (int p = 0; p < kI8Loads; ++p)
        cv.w[p] = *reinterpret_cast<const u32x4*>((group == 0 ? rg.k8 : rg.v8) + (p * 256 + wq * 64 + lane) * 16);
    }
#pragma unroll
    for (int p = 0; p < kI8Loads; ++p) {
      if (i != 4 + 4 * p) continue;
      const int o = (p * 256 + wq * 64 + lane) * 16;
      const bf16x8 lo = i8x8_bf16(cv.w[p][0], cv.w[p][1]);
      const bf16x8 hi = i8x8_bf16(cv.w[p][2], cv.w[p][3]);
      if (group == 0) {
        const int row = o / D, g = (o % D) / 8;
        char* dst = reinterpret_cast<char*>(stage[j % kI8Stages].k);
        *reinterpret_cast<bf16x8*>(dst + k_swz<D>(row, g)) = lo;
        *reinterpret_cast<bf16x8*>(dst + k_swz<D>(row, g + 1)) = hi;
      } else {
        const int d = o / kBN, g = (o % kBN) / 8;
        char* dst = reinterpret_cast<char*>(stage[j % kI8Stages].v) + d * 128;
        *reinterpret_cast<bf16x8*>(dst + ((g ^ ((d >> 1) & 7)) << 4)) = lo;
        *reinterpret_cast<bf16x8*>(dst + (((g + 1) ^ ((d >> 1) & 7)) << 4)) = hi;
      }
    }
  };
  // In MFMA phase t group A converts K(t+1) (loaded in phase t-2; phase t-1
  // issued after it), group B V(t) (loaded in phase t-3; phases t-2 and t-1
  // after it).
  auto conv_of_phase = [&](int t, int& j, int& behind) -> bool {
    j = group == 0 ? t + 1 : t;
    behind = group == 0 ? c1 : c1 + c2;
    return j < n8;
  };

  const std::true_type scaled{}, may_i8{};
  const std::false_type plain{}, bf16_only{};
  // Prologue: issuing phases -3..-1 (int8 tiles 0..2 / bf16 tiles up to 1);
  // group A converts K(0) (group B converts V(0) in its MFMA phase 0).
  issue_phase(-3, may_i8);
  issue_phase(-2, may_i8);
  issue_phase(-1, may_i8);
  if (group == 0) {
    if (n8 > 0) {
      Conv cv;
      for (int i = 1; i <= 8; ++i) conv_step(i, 0, c1 + c2, cv);
    } else {
      wait_vmcnt_dyn(c1);  // bf16 K(0)
    }
  }
  bf16x8 qf[D / 16];
#pragma unroll
  for (int j = 0; j < D / 16; ++j) {
    f32x8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __builtin_bit_cast(float, qw[j][i] << 16) * c;
      f[2 * i + 1] = __builtin_bit_cast(float, qw[j][i] & 0xffff0000u) * c;
    }
    qf[j] = __builtin_convertvector(f, bf16x8);
  }
  wg_barrier();
  if (group == 1) wg_barrier();  // group B runs one interval behind

  f32x16 s[2];

  // After MFMA phase t: group B makes sure a bf16 V(t) has landed (A's MFMA
  // phase t+1 reads it); it was loaded in phase t-2, phase t-1 after it.
  auto after_mfma = [&](int t) {
    if (group == 1 && t >= n8 && t < n) wait_vmcnt_dyn(c1);
  };

  // Softmax phase t (kScaled: tile t is int8; kMayI8: an int8 tile can be
  // due for loading): the loads of issuing phase t, then the online softmax
  // of S(t); group A then makes sure a bf16 K(t+1) has landed.
  auto softmax_phase = [&](int t, auto scaled_tag, auto may_i8_tag) {
    constexpr bool kScaled = decltype(scaled_tag)::value;
    issue_phase(t, may_i8_tag);
    const int valid = min(kBN, cu.len - cu.tile * kBN);
    cu.advance(a, head);
    const float* ksl = sring[t % kScaleStages].ks;
    const float* vsl = sring[t % kScaleStages].vs;
    if constexpr (kScaled) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 k4 = *reinterpret_cast<const float4*>(ksl + kb * 32 + 8 * i + 4 * half);
          s[kb][4 * i + 0] = fmaf(s[kb][4 * i + 0], k4.x, -m_run);
          s[kb][4 * i + 1] = fmaf(s[kb][4 * i + 1], k4.y, -m_run);
          s[kb][4 * i + 2] = fmaf(s[kb][4 * i + 2], k4.z, -m_run);
          s[kb][4 * i + 3] = fmaf(s[kb][4 * i + 3], k4.w, -m_run);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] -= m_run;
    }
    if (valid < kBN) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= valid) s[kb][r] = -INFINITY;
        }
    }
    auto tile_max = [&]() {
      float mp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) mp[i] = fmaxf(s[i >> 1][8 * (i & 1)], s[i >> 1][8 * (i & 1) + 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 2; r < 8; ++r) mp[i] = fmaxf(mp[i], s[i >> 1][8 * (i & 1) + r]);
      return swap_halves_max(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3])));
    };
    auto shift_reference = [&](float sh, bool rescale) {
      if (rescale) {
        const float alpha = __builtin_amdgcn_exp2f(-sh);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      }
      m_run += sh;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] -= sh;
    };
    // P = 2^s; the PV operand takes bf16(P * vs) (V scale folded in), the
    // row sum P itself.
    auto form_p = [&]() {
      float ls[2] = {0.f, 0.f};
#pragma unroll
      for (int step = 0; step < 4; ++step) {
        const int kb = step >> 1, r0 = 8 * (step & 1);
        float4 v4[2];
        if constexpr (kScaled) {
          v4[0] = *reinterpret_cast<const float4*>(vsl + kb * 32 + 2 * r0 + 4 * half);
          v4[1] = *reinterpret_cast<const float4*>(vsl + kb * 32 + 2 * r0 + 8 + 4 * half);
        }
        u32x4 pw;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = __builtin_amdgcn_exp2f(s[kb][r0 + 2 * i]);
          const float p1 = __builtin_amdgcn_exp2f(s[kb][r0 + 2 * i + 1]);
          ls[i & 1] += p0 + p1;
          f32x2 f = {p0, p1};
          if constexpr (kScaled) {
            const float4& vv = v4[i >> 1];
            f[0] *= (i & 1) ? vv.z : vv.x;
            f[1] *= (i & 1) ? vv.w : vv.y;
          }
          pw[i] = __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
        }
        pb[step] = __builtin_bit_cast(bf16x8, pw);
      }
      return ls[0] + ls[1];
    };
    if (t == 0) shift_reference(tile_max(), false);
    float lt = form_p();
    if (__builtin_amdgcn_ballot_w64(!(lt <= kTileSumLimit))) {
      shift_reference(fmaxf(tile_max(), 0.f), true);
      lt = form_p();
    }
    l_run += lt;
    if (group == 0 && t + 1 >= n8 && t + 1 < n) wait_vmcnt_dyn(c1);  // bf16 K(t+1)
  };

  auto kt = [&](int t) { return reinterpret_cast<const char*>(stage[t % kI8Stages].k); };
  auto vt = [&](int t) { return reinterpret_cast<const char*>(stage[t % kI8Stages].v); };

  // MFMA phase t with the conversion due in it (if any; kConv: one can be
  // due in this phase variant) between its MFMAs.
  auto run_mfma = [&](int t, auto qk_tag, auto pv_tag, auto vt_tag, auto conv_tag) {
    constexpr bool kQK = decltype(qk_tag)::value, kPV = decltype(pv_tag)::value;
    constexpr bool kVTl = decltype(vt_tag)::value, kConv = decltype(conv_tag)::value;
    int j = 0, behind = 0;
    const bool conv = kConv && conv_of_phase(t, j, behind);
    Conv cv;
    auto extra = [&](int i) {
      if (kConv && conv) conv_step(i, j, behind, cv);
    };
    __builtin_amdgcn_s_setprio(1);
    mfma_phase<D, kQK, kPV, kVTl>(kt(t), vt(t - 1), k_row, k_x, voff, vb, qf, zero, s, o, pb, extra);
    __builtin_amdgcn_s_setprio(0);
    after_mfma(t);
  };

  const std::true_type yes{};
  const std::false_type no{};
  run_mfma(0, yes, no, no, yes);
  wg_barrier();
  if (n8 > 0) softmax_phase(0, scaled, may_i8);
  else softmax_phase(0, plain, bf16_only);
  wg_barrier();
  // t < n8: QK of an int8 tile, PV of an int8 tile (transposed V);
  // t == n8: QK of the first bf16 tile, PV of the last int8 tile;
  // t > n8: bf16 tiles, row-major V (transpose reads).
  const int t1 = min(n8, n);
  for (int t = 1; t < t1; ++t) {
    run_mfma(t, yes, yes, yes, yes);
    wg_barrier();
    softmax_phase(t, scaled, may_i8);
    wg_barrier();
  }
  if (n8 >= 1 && n8 < n) {
    const int t = n8;
    run_mfma(t, yes, yes, yes, no);
    wg_barrier();
    softmax_phase(t, plain, bf16_only);
    wg_barrier();
  }
  for (int t = max(n8 + 1, 1); t < n; ++t) {
    run_mfma(t, yes, yes, no, no);
    wg_barrier();
    softmax_phase(t, plain, bf16_only);
    wg_barrier();
  }
  if (n - 1 < n8) run_mfma(n, no, yes, yes, no);
  else run_mfma(n, no, yes, no, no);
  wg_barrier();
  wg_barrier();  // the softmax phase n does not exist; keep the two groups' barrier counts equal
  if (group == 0) wg_barrier();

  const float l_tot = swap_halves_sum(l_run);
  if (!q_ok) return;
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d0 = db * 32 + 8 * gq + 4 * half;
      float4 f = make_float4(o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv, o[db][4 * gq + 2] * inv,
                             o[db][4 * gq + 3] * inv);
      const bf16x4 b = __builtin_convertvector(*reinterpret_cast<float __attribute__((__vector_size__(16)))*>(&f), bf16x4);
      *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.out) + qrow + d0) = b;
    }
  if (a.lse && half == 0) a.lse[int64_t(head) * a.n_q + qi] = (m_run + __log2f(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------
// fp32 activations: same run/tile walk and online softmax, fp32 MFMA 32x32x2,
// single LDS stage (small correctness-first shapes).
// ---------------------------------------------------------------------------
template <int D>
struct F32Stage {
  static constexpr int KS = D + 4;
  float k[kBN * KS];
  float v[kBN * KS];
};

template <int D>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(AttnArgs a) {
  using S = F32Stage<D>;
  __shared__ __attribute__((aligned(16))) S st;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31;
  const int half = lane >> 5;
  const QueryTile qt = query_tile(a, blockIdx.x, kBM);
  const int qi = qt.q0 + wave * 32 + r32;
  const bool q_ok = qi < qt.q_end;
  const float c = a.scale * kLog2e;
  const int64_t qrow = (int64_t(qi) * a.H + head) * D;

  float qf[D / 2];
  {
    const float* q = static_cast<const float*>(a.q) + qrow;
#pragma unroll
    for (int j = 0; j < D / 2; ++j) qf[j] = q_ok ? q[2 * j + half] : 0.f;
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  constexpr int kVec = D / 4;
  constexpr int kItems = kBN * kVec / kThreads;
  const int n_tiles = count_tiles(a, qt.n_seg);
  TileCursor cu{0, 0};
  for (int g = 0; g < n_tiles; ++g) {
    const KvSeg& sg = a.seg[cu.run];
    const int row0 = cu.tile * kBN;
    const int valid = min(kBN, sg.len - row0);
    {
      const uint32_t rs = uint32_t(sg.row_stride) * 4;
      const auto rk = make_rsrc(static_cast<const float*>(sg.k) + int64_t(head) * sg.head_stride, uint32_t(sg.len) * rs);
      const auto rv = make_rsrc(static_cast<const float*>(sg.v) + int64_t(head) * sg.head_stride, uint32_t(sg.len) * rs);
#pragma unroll
      for (int it = 0; it < kItems; ++it) {
        const int item = tid + it * kThreads;
        const int row = item / kVec, vec = item % kVec;
        const uint32_t off = uint32_t(row0 + row) * rs + vec * 16;
        *reinterpret_cast<u32x4*>(&st.k[row * S::KS + vec * 4]) = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
        *reinterpret_cast<u32x4*>(&st.v[row * S::KS + vec * 4]) = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
      }
    }
    cu.advance(a);
    __syncthreads();

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int j = 0; j < D / 2; ++j)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(st.k[(kb * 32 + r32) * S::KS + 2 * j + half], qf[j], s[kb], 0, 0, 0);
    if (valid < kBN) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= valid) s[kb][r] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = swap_halves_max(mx);
    const float m_new = fmaxf(m_run, mx);
    if (__builtin_amdgcn_ballot_w64((m_new - m_run) * c > kRescaleLog2)) {
      const float alpha = exp2f((m_run - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run * c;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(fmaf(s[kb][r], c, -mc));
        l_run += p;
        s[kb][r] = p;
      }
    // O^T[d][q] += V^T P^T with k = the half's key for accumulator r.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(st.v[key * S::KS + db * 32 + r32], s[kb][r], o[db], 0, 0, 0);
      }
    __syncthreads();
  }
  const float l_tot = swap_halves_sum(l_run);
  if (!q_ok) return;
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d0 = db * 32 + 8 * gq + 4 * half;
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + qrow + d0) =
          make_float4(o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv, o[db][4 * gq + 2] * inv, o[db][4 * gq + 3] * inv);
    }
  if (a.lse && half == 0) a.lse[int64_t(head) * a.n_q + qi] = (m_run * c + __log2f(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------
// Cache writers (append / recache of whole chunks).
// ---------------------------------------------------------------------------

// fp32 cache (K and V row-major).  Grid: x over (head, row, 16-byte vector)
// of one chunk, y = chunk * 2 + (0: K, 1: V), z = layer.  Destination rows
// are contiguous per head (coalesced writes); each source row is one
// contiguous D-vector.
__global__ __launch_bounds__(256) void copy_chunks_kernel(CopyArgs a) {
  constexpr int kElt = 4;  // fp32
  // 32-bit indexing: the host bounds ctok * H * D by 2^30.
  const unsigned vpr = unsigned(a.D) * kElt / 16;  // 32 or 16
  const unsigned e = blockIdx.x * 256u + threadIdx.x;
  if (e >= unsigned(a.ctok) * unsigned(a.H) * vpr) return;
  const int chunk = blockIdx.y >> 1;
  const int isv = blockIdx.y & 1;
  const int z = blockIdx.z;
  const int vec = int(e % vpr);
  const unsigned rh = e / vpr;
  const int row = int(rh % unsigned(a.ctok));
  const int h = int(rh / unsigned(a.ctok));
  const char* src = static_cast<const char*>(isv ? a.src_v : a.src_k) +
                    (int64_t(z) * a.src_layer_elems + (int64_t(chunk) * a.ctok + row) * a.H * a.D +
                     int64_t(h) * a.D) * kElt + vec * 16;
  char* dst = a.dst + int64_t(z) * a.dst_layer_bytes + (isv ? a.v_off : a.k_off) +
              ((int64_t(h) * a.rows + a.dst_row0[chunk] + row) * a.D) * kElt + vec * 16;
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

// bf16 cache, K rows and transposed V tiles in one launch.  Grid: x over
// (head, 64-key tile) of one chunk, y = chunk * 2 + (0: K, 1: V), z = layer.
// A K block copies the tile's rows into the head-major cache rows (16 KB
// contiguous for D = 128).  A V block stages the tile key-major in LDS and
// writes it as [D][64] into the chunk slot's tile, physical column p holding
// key p with bits 2 and 3 swapped (the key order of the PV operand); keys
// past the chunk's end are written as zeros.
template <int D>
__global__ __launch_bounds__(256) void append_bf16_kernel(CopyArgs a) {
  constexpr int kG = D / 8;  // 16-byte granules per key row
  __shared__ __attribute__((aligned(16))) __bf16 t[kBN][D + 8];
  const int h = blockIdx.x / a.tps;
  const int tile = blockIdx.x % a.tps;
  const int chunk = blockIdx.y >> 1;
  const bool isv = blockIdx.y & 1;
  const int z = blockIdx.z;
  const int tid = threadIdx.x;
  const __bf16* src = static_cast<const __bf16*>(isv ? a.src_v : a.src_k) + int64_t(z) * a.src_layer_elems +
                      int64_t(chunk) * a.ctok * a.H * D + int64_t(h) * D;
  constexpr int kPer = kBN * kG / 256;  // 16-byte loads per thread
  // all loads of the thread first, then the stores
  uint4 w[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int it = tid + 256 * i;
    const int row = tile * kBN + it / kG, g = it % kG;
    w[i] = row < a.ctok ? *reinterpret_cast<const uint4*>(src + int64_t(row) * a.H * D + g * 8)
                        : make_uint4(0, 0, 0, 0);
  }
  if (!isv) {
    __bf16* dst = reinterpret_cast<__bf16*>(a.dst + int64_t(z) * a.dst_layer_bytes + a.k_off) +
                  (int64_t(h) * a.rows + a.dst_row0[chunk]) * D;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int it = tid + 256 * i;
      const int row = tile * kBN + it / kG, g = it % kG;
      if (row < a.ctok) *reinterpret_cast<uint4*>(dst + int64_t(row) * D + g * 8) = w[i];
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int it = tid + 256 * i;
    *reinterpret_cast<uint4*>(&t[it / kG][(it % kG) * 8]) = w[i];
  }
  __syncthreads();
  __bf16* dst = reinterpret_cast<__bf16*>(a.dst + int64_t(z) * a.dst_layer_bytes + a.v_off) +
                int64_t(h) * a.vt_head_elems + (int64_t(a.dst_slot[chunk]) * a.tps + tile) * (kBN * D);
#pragma unroll
  for (int it = tid; it < D * (kBN / 8); it += 256) {
    const int d = it / (kBN / 8), p0 = (it % (kBN / 8)) * 8;
    bf16x8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = p0 + j;
      const int key = (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
      o[j] = t[key][d];
    }
    *reinterpret_cast<bf16x8*>(dst + d * kBN + p0) = o;
  }
}

// bf16 staging of an I8 layer (the attention's default INT8 mode, the backward
// and the linear-attention variant), one workgroup per (head, 64-key tile,
// listed chunk): every code becomes bf16(q * s) with its key's fp32 scale.  K
// rows are written in place of the same rows of the staging K; the V tile
// ([D][64], column p holding key p with bits 2 and 3 swapped) goes to the same
// tile of the staging V, zeros past the chunk.
template <int D>
__global__ __launch_bounds__(256) void stage_int8_kernel(StageArgs a) {
  constexpr int kG = D / 8;                   // 8-code groups per row
  constexpr int kKPer = kBN * kG / 256;       // K groups per thread
  constexpr int kVPer = D * (kBN / 8) / 256;  // V^T groups (8 columns of one dim) per thread
  const int h = blockIdx.x / a.tps;
  const int tile = blockIdx.x % a.tps;
  const int chunk = blockIdx.y;
  const int tid = threadIdx.x;
  const int valid = min(kBN, a.ctok - tile * kBN);
  const int64_t row_base = int64_t(h) * a.rows + a.row0[chunk] + tile * kBN;  // head-major row index
  const char* kq = a.layer + a.k_off;
  const float* ks = reinterpret_cast<const float*>(a.layer + a.ks_off);
  const float* vs = reinterpret_cast<const float*>(a.layer + a.vs_off);
  const int64_t vt_off = int64_t(h) * a.vt_head_elems + (int64_t(a.slot[chunk]) * a.tps + tile) * (kBN * D);
  const char* vq = a.layer + a.v_off + vt_off;
  // All loads first (keys past the chunk read the last valid key, in bounds,
  // and are dropped), so their latencies overlap.  Column p of the V tile
  // holds key p with bits 2 and 3 swapped; its scale goes to LDS in column
  // order, zero past the chunk (the padding codes are 0 too).
  const int pcol = tid & (kBN - 1);
  const int pkey = (pcol & ~12) | ((pcol & 4) << 1) | ((pcol & 8) >> 1);
  const float vsl = vs[row_base + min(pkey, valid - 1)];
  uint2 kc[kKPer];
  float ksl[kKPer];
#pragma unroll
  for (int i = 0; i < kKPer; ++i) {
    const int it = tid + 256 * i;
    const int64_t r = row_base + min(it / kG, valid - 1);
    kc[i] = *reinterpret_cast<const uint2*>(kq + r * D + (it % kG) * 8);
    ksl[i] = ks[r];
  }
  uint2 vc[kVPer];
#pragma unroll
  for (int i = 0; i < kVPer; ++i) {
    const int it = tid + 256 * i;
    vc[i] = *reinterpret_cast<const uint2*>(vq + (it / (kBN / 8)) * kBN + (it % (kBN / 8)) * 8);
  }
  __shared__ float vsc[kBN];
  if (tid < kBN) vsc[tid] = pkey < valid ? vsl : 0.f;
  __bf16* dk = reinterpret_cast<__bf16*>(a.dst_k);
#pragma unroll
  for (int i = 0; i < kKPer; ++i) {
    const int it = tid + 256 * i;
    const int key = it / kG;
    if (key < valid)
      *reinterpret_cast<u32x4*>(dk + (row_base + key) * D + (it % kG) * 8) =
          int8x8_dequant_bf16x8(u32x2{kc[i].x, kc[i].y}, ksl[i]);
  }
  __syncthreads();
  __bf16* dv = reinterpret_cast<__bf16*>(a.dst_v) + vt_off;
#pragma unroll
  for (int i = 0; i < kVPer; ++i) {
    const int it = tid + 256 * i;
    const int d = it / (kBN / 8), p0 = (it % (kBN / 8)) * 8;
    const uint32_t wv[2] = {vc[i].x, vc[i].y};
    bf16x8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      o[j] = (__bf16)(float(int8_t(wv[j >> 2] >> (8 * (j & 3)))) * vsc[p0 + j]);
    *reinterpret_cast<bf16x8*>(dv + d * kBN + p0) = o;
  }
}

// Max over aligned groups of G = 8 or 16 lanes (one DPP row or half-row), in
// every lane of the group: quad swaps (xor 1, xor 2), then the half-row mirror
// (lane i <-> 7 - i) and, for 16, the row mirror (i <-> 15 - i).
template <int G>
__device__ __forceinline__ float group_max(float v) {
  static_assert(G == 8 || G == 16, "group of 8 or 16 lanes");
  auto dpp = [](float x, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), decltype(ctrl)::value,
                                                                 0xf, 0xf, false));
  };
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0xB1>{}));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x4E>{}));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x141>{}));  // row_half_mirror
  if constexpr (G == 16) v = fmaxf(v, dpp(v, std::integral_constant<int, 0x140>{}));  // row_mirror
  return v;
}

// The 8 codes of one lane, q = clamp(rne(fl32(x / s)), -127, 127), bit-identical
// to the IEEE division.  For s > 0, r = x * rcp(s) (rcp within 1 ulp) lies
// within 127.5 * 1.5 * 2^-23 + 2^-18 < 3e-5 of fl32(x / s) (|x / s| <= 127.5),
// so rne(r) is the code unless r is within that distance of a half-integer,
// i.e. |r - rne(r)| > 0.5 - 1e-4 (or r is not finite, from a subnormal s).
// Such codes are rare (about 2e-4 of them); if any lane of the wave has one,
// the flagged codes take the division itself, so the common path costs a
// multiply, a rounding and a compare per code.  s == 0 (an all-zero vector)
// gives r = 0, q = 0.
__device__ __forceinline__ u32x2 quant_codes8(const float (&x)[8], float s) {
  constexpr float kNearHalf = 0.5f - 1e-4f;
  const float inv = s != 0.f ? __builtin_amdgcn_rcpf(s) : 0.f;
  float q[8];
  uint64_t tie = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float r = x[e] * inv;
    q[e] = rintf(r);
    tie |= __builtin_amdgcn_ballot_w64(!(fabsf(r - q[e]) < kNearHalf));
  }
  if (tie != 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float r = x[e] * inv;
      if (!(fabsf(r - q[e]) < kNearHalf)) q[e] = rintf(x[e] / s);
    }
  }
  u32x2 packed = {0, 0};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = int(fminf(fmaxf(q[e], -127.f), 127.f));
    packed[e >> 2] |= uint32_t(c & 0xff) << (8 * (e & 3));
  }
  return packed;
}

// INT8 writer, one workgroup per (head, 64-token tile, chunk, K or V): each
// token's D values of the head are quantised with s = max|x| / 127 (IEEE fp32
// division) and q = clamp(rne(x / s), -127, 127) (s = 0, q = 0 for an
// all-zero vector).  Thread groups of D/8 lanes hold one token (8 values per
// lane), so max|x| is a reduction over those lanes.  K codes go to the cache
// rows ([H][rows][D]); V codes are staged in LDS and written as the chunk
// slot's transposed tile ([D][64], physical column p holding key p with bits
// 2 and 3 swapped, zeros after the chunk's last key).  Scales go to the
// [H][rows] fp32 arrays at the token's row.
template <int D>
__global__ __launch_bounds__(256) void quant_tile_kernel(CopyArgs a) {
  constexpr int kG = D / 8;             // lanes per token
  constexpr int kPer = kBN * kG / 256;  // tokens' groups per thread
  constexpr int kRowW = D / 4 + 1;      // staged code row in words (odd: conflict-free column reads)
  __shared__ uint32_t c8[kBN * kRowW];
  const int h = blockIdx.x / a.tps;
  const int tile = blockIdx.x % a.tps;
  const int chunk = blockIdx.y >> 1;
  const bool isv = blockIdx.y & 1;
  const int z = blockIdx.z;
  const int tid = threadIdx.x;
  const __bf16* src = static_cast<const __bf16*>(isv ? a.src_v : a.src_k) + int64_t(z) * a.src_layer_elems +
                      int64_t(chunk) * a.ctok * a.H * D + int64_t(h) * D;
  char* layer = a.dst + int64_t(z) * a.dst_layer_bytes;
  float* scales = reinterpret_cast<float*>(layer + (isv ? a.vs_off : a.ks_off));
  const int64_t row_base = int64_t(h) * a.rows + a.dst_row0[chunk] + tile * kBN;  // head-major row
  const int valid = min(kBN, a.ctok - tile * kBN);
  // Every load is issued before any is used: keys past the chunk read the
  // last valid key (in bounds) and are zeroed afterwards, so no load sits in
  // a branch of its own with a wait behind it.
  uint4 w[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int it = tid + 256 * i;
    const int key = it / kG, g = it % kG;
    w[i] = *reinterpret_cast<const uint4*>(src + int64_t(tile * kBN + min(key, valid - 1)) * a.H * D + g * 8);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of any use
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if ((tid + 256 * i) / kG >= valid) w[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int it = tid + 256 * i;
    const int key = it / kG, g = it % kG;
    const uint32_t ww[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __builtin_bit_cast(float, ww[e] << 16);
      x[2 * e + 1] = __builtin_bit_cast(float, ww[e] & 0xffff0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
    amax = group_max<kG>(amax);
    const float sc = amax / 127.0f;
    const u32x2 packed = quant_codes8(x, sc);
    if (key < valid) {
      if (g == 0) scales[row_base + key] = sc;
      if (!isv) *reinterpret_cast<uint2*>(layer + a.k_off + (row_base + key) * D + g * 8) = make_uint2(packed[0], packed[1]);
    }
    if (isv) {  // zeros past the chunk
      c8[key * kRowW + 2 * g] = packed[0];
      c8[key * kRowW + 2 * g + 1] = packed[1];
    }
  }
  if (!isv) return;
  __syncthreads();
  // [D][64] tile: thread (4 dims, 8 columns) reads one word (4 dims) of each
  // of its 8 keys and transposes the 8 x 4 bytes into 4 rows of 8 columns.
  char* dst = layer + a.v_off + int64_t(h) * a.vt_head_elems + (int64_t(a.dst_slot[chunk]) * a.tps + tile) * (kBN * D);
  if (tid < D / 4 * 8) {
    const int d4 = tid / 8, p0 = (tid % 8) * 8;
    uint32_t in[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = p0 + j;
      const int key = (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
      in[j] = c8[key * kRowW + d4];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // byte i of in[0..3] -> word lo, of in[4..7] -> word hi
      const uint32_t s01 = __builtin_amdgcn_perm(in[1], in[0], 0x0c0c0400u + 0x0101u * i);
      const uint32_t s23 = __builtin_amdgcn_perm(in[3], in[2], 0x04000c0cu + 0x01010000u * i);
      const uint32_t s45 = __builtin_amdgcn_perm(in[5], in[4], 0x0c0c0400u + 0x0101u * i);
      const uint32_t s67 = __builtin_amdgcn_perm(in[7], in[6], 0x04000c0cu + 0x01010000u * i);
      *reinterpret_cast<uint2*>(dst + (4 * d4 + i) * kBN + p0) = make_uint2(s01 | s23, s45 | s67);
    }
  }
}

template <typename K>
int launch(K kernel, dim3 grid, dim3 block, const void* arg, void* stream) {
  void* args[] = {const_cast<void*>(arg)};
  return int(hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0,
                             static_cast<hipStream_t>(stream)));
}

// Query tiles per head for tile height bm; fills in q_tiles for chunk-causal
// queries (the host checks that q_chunk divides n_q).
int query_tiles(AttnArgs& a, int bm) {
  if (a.q_chunk == 0) return (a.n_q + bm - 1) / bm;
  a.q_tiles = (a.q_chunk + bm - 1) / bm;
  return a.n_q / a.q_chunk * a.q_tiles;
}

template <int D>
int launch_attention_d(const AttnArgs& args, void* stream) {
  AttnArgs a = args;
  if (a.act == LL_F32) {
    const dim3 grid(query_tiles(a, kBM), a.H);
    return launch(attn_f32_kernel<D>, grid, dim3(kThreads), &a, stream);
  }
  const dim3 grid(query_tiles(a, kPPBM), a.H);
  const dim3 block(kPPThreads);
  if (a.seg[0].i8) return launch(attn_i8_kernel<D>, grid, block, &a, stream);
  if (a.n_seg == 1) return launch(attn_pp_kernel<D, true>, grid, block, &a, stream);
  return launch(attn_pp_kernel<D, false>, grid, block, &a, stream);
}

}  // namespace

int launch_attention(const AttnArgs& a, void* stream) {
  if (a.n_q <= 0) return 0;
  return a.D == 64 ? launch_attention_d<64>(a, stream) : launch_attention_d<128>(a, stream);
}

int launch_copy_chunks(const CopyArgs& a, void* stream) {
  if (a.n_chunks <= 0) return 0;
  if (a.kv == LL_I8) {
    const dim3 grid(unsigned(a.H * a.tps), a.n_chunks * 2, a.n_layers);
    return a.D == 64 ? launch(quant_tile_kernel<64>, grid, dim3(256), &a, stream)
                     : launch(quant_tile_kernel<128>, grid, dim3(256), &a, stream);
  }
  if (a.vt) {  // bf16 cache
    const dim3 grid(unsigned(a.H * a.tps), a.n_chunks * 2, a.n_layers);
    return a.D == 64 ? launch(append_bf16_kernel<64>, grid, dim3(256), &a, stream)
                     : launch(append_bf16_kernel<128>, grid, dim3(256), &a, stream);
  }
  // fp32 cache (fp32 activations)
  const int64_t threads = int64_t(a.ctok) * a.H * (a.D * 4 / 16);
  const dim3 grid(unsigned((threads + 255) / 256), a.n_chunks * 2, a.n_layers);
  return launch(copy_chunks_kernel, grid, dim3(256), &a, stream);
}

int launch_stage_int8(const StageArgs& a, void* stream) {
  if (a.n_chunks <= 0) return 0;
  const dim3 grid(unsigned(a.H * a.tps), a.n_chunks);
  return a.D == 64 ? launch(stage_int8_kernel<64>, grid, dim3(256), &a, stream)
                   : launch(stage_int8_kernel<128>, grid, dim3(256), &a, stream);
}

const char* hip_error_string(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

}  // namespace ll
