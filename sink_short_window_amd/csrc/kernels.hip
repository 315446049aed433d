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
// head.  Per 64-key tile:
//   S^T[key][q] = K Q^T      bf16 MFMA 32x32x16, A = K rows from LDS, B = the
//                            wave's Q fragment kept in registers.  Each lane
//                            owns one query and 16 keys per 32-key block, so
//                            row max / row sum are lane-local plus one swap
//                            between the two 32-lane halves.
//   online softmax in the log2 domain against a reference that the first
//   tile sets to its max and that moves only when a tile's P would leave the
//   safe fp32/bf16 range (exact: any reference gives the same softmax).
//   O^T[d][q] += V^T P^T     bf16 MFMA; B = P straight from the S^T
//                            accumulators; A = V^T: for the bf16 cache, whose
//                            V is stored transposed in 64-key tiles, a plain
//                            16-byte LDS read; for row-major V (the caller's
//                            current chunk, text K/V) the gfx950 transpose
//                            read (ds_read_b64_tr_b16).
// The two halves of the workgroup alternate between an MFMA phase and a
// softmax phase (details above attn_pp_kernel); K/V tiles reach LDS by
// direct-to-LDS buffer loads.  An int8 cache is read through a bf16 staging
// copy in the bf16 cache's layout (stage_int8_kernel, one launch per call:
// every code becomes bf16(q * s) once, not once per query tile).
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
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

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
// granules of row r XOR-swizzled by (r mod granules-per-row) so the MFMA
// operand reads of 32 consecutive rows spread over the banks.  bf16 tiles are
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
  uint32_t rs;  // row stride in bytes
  __amdgpu_buffer_rsrc_t rk, rv;

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
    constexpr int elt = 2;  // bf16
    rs = __builtin_amdgcn_readfirstlane(uint32_t(s.row_stride) * elt);
    const int64_t hoff = int64_t(head) * s.head_stride * elt;
    rk = make_rsrc(uni(static_cast<const char*>(s.k) + hoff), uint32_t(len) * rs);
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

// LDS-DMA load of rows [row_lo, row_lo + 16) of a tile (bf16 runs).
template <int D>
__device__ __forceinline__ void dma_rows(const RunCursor& c, bool v_side, __bf16* tile_base, int row_lo,
                                         int lane) {
  using S = SwzStage<D>;
  const int row0 = c.tile * kBN;
#pragma unroll
  for (int r0 = 0; r0 < 16; r0 += S::kRowsPerLoad) {
    const int row = row_lo + r0 + lane / S::kGran;
    const int pg = lane % S::kGran;
    const int lg = v_side ? v_swz_gran<D>(row, pg) : k_swz_gran<D>(row, pg);  // XOR: its own inverse
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

// One MFMA phase of a wave: S(t) = K(t) Q^T (kQK) and O += V(t-1)^T P(t-1)^T
// (kPV), as 16 + 16 MFMAs 32x32x16.  The operand reads are software
// pipelined by hand: kAhead LDS reads are in flight ahead of the MFMA that
// consumes them, and sched_barrier keeps the compiler from regrouping them
// (left alone it waits for every pair of reads before each pair of MFMAs).
// Five reads ahead measured as fast as six with fewer registers spilled.
constexpr int kAhead = 5;

template <int D, bool kQK, bool kPV, bool kVT>
__device__ __forceinline__ void mfma_phase(const char* kt, const char* vt, int k_row, int k_x,
                                           const int (&voff)[2][D / 32], const int (&vb)[4],
                                           const bf16x8 (&qf)[D / 16], const f32x16& cinit, f32x16 (&s)[2],
                                           f32x16 (&o)[D / 32], const bf16x8 (&pb)[4]) {
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
  xcd_unit(head, qtile);
  const int lane = threadIdx.x & 63;
  // wave-uniform by construction; readfirstlane lets the compiler keep the
  // group's branches and the buffer descriptors scalar
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

  // The wave's queries, raw; converted to the MFMA fragment once the first
  // K/V tiles' loads are in flight, so the two memory latencies overlap.
  // (They are issued before any LDS-DMA load, so every vmcnt wait below that
  // covers a tile also covers them.)
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
  // Running reference max in log2 units; the S accumulators start at -m_run
  // (cinit), so the MFMA output is already c*q.k - m_run.
  float m_run = 0.f;
  f32x16 cinit;
#pragma unroll
  for (int r = 0; r < 16; ++r) cinit[r] = 0.f;
  float l_run = 0.f;
  bf16x8 pb[4];  // P of the last softmaxed tile, one bf16x8 per 16-key step

  // Byte offsets of this lane's operand reads.
  // K (A of S^T): row kb*32 + r32, logical granule 2j + half, i.e. physical
  // granule (2j ^ (r32 & ~1 & mask)) | (half ^ (r32 & 1)), formed per j.
  const int k_row = r32 * S::kRowB + ((half ^ (r32 & 1)) << 4);
  const int k_x = r32 & (S::kGran - 2);
  // V (transpose reads): 16-lane group g16, lane j16 reads 4 elements of row
  // 16*step + 8*a + 4*(g16 >> 1) + (j16 >> 2) at column
  // 32*db + 16*(g16 & 1) + 4*(j16 & 3); the lane then holds V[4 keys][d].
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
  // V^T tiles (128-byte rows, see dma_vt): lane (r32, half) reads row
  // 32*db + r32 at logical granule 2*step + half, stored at granule
  // (2*step + half) ^ ((r32 >> 1) & 7).
  int vb[4];
  {
    const int f = (r32 >> 1) & 7;
#pragma unroll
    for (int step = 0; step < 4; ++step)
      vb[step] = r32 * 128 + ((((2 * step) ^ (f & 6)) | (half ^ (f & 1))) << 4);
  }

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
      if (group == 0) dma_rows<D>(ld, false, stage[j].k, 16 * wq, lane);
      else if (ld.vt) dma_vt<D>(ld, stage[j].v, wq, lane);
      else dma_rows<D>(ld, true, stage[j].v, 16 * wq, lane);
      ld.advance(a, head);
    }
    if (group == 0) {
      if (pre == 3) wait_vmcnt<2 * kLoads>();
      else if (pre == 2) wait_vmcnt<kLoads>();
      else wait_vmcnt<0>();
    }
  }
  // Q fragment with the logit scale folded in: Q' = bf16(Q * scale * log2 e),
  // so the MFMA yields scores in log2 units.
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
      if (group == 0) dma_rows<D>(ld, false, stage[(t + 3) % kPPStages].k, 16 * wq, lane);
      else if (ld.vt) dma_vt<D>(ld, stage[(t + 3) % kPPStages].v, wq, lane);
      else dma_rows<D>(ld, true, stage[(t + 3) % kPPStages].v, 16 * wq, lane);
      ld.advance(a, head);
    }
    const int valid = min(kBN, cu.len - cu.tile * kBN);
    cu.advance(a, head);
    if (valid < kBN) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= valid) s[kb][r] = -INFINITY;
        }
    }
    // Scores are relative to the reference m_run (cinit).  The first tile
    // sets the reference to its max.  Later tiles skip the max: P = 2^s is
    // formed and summed first, and only a tile whose sum leaves the safe range
    // (a score more than ~2^60 above the reference, or an overflow to inf)
    // takes the slow path that raises the reference and redoes P.  Any
    // reference gives the same softmax; the bound keeps P, the row sum and O
    // finite in fp32 and bf16.
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
    // Move the reference up by sh (all lanes; sh = 0 leaves a lane as is).
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
#pragma unroll
      for (int r = 0; r < 16; ++r) cinit[r] = -m_run;
    };
    // P = 2^s as bf16 pairs (one 32-bit word each) for the PV operand; the
    // row sum adds exactly these rounded values, two per dot2.  s is kept.
    auto form_p = [&]() {
      float ls[2] = {0.f, 0.f};
#pragma unroll
      for (int step = 0; step < 4; ++step) {
        u32x4 pw;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x2 f = {__builtin_amdgcn_exp2f(s[step >> 1][8 * (step & 1) + 2 * i]),
                           __builtin_amdgcn_exp2f(s[step >> 1][8 * (step & 1) + 2 * i + 1])};
          const bf16x2 b = __builtin_convertvector(f, bf16x2);
          pw[i] = __builtin_bit_cast(unsigned, b);
          ls[i & 1] = __builtin_amdgcn_fdot2_f32_bf16(b, kOnes2, ls[i & 1], false);
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
  mfma_phase<D, true, false, false>(kt(0), vt(0), k_row, k_x, voff, vb, qf, cinit, s, o, pb);
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
    mfma_phase<D, true, true, true>(kt(t), vt(t - 1), k_row, k_x, voff, vb, qf, cinit, s, o, pb);
    __builtin_amdgcn_s_setprio(0);
    after_mfma(t);
    wg_barrier();
    softmax_phase(t);
    wg_barrier();
  }
  for (int t = t1; t < n; ++t) {  // row-major V: transpose reads
    __builtin_amdgcn_s_setprio(1);
    mfma_phase<D, true, true, false>(kt(t), vt(t - 1), k_row, k_x, voff, vb, qf, cinit, s, o, pb);
    __builtin_amdgcn_s_setprio(0);
    after_mfma(t);
    wg_barrier();
    softmax_phase(t);
    wg_barrier();
  }
  __builtin_amdgcn_s_setprio(1);
  if (n - 1 < n_vt) mfma_phase<D, false, true, true>(kt(n), vt(n - 1), k_row, k_x, voff, vb, qf, cinit, s, o, pb);
  else mfma_phase<D, false, true, false>(kt(n), vt(n - 1), k_row, k_x, voff, vb, qf, cinit, s, o, pb);
  __builtin_amdgcn_s_setprio(0);
  after_mfma(n);
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

// bf16 staging of an I8 layer for the attention, one workgroup per (head,
// 64-key tile, listed chunk): every code becomes bf16(q * s) with the row's
// fp32 scale (the fma of int8x8_dequant_bf16x8), once per call instead of
// once per query tile.  K rows are written in place of the same rows of the
// staging K; V goes through LDS to the transposed tile of the chunk's slot
// (column p holds key p with bits 2 and 3 swapped; zeros past the chunk).
template <int D>
__global__ __launch_bounds__(256) void stage_int8_kernel(StageArgs a) {
  constexpr int kG = D / 8;  // 8-code groups per row
  __shared__ __attribute__((aligned(16))) __bf16 t[kBN][D + 8];
  const int h = blockIdx.x / a.tps;
  const int tile = blockIdx.x % a.tps;
  const int chunk = blockIdx.y;
  const int tid = threadIdx.x;
  const int valid = min(kBN, a.ctok - tile * kBN);
  const int64_t row_base = int64_t(h) * a.rows + a.row0[chunk] + tile * kBN;  // head-major row index
  const char* kq = a.layer + a.k_off;
  const char* vq = a.layer + a.v_off;
  const float* ks = reinterpret_cast<const float*>(a.layer + a.ks_off);
  const float* vs = reinterpret_cast<const float*>(a.layer + a.vs_off);
  __bf16* dk = reinterpret_cast<__bf16*>(a.dst_k);
#pragma unroll
  for (int it = tid; it < kBN * kG; it += 256) {
    const int key = it / kG, g = it % kG;
    u32x4 vw = {0, 0, 0, 0};
    if (key < valid) {
      const int64_t r = row_base + key;
      const uint2 kc = *reinterpret_cast<const uint2*>(kq + r * D + g * 8);
      const uint2 vc = *reinterpret_cast<const uint2*>(vq + r * D + g * 8);
      *reinterpret_cast<u32x4*>(dk + r * D + g * 8) = int8x8_dequant_bf16x8(u32x2{kc.x, kc.y}, ks[r]);
      vw = int8x8_dequant_bf16x8(u32x2{vc.x, vc.y}, vs[r]);
    }
    *reinterpret_cast<u32x4*>(&t[key][g * 8]) = vw;
  }
  __syncthreads();
  __bf16* dst = reinterpret_cast<__bf16*>(a.dst_v) + int64_t(h) * a.vt_head_elems +
                (int64_t(a.slot[chunk]) * a.tps + tile) * (kBN * D);
#pragma unroll
  for (int it = tid; it < D * (kBN / 8); it += 256) {
    const int d = it / (kBN / 8), p0 = (it % (kBN / 8)) * 8;
    bf16x8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = p0 + j;
      o[j] = t[(p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1)][d];
    }
    *reinterpret_cast<bf16x8*>(dst + d * kBN + p0) = o;
  }
}

// INT8 writer: one group of D/8 lanes per (head, row); each lane quantises
// 8 values.  s = max|x| / 127 (IEEE fp32 division), q = clamp(rne(x / s)).
__global__ __launch_bounds__(256) void quant_chunks_kernel(CopyArgs a) {
  // 32-bit indexing: the host's grid covers ctok * H groups, far below 2^31.
  const unsigned gl = unsigned(a.D) / 8;  // 16 or 8
  const unsigned grp = (blockIdx.x * 256u + threadIdx.x) / gl;
  const int li = int(threadIdx.x % gl);
  const bool valid = grp < unsigned(a.ctok) * unsigned(a.H);
  const int chunk = blockIdx.y >> 1;
  const int isv = blockIdx.y & 1;
  const int z = blockIdx.z;
  const int row = valid ? int(grp % unsigned(a.ctok)) : 0;
  const int h = valid ? int(grp / unsigned(a.ctok)) : 0;
  float x[8];
  if (valid) {
    const __bf16* src = static_cast<const __bf16*>(isv ? a.src_v : a.src_k) + int64_t(z) * a.src_layer_elems +
                        (int64_t(chunk) * a.ctok + row) * a.H * a.D + int64_t(h) * a.D + li * 8;
    const uint4 w = *reinterpret_cast<const uint4*>(src);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __builtin_bit_cast(float, ww[i] << 16);
      x[2 * i + 1] = __builtin_bit_cast(float, ww[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  for (int m = 1; m < int(gl); m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  if (!valid) return;
  const float s = amax / 127.0f;
  uint32_t packed[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int qv = 0;
    if (s != 0.f) qv = int(fminf(fmaxf(rintf(x[i] / s), -127.f), 127.f));
    packed[i >> 2] |= uint32_t(qv & 0xff) << (8 * (i & 3));
  }
  char* base = a.dst + int64_t(z) * a.dst_layer_bytes;
  const int64_t r = int64_t(h) * a.rows + a.dst_row0[chunk] + row;
  *reinterpret_cast<uint2*>(base + (isv ? a.v_off : a.k_off) + r * a.D + li * 8) = make_uint2(packed[0], packed[1]);
  if (li == 0) reinterpret_cast<float*>(base + (isv ? a.vs_off : a.ks_off))[r] = s;
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
    const int64_t threads = int64_t(a.ctok) * a.H * (a.D / 8);
    const dim3 grid(unsigned((threads + 255) / 256), a.n_chunks * 2, a.n_layers);
    return launch(quant_chunks_kernel, grid, dim3(256), &a, stream);
  }
  if (a.vt) {  // bf16 cache (the only one with transposed V)
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
