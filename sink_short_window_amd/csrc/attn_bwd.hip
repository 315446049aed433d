// HIP kernels for gfx950 (MI355X): backward of the sink + short-window
// attention call for the training step.
//
// LongLive: Real-time Interactive Long Video Generation, §3.2 (streaming long
// tuning: frames generated earlier are detached, gradients flow through the
// current clip only) and §3.3 (training keeps the last W frames' K/V without
// gradient, the current clip's K/V with gradient, and the sink tokens
// concatenated to every layer).  The call's key set is the forward's run table
// (sink and window runs from the cache, then the caller's current chunk); only
// the last run, the current chunk, receives dK/dV.
//
// With P = softmax(S), S = scale q.k over the runs, O = P V and upstream dO:
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - delta),  delta = rowsum(dO O),
//   dQ = scale dS K,  dK = scale dS^T Q.
// Three kernels on the stream:
//   bwd_delta_kernel  delta[h][i] = dO_i . O_i (fp32); when dK/dV are asked
//                     for, also Q' (below) as bf16 into the first half of dq.
//   bwd_dkv_kernel    per 256 keys of the current chunk (8 waves x 32):
//                     loop over 64-query tiles; S = Q' K^T, dP = dO V^T (K/V
//                     fragments in registers, starting from -lse2 and
//                     -delta of each query), then dV^T += dO^T P and
//                     dK^T += Q'^T dS with dO^T and Q'^T from transpose reads.
//                     The Q' and dO tiles stream straight into a 3-stage LDS
//                     ring (LDS-DMA), two tiles ahead.
//   bwd_dq_kernel     per 256 queries of one head (8 waves x 32): walk every
//                     64-key tile of every run; S^T = K Q'^T and dP^T = V dO^T
//                     (K/V rows from LDS, Q' and dO in registers), starting
//                     from -lse2 and -delta, P = 2^(S^T) from the forward's
//                     log-sum-exp, dS^T in fp32 rounded to bf16, then
//                     dQ^T += K^T dS^T with K^T from gfx950 transpose reads.
//                     The K/V tiles stream straight into a 2-stage LDS ring
//                     (LDS-DMA), one tile ahead.  It runs last: it
//                     overwrites the Q' copy in dq.
// Both MFMA kernels use bf16 MFMA 16x16x32 with two 16-row blocks per wave
// sharing every LDS operand read; the accumulators of the two 16-row blocks
// of a 32-row step pack into the B operand of the next product, and the
// transpose reads that form its A operand take rows in that same order.
// Q' = bf16(Q * scale * log2 e) exactly as the forward kernel forms it, so P is
// recomputed from the same rounded scores the forward normalised.  Gradients
// are written in fp32 (token-major [n][H][D]).
//
// Tiles sit in LDS in layouts (RowTile, VtTile) whose XOR swizzles or skewed
// padding spread the 16-byte row reads and the transpose reads over the LDS
// banks (conflict-free in the dQ kernel; the dK/dV kernel's padded tile
// leaves its transpose reads one 2-way conflict).  In the dQ kernel the cache's V stays transposed ([D][64]
// per 64 keys, as the bf16 cache stores it) and its rows are read back with
// transpose reads; the caller's row-major current chunk is read as rows.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <type_traits>

#include "launch.hpp"

namespace ll {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x8 __attribute__((__vector_size__(8 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef unsigned int u32x4 __attribute__((__vector_size__(4 * sizeof(unsigned))));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kBwdThreads = 512;  // 8 waves
// Waves of 32 queries per dq workgroup.  (Four, i.e. two workgroups per CU
// whose waves are not barrier-locked to each other, measured 4% slower for
// the whole backward: each workgroup streams every K/V tile, so the LDS-DMA
// traffic per flop doubles.)
constexpr int kBwdDqWaves = 8;
constexpr int kBwdBK = 256;       // current-chunk keys per dk/dv workgroup (8 waves x 32)
constexpr int kTile = 64;         // keys (dq) or queries (dk/dv) per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

// gfx950 LDS transpose read of 4 bf16: within each group of 16 lanes, lane i
// receives element (i & 3) of the 8 bytes addressed by lane 4*e + (i >> 2),
// for e = 0..3.
__device__ __forceinline__ bf16x4 tr_read(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

__device__ __forceinline__ float bf_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// 8 bf16 (one 16-byte word) times c, rounded to bf16.
__device__ __forceinline__ bf16x8 scale_bf16x8(u32x4 w, float c) {
  f32x8 f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf_lo(w[i]) * c;
    f[2 * i + 1] = bf_hi(w[i]) * c;
  }
  return __builtin_convertvector(f, bf16x8);
}

// Column p of a transposed V tile of the cache holds key p with bits 2 and 3
// swapped (the involution the forward kernel's PV operand order asks for);
// the dQ kernel's transpose-read offsets undo it.

// Row-major [kTile][D] bf16 LDS tile (K, Q' or dO), read both as rows
// (16-byte reads: per 16 lanes, 16 consecutive rows at one granule) and by
// transpose reads (8-byte reads: 16 lanes read 4 consecutive rows 4 j .. at
// two adjacent granules, j being the lane group).  For D = 128 rows are 256
// bytes (all 64 banks) and granule g of row r is stored at g ^ swz(r), with
// swz(r) = (a << 1) | ((b ^ c) << 3) | c for a = r & 3, b = (r >> 2) & 1,
// c = (r >> 3) & 1: swz is a bijection on r mod 16, so the row reads cover 16
// distinct granules; and swz(r) >> 1 is a bijection on the 8 rows of any two
// lane groups served together (rows 0..7 or 8..15, and rows {0..3, 8..11} or
// {4..7, 12..15}), so the transpose reads' granule pairs {x, x ^ 1} are
// disjoint however the hardware pairs the groups.
// For D = 64, and in the dK/dV kernel (whose register allocation holds with
// it), rows are padded by 64 bytes and skewed: granule g of row r is stored
// at granule g + skew(r), skew(r) = (b << 1) | c.  Rows r and r + 4 start on
// the same bank (a row is 80 or 48 banks) and their skews differ by two
// granules, so the transpose reads of lane groups j and j + 1 do not overlap
// (those of groups j and j + 2, rows r and r + 8, overlap by one granule if
// the hardware serves them together); the four skews of a 16-row block are
// distinct, so the row reads do not overlap either.
template <int D, bool kPadded = false>
struct RowTile {
  static constexpr bool kSwz = !kPadded && D == 128;
  static constexpr int RB = kSwz ? D * 2 : (D + 32) * 2;
  static constexpr int kBytes = kTile * RB;
  static __device__ __forceinline__ int swz(int row) {
    return ((row & 3) << 1) | ((((row >> 2) ^ (row >> 3)) & 1) << 3) | ((row >> 3) & 1);
  }
  static __device__ __forceinline__ int skew(int row) { return (((row >> 2) & 1) << 1) | ((row >> 3) & 1); }
  static __device__ __forceinline__ int off(int row, int gran) {
    if constexpr (kSwz) return row * RB + ((gran ^ swz(row)) << 4);
    else return row * RB + ((gran + skew(row)) << 4);
  }
};

// Transposed [D][64] bf16 V tile of the dQ kernel, read by transpose reads
// only (16 lanes read rows d = 8 j + {0..3} at two adjacent granules, j being
// the lane group).  Rows are 128 bytes, so rows of one parity share 32
// banks; granule g of row d is stored at g ^ swz(d), swz(d) =
// (((d >> 1) & 1) << 2) | ((((d >> 3) ^ (d >> 4)) & 1) << 1), which gives the
// four same-parity rows of any two lane groups served together distinct
// granule pairs.
template <int D>
struct VtTile {
  static constexpr int RB = kTile * 2;
  static constexpr int kBytes = D * RB;
  static __device__ __forceinline__ int swz(int d) { return (((d >> 1) & 1) << 2) | ((((d >> 3) ^ (d >> 4)) & 1) << 1); }
  static __device__ __forceinline__ int off(int d, int gran) { return d * RB + ((gran ^ swz(d)) << 4); }
};

// The A operand of an MFMA 16x16x32 (8 bf16 per lane) from two transpose
// reads, at `lo` and `hi_off` bytes further on.
__device__ __forceinline__ bf16x8 tr_pair(const char* lo, int hi_off) {
  return __builtin_shufflevector(tr_read(lo), tr_read(lo + hi_off), 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------
// delta[h][i] = sum_d dO[i][h][d] * O[i][h][d]; and, when the dK/dV kernel
// runs, Q' = bf16(Q * scale * log2 e) ([n_q][H][D] bf16) in the first half of
// dq, which that kernel streams into LDS as it is.  The dQ kernel runs last
// and overwrites dq.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(AttnBwdArgs p) {
  constexpr int kLanes = D / 8;  // lanes per (query, head) row, 8 elements each
  const int64_t rows = int64_t(p.a.n_q) * p.a.H;
  const int64_t row = (int64_t(blockIdx.x) * 256 + threadIdx.x) / kLanes;
  const int part = threadIdx.x % kLanes;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 o = reinterpret_cast<const u32x4*>(p.out)[row * kLanes + part];
    const u32x4 g = reinterpret_cast<const u32x4*>(p.dout)[row * kLanes + part];
    if (p.dk) {
      const u32x4 q = reinterpret_cast<const u32x4*>(p.a.q)[row * kLanes + part];
      reinterpret_cast<bf16x8*>(p.dq)[row * kLanes + part] = scale_bf16x8(q, p.a.scale * kLog2e);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += bf_lo(o[i]) * bf_lo(g[i]) + bf_hi(o[i]) * bf_hi(g[i]);
  }
#pragma unroll
  for (int m = kLanes / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, kLanes);
  if (row < rows && part == 0) {
    const int qi = int(row / p.a.H), h = int(row % p.a.H);
    p.delta[int64_t(h) * p.a.n_q + qi] = acc;
  }
}

// Workgroups are dispatched to the 8 XCDs round-robin by linear id, and each
// XCD has its own L2: XCD x gets a contiguous, head-major range of (head,
// tile) units, so the workgroups that share a head's K/V (dQ) or Q/dO (dK/dV)
// run on the same XCD.
constexpr int kXcds = 8;
__device__ __forceinline__ void xcd_unit(int& head, int& tile) {
  const int nt = gridDim.x;
  const int total = nt * gridDim.y;
  const int lin = blockIdx.y * nt + blockIdx.x;
  const int xcd = lin % kXcds;
  const int slot = lin / kXcds;
  const int per = total / kXcds, extra = total % kXcds;
  const int unit = xcd * per + min(xcd, extra) + slot;
  head = unit / nt;
  tile = unit % nt;
}

// s_waitcnt vmcnt(N) (N <= 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 15, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
  __asm__ __volatile__("" ::: "memory");
}

// Workgroup barrier that waits only for this wave's LDS operations; LDS-DMA
// loads stay in flight (their waits are explicit).
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// Stage of the dQ kernel's LDS ring: one K tile (RowTile rows) and one V tile,
// either a transposed [D][64] tile (cache runs) or row-major rows in the K
// tile's layout (the caller's current chunk).
template <int D>
struct DqStage {
  static constexpr int kVBytes =
      RowTile<D>::kBytes > VtTile<D>::kBytes ? RowTile<D>::kBytes : VtTile<D>::kBytes;
  char k[RowTile<D>::kBytes];
  char v[kVBytes];
};

// LDS-DMA load `ins` (1 KB: 64 lanes x 16 bytes) of a RowTile: slot
// s = 64 ins + lane is LDS row s / G, slot s % G, which holds granule
// slot ^ swz(row) (XOR layout, an involution) or slot - skew(row) (padded
// layout; padding slots take a duplicate in-row granule and are never read)
// of tile row `row`, i.e. source row row0 + row at byte stride rs.  Rows
// past the buffer range load as zeros.
template <int D, typename T>
__device__ __forceinline__ void dma_rowtile(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t rs, uint32_t row0, int ins,
                                            int lane) {
  constexpr int G = T::RB / 16;
  const int s = ins * 64 + lane;
  const int row = s / G, sg = s % G;
  int gran;
  if constexpr (T::kSwz) gran = sg ^ T::swz(row);
  else gran = min(max(sg - T::skew(row), 0), D / 8 - 1);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds + ins * 1024), 16,
                                           (row0 + uint32_t(row)) * rs + uint32_t(gran) * 16, 0, 0, 0);
}

// LDS-DMA load `ins` of a transposed [D][64] V tile stored at byte offset
// `tile` of the buffer: slot s is row d = s / 8, slot s % 8, holding granule
// slot ^ swz(d) (VtTile's layout, an involution).
template <int D>
__device__ __forceinline__ void dma_vttile(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t tile, int ins, int lane) {
  const int s = ins * 64 + lane;
  const int d = s >> 3, sg = s & 7;
  const int gran = sg ^ VtTile<D>::swz(d);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds + ins * 1024), 16,
                                           tile + uint32_t(d) * 128 + uint32_t(gran) * 16, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
// W waves of 32 queries each.  Tiles reach LDS by LDS-DMA into a two-stage
// ring, one tile ahead: the first W/2 waves load the K tile, the others the V
// tile.  Each stage is its own __shared__ variable and the loops are unrolled
// by two, so the compiler can tell the stage being filled from the stage
// being read and inserts no wait for the fill before the reads.
template <int D, int W>
__global__ __launch_bounds__(64 * W, 8 / W) void bwd_dq_kernel(AttnBwdArgs p) {
  using KT = RowTile<D>;
  using VT = VtTile<D>;
  constexpr int BQ = 32 * W;           // queries per workgroup
  constexpr int HW = W / 2;            // waves per tile side
  constexpr int NKL = (KT::RB / 16) / HW;  // 1 KB loads per wave: K tile, or row-major V rows
  constexpr int NVL = (D / 8) / HW;        // 1 KB loads per wave: transposed V tile
  static_assert((KT::RB / 16) % HW == 0 && (D / 8) % HW == 0, "tile loads split evenly over the waves");
  __shared__ __attribute__((aligned(16))) DqStage<D> st0;
  __shared__ __attribute__((aligned(16))) DqStage<D> st1;
  const AttnArgs& a = p.a;
  int head, qtile;
  xcd_unit(head, qtile);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // MFMA 16x16x32 lane roles: r16 = lane % 16 is the query column of each
  // 16-query block (and the row of an A operand), g = lane / 16 the 8-wide
  // slice of the contraction and the 4-row slice of the result.
  const int r16 = lane & 15, g = lane >> 4;
  const float c = a.scale * kLog2e;

  // B operands: Q' and dO of query 16 qb + r16 of the wave's 32, d = 32 ks + 8 g .. +7.
  int qi[2];
  bool q_ok[2];
  bf16x8 qf[2][D / 32], dof[2][D / 32];
  float lse2[2], dl[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    qi[qb] = qtile * BQ + wave * 32 + 16 * qb + r16;
    q_ok[qb] = qi[qb] < a.n_q;
    const int64_t qrow = (int64_t(qi[qb]) * a.H + head) * D;
    const u32x4* q = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(a.q) + qrow);
    const u32x4* gp = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(p.dout) + qrow);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const u32x4 wq = q_ok[qb] ? q[4 * ks + g] : u32x4{0, 0, 0, 0};
      const u32x4 wg = q_ok[qb] ? gp[4 * ks + g] : u32x4{0, 0, 0, 0};
      qf[qb][ks] = scale_bf16x8(wq, c);
      dof[qb][ks] = __builtin_bit_cast(bf16x8, wg);
    }
    // log2-domain log-sum-exp; +inf for padding queries makes their P exactly 0
    lse2[qb] = q_ok[qb] ? p.lse[int64_t(head) * a.n_q + qi[qb]] * kLog2e : INFINITY;
    dl[qb] = q_ok[qb] ? p.delta[int64_t(head) * a.n_q + qi[qb]] : 0.f;
  }

  f32x4 sinit[2], dinit[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sinit[qb][r] = -lse2[qb];
      dinit[qb][r] = -dl[qb];
    }

  // dQ^T accumulators: element i of lane (r16, g) in block (db, qb) is
  // dimension 16 db + 4 g + i of query 16 qb + r16.
  f32x4 dq[D / 16][2];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dq[db][qb][r] = 0.f;
  // Byte offsets of this lane's LDS operand reads.  Both tile layouts depend
  // on the row mod 16 only, so the key block (16 rows), the upper half of a
  // key step (16 rows) and the key step (32 rows) are plain offsets.
  //  * K rows (A of S^T) and row-major V rows (A of dP^T): key 16 kb + r16,
  //    granule 4 ks + g.
  int koff[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) koff[ks] = KT::off(r16, 4 * ks + g);
  //  * K^T (A of dQ^T) by two transpose reads: the address lane (e = r16 >> 2,
  //    m = r16 & 3) of group g points at key row 4 g + e (+16 for the second
  //    read) at dimensions 16 db + 4 m .. +3, so lane r16 receives dimension
  //    16 db + r16 of keys 4 g .. 4 g + 3 (and 16 + 4 g .. 16 + 4 g + 3): the
  //    key order in which the S^T accumulators of the step's two key blocks
  //    pack into the dS^T operand.
  int ktoff[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    const int col = 16 * db + 4 * (r16 & 3);
    ktoff[db] = KT::off(4 * g + (r16 >> 2), col >> 3) + (col & 7) * 2;
  }
  //  * V rows from a transposed [D][64] tile (A of dP^T) by two transpose
  //    reads: the address lane (e, m) of group g points at dimension row
  //    8 g + e (+4 for the second read, +32 per ks) at the columns holding
  //    keys 16 kb + 4 m .. +3, i.e. columns 16 kb + 4 swap(m), where swap
  //    exchanges m's two bits (the cache's column order); lane r16 receives
  //    key 16 kb + r16 at four consecutive dimensions.  The tile's swizzle
  //    depends on (d >> 1) & 1 = (e >> 1) & 1 only.
  int vtoff[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int m = r16 & 3;
    const int col = 16 * kb + 4 * (((m & 1) << 1) | (m >> 1));
    vtoff[kb] = VT::off(8 * g + (r16 >> 2), col >> 3) + (col & 7) * 2;
  }

  const int side = __builtin_amdgcn_readfirstlane(wave / HW);
  const int wq = __builtin_amdgcn_readfirstlane(wave % HW);
  // The loads of key tile (run, t0) into stage s.  Rows past the run's end
  // lie past the end of its buffer range and load as zeros (their scores are
  // masked below).
  auto issue = [&](DqStage<D>& s, int run, int t0) __attribute__((always_inline)) {
    const KvSeg& sg = a.seg[run];
    const int len = sg.len;
    const uint32_t rs = uint32_t(sg.row_stride) * 2;
    if (side == 0) {
      const auto rk = rsrc(static_cast<const char*>(sg.k) + int64_t(head) * sg.head_stride * 2, uint32_t(len) * rs);
#pragma unroll
      for (int k = 0; k < NKL; ++k) dma_rowtile<D, KT>(rk, s.k, rs, uint32_t(t0), wq * NKL + k, lane);
    } else if (sg.v_tiled) {
      const uint32_t tiles = uint32_t(len + kTile - 1) / kTile;
      const auto rv = rsrc(static_cast<const char*>(sg.v) + int64_t(head) * sg.v_head_stride * 2, tiles * kTile * D * 2);
#pragma unroll
      for (int k = 0; k < NVL; ++k) dma_vttile<D>(rv, s.v, uint32_t(t0) * D * 2, wq * NVL + k, lane);
    } else {
      const auto rv = rsrc(static_cast<const char*>(sg.v) + int64_t(head) * sg.head_stride * 2, uint32_t(len) * rs);
#pragma unroll
      for (int k = 0; k < NKL; ++k) dma_rowtile<D, KT>(rv, s.v, rs, uint32_t(t0), wq * NKL + k, lane);
    }
  };

  // dQ^T += K^T dS^T for one key tile, one 32-key step at a time: S^T and
  // dP^T of the step's two 16-key blocks (MFMA 16x16x32, each A read serving
  // both query blocks), dS^T = P (dP^T - delta) in fp32, packed to bf16 as the
  // B operand of dQ^T.  V comes from a transposed tile (kVt) or row-major rows.
  auto compute = [&](const DqStage<D>& s, int valid, auto vt_tag) __attribute__((always_inline)) {
    constexpr bool kVt = decltype(vt_tag)::value;
#pragma unroll
    for (int kst = 0; kst < 2; ++kst) {
      // The accumulators start at -lse2 and -delta of their query, so S^T
      // comes out as the log2 P and dP^T as dP - delta.
      f32x4 sc[2][2], dp[2][2];  // [key block of the step][query block]
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          sc[kk][qb] = sinit[qb];
          dp[kk][qb] = dinit[qb];
        }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int kb = 2 * kst + kk;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(s.k + 16 * kb * KT::RB + koff[ks]);
          bf16x8 va;
          if constexpr (kVt) {
            va = tr_pair(s.v + (32 * ks) * VT::RB + vtoff[kb], 4 * VT::RB);
          } else {
            va = *reinterpret_cast<const bf16x8*>(s.v + 16 * kb * KT::RB + koff[ks]);
          }
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            sc[kk][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[qb][ks], sc[kk][qb], 0, 0, 0);
            dp[kk][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, dof[qb][ks], dp[kk][qb], 0, 0, 0);
          }
        }
      }
      // element i of lane (r16, g) in block (kk, qb): key 32 kst + 16 kk + 4 g + i
      if (valid < kTile) {  // keys past the run's end: P = 0
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              if (32 * kst + 16 * kk + 4 * g + i >= valid) sc[kk][qb][i] = -INFINITY;
      }
      bf16x8 bds[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x8 f;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            f[4 * kk + i] = __builtin_amdgcn_exp2f(sc[kk][qb][i]) * dp[kk][qb][i];
        bds[qb] = __builtin_convertvector(f, bf16x8);
      }
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const bf16x8 ka = tr_pair(s.k + (32 * kst) * KT::RB + ktoff[db], 16 * KT::RB);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          dq[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, bds[qb], dq[db][qb], 0, 0, 0);
      }
    }
  };

  // Tiles in run order (runs are never empty); the runs with transposed V
  // tiles (the cache's) come first, then the caller's row-major current
  // chunk.  Step t: wait for this wave's loads of tile t (the only ones in
  // flight), one barrier (every wave's tile t has landed and every wave is
  // done with tile t-1), load tile t+1 into the other stage, compute tile t.
  int n_vt = 0, n = 0;
  for (int r = 0; r < a.n_seg; ++r) {
    const int tl = (a.seg[r].len + kTile - 1) / kTile;
    n += tl;
    if (a.seg[r].v_tiled && n_vt == n - tl) n_vt = n;
  }
  int run = 0, t0 = 0;    // tile being computed
  int lrun = 0, lt0 = 0;  // next tile to load
  auto advance = [&](int& r, int& t) __attribute__((always_inline)) {
    t += kTile;
    if (t >= a.seg[r].len) {
      ++r;
      t = 0;
    }
  };
  issue(st0, 0, 0);
  advance(lrun, lt0);
  auto step = [&](const DqStage<D>& cur, DqStage<D>& nxt, auto vt_tag) __attribute__((always_inline)) {
    wait_vmcnt<0>();
    wg_barrier();
    if (lrun < a.n_seg) {
      issue(nxt, lrun, lt0);
      advance(lrun, lt0);
    }
    compute(cur, min(kTile, a.seg[run].len - t0), vt_tag);
    advance(run, t0);
  };
  auto loop = [&](int tb, int te, auto vt_tag) __attribute__((always_inline)) {
    int t = tb;
    if (t < te && (t & 1)) {
      step(st1, st0, vt_tag);
      ++t;
    }
    for (; t + 1 < te; t += 2) {
      step(st0, st1, vt_tag);
      step(st1, st0, vt_tag);
    }
    if (t < te) step(st0, st1, vt_tag);
  };
  loop(0, n_vt, std::true_type{});
  loop(n_vt, n, std::false_type{});

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (!q_ok[qb]) continue;
    float* out = p.dq + (int64_t(qi[qb]) * a.H + head) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<float4*>(out + 16 * db + 4 * g) =
          make_float4(dq[db][qb][0] * a.scale, dq[db][qb][1] * a.scale, dq[db][qb][2] * a.scale,
                      dq[db][qb][3] * a.scale);
  }
}

// ---------------------------------------------------------------------------
// dK, dV of the current chunk (the last run)
// ---------------------------------------------------------------------------
// The tile ring: Q' rows and dO rows in the padded, skewed RowTile layout,
// plus the tile's forward log-sum-exp and delta.  Three stages, each its own
// __shared__ variable so that the compiler can tell a stage being filled by
// LDS-DMA from the stage being read and does not wait for the fill.
template <int D>
struct DkvStage {
  char q[RowTile<D, true>::kBytes];
  char g[RowTile<D, true>::kBytes];
  float lse[kTile];
  float dl[kTile];
};

template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_dkv_kernel(AttnBwdArgs p) {
  using QT = RowTile<D, true>;  // padded and skewed
  constexpr int G = QT::RB / 16;  // 16-byte slots per LDS row, padding included
  constexpr int NI = G / 4;       // 1 KB LDS-DMA loads per wave per tile side (4 waves per side)
  static_assert(G % 4 == 0, "tile side splits over four waves");
  __shared__ __attribute__((aligned(16))) DkvStage<D> st0;
  __shared__ __attribute__((aligned(16))) DkvStage<D> st1;
  __shared__ __attribute__((aligned(16))) DkvStage<D> st2;
  const AttnArgs& a = p.a;
  const KvSeg& cur = a.seg[a.n_seg - 1];
  int head, ktile;
  xcd_unit(head, ktile);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // MFMA 16x16x32 lane roles: r16 = lane % 16 is the key column of each
  // 16-key block (and the row of an A operand), g = lane / 16 the 8-wide
  // slice of the contraction and the 4-row slice of the result.
  const int r16 = lane & 15, g = lane >> 4;

  // B operands: K and V of key 16 kb + r16 of the wave's 32, d = 32 ks + 8 g .. +7.
  int key[2];
  bool k_ok[2];
  bf16x8 kf[2][D / 32], vf[2][D / 32];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    key[kb] = ktile * kBwdBK + wave * 32 + 16 * kb + r16;
    k_ok[kb] = key[kb] < cur.len;
    const int64_t off = int64_t(key[kb]) * cur.row_stride + int64_t(head) * cur.head_stride;
    const u32x4* kp = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(cur.k) + off);
    const u32x4* vp = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(cur.v) + off);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      kf[kb][ks] = __builtin_bit_cast(bf16x8, k_ok[kb] ? kp[4 * ks + g] : u32x4{0, 0, 0, 0});
      vf[kb][ks] = __builtin_bit_cast(bf16x8, k_ok[kb] ? vp[4 * ks + g] : u32x4{0, 0, 0, 0});
    }
  }
  // dK^T and dV^T accumulators: element i of lane (r16, g) in block (db, kb)
  // is dimension 16 db + 4 g + i of key 16 kb + r16.
  f32x4 dk[D / 16][2], dv[D / 16][2];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dk[db][kb][r] = dv[db][kb][r] = 0.f;
  // Byte offsets of this lane's LDS operand reads (the tile layout depends
  // on the row mod 16 only, so query blocks and steps are plain offsets):
  //  * Q' and dO rows (A of S and dP): query 16 qb + r16, granule 4 ks + g;
  //  * dO^T and Q'^T (A of dV^T and dK^T) by two transpose reads: the address
  //    lane (e = r16 >> 2, m = r16 & 3) of group g points at query row
  //    4 g + e (+16 for the second read, +32 per query step) at dimensions
  //    16 db + 4 m .. +3, so lane r16 receives dimension 16 db + r16 of
  //    queries 4 g .. 4 g + 3 (and 16 + 4 g ..): the query order in which the
  //    S and dS accumulators of the step's two query blocks pack into the
  //    P and dS operands.
  //  The skewed layout advances a row's granules linearly, so one base
  //  offset serves every ks (+64 bytes a step) and one every db (+32 bytes).
  const int qoff0 = QT::off(r16, g);
  const int toff0 = QT::off(4 * g + (r16 >> 2), (4 * (r16 & 3)) >> 3) + ((4 * (r16 & 3)) & 7) * 2;

  // Tile loads, straight into LDS (dma_rowtile).  Waves 0-3 fill the Q' side
  // (the delta kernel's bf16(Q c) copy at the start of dq), waves 4-7 the dO
  // side; wave 0 also loads the tile's lse and wave 4 its delta.  Query rows
  // past n_q lie past the end of every buffer range and load as zeros:
  // Q' = dO = 0 and lse = delta = 0 give P = 1 and dS = 0, and a zero dO
  // row, so those rows add nothing to dK or dV.
  const int side = __builtin_amdgcn_readfirstlane(wave >> 2);
  const int wq = __builtin_amdgcn_readfirstlane(wave & 3);
  const uint32_t row_bytes = uint32_t(a.H) * D * 2;  // one query's row of all heads
  const uint32_t head_off = uint32_t(head) * D * 2;
  const __amdgpu_buffer_rsrc_t rside =
      rsrc(static_cast<const char*>(side ? p.dout : static_cast<const void*>(p.dq)) + head_off,
           uint32_t(a.n_q) * row_bytes - head_off);
  const __amdgpu_buffer_rsrc_t rvec = rsrc(side ? static_cast<const void*>(p.delta + int64_t(head) * a.n_q)
                                                : static_cast<const void*>(p.lse + int64_t(head) * a.n_q),
                                           uint32_t(a.n_q) * 4);
  auto issue = [&](DkvStage<D>& s, int t) __attribute__((always_inline)) {
    // The lane's slot addresses are recomputed per tile from an opaque copy of
    // the lane id, so the compiler does not keep them in registers across the
    // loop (the MFMA accumulators and K/V fragments fill the register file).
    int ln = lane;
    __asm__ __volatile__("" : "+v"(ln));
    char* dst = side ? s.g : s.q;
#pragma unroll
    for (int k = 0; k < NI; ++k) dma_rowtile<D, QT>(rside, dst, row_bytes, uint32_t(t) * kTile, wq * NI + k, ln);
    if (wq == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rvec, (__attribute__((address_space(3))) void*)(side ? s.dl : s.lse),
                                               4, uint32_t(t * kTile + ln) * 4, 0, 0, 0);
  };

  // One 64-query tile, one 32-query step at a time: S and dP of the step's
  // two 16-query blocks (MFMA 16x16x32, each A read serving both key blocks),
  // P = 2^(S - lse2) and dS = P (dP - delta) in fp32, packed to bf16 as the
  // B operands of dV^T += dO^T P and dK^T += Q'^T dS.
  auto compute = [&](const DkvStage<D>& s) __attribute__((always_inline)) {
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      // element i of lane (r16, g) in block (qq, kb): query 32 qs + 16 qq + 4 g + i.
      // The accumulators start at -lse2 and -delta of their query, so S comes
      // out as log2 P and dP as dP - delta.
      f32x4 sc[2][2], dp[2][2];  // [query block of the step][key block]
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int q4 = 32 * qs + 16 * qq + 4 * g;
        const float4 l4 = *reinterpret_cast<const float4*>(&s.lse[q4]);
        const float4 d4 = *reinterpret_cast<const float4*>(&s.dl[q4]);
        const f32x4 si = {-l4.x * kLog2e, -l4.y * kLog2e, -l4.z * kLog2e, -l4.w * kLog2e};
        const f32x4 di = {-d4.x, -d4.y, -d4.z, -d4.w};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          sc[qq][kb] = si;
          dp[qq][kb] = di;
        }
      }
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int row0 = 16 * (2 * qs + qq) * QT::RB;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(s.q + row0 + 64 * ks + qoff0);
          const bf16x8 ga = *reinterpret_cast<const bf16x8*>(s.g + row0 + 64 * ks + qoff0);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            sc[qq][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[kb][ks], sc[qq][kb], 0, 0, 0);
            dp[qq][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga, vf[kb][ks], dp[qq][kb], 0, 0, 0);
          }
        }
      }
      bf16x8 pb[2], db8[2];
      {
        f32x8 pf[2], df[2];
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float pr = __builtin_amdgcn_exp2f(sc[qq][kb][i]);
              pf[kb][4 * qq + i] = pr;
              df[kb][4 * qq + i] = pr * dp[qq][kb][i];
            }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          pb[kb] = __builtin_convertvector(pf[kb], bf16x8);
          db8[kb] = __builtin_convertvector(df[kb], bf16x8);
        }
      }
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const int to = (32 * qs) * QT::RB + 32 * db + toff0;
        const bf16x8 ga = tr_pair(s.g + to, 16 * QT::RB);
        const bf16x8 qa = tr_pair(s.q + to, 16 * QT::RB);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          dv[db][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga, pb[kb], dv[db][kb], 0, 0, 0);
          dk[db][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, db8[kb], dk[db][kb], 0, 0, 0);
        }
      }
    }
  };

  // Tile t sits in stage t mod 3.  Step t: wait for this wave's loads of tile
  // t (tile t+1's may stay in flight), one barrier (every wave's tile t has
  // landed and every wave is done with tile t-1), then load tile t+2 into the
  // stage tile t-1 used, and compute tile t.
  const int nt = (a.n_q + kTile - 1) / kTile;
  issue(st0, 0);
  if (nt > 1) issue(st1, 1);
  auto step = [&](const DkvStage<D>& cur_st, DkvStage<D>& next2, int t) __attribute__((always_inline)) {
    if (t + 1 < nt) {
      if (wq == 0) wait_vmcnt<NI + 1>();
      else wait_vmcnt<NI>();
    } else {
      wait_vmcnt<0>();
    }
    wg_barrier();
    if (t + 2 < nt) issue(next2, t + 2);
    compute(cur_st);
  };
  for (int t = 0; t < nt; t += 3) {
    step(st0, st2, t);
    if (t + 1 < nt) step(st1, st0, t + 1);
    if (t + 2 < nt) step(st2, st1, t + 2);
  }
  // dK = scale dS^T Q = (dS^T Q') / log2 e
  const float kscale = 1.f / kLog2e;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if (!k_ok[kb]) continue;
    const int64_t orow = (int64_t(key[kb]) * a.H + head) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const int d0 = 16 * db + 4 * g;
      *reinterpret_cast<float4*>(p.dv + orow + d0) =
          make_float4(dv[db][kb][0], dv[db][kb][1], dv[db][kb][2], dv[db][kb][3]);
      *reinterpret_cast<float4*>(p.dk + orow + d0) =
          make_float4(dk[db][kb][0] * kscale, dk[db][kb][1] * kscale, dk[db][kb][2] * kscale,
                      dk[db][kb][3] * kscale);
    }
  }
}

template <typename K>
int launch(K kernel, dim3 grid, dim3 block, const void* arg, void* stream) {
  void* args[] = {const_cast<void*>(arg)};
  return int(hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0,
                             static_cast<hipStream_t>(stream)));
}

template <int D>
int launch_bwd_d(const AttnBwdArgs& p, void* stream) {
  const AttnArgs& a = p.a;
  const int64_t lanes = int64_t(a.n_q) * a.H * (D / 8);
  int err = launch(bwd_delta_kernel<D>, dim3(unsigned((lanes + 255) / 256)), dim3(256), &p, stream);
  if (err) return err;
  if (p.dk) {  // before the dQ kernel, which overwrites the Q' copy in dq
    const int len = a.seg[a.n_seg - 1].len;
    err = launch(bwd_dkv_kernel<D>, dim3((len + kBwdBK - 1) / kBwdBK, a.H), dim3(kBwdThreads), &p, stream);
    if (err) return err;
  }
  constexpr int W = kBwdDqWaves;
  return launch(bwd_dq_kernel<D, W>, dim3((a.n_q + 32 * W - 1) / (32 * W), a.H), dim3(64 * W), &p, stream);
}

}  // namespace

// Workspace of the allocation-free backward (ll_sink_window_attn_bwd_noalloc):
// delta, [H][n_q] fp32, rewritten by every call before it is read.  Each GPU
// holds its own copy for the life of the process; calls that overlap on one
// GPU share it and race.
static __device__ __align__(256) float scratch[kBwdScratchFloats];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {};
}  // namespace

// The current device's address of `scratch`, looked up once per device (the
// array's name is a host-side stand-in, not a device address).
int bwd_scratch(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  if (dev < 0 || dev >= kMaxDevices) return int(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return int(e);
    g_scratch[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch[dev];
  return 0;
}

int launch_attention_bwd(const AttnBwdArgs& p, void* stream) {
  if (p.a.n_q <= 0) return 0;
  return p.a.D == 64 ? launch_bwd_d<64>(p, stream) : launch_bwd_d<128>(p, stream);
}

}  // namespace ll
