// HIP kernels for gfx950 (MI355X): linear-attention variant of the sink +
// short-window attention call.
//
// LongLive: Real-time Interactive Long Video Generation, §4 "Implementation"
// (the method was also built on a linear-attention video model, for more
// speed; the pages give no formulation).  Reading: the softmax call's key set
// (frame sink, resident window, current chunk) with the weights
// w_ij = phi(q_i) . phi(k_j), phi(x) = max(x, 0), and
// out_i = sum_j w_ij v_j / (sum_j w_ij + eps).
// The weights factor, so the call runs in its associative form: per head
//   S = sum_j phi(k_j) v_j^T ([D][D]),  z = sum_j phi(k_j) ([D]),
//   out_i = phi(q_i)^T S / (phi(q_i) . z + eps),
// O((n_keys + n_q) D^2) work instead of O(n_q n_keys D).  Three kernels:
//   lin_state_kernel   per (key split, head): partial S and z over a range of
//                      64-key tiles; bf16 MFMA 32x32x16 with A = phi(K)^T
//                      (transpose reads of the row-major K tile, then max(., 0))
//                      and B = V (rows of the cache's transposed V tile, or
//                      transpose reads of a row-major V tile); z is the same
//                      product with B = ones.  Two load waves fill a 4-stage
//                      LDS ring by direct-to-LDS buffer loads, three tiles
//                      ahead of the four MFMA waves.  Keys past a run's end
//                      read as zero, so they add nothing and need no mask.
//   lin_reduce_kernel  sums the partials (written transposed) elementwise in a
//                      fixed order (deterministic) and stores S^T as a bf16
//                      pair hi + lo (hi = bf16(S), lo = bf16(S - hi)), which
//                      keeps ~16 significant bits.
//   lin_apply_kernel   per 128 queries of one head: O^T = S^T phi(Q)^T as two
//                      MFMA sums (hi and lo), the normaliser phi(q) . z on the
//                      VALU, bf16 output.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.hpp"

namespace ll {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef unsigned int u32x4 __attribute__((__vector_size__(4 * sizeof(unsigned))));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kTile = 64;          // keys per LDS tile
constexpr int kStateWaves = 6;      // state kernel: 4 MFMA waves + 2 load waves
constexpr int kStateThreads = 64 * kStateWaves;
constexpr int kStateStages = 4;     // LDS ring depth of the state kernel
constexpr int kApplyThreads = 256;  // 4 waves x 32 queries (two workgroups fit a CU)
constexpr int kApplyBQ = 128;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

// gfx950 LDS transpose read of 4 bf16: within each group of 16 lanes, lane i
// receives element (i & 3) of the 8 bytes addressed by lane 4*e + (i >> 2).
__device__ __forceinline__ bf16x4 tr_read(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// max(x, 0) of 8 bf16: a negative value (sign bit set) becomes +0.
__device__ __forceinline__ bf16x8 relu8(bf16x8 x) {
  u32x4 w = __builtin_bit_cast(u32x4, x);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned neg = (w[i] >> 15) & 0x00010001u;
    w[i] &= ~(neg * 0xffffu);
  }
  return __builtin_bit_cast(bf16x8, w);
}

// Key order (vt_key): column p of the cache's transposed V tiles holds key p
// with bits 2 and 3 swapped, the order in which an MFMA k-block of 16 keys is
// split between the two half waves (keys 0..3, 8..11 in half 0; 4..7, 12..15
// in half 1).  The transpose reads of row-major tiles produce the same order.

// Row-major [64][D] tile (K, or a row-major V), unpadded so that direct-to-LDS
// loads can fill it, read by transpose reads (per 32 lanes: 4 consecutive
// rows x 4 granules).  Granule g of row r sits at g ^ f(r), which spreads those
// 16 (row, granule) pairs over all 64 banks: D = 128 (256-byte rows):
// f(r) = ((r & 3) << 2) | ((r >> 2) & 3); D = 64 (128-byte rows, two per bank
// sweep): f(r) = 4 * (bit 1 of r).
template <int D>
struct KTile {
  static constexpr int RB = D * 2;
  static constexpr int kBytes = kTile * RB;
  static __device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return ((row >> 1) & 1) << 2;
  }
  static __device__ __forceinline__ int off(int row, int gran) { return row * RB + ((gran ^ swz(row)) << 4); }
};

// Transposed [D][64] V tile (128-byte rows, columns in vt_key order), read by
// 16-byte row reads of 32 consecutive rows; granule g of row d at
// g ^ ((d >> 1) & 7).
template <int D>
struct VTile {
  static constexpr int RB = kTile * 2;
  static constexpr int kBytes = D * RB;
  static __device__ __forceinline__ int off(int d, int gran) { return d * RB + ((gran ^ ((d >> 1) & 7)) << 4); }
};

// ---------------------------------------------------------------------------
// State: partial S and z of one key split
// ---------------------------------------------------------------------------
// s_waitcnt vmcnt(N): this wave's oldest loads up to all but N have landed.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  __asm__ __volatile__("" ::: "memory");
}

// Workgroup barrier that waits only for this wave's LDS operations, so the
// ring's direct-to-LDS loads stay in flight across it.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// Position (run, first key) of a tile in the sequence of 64-key tiles over
// the runs; all fields are uniform.
struct TileCursor {
  int run = 0, t0 = 0;
  __device__ void seek(const AttnArgs& a, int t) {
    run = 0;
    t0 = t * kTile;
    skip(a, 0);
  }
  // Moves k tiles on (a run's last tile may be partial).
  __device__ void skip(const AttnArgs& a, int k) {
    t0 += k * kTile;
    while (run < a.n_seg) {
      const int span = (a.seg[run].len + kTile - 1) / kTile * kTile;
      if (t0 < span) break;
      t0 -= span;
      ++run;
    }
  }
};

// A wave's LDS reads wait behind its own direct-to-LDS loads still in flight,
// so the roles are split: waves 4 and 5 only load (K and V of tile j + 3 into
// the ring stage that tile j - 1 left), waves 0..3 only read LDS and issue
// MFMAs.  One workgroup barrier per tile both publishes tile j (each load
// wave waits for its part of it first) and frees the stage of tile j - 1.
template <int D>
__global__ __launch_bounds__(kStateThreads) void lin_state_kernel(LinArgs p) {
  using KT = KTile<D>;
  using VT = VTile<D>;
  constexpr int G = D / 8;                        // 16-byte granules per K row
  constexpr int NB = D / 32;                      // 32-wide blocks of S per dimension
  constexpr int NPW = NB * NB / 4;                // S blocks per MFMA wave
  constexpr int RPI = 1024 / KT::RB;              // rows per 1 KB load
  constexpr int NI = KT::kBytes / 1024;           // 1 KB loads per operand and tile
  constexpr int kStage = KT::kBytes + VT::kBytes;
  static_assert(NPW >= 1 && 2 * NI < 64 && KT::kBytes == VT::kBytes, "shape");
  __shared__ __attribute__((aligned(16))) char ring[kStateStages * kStage];
  const AttnArgs& a = p.a;
  const int split = blockIdx.x;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, r32 = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // This split's tiles split, split + n_split, ... of the tile sequence over
  // the runs: interleaved, so every split gets the same mix of the cache's
  // transposed V tiles and the current chunk's row-major ones (which need
  // more LDS reads).
  int n_tiles = 0;
  for (int r = 0; r < a.n_seg; ++r) n_tiles += (a.seg[r].len + kTile - 1) / kTile;
  const int n_loc = split < n_tiles ? (n_tiles - split + p.n_split - 1) / p.n_split : 0;

  if (wave >= 4) {
    // Load wave: 4 -> K, 5 -> V.
    if (n_loc <= 0) return;
    const bool v_side = wave == 5;
    TileCursor c;
    c.seek(a, split);
    auto issue = [&](int st) {
      const KvSeg& sg = a.seg[c.run];
      const int len = sg.len;
      const uint32_t rs = uint32_t(sg.row_stride) * 2;
      char* dst = ring + st * kStage + (v_side ? KT::kBytes : 0);
      if (v_side && sg.v_tiled) {
        // the cache's [D][64] tile: 8 rows of 128 bytes per 1 KB load
        const uint32_t tiles = uint32_t(len + kTile - 1) / kTile;
        const auto rv = rsrc(static_cast<const char*>(sg.v) + int64_t(head) * sg.v_head_stride * 2,
                             tiles * kTile * D * 2);
        const uint32_t tbase = uint32_t(c.t0 / kTile) * kTile * D * 2;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int d = i * 8 + (lane >> 3);
          const uint32_t off = tbase + uint32_t(d * VT::RB + (((lane & 7) ^ ((d >> 1) & 7)) << 4));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(dst + i * 1024), 16, off, 0, 0, 0);
        }
      } else {
        // row-major rows: lane -> (row, stored granule); it fetches the
        // logical granule that belongs there (the XOR is its own inverse)
        const void* base = v_side ? sg.v : sg.k;
        const auto rr = rsrc(static_cast<const char*>(base) + int64_t(head) * sg.head_stride * 2, uint32_t(len) * rs);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int row = i * RPI + lane / G;
          const uint32_t off = uint32_t(c.t0 + row) * rs + (uint32_t((lane % G) ^ KT::swz(row)) << 4);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void*)(dst + i * 1024), 16, off, 0, 0, 0);
        }
      }
      c.skip(a, p.n_split);
    };
    for (int j = 0; j < kStateStages - 1 && j < n_loc; ++j) issue(j);
    for (int j = 0; j < n_loc; ++j) {
      // tile j has landed once only the tiles issued after it are in flight
      const int after = min(kStateStages - 2, n_loc - 1 - j);
      if (after >= 2) wait_vmcnt<2 * NI>();
      else if (after == 1) wait_vmcnt<NI>();
      else wait_vmcnt<0>();
      wg_barrier();
      if (j + kStateStages - 1 < n_loc) issue((j + kStateStages - 1) % kStateStages);
    }
    return;
  }

  // MFMA wave: S blocks (d1b, d2b0 .. d2b0 + NPW - 1); z with the first.
  const int d1b = (wave * NPW) / NB;
  const int d2b0 = (wave * NPW) % NB;
  const bool do_z = d2b0 == 0;
  f32x16 acc[NPW], zacc;
#pragma unroll
  for (int i = 0; i < NPW; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) zacc[r] = 0.f;

  if (n_loc > 0) {
    // Transpose-read offsets inside a row-major tile, per 16-key step: lane
    // r32 takes column 32*blk + r32 at keys {0..3, 8..11} (half 0) or
    // {4..7, 12..15} (half 1), the vt_key order of the V^T tiles' columns.
    auto tr_off = [&](int blk, int aa) {
      const int g16 = lane >> 4, j16 = lane & 15;
      const int row = 8 * aa + 4 * (g16 >> 1) + (j16 >> 2);
      const int col = 32 * blk + 16 * (g16 & 1) + 4 * (j16 & 3);
      return KT::off(row, col >> 3) + (col & 7) * 2;
    };
    const int ka0 = tr_off(d1b, 0), ka1 = tr_off(d1b, 1);
    int vb0[NPW], vb1[NPW];
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      vb0[i] = tr_off(d2b0 + i, 0);
      vb1[i] = tr_off(d2b0 + i, 1);
    }
    // V^T tile rows d2 = 32*d2b + r32 at columns 16*step + 8*half .. +7.
    const int vrow = r32 * VT::RB;
    const int vx = (r32 >> 1) & 7;  // the row's granule swizzle (32*d2b keeps it)
    const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                         (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
    TileCursor c;
    c.seek(a, split);
    for (int j = 0; j < n_loc; ++j) {
      wg_barrier();
      const int st = j % kStateStages;
      const char* ks = ring + st * kStage;
      const char* vs = ks + KT::kBytes;
      if (a.seg[c.run].v_tiled) {
#pragma unroll
        for (int step = 0; step < kTile / 16; ++step) {
          const char* kb = ks + 16 * step * KT::RB;
          const bf16x8 fa = relu8(__builtin_shufflevector(tr_read(kb + ka0), tr_read(kb + ka1), 0, 1, 2, 3, 4, 5, 6, 7));
          const int g = ((2 * step) ^ (vx & 6)) | (half ^ (vx & 1));
#pragma unroll
          for (int i = 0; i < NPW; ++i) {
            const bf16x8 vb = *reinterpret_cast<const bf16x8*>(vs + (32 * (d2b0 + i)) * VT::RB + vrow + (g << 4));
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, vb, acc[i], 0, 0, 0);
          }
          if (do_z) zacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, ones, zacc, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int step = 0; step < kTile / 16; ++step) {
          const char* kb = ks + 16 * step * KT::RB;
          const char* vbp = vs + 16 * step * KT::RB;
          const bf16x8 fa = relu8(__builtin_shufflevector(tr_read(kb + ka0), tr_read(kb + ka1), 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int i = 0; i < NPW; ++i) {
            const bf16x8 vb = __builtin_shufflevector(tr_read(vbp + vb0[i]), tr_read(vbp + vb1[i]), 0, 1, 2, 3, 4, 5, 6, 7);
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, vb, acc[i], 0, 0, 0);
          }
          if (do_z) zacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, ones, zacc, 0, 0, 0);
        }
      }
      c.skip(a, p.n_split);
    }
  }

  // Partial S, stored transposed ([d2][d1], the layout the apply kernel
  // reads): acc[i][4g + e] is d1 = 32*d1b + 8g + 4*half + e, d2 =
  // 32*(d2b0 + i) + r32, so each lane stores 4 consecutive d1 at once.
  float* ps = p.part_s + (int64_t(split) * a.H + head) * D * D;
#pragma unroll
  for (int i = 0; i < NPW; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 v = {acc[i][4 * g], acc[i][4 * g + 1], acc[i][4 * g + 2], acc[i][4 * g + 3]};
      *reinterpret_cast<f32x4*>(ps + (32 * (d2b0 + i) + r32) * D + 32 * d1b + 8 * g + 4 * half) = v;
    }
  if (do_z && r32 == 0) {
    float* pz = p.part_z + (int64_t(split) * a.H + head) * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) pz[32 * d1b + 8 * (r >> 2) + 4 * half + (r & 3)] = zacc[r];
  }
}

// ---------------------------------------------------------------------------
// Reduce: S^T = sum of the transposed partials in split order, stored as
// bf16 hi + lo; z likewise in fp32.  Elementwise: each thread sums one
// 16-byte group of 4 floats over the splits with every load in flight at once
// (a fixed order, so the result is deterministic).
// ---------------------------------------------------------------------------
constexpr int kReduceThreads = 128;

template <int D>
__global__ __launch_bounds__(kReduceThreads) void lin_reduce_kernel(LinArgs p) {
  const int H = p.a.H;
  const int64_t n4 = int64_t(H) * D * D / 4;  // float4 groups of S^T
  const int64_t e = int64_t(blockIdx.x) * kReduceThreads + threadIdx.x;
  if (e < n4) {
    const f32x4* src = reinterpret_cast<const f32x4*>(p.part_s) + e;
    f32x4 v[kLinMaxSplits];
#pragma unroll
    for (int k = 0; k < kLinMaxSplits; ++k)
      if (k < p.n_split) v[k] = src[int64_t(k) * n4];
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kLinMaxSplits; ++k)
      if (k < p.n_split) s += v[k];
    bf16x4 hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hi[i] = (__bf16)s[i];
      lo[i] = (__bf16)(s[i] - float(hi[i]));
    }
    reinterpret_cast<bf16x4*>(p.st_hi)[e] = hi;
    reinterpret_cast<bf16x4*>(p.st_lo)[e] = lo;
  } else if (e < n4 + H * D) {
    const int64_t z = e - n4;
    float v[kLinMaxSplits];
#pragma unroll
    for (int k = 0; k < kLinMaxSplits; ++k)
      if (k < p.n_split) v[k] = p.part_z[int64_t(k) * H * D + z];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kLinMaxSplits; ++k)
      if (k < p.n_split) s += v[k];
    p.z[z] = s;
  }
}

// ---------------------------------------------------------------------------
// Apply: out_i = phi(q_i)^T S / (phi(q_i) . z + eps)
// ---------------------------------------------------------------------------
// Value held by lane l ^ 32 (v_permlane32_swap; see the attention kernels).
__device__ __forceinline__ float partner_half(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                   __builtin_bit_cast(unsigned, x), false, false);
  const unsigned lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  return __builtin_bit_cast(float, lane < 32 ? pr[1] : pr[0]);
}

template <int D>
__global__ __launch_bounds__(kApplyThreads) void lin_apply_kernel(LinArgs p) {
  constexpr int G = D / 8;    // 16-byte granules per row of S^T
  constexpr int NB = D / 32;  // 32-row blocks of S^T (output column blocks)
  constexpr int RB = D * 2;
  constexpr int kWaves = kApplyThreads / 64;
  constexpr int kSBytes = D * RB;            // one part (hi or lo) of S^T
  constexpr int kOBytes = kWaves * 32 * RB;  // output staging, 32 rows per wave
  constexpr int kLds = 2 * kSBytes > kOBytes ? 2 * kSBytes : kOBytes;
  // S^T rows (d2), granule g stored at g ^ (d2 mod G): 16-byte reads of
  // consecutive rows at one granule fall in distinct banks.  The same memory
  // stages the output once every wave is done with S^T.
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  __shared__ float zs[D];
  char* const sh = lds;
  char* const sl = lds + kSBytes;
  const AttnArgs& a = p.a;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, r32 = lane & 31, half = lane >> 5;

  const int qi = blockIdx.x * kApplyBQ + wave * 32 + r32;
  const bool q_ok = qi < a.n_q;
  const int64_t qrow = (int64_t(qi) * a.H + head) * D;
  // B operand: phi(q) of the lane's query at d1 = 16j + 8*half .. +7; its
  // loads go out first, then every load of S^T, then the LDS stores.
  bf16x8 qf[D / 16];
  {
    const u32x4* q = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(a.q) + qrow);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) qf[j] = __builtin_bit_cast(bf16x8, q_ok ? q[2 * j + half] : u32x4{0, 0, 0, 0});
  }
  {
    constexpr int NS = D * G / kApplyThreads;  // 16-byte loads per thread per part
    const u32x4* gh = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(p.st_hi) + int64_t(head) * D * D);
    const u32x4* gl = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(p.st_lo) + int64_t(head) * D * D);
    u32x4 wh[NS], wl[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      wh[i] = gh[tid + i * kApplyThreads];
      wl[i] = gl[tid + i * kApplyThreads];
    }
    const float zv = tid < D ? p.z[int64_t(head) * D + tid] : 0.f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int it = tid + i * kApplyThreads;
      const int row = it / G, g = it % G;
      const int o = row * RB + ((g ^ (row & (G - 1))) << 4);
      *reinterpret_cast<u32x4*>(sh + o) = wh[i];
      *reinterpret_cast<u32x4*>(sl + o) = wl[i];
    }
    if (tid < D) zs[tid] = zv;
  }
#pragma unroll
  for (int j = 0; j < D / 16; ++j) qf[j] = relu8(qf[j]);
  __syncthreads();

  // normaliser phi(q) . z: this half's 64 dims, then the other half's
  float den = 0.f;
#pragma unroll
  for (int j = 0; j < D / 16; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) den = fmaf(float(qf[j][i]), zs[16 * j + 8 * half + i], den);
  den += partner_half(den);

  f32x16 o[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[b][r] = 0.f;
#pragma unroll
  for (int j = 0; j < D / 16; ++j)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int row = 32 * b + r32;
      const int off = row * RB + (((2 * j + half) ^ (row & (G - 1))) << 4);
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(sh + off);
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(sl + off);
      o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, qf[j], o[b], 0, 0, 0);
      o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, qf[j], o[b], 0, 0, 0);
    }

  // Output through LDS: the lane's 4-dim pieces of its query row go into the
  // wave's 32-row block, which is read back as whole rows, so that each
  // global store covers complete rows of out.  Row r keeps granule g at
  // g ^ sw(r) and its 8-byte half s at s ^ (bit 4 of r): the writes (32
  // rows at one granule) and the row reads are both free of bank conflicts.
  const float inv = 1.f / (den + p.eps);
  auto sw = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  char* const ob = lds + wave * 32 * RB;
  __syncthreads();  // every wave's reads of S^T are done
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      bf16x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (__bf16)(o[b][4 * gq + i] * inv);
      const int g = 4 * b + gq;
      *reinterpret_cast<bf16x4*>(ob + r32 * RB + ((g ^ sw(r32)) << 4) + ((half ^ (r32 >> 4)) << 3)) = w;
    }
  __syncthreads();
  constexpr int RPI = 64 / G;  // rows per 64-lane read
  const int gg = lane % G;
  const int64_t obase = (int64_t(blockIdx.x) * kApplyBQ + wave * 32) * a.H + head;
  const int q = blockIdx.x * kApplyBQ + wave * 32;
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int row = k * RPI + lane / G;
    u32x4 v = *reinterpret_cast<const u32x4*>(ob + row * RB + ((gg ^ sw(row)) << 4));
    if ((k * RPI) & 16) v = u32x4{v[2], v[3], v[0], v[1]};  // rows 16..31 hold their halves swapped
    if (q + row < a.n_q)
      *reinterpret_cast<u32x4*>(static_cast<__bf16*>(a.out) + (obase + int64_t(row) * a.H) * D + gg * 8) = v;
  }
}

template <typename K>
int launch(K kernel, dim3 grid, dim3 block, const void* arg, void* stream) {
  void* args[] = {const_cast<void*>(arg)};
  return int(hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0,
                             static_cast<hipStream_t>(stream)));
}

template <int D>
int launch_linear_d(const LinArgs& p, void* stream) {
  int err = launch(lin_state_kernel<D>, dim3(p.n_split, p.a.H), dim3(kStateThreads), &p, stream);
  if (err) return err;
  const int64_t n_red = int64_t(p.a.H) * D * D / 4 + int64_t(p.a.H) * D;
  err = launch(lin_reduce_kernel<D>, dim3(unsigned((n_red + kReduceThreads - 1) / kReduceThreads)),
               dim3(kReduceThreads), &p, stream);
  if (err || p.a.n_q <= 0) return err;
  return launch(lin_apply_kernel<D>, dim3((p.a.n_q + kApplyBQ - 1) / kApplyBQ, p.a.H), dim3(kApplyThreads), &p,
                stream);
}

}  // namespace

int launch_linear_attention(const LinArgs& p, void* stream) {
  return p.a.D == 64 ? launch_linear_d<64>(p, stream) : launch_linear_d<128>(p, stream);
}

}  // namespace ll
