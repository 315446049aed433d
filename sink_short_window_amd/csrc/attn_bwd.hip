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
//   bwd_delta_kernel  delta[h][i] = dO_i . O_i (fp32).
//   bwd_dq_kernel     per 256 queries of one head (8 waves x 32): walk every
//                     64-key tile of every run; S^T = K Q'^T and dP^T = V dO^T
//                     (bf16 MFMA 32x32x16, K/V rows from LDS, Q' and dO in
//                     registers), P = 2^(S^T - lse2) from the forward's
//                     log-sum-exp, dS^T in fp32 rounded to bf16, then
//                     dQ^T += K^T dS^T with K^T from gfx950 transpose reads.
//   bwd_dkv_kernel    per 256 keys of the current chunk: loop over 64-query
//                     tiles; S = Q' K^T, dP = dO V^T (K/V fragments in
//                     registers), then dV^T += dO^T P and dK^T += Q'^T dS with
//                     dO^T and Q'^T from transpose reads.
// Q' = bf16(Q * scale * log2 e) exactly as the forward kernel forms it, so P is
// recomputed from the same rounded scores the forward normalised.  Gradients
// are written in fp32 (token-major [n][H][D]).
//
// Tiles reach LDS through registers, in layouts (RowTile, VtTile) whose XOR
// swizzles keep both the 16-byte row reads and the transpose reads free of
// bank conflicts.  In the dQ kernel V stays transposed ([D][64] per 64 keys,
// as the bf16 cache stores it; the caller's row-major current chunk is
// transposed while staged) and its rows are read back with transpose reads.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.hpp"

namespace ll {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x8 __attribute__((__vector_size__(8 * sizeof(float))));
typedef unsigned int u32x4 __attribute__((__vector_size__(4 * sizeof(unsigned))));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kBwdThreads = 512;  // 8 waves
constexpr int kBwdBQ = 256;       // queries per dq workgroup (8 waves x 32)
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

// Column p of a transposed V tile holds key p with bits 2 and 3 swapped (the
// involution the forward kernel's PV operand order asks for).
__device__ __forceinline__ int vt_key(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

// Row-major [kTile][D] bf16 LDS tile (K, Q' or dO), read both as rows
// (16-byte reads, 16 consecutive rows at one granule) and by transpose reads
// (per 32 lanes: 4 consecutive rows x 4 granules).  For D = 128 rows are 256
// bytes and granule g of row r is stored at g ^ f(r), f(r) = ((r & 3) << 2) |
// ((r >> 2) & 3), a rotation of r mod 16: both patterns then cover 16
// distinct granules, i.e. all 64 banks.  Otherwise (D = 64, or a kernel
// whose registers cannot spare the per-read address arithmetic) rows are
// padded by 32 bytes, to a stride of 8 (mod 64) dwords, which keeps the
// transpose reads conflict-free within 16 lanes.
template <int D, bool kSwzOn = true>
struct RowTile {
  static constexpr bool kSwz = kSwzOn && D == 128;
  static constexpr int RB = kSwz ? D * 2 : (D + 16) * 2;
  static constexpr int kBytes = kTile * RB;
  static __device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
  static __device__ __forceinline__ int off(int row, int gran) {
    if constexpr (kSwz) return row * RB + ((gran ^ swz(row)) << 4);
    else return row * RB + gran * 16;
  }
};

// Transposed [D][64] bf16 V tile of the dQ kernel, read by transpose reads
// only (per 32 lanes: 4 consecutive rows d, two of each parity).  Rows are
// 128 bytes; granule g of row d is stored at g ^ (((d >> 1) & 1) << 2) so the
// two rows of one parity fall in different halves of their 32 banks.
template <int D>
struct VtTile {
  static constexpr int RB = kTile * 2;
  static constexpr int kBytes = D * RB;
  static __device__ __forceinline__ int off(int d, int gran) { return d * RB + ((gran ^ (((d >> 1) & 1) << 2)) << 4); }
};

// Byte offsets (within a RowTile) of the two transpose
// reads that give lane (r32, half) the A operand of a 32x32x16 MFMA whose
// rows are the tile's columns 32*db + r32 and whose 16 k values are tile rows
// 16*step + {0..3, 8..11} (half 0) or {4..7, 12..15} (half 1): the row order
// in which the C accumulator of the previous MFMA packs into a B operand.
// (The swizzle depends on row mod 16 only, so the offsets of rows 0..15 serve
// every 16-row step.)
template <int D, typename T>
__device__ __forceinline__ void tr_offsets(int lane, int (&off)[2][D / 32]) {
  const int g16 = lane >> 4, j16 = lane & 15;
#pragma unroll
  for (int aa = 0; aa < 2; ++aa)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int row = 8 * aa + 4 * (g16 >> 1) + (j16 >> 2);
      const int col = 32 * db + 16 * (g16 & 1) + 4 * (j16 & 3);
      if constexpr (T::kSwz) off[aa][db] = T::off(row, col >> 3) + (col & 7) * 2;
      else off[aa][db] = row * T::RB + col * 2;  // (this form keeps the compiler from spilling)
    }
}

// 16-byte read of granule gran of row `row` of a RowTile.
template <typename T>
__device__ __forceinline__ bf16x8 row_read(const char* tile, int row, int gran) {
  return *reinterpret_cast<const bf16x8*>(tile + T::off(row, gran));
}

template <int D, typename T>
__device__ __forceinline__ bf16x8 tr_operand(const char* tile, int step, const int (&off)[2][D / 32], int db) {
  constexpr int RB = T::RB;
  const char* base = tile + 16 * step * RB;
  const bf16x4 lo = tr_read(base + off[0][db]);
  const bf16x4 hi = tr_read(base + off[1][db]);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Pack C accumulator elements 8*s2 .. 8*s2+7 (scaled) as one bf16 B operand.
__device__ __forceinline__ bf16x8 pack8(const float (&x)[16], int s2) {
  f32x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = x[8 * s2 + e];
  return __builtin_convertvector(f, bf16x8);
}

// ---------------------------------------------------------------------------
// delta[h][i] = sum_d dO[i][h][d] * O[i][h][d]
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

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(AttnBwdArgs p) {
  using KT = RowTile<D, true>;
  using VT = VtTile<D>;
  constexpr int NV = D / 8;        // 16-byte vectors per row
  // two LDS buffers: tile t is read from one while tile t+1 is written to the other
  __shared__ __attribute__((aligned(16))) char ks2[2][KT::kBytes];
  __shared__ __attribute__((aligned(16))) char vs2[2][VT::kBytes];  // [d][column], column p = key vt_key(p)
  const AttnArgs& a = p.a;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, r32 = lane & 31, half = lane >> 5;
  const int qi = blockIdx.x * kBwdBQ + wave * 32 + r32;
  const bool q_ok = qi < a.n_q;
  const float c = a.scale * kLog2e;
  const int64_t qrow = (int64_t(qi) * a.H + head) * D;

  // B operands: Q' and dO of the lane's query, d = 16j + 8*half .. +7.
  bf16x8 qf[D / 16], dof[D / 16];
  {
    const u32x4* q = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(a.q) + qrow);
    const u32x4* g = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(p.dout) + qrow);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const u32x4 wq = q_ok ? q[2 * j + half] : u32x4{0, 0, 0, 0};
      const u32x4 wg = q_ok ? g[2 * j + half] : u32x4{0, 0, 0, 0};
      qf[j] = scale_bf16x8(wq, c);
      dof[j] = __builtin_bit_cast(bf16x8, wg);
    }
  }
  // log2-domain log-sum-exp; +inf for padding lanes makes their P exactly 0
  const float lse2 = q_ok ? p.lse[int64_t(head) * a.n_q + qi] * kLog2e : INFINITY;
  const float dl = q_ok ? p.delta[int64_t(head) * a.n_q + qi] : 0.f;

  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[i][r] = 0.f;
  int toff[2][D / 32];
  tr_offsets<D, KT>(lane, toff);
  // V rows (A of dP^T: key 32*kb + r32, d = 16j + 8*half + 0..7) from the
  // transposed tile by two transpose reads: the address lane (e = j16 >> 2,
  // m = j16 & 3) of a 16-lane group points at row d = 16j + 8*half + 4*aa + e,
  // at the column holding keys 32*kb + 16*(g16 & 1) + 4m .. +3, i.e. column
  // 32*kb + 16*(g16 & 1) + 4*swap(m) where swap exchanges m's two bits.  The
  // swizzle depends on (d >> 1) & 1 = (e >> 1) & 1 only, so 16j is a plain
  // offset.
  int voff[2][2];
  {
    const int g16 = lane >> 4, j16 = lane & 15, m = j16 & 3;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
        const int col = 32 * kb + 16 * (g16 & 1) + 4 * (((m & 1) << 1) | (m >> 1));
        voff[kb][aa] = VT::off(8 * (g16 >> 1) + 4 * aa + (j16 >> 2), col >> 3) + (col & 7) * 2;
      }
  }

  // Loads of one 64-key tile, held in registers from issue to LDS write.
  constexpr int NL = kTile * NV / kBwdThreads;  // 16-byte loads per thread per side
  u32x4 kreg[NL], vreg[NL];
  bool vt_reg = false;
  auto issue = [&](int run, int t0) {
    const KvSeg& sg = a.seg[run];
    const int len = sg.len;
    const uint32_t rs = uint32_t(sg.row_stride) * 2;
    const auto rk = rsrc(static_cast<const char*>(sg.k) + int64_t(head) * sg.head_stride * 2, uint32_t(len) * rs);
    vt_reg = sg.v_tiled != 0;
    const uint32_t tiles = uint32_t(len + kTile - 1) / kTile;
    const auto rv = vt_reg ? rsrc(static_cast<const char*>(sg.v) + int64_t(head) * sg.v_head_stride * 2,
                                  tiles * kTile * D * 2)
                           : rsrc(static_cast<const char*>(sg.v) + int64_t(head) * sg.head_stride * 2, uint32_t(len) * rs);
    const uint32_t tbase = uint32_t(t0 / kTile) * kTile * D * 2;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int it = tid + i * kBwdThreads;
      const int row = it / NV, vec = it % NV;
      // K rows (rows past the run read as zero)
      kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, uint32_t(t0 + row) * rs + vec * 16, 0, 0);
      // V: a stored [D][64] tile (row d = it / 8, granule it % 8), or
      // row-major rows with the key in the low bits of it (see stage)
      vreg[i] = vt_reg ? __builtin_amdgcn_raw_buffer_load_b128(rv, tbase + (it >> 3) * 128 + (it & 7) * 16, 0, 0)
                       : __builtin_amdgcn_raw_buffer_load_b128(rv, uint32_t(t0 + it % kTile) * rs + it / kTile * 16, 0, 0);
    }
  };
  auto stage = [&](char* kbuf, char* vbuf) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int it = tid + i * kBwdThreads;
      const int row = it / NV, vec = it % NV;
      *reinterpret_cast<u32x4*>(kbuf + KT::off(row, vec)) = kreg[i];
      if (vt_reg) {  // columns already in vt_key order: copy
        *reinterpret_cast<u32x4*>(vbuf + VT::off(it >> 3, it & 7)) = vreg[i];
      } else {
        // Row-major V (the current chunk): the 64 lanes of a wave hold the 64
        // keys of one 16-byte column (dims 8*vv .. 8*vv+7), so each 2-byte
        // store below fills one whole 128-byte row d of the transposed tile
        // (key -> column vt_key(key)) without bank conflicts.
        const bf16x8 b = __builtin_bit_cast(bf16x8, vreg[i]);
        const int key = it % kTile, vv = it / kTile;
        const int p = vt_key(key);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<__bf16*>(vbuf + VT::off(vv * 8 + e, p >> 3) + (p & 7) * 2) = b[e];
      }
    }
  };

  // Tiles in run order; runs are never empty.  Tile t is computed from
  // buffer t & 1 while tile t+1's loads are in flight, then written to the
  // other buffer; one barrier per tile.
  int run = 0, t0 = 0;
  issue(0, 0);
  stage(ks2[0], vs2[0]);
  __syncthreads();
  for (int t = 0;; ++t) {
    int nrun = run, nt0 = t0 + kTile;
    if (nt0 >= a.seg[run].len) {
      ++nrun;
      nt0 = 0;
    }
    const bool has_next = nrun < a.n_seg;
    if (has_next) issue(nrun, nt0);
    const char* ks = ks2[t & 1];
    const char* vs = vs2[t & 1];
    const int valid = min(kTile, a.seg[run].len - t0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
      for (int j = 0; j < D / 16; ++j) {
        const bf16x8 ka = row_read<KT>(ks, kb * 32 + r32, 2 * j + half);
        const char* vb = vs + j * 16 * VT::RB;
        const bf16x8 va = __builtin_shufflevector(tr_read(vb + voff[kb][0]), tr_read(vb + voff[kb][1]), 0, 1, 2, 3, 4, 5, 6, 7);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[j], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, dof[j], dp, 0, 0, 0);
      }
      float ds[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kb * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
        const float pr = key < valid ? __builtin_amdgcn_exp2f(s[e] - lse2) : 0.f;
        ds[e] = pr * (dp[e] - dl);
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 b = pack8(ds, s2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D, KT>(ks, 2 * kb + s2, toff, db), b, dq[db], 0, 0, 0);
      }
    }
    if (has_next) stage(ks2[(t + 1) & 1], vs2[(t + 1) & 1]);
    __syncthreads();
    if (!has_next) break;
    run = nrun;
    t0 = nt0;
  }
  if (!q_ok) return;
  float* out = p.dq + qrow;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d0 = db * 32 + 8 * gq + 4 * half;
      *reinterpret_cast<float4*>(out + d0) = make_float4(dq[db][4 * gq] * a.scale, dq[db][4 * gq + 1] * a.scale,
                                                         dq[db][4 * gq + 2] * a.scale, dq[db][4 * gq + 3] * a.scale);
    }
}

// ---------------------------------------------------------------------------
// dK, dV of the current chunk (the last run)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_dkv_kernel(AttnBwdArgs p) {
  using QT = RowTile<D, false>;  // padded: the swizzle's address arithmetic spills here
  constexpr int NV = D / 8;
  __shared__ __attribute__((aligned(16))) char qs[QT::kBytes];   // Q' rows
  __shared__ __attribute__((aligned(16))) char gs[QT::kBytes];   // dO rows
  __shared__ __attribute__((aligned(16))) float lse2s[kTile];
  __shared__ __attribute__((aligned(16))) float dls[kTile];
  const AttnArgs& a = p.a;
  const KvSeg& cur = a.seg[a.n_seg - 1];
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, r32 = lane & 31, half = lane >> 5;
  const int key = blockIdx.x * kBwdBK + wave * 32 + r32;
  const bool k_ok = key < cur.len;
  const float c = a.scale * kLog2e;

  // B operands: K and V of the lane's key, d = 16j + 8*half .. +7.
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const int64_t off = int64_t(key) * cur.row_stride + int64_t(head) * cur.head_stride;
    const u32x4* kp = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(cur.k) + off);
    const u32x4* vp = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(cur.v) + off);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      kf[j] = __builtin_bit_cast(bf16x8, k_ok ? kp[2 * j + half] : u32x4{0, 0, 0, 0});
      vf[j] = __builtin_bit_cast(bf16x8, k_ok ? vp[2 * j + half] : u32x4{0, 0, 0, 0});
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[i][r] = dv[i][r] = 0.f;
  int toff[2][D / 32];
  tr_offsets<D, QT>(lane, toff);
  const __bf16* q = static_cast<const __bf16*>(a.q);
  const __bf16* g = static_cast<const __bf16*>(p.dout);

  for (int q0 = 0; q0 < a.n_q; q0 += kTile) {
    __syncthreads();
#pragma unroll
    for (int it = tid; it < kTile * NV; it += kBwdThreads) {
      const int row = it / NV, vec = it % NV;
      const int qi = q0 + row;
      u32x4 wq = {0, 0, 0, 0}, wg = {0, 0, 0, 0};
      if (qi < a.n_q) {
        const int64_t e = (int64_t(qi) * a.H + head) * D + vec * 8;
        wq = *reinterpret_cast<const u32x4*>(q + e);
        wg = *reinterpret_cast<const u32x4*>(g + e);
      }
      *reinterpret_cast<bf16x8*>(qs + QT::off(row, vec)) = scale_bf16x8(wq, c);
      *reinterpret_cast<u32x4*>(gs + QT::off(row, vec)) = wg;
    }
    if (tid < kTile) {
      const int qi = q0 + tid;
      lse2s[tid] = qi < a.n_q ? p.lse[int64_t(head) * a.n_q + qi] * kLog2e : INFINITY;
      dls[tid] = qi < a.n_q ? p.delta[int64_t(head) * a.n_q + qi] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
      for (int j = 0; j < D / 16; ++j) {
        const bf16x8 qa = row_read<QT>(qs, qb * 32 + r32, 2 * j + half);
        const bf16x8 ga = row_read<QT>(gs, qb * 32 + r32, 2 * j + half);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[j], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf[j], dp, 0, 0, 0);
      }
      // rows of the accumulators: queries qb*32 + 8*(e >> 2) + 4*half + (e & 3)
      float pr[16], ds[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int q4 = qb * 32 + 8 * g4 + 4 * half;
        const float4 l4 = *reinterpret_cast<const float4*>(&lse2s[q4]);
        const float4 d4 = *reinterpret_cast<const float4*>(&dls[q4]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * g4 + i;
          pr[e] = __builtin_amdgcn_exp2f(s[e] - lv[i]);
          ds[e] = pr[e] * (dp[e] - dv4[i]);
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 pb = pack8(pr, s2);
        const bf16x8 db8 = pack8(ds, s2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D, QT>(gs, 2 * qb + s2, toff, db), pb, dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D, QT>(qs, 2 * qb + s2, toff, db), db8, dk[db], 0, 0, 0);
        }
      }
    }
  }
  if (!k_ok) return;
  // dK = scale dS^T Q = (dS^T Q') / log2 e
  const float kscale = 1.f / kLog2e;
  const int64_t orow = (int64_t(key) * a.H + head) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d0 = db * 32 + 8 * gq + 4 * half;
      *reinterpret_cast<float4*>(p.dv + orow + d0) =
          make_float4(dv[db][4 * gq], dv[db][4 * gq + 1], dv[db][4 * gq + 2], dv[db][4 * gq + 3]);
      *reinterpret_cast<float4*>(p.dk + orow + d0) =
          make_float4(dk[db][4 * gq] * kscale, dk[db][4 * gq + 1] * kscale, dk[db][4 * gq + 2] * kscale,
                      dk[db][4 * gq + 3] * kscale);
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
  err = launch(bwd_dq_kernel<D>, dim3((a.n_q + kBwdBQ - 1) / kBwdBQ, a.H), dim3(kBwdThreads), &p, stream);
  if (err || !p.dk) return err;
  const int len = a.seg[a.n_seg - 1].len;
  return launch(bwd_dkv_kernel<D>, dim3((len + kBwdBK - 1) / kBwdBK, a.H), dim3(kBwdThreads), &p, stream);
}

}  // namespace

int launch_attention_bwd(const AttnBwdArgs& p, void* stream) {
  if (p.a.n_q <= 0) return 0;
  return p.a.D == 64 ? launch_bwd_d<64>(p, stream) : launch_bwd_d<128>(p, stream);
}

}  // namespace ll
