// HIP kernels for gfx950 (MI355X): sink + short-window attention (also used
// for text cross-attention) and the cache chunk writers (append / recache,
// copy or int8 quantise).
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
// bf16 kernel, per workgroup: 4 waves x 32 queries of one head.  Per tile:
//   S^T[key][q] = K Q^T      bf16 MFMA 32x32x16, A = K rows from LDS, B = the
//                            wave's Q fragment kept in registers.  Each lane
//                            owns one query and 16 keys per 32-key block, so
//                            row max / row sum are lane-local plus one swap
//                            between the two 32-lane halves.
//   online softmax in the log2 domain; O is rescaled only when the running
//   max grows by more than 2^8 (exact: any reference max works, the bound
//   keeps P within bf16/fp32 range).
//   O^T[d][q] += V^T P^T     bf16 MFMA; B = P straight from the S^T
//                            accumulators; A = V^T produced from row-major V
//                            in LDS by the gfx950 transpose read
//                            (ds_read_b64_tr_b16).
// K/V tiles are staged through registers into a double-buffered LDS: the next
// tile's global loads are in flight while the current tile is computed, with
// one barrier per tile.
// INT8 runs are converted exactly to bf16 (|q| <= 127) while staged; the K
// scale multiplies the score and the V scale multiplies P before its bf16
// cast.  fp32 activations use a plainer kernel with the fp32 MFMA 32x32x2.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "launch.hpp"

namespace ll {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x8 __attribute__((__vector_size__(8 * sizeof(float))));
typedef unsigned int u32x4 __attribute__((__vector_size__(4 * sizeof(unsigned))));
typedef unsigned int u32x2 __attribute__((__vector_size__(2 * sizeof(unsigned))));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // queries per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

// Combine a per-lane value with the one held by lane l^32 (the other half of
// the wave, which owns the same query column).
__device__ __forceinline__ float swap_halves_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float swap_halves_sum(float x) { return x + __shfl_xor(x, 32); }

// gfx950 LDS transpose read of 4 bf16.  Within each group of 16 lanes, lane
// i receives element (i & 3) of the 8 bytes addressed by lane 4*e + (i >> 2),
// for e = 0..3.
__device__ __forceinline__ bf16x4 tr_read(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// 8 int8 -> 8 bf16, exact for |q| <= 127.
__device__ __forceinline__ u32x4 int8x8_to_bf16x8(u32x2 w) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t src = i < 2 ? w[0] : w[1];
    const int sh = (i & 1) * 16;
    const float f0 = float(int8_t((src >> sh) & 0xff));
    const float f1 = float(int8_t((src >> (sh + 8)) & 0xff));
    o[i] = (__builtin_bit_cast(uint32_t, f0) >> 16) | (__builtin_bit_cast(uint32_t, f1) & 0xffff0000u);
  }
  return o;
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

__device__ __forceinline__ int count_tiles(const AttnArgs& a) {
  int n = 0;
  for (int r = 0; r < a.n_seg; ++r) n += (a.seg[r].len + kBN - 1) / kBN;
  return n;
}

// ---------------------------------------------------------------------------
// bf16 activations (bf16 or int8 cache)
// ---------------------------------------------------------------------------
template <int D>
struct Bf16Stage {
  static constexpr int KS = D + 8;   // K row stride (elements): rows shift by 4 banks
  static constexpr int VS = D + 32;  // V row stride (elements): rows shift by 16 banks
  __bf16 k[kBN * KS];
  __bf16 v[kBN * VS];
  float ksc[kBN];
  float vsc[kBN];
};

// Per-thread share of one tile: kItems 16-byte vectors of K and of V.
template <int D>
struct Bf16Regs {
  static constexpr int kVec = D / 8;                   // 8 bf16 per vector
  static constexpr int kItems = kBN * kVec / kThreads; // per thread
  u32x4 k[kItems];  // bf16 rows, or raw int8 bytes in the low 8 bytes
  u32x4 v[kItems];
  float ks, vs;
  bool q8;          // the staged tile comes from an int8 run
};

template <int D, bool kQ8>
__device__ __forceinline__ void load_tile_bf16(const AttnArgs& a, int head, TileCursor cur,
                                               Bf16Regs<D>& r) {
  using R = Bf16Regs<D>;
  const KvSeg& s = a.seg[cur.run];
  const int tid = threadIdx.x;
  const int row0 = cur.tile * kBN;
  const bool q8 = kQ8 && s.quant;
  const int elt = q8 ? 1 : 2;
  const uint32_t rs = uint32_t(s.row_stride) * elt;
  const char* kb = static_cast<const char*>(s.k) + int64_t(head) * s.head_stride * elt;
  const char* vb = static_cast<const char*>(s.v) + int64_t(head) * s.head_stride * elt;
  const uint32_t bytes = uint32_t(s.len) * rs;
  const auto rk = make_rsrc(kb, bytes);
  const auto rv = make_rsrc(vb, bytes);
#pragma unroll
  for (int it = 0; it < R::kItems; ++it) {
    const int item = tid + it * kThreads;
    const int row = item / R::kVec, vec = item % R::kVec;
    const uint32_t off = uint32_t(row0 + row) * rs;
    if (q8) {
      // converted when staged into LDS, so the loads stay in flight
      const u32x2 kq = __builtin_amdgcn_raw_buffer_load_b64(rk, off + vec * 8, 0, 0);
      const u32x2 vq = __builtin_amdgcn_raw_buffer_load_b64(rv, off + vec * 8, 0, 0);
      r.k[it] = u32x4{kq[0], kq[1], 0, 0};
      r.v[it] = u32x4{vq[0], vq[1], 0, 0};
    } else {
      r.k[it] = __builtin_amdgcn_raw_buffer_load_b128(rk, off + vec * 16, 0, 0);
      r.v[it] = __builtin_amdgcn_raw_buffer_load_b128(rv, off + vec * 16, 0, 0);
    }
  }
  r.q8 = q8;
  if constexpr (kQ8) {
    // one scale per key row: threads 0..63 load the K and V scales
    const int row = tid & (kBN - 1);
    if (q8) {
      const uint32_t sb = uint32_t(s.len) * 4;
      const auto rks = make_rsrc(s.ks + int64_t(head) * s.sc_head_stride, sb);
      const auto rvs = make_rsrc(s.vs + int64_t(head) * s.sc_head_stride, sb);
      r.ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rks, uint32_t(row0 + row) * 4, 0, 0));
      r.vs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvs, uint32_t(row0 + row) * 4, 0, 0));
    } else {
      r.ks = 1.f;
      r.vs = 1.f;
    }
  }
}

template <int D, bool kQ8>
__device__ __forceinline__ void store_tile_bf16(Bf16Stage<D>& st, const Bf16Regs<D>& r) {
  using R = Bf16Regs<D>;
  using S = Bf16Stage<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < R::kItems; ++it) {
    const int item = tid + it * kThreads;
    const int row = item / R::kVec, vec = item % R::kVec;
    u32x4 kw = r.k[it], vw = r.v[it];
    if (kQ8 && r.q8) {
      kw = int8x8_to_bf16x8(u32x2{kw[0], kw[1]});
      vw = int8x8_to_bf16x8(u32x2{vw[0], vw[1]});
    }
    *reinterpret_cast<u32x4*>(&st.k[row * S::KS + vec * 8]) = kw;
    *reinterpret_cast<u32x4*>(&st.v[row * S::VS + vec * 8]) = vw;
  }
  if constexpr (kQ8) {
    if (tid < kBN) {
      st.ksc[tid] = r.ks;
      st.vsc[tid] = r.vs;
    }
  }
}

template <int D, bool kQ8, bool kOneRun>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(AttnArgs a) {
  using S = Bf16Stage<D>;
  __shared__ __attribute__((aligned(16))) S stage[2];

  const int head = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r32 = lane & 31;
  const int half = lane >> 5;
  const int qi = blockIdx.x * kBM + wave * 32 + r32;
  const bool q_ok = qi < a.n_q;
  const float c = a.scale * kLog2e;
  const int64_t qrow = (int64_t(qi) * a.H + head) * D;

  // Q fragment (B operand of S^T = K Q^T): lane holds Q[q][16j + 8*half + 0..7].
  bf16x8 qf[D / 16];
  {
    const u32x4* q = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(a.q) + qrow);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const u32x4 w = q_ok ? q[2 * j + half] : u32x4{0, 0, 0, 0};
      qf[j] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  // Lane-constant LDS offsets (elements).
  // K A-operand: row = kb*32 + r32, cols 16j + 8*half.
  const int k_off = r32 * S::KS + 8 * half;
  // V transpose read: 16-lane group g, lane j in group.  The group reads rows
  // 4*(g>>1) + (j>>2) (+ 16*step + 8*a) at cols 16*(g&1) + 4*(j&3) (+ 32*db);
  // lane receives V[4 consecutive keys][d = 32*db + (lane & 31)].
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_off = (4 * (g16 >> 1) + (j16 >> 2)) * S::VS + 16 * (g16 & 1) + 4 * (j16 & 3);

  const int n_tiles = kOneRun ? (a.seg[0].len + kBN - 1) / kBN : count_tiles(a);
  TileCursor ld{0, 0};       // next tile to load
  TileCursor cu{0, 0};       // tile being computed
  Bf16Regs<D> regs;
  load_tile_bf16<D, kQ8>(a, head, ld, regs);
  ld.advance(a);
  store_tile_bf16<D, kQ8>(stage[0], regs);
  if (n_tiles > 1) {
    load_tile_bf16<D, kQ8>(a, head, ld, regs);
    ld.advance(a);
  }
  __syncthreads();

  for (int g = 0; g < n_tiles; ++g) {
    S& st = stage[g & 1];
    // Stage tile g+1 (already in registers) and start loading tile g+2.
    if (g + 1 < n_tiles) {
      store_tile_bf16<D, kQ8>(stage[(g + 1) & 1], regs);
      if (g + 2 < n_tiles) {
        load_tile_bf16<D, kQ8>(a, head, ld, regs);
        ld.advance(a);
      }
    }
    const int valid = min(kBN, a.seg[cu.run].len - cu.tile * kBN);
    cu.advance(a);

    // ---- S^T = K Q^T for two 32-key blocks ----
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&st.k[k_off + kb * 32 * S::KS + 16 * j]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[j], s[kb], 0, 0, 0);
      }
    }

    // Lane (q = r32, half) holds keys kb*32 + 8*(r/4) + 4*half + r%4.
    if constexpr (kQ8) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const float4 sc = *reinterpret_cast<const float4*>(&st.ksc[kb * 32 + 8 * gq + 4 * half]);
          s[kb][4 * gq + 0] *= sc.x; s[kb][4 * gq + 1] *= sc.y;
          s[kb][4 * gq + 2] *= sc.z; s[kb][4 * gq + 3] *= sc.w;
        }
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

    // ---- online softmax (log2 domain) ----
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = swap_halves_max(mx);
    const float m_new = fmaxf(m_run, mx);
    if (__builtin_amdgcn_ballot_w64((m_new - m_run) * c > kRescaleLog2)) {
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
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
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -mc));
        l_run += p;
        s[kb][r] = p;
      }
    if constexpr (kQ8) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const float4 sc = *reinterpret_cast<const float4*>(&st.vsc[kb * 32 + 8 * gq + 4 * half]);
          s[kb][4 * gq + 0] *= sc.x; s[kb][4 * gq + 1] *= sc.y;
          s[kb][4 * gq + 2] *= sc.z; s[kb][4 * gq + 3] *= sc.w;
        }
    }

    // ---- O^T += V^T P^T: 4 steps of 16 keys ----
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      const f32x16& sv = s[step >> 1];
      const int t8 = 8 * (step & 1);
      f32x8 pf;
#pragma unroll
      for (int i = 0; i < 8; ++i) pf[i] = sv[t8 + i];
      const bf16x8 pb = __builtin_convertvector(pf, bf16x8);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int base = v_off + 16 * step * S::VS + 32 * db;
        const bf16x4 lo = tr_read(&st.v[base]);
        const bf16x4 hi = tr_read(&st.v[base + 8 * S::VS]);
        const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[db], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, optional LSE ----
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
  if (a.lse && half == 0) a.lse[int64_t(head) * a.n_q + qi] = (m_run * c + __log2f(l_tot)) * kLn2;
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
  const int qi = blockIdx.x * kBM + wave * 32 + r32;
  const bool q_ok = qi < a.n_q;
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
  const int n_tiles = count_tiles(a);
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
// Cache writers.  Grid: x over (head, row, 16-byte vector) of one chunk,
// y = chunk * 2 + (0: K, 1: V), z = layer.  Destination rows are contiguous
// per head (coalesced writes); each source row is one contiguous D-vector.
// ---------------------------------------------------------------------------
template <int kElt>
__global__ __launch_bounds__(256) void copy_chunks_kernel(CopyArgs a) {
  const int vpr = a.D * kElt / 16;
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = int64_t(a.ctok) * a.H * vpr;
  if (e >= total) return;
  const int chunk = blockIdx.y >> 1;
  const int isv = blockIdx.y & 1;
  const int z = blockIdx.z;
  const int vec = int(e % vpr);
  const int64_t rh = e / vpr;
  const int row = int(rh % a.ctok);
  const int h = int(rh / a.ctok);
  const char* src = static_cast<const char*>(isv ? a.src_v : a.src_k) +
                    (int64_t(z) * a.src_layer_elems + (int64_t(chunk) * a.ctok + row) * a.H * a.D +
                     int64_t(h) * a.D) * kElt + vec * 16;
  char* dst = a.dst + int64_t(z) * a.dst_layer_bytes + (isv ? a.v_off : a.k_off) +
              ((int64_t(h) * a.rows + a.dst_row0[chunk] + row) * a.D) * kElt + vec * 16;
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

// INT8 writer: one group of D/8 lanes per (head, row); each lane quantises
// 8 values.  s = max|x| / 127 (IEEE fp32 division), q = clamp(rne(x / s)).
__global__ __launch_bounds__(256) void quant_chunks_kernel(CopyArgs a) {
  const int gl = a.D / 8;
  const int64_t grp = (int64_t(blockIdx.x) * 256 + threadIdx.x) / gl;
  const int li = threadIdx.x % gl;
  const bool valid = grp < int64_t(a.ctok) * a.H;
  const int chunk = blockIdx.y >> 1;
  const int isv = blockIdx.y & 1;
  const int z = blockIdx.z;
  const int row = valid ? int(grp % a.ctok) : 0;
  const int h = valid ? int(grp / a.ctok) : 0;
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
  for (int m = 1; m < gl; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
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

template <int D>
int launch_attention_d(const AttnArgs& a, dim3 grid, void* stream) {
  const dim3 block(kThreads);
  if (a.act == LL_F32) return launch(attn_f32_kernel<D>, grid, block, &a, stream);
  if (a.kv == LL_I8) return launch(attn_bf16_kernel<D, true, false>, grid, block, &a, stream);
  if (a.n_seg == 1) return launch(attn_bf16_kernel<D, false, true>, grid, block, &a, stream);
  return launch(attn_bf16_kernel<D, false, false>, grid, block, &a, stream);
}

}  // namespace

int launch_attention(const AttnArgs& a, void* stream) {
  if (a.n_q <= 0) return 0;
  const dim3 grid((a.n_q + kBM - 1) / kBM, a.H);
  return a.D == 64 ? launch_attention_d<64>(a, grid, stream) : launch_attention_d<128>(a, grid, stream);
}

int launch_copy_chunks(const CopyArgs& a, void* stream) {
  if (a.n_chunks <= 0) return 0;
  if (a.kv == LL_I8) {
    const int64_t threads = int64_t(a.ctok) * a.H * (a.D / 8);
    const dim3 grid(unsigned((threads + 255) / 256), a.n_chunks * 2, a.n_layers);
    return launch(quant_chunks_kernel, grid, dim3(256), &a, stream);
  }
  const int elt = a.act == LL_F32 ? 4 : 2;
  const int64_t threads = int64_t(a.ctok) * a.H * (a.D * elt / 16);
  const dim3 grid(unsigned((threads + 255) / 256), a.n_chunks * 2, a.n_layers);
  if (elt == 4) return launch(copy_chunks_kernel<4>, grid, dim3(256), &a, stream);
  return launch(copy_chunks_kernel<2>, grid, dim3(256), &a, stream);
}

const char* hip_error_string(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

}  // namespace ll
