// HIP kernels for gfx950 (MI355X): sink + short-window attention (also used
// for text cross-attention) and the cache chunk writers (append / recache,
// copy or int8 quantise).
//
// Attention (LongLive: Real-time Interactive Long Video Generation, §3.3):
// one softmax over the union of the frame-sink tokens, the resident window
// chunks and the current chunk, no mask inside the set.  The key set arrives
// as a table of runs (KvSeg) that point into the cache or the caller's
// buffers, so nothing is concatenated; a key tile may straddle runs.
//
// Per workgroup: 4 waves x 32 queries of one head.  Per key tile of 64 keys:
//   S^T[key][q] = K Q^T      bf16 MFMA 32x32x16 (A = K tile from LDS, B = Q
//                            kept in registers); each lane owns one query and
//                            16 keys per 32-key block, so row max / row sum
//                            are lane-local plus one exchange between the two
//                            32-lane halves.
//   online softmax in the log2 domain, rescaling O only when the running max
//   grows by more than 2^8 (exact: any reference max works, the bound only
//   keeps P in bf16/fp32 range).
//   O^T[d][q] += V^T P^T      bf16 MFMA; B = P straight from the S^T
//                            accumulators, A = V^T read from LDS.  V is
//                            transposed while it is staged into LDS, with the
//                            keys of each 16-key group permuted so each lane's
//                            8 keys are contiguous.
// fp32 activations use the fp32 MFMA 32x32x2 with the same structure.
// INT8 runs are converted exactly to bf16 (|q| <= 127) while staged; the K
// scale multiplies the score, the V scale multiplies P before the bf16 cast.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "launch.hpp"

namespace ll {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // queries per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;

// Physical LDS column of logical key k inside a 16-key group: swap bits 2, 3.
__device__ __forceinline__ int vt_col(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Pointers to key `key`'s K and V rows for head `head` (null past the end).
__device__ __forceinline__ void key_rows(const AttnArgs& a, int head, int key, int elt,
                                         const char*& kp, const char*& vp,
                                         const float*& ksp, const float*& vsp, int& quant) {
  kp = vp = nullptr;
  ksp = vsp = nullptr;
  quant = 0;
  for (int i = 0; i < a.n_seg; ++i) {
    const KvSeg& s = a.seg[i];
    const int rel = key - s.key_start;
    if (rel >= 0 && rel < s.len) {
      const int e = s.quant ? 1 : elt;
      const int64_t off = (int64_t(head) * s.head_stride + int64_t(rel) * s.row_stride) * e;
      kp = static_cast<const char*>(s.k) + off;
      vp = static_cast<const char*>(s.v) + off;
      if (s.quant) {
        ksp = s.ks + int64_t(head) * s.sc_head_stride + rel;
        vsp = s.vs + int64_t(head) * s.sc_head_stride + rel;
      }
      quant = s.quant;
    }
  }
}

__device__ __forceinline__ uint4 int8x8_to_bf16x8(uint2 w) {
  // int8 -> fp32 -> bf16 is exact for |q| <= 127.
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t src = i < 2 ? w.x : w.y;
    const int sh = (i & 1) * 16;
    const float f0 = float(int8_t((src >> sh) & 0xff));
    const float f1 = float(int8_t((src >> (sh + 8)) & 0xff));
    const uint32_t b0 = __builtin_bit_cast(uint32_t, f0) >> 16;  // exact: low bits are 0
    const uint32_t b1 = __builtin_bit_cast(uint32_t, f1) >> 16;
    o[i] = b0 | (b1 << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

template <typename Act, int D>
struct Smem;

template <int D>
struct Smem<__bf16, D> {
  static constexpr int KS = D + 8;    // K row stride (elements)
  static constexpr int VS = kBN + 8;  // V^T row stride (elements)
  __bf16 k[kBN * KS];
  __bf16 vt[D * VS];
  float ksc[kBN];
  float vsc[kBN];
};

template <int D>
struct Smem<float, D> {
  static constexpr int KS = D + 4;
  float k[kBN * KS];
  float v[kBN * KS];
};

template <typename Act, int D, bool kQ8>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
  constexpr bool kF32 = std::is_same<Act, float>::value;
  static_assert(!(kF32 && kQ8), "int8 K/V pairs with bf16 activations");
  constexpr int kElt = sizeof(Act);
  constexpr int kVpr = D * kElt / 16;  // 16-byte vectors per row
  using S = Smem<Act, D>;
  __shared__ __attribute__((aligned(16))) S sm;

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

  // Q fragment in registers: B operand of S^T = K Q^T.
  constexpr int kQf = kF32 ? D / 2 : D / 16;
  typename std::conditional<kF32, float, bf16x8>::type qf[kQf];
  if constexpr (kF32) {
    const float* q = static_cast<const float*>(a.q) + qrow;
#pragma unroll
    for (int j = 0; j < kQf; ++j) qf[j] = q_ok ? q[2 * j + half] : 0.f;
  } else {
    const uint4* q = reinterpret_cast<const uint4*>(static_cast<const __bf16*>(a.q) + qrow);
#pragma unroll
    for (int j = 0; j < kQf; ++j) {
      uint4 w = q_ok ? q[2 * j + half] : make_uint4(0, 0, 0, 0);
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

  for (int t0 = 0; t0 < a.n_keys; t0 += kBN) {
    __syncthreads();  // the previous tile has been consumed
    // ---- stage K (and V / V^T) rows of this tile into LDS ----
    if constexpr (kF32) {
      constexpr int kItems = kBN * kVpr / kThreads;
#pragma unroll
      for (int it = 0; it < kItems; ++it) {
        const int item = tid + it * kThreads;
        const int row = item / kVpr, vec = item % kVpr;
        const char *kp, *vp; const float *ksp, *vsp; int qt;
        key_rows(a, head, t0 + row, kElt, kp, vp, ksp, vsp, qt);
        uint4 kw = make_uint4(0, 0, 0, 0), vw = kw;
        if (kp) {
          kw = reinterpret_cast<const uint4*>(kp)[vec];
          vw = reinterpret_cast<const uint4*>(vp)[vec];
        }
        *reinterpret_cast<uint4*>(&sm.k[row * S::KS + vec * 4]) = kw;
        *reinterpret_cast<uint4*>(&sm.v[row * S::KS + vec * 4]) = vw;
      }
    } else {
      constexpr int kVec = D / 8;  // 8 bf16 per 16-byte vector
      constexpr int kItems = kBN * kVec / kThreads;
#pragma unroll
      for (int it = 0; it < kItems; ++it) {
        const int item = tid + it * kThreads;
        const int row = item / kVec, vec = item % kVec;
        const char *kp, *vp; const float *ksp, *vsp; int qt;
        key_rows(a, head, t0 + row, kElt, kp, vp, ksp, vsp, qt);
        uint4 kw = make_uint4(0, 0, 0, 0);
        if (kp) {
          if (kQ8 && qt) kw = int8x8_to_bf16x8(reinterpret_cast<const uint2*>(kp)[vec]);
          else kw = reinterpret_cast<const uint4*>(kp)[vec];
        }
        *reinterpret_cast<uint4*>(&sm.k[row * S::KS + vec * 8]) = kw;
        if (kQ8 && vec == 0) {
          sm.ksc[row] = kp ? (qt ? *ksp : 1.f) : 0.f;
          sm.vsc[row] = kp ? (qt ? *vsp : 1.f) : 0.f;
        }
      }
      // V^T: a thread takes two adjacent keys x one 8-wide d vector and
      // writes 8 words of (key, key+1) pairs.
      constexpr int kPairs = kBN / 2 * kVec / kThreads;
#pragma unroll
      for (int it = 0; it < kPairs; ++it) {
        const int item = tid + it * kThreads;
        const int pr = item / kVec, vec = item % kVec;
        const int k0 = 2 * pr;
        uint4 w[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const char *kp, *vp; const float *ksp, *vsp; int qt;
          key_rows(a, head, t0 + k0 + u, kElt, kp, vp, ksp, vsp, qt);
          w[u] = make_uint4(0, 0, 0, 0);
          if (vp) {
            if (kQ8 && qt) w[u] = int8x8_to_bf16x8(reinterpret_cast<const uint2*>(vp)[vec]);
            else w[u] = reinterpret_cast<const uint4*>(vp)[vec];
          }
        }
        const uint32_t a4[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
        const uint32_t b4[4] = {w[1].x, w[1].y, w[1].z, w[1].w};
        const int col = vt_col(k0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t x = a4[e >> 1], y = b4[e >> 1];
          const uint32_t word = (e & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
          *reinterpret_cast<uint32_t*>(&sm.vt[(vec * 8 + e) * S::VS + col]) = word;
        }
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for two 32-key blocks ----
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
    if constexpr (kF32) {
#pragma unroll
      for (int j = 0; j < kQf; ++j) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const float ka = sm.k[(kb * 32 + r32) * S::KS + 2 * j + half];
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(ka, qf[j], s[kb], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kQf; ++j) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&sm.k[(kb * 32 + r32) * S::KS + j * 16 + half * 8]);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[j], s[kb], 0, 0, 0);
        }
      }
    }

    // Lane (q = r32, half) holds keys kb*32 + 8*(r/4) + 4*half + r%4.
    if constexpr (kQ8) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 sc = *reinterpret_cast<const float4*>(&sm.ksc[kb * 32 + 8 * g + 4 * half]);
          s[kb][4 * g + 0] *= sc.x; s[kb][4 * g + 1] *= sc.y;
          s[kb][4 * g + 2] *= sc.z; s[kb][4 * g + 3] *= sc.w;
        }
    }
    if (t0 + kBN > a.n_keys) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= a.n_keys) s[kb][r] = -INFINITY;
        }
    }

    // ---- online softmax (log2 domain) ----
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const bool need = (m_new - m_run) * c > kRescaleLog2;
    if (__ballot(need)) {
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
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -mc));
        l_run += p;
        s[kb][r] = p;
      }

    // ---- O^T += V^T P^T ----
    if constexpr (kF32) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const float va = sm.v[key * S::KS + db * 32 + r32];
            o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, s[kb][r], o[db], 0, 0, 0);
          }
        }
    } else {
      if constexpr (kQ8) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 sc = *reinterpret_cast<const float4*>(&sm.vsc[kb * 32 + 8 * g + 4 * half]);
            s[kb][4 * g + 0] *= sc.x; s[kb][4 * g + 1] *= sc.y;
            s[kb][4 * g + 2] *= sc.z; s[kb][4 * g + 3] *= sc.w;
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          bf16x8 pb;
#pragma unroll
          for (int i = 0; i < 8; ++i) pb[i] = static_cast<__bf16>(s[kb][8 * t + i]);
          const int step = kb * 2 + t;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const bf16x8 va = *reinterpret_cast<const bf16x8*>(&sm.vt[(db * 32 + r32) * S::VS + step * 16 + half * 8]);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[db], 0, 0, 0);
          }
        }
    }
  }

  // ---- epilogue: O = O^T / l, optional LSE ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!q_ok) return;
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = db * 32 + 8 * g + 4 * half;
      if constexpr (kF32) {
        float4 v = make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                               o[db][4 * g + 3] * inv);
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + qrow + d0) = v;
      } else {
        const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(o[db][4 * g] * inv)) |
                            (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(o[db][4 * g + 1] * inv))) << 16);
        const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(o[db][4 * g + 2] * inv)) |
                            (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(o[db][4 * g + 3] * inv))) << 16);
        *reinterpret_cast<uint2*>(static_cast<__bf16*>(a.out) + qrow + d0) = make_uint2(lo, hi);
      }
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

}  // namespace

int launch_attention(const AttnArgs& a, void* stream) {
  if (a.n_q <= 0) return 0;
  const dim3 grid((a.n_q + kBM - 1) / kBM, a.H);
  const dim3 block(kThreads);
  if (a.act == LL_F32) {
    if (a.D == 64) return launch(attn_kernel<float, 64, false>, grid, block, &a, stream);
    return launch(attn_kernel<float, 128, false>, grid, block, &a, stream);
  }
  if (a.kv == LL_I8) {
    if (a.D == 64) return launch(attn_kernel<__bf16, 64, true>, grid, block, &a, stream);
    return launch(attn_kernel<__bf16, 128, true>, grid, block, &a, stream);
  }
  if (a.D == 64) return launch(attn_kernel<__bf16, 64, false>, grid, block, &a, stream);
  return launch(attn_kernel<__bf16, 128, false>, grid, block, &a, stream);
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
