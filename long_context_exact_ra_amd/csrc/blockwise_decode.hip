// One incremental-decoding step of Ring Attention over a KV cache, for bf16
// and float32 inputs ("RingAttention与传统注意力机制对比为什么它是大语言模型
// 的终极解决方案", sections "3. 推理成本显著降低" and "关键参数配置": the
// inference cache index cache_idx; "从论文到代码：深入理解RingAttention的块
// 注意力计算逻辑", section "RingAttention的算法原理": cache_idx beside the
// segment ids in the ring forward's arguments).
//
// The step's n_new query tokens sit at positions cache_idx .. cache_idx +
// n_new - 1 and their keys and values already in the cache rows of those
// positions; query t attends to cache rows 0 .. cache_idx + t (token causal,
// "3. 因果注意力掩码支持") with exact softmax(q K^T / sqrt(D)) V.
//
// A decoding step reads every valid cache row once and does 4 D flop per
// (query, key) pair: for a handful of queries it is bound by HBM bandwidth,
// not by the matrix cores.  So the kernel streams K and V rows straight into
// registers with whole-row loads (LPR lanes x 16 bytes = one row of one
// head) and does the arithmetic on the vector ALUs:
//   * a group of LPR lanes owns one key per step: each lane holds 16 bytes
//     of the key's row and of the value row, forms its share of q.k for
//     each query (bf16: v_dot2_f32_bf16, exact products, float32 sums) and
//     the group sums the shares with DPP row operations (every lane ends
//     with the full logit);
//   * each group keeps, per query, the running max (base 2, kept lazily:
//     it moves only when a logit would exceed it by 2^8, as in the forward),
//     the denominator and its 8 (bf16) or 4 (float32) columns of the
//     numerator ("2. 数值稳定的注意力计算": the carry and its correction);
//   * the groups of a workgroup walk interleaved keys of one contiguous key
//     range, U keys each per iteration, loaded one iteration ahead with
//     nontemporal loads, and fold their carries at the end (within a wave by
//     lane exchanges, across waves through LDS).
// Key splits: the valid cache rows are cut into key_splits contiguous
// ranges, one workgroup each per (batch, head, group of NQ queries); with
// more than one split, each workgroup writes its kept max, denominator and
// unnormalised numerator, and decode_combine_kernel folds the splits with
// the same carry (the ring's fold of per-block partials: the blocks may be
// folded in any order, "Ring Attention with Blockwise Transformers for
// Near-Infinite Context", section 三, 排列不变性).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ra_device.h"
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int kDecThreads = 256;  // 4 waves
constexpr int kDecWaves = kDecThreads / 64;
// Largest log2 of a probability weight before the running max must move.
constexpr float kDecLazy = 8.f;

// 16 bytes of a row: 8 bf16 or 4 float32.
template <typename T>
struct Slice;
template <>
struct Slice<__bf16> {
  using vec = bf16x8_t;
  static constexpr int kElems = 8;
};
template <>
struct Slice<float> {
  using vec = float4;
  static constexpr int kElems = 4;
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the LPR consecutive lanes of a group (LPR = 8, 16 or 32): two
// quad exchanges, the half-row mirror (8 lanes), the row mirror (16 lanes)
// and, for 32, one exchange between rows.  Every lane of the group gets
// the sum.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp<0x141>(x);  // row_half_mirror: lane i of 8 reads lane 7 - i
  if constexpr (LPR >= 16) x += dpp<0x140>(x);  // row_mirror: lane i of 16 reads 15 - i
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "group of 8, 16 or 32 lanes");
  return x;
}

// The lane's share of q.k (EPL elements; float32 sum).
__device__ __forceinline__ float dot_share(const bf16x8_t& q, const bf16x8_t& k) {
  float s = __builtin_amdgcn_fdot2_f32_bf16(q.s01, k.s01, 0.f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(q.s23, k.s23, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(q.s45, k.s45, s, false);
  return __builtin_amdgcn_fdot2_f32_bf16(q.s67, k.s67, s, false);
}
__device__ __forceinline__ float dot_share(const float4& q, const float4& k) {
  float s = q.x * k.x;
  s = __builtin_fmaf(q.y, k.y, s);
  s = __builtin_fmaf(q.z, k.z, s);
  return __builtin_fmaf(q.w, k.w, s);
}

__device__ __forceinline__ void to_f32(const bf16x8_t& v, float* f) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (float)v[e];
}
__device__ __forceinline__ void to_f32(const float4& v, float* f) {
  f[0] = v.x;
  f[1] = v.y;
  f[2] = v.z;
  f[3] = v.w;
}

// Weight of a carry with kept max m under the common max mn (0 for an
// empty carry, whose m is -inf).
__device__ __forceinline__ float carry_weight(float m, float mn) {
  return m == ninf() ? 0.f : __builtin_amdgcn_exp2f(m - mn);
}

template <int D, typename T, int NQ>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(const DecParams p) {
  using vec = typename Slice<T>::vec;
  constexpr int EPL = Slice<T>::kElems;  // elements per lane
  constexpr int LPR = D / EPL;           // lanes per row
  constexpr int GPW = 64 / LPR;          // groups (keys per step) per wave
  constexpr int G = kDecWaves * GPW;     // groups per workgroup
  constexpr int U = NQ <= 2 ? 8 : 4;     // keys per group per iteration
  constexpr int KB = G * U;              // keys per workgroup per iteration
  __shared__ float sm_o[kDecWaves][NQ][D];
  __shared__ float sm_ml[kDecWaves][NQ][2];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int part = lane % LPR;
  const int grp = wave * GPW + lane / LPR;
  const int wg = blockIdx.x;
  const int split = wg % p.key_splits;
  const int rest = wg / p.key_splits;
  const int qg = rest % p.q_groups;
  const int bh = rest / p.q_groups;
  const int b = bh / p.heads, h = bh % p.heads;
  const int t0 = qg * NQ;
  const int nq = min(NQ, p.n_new - t0);
  const int64_t kb = (int64_t)split * p.split_keys;
  const int64_t ke = kb + p.split_keys < p.n_keys ? kb + p.split_keys : p.n_keys;
  const int64_t rs = (int64_t)p.heads * D;  // elements per cache or query row
  const int64_t col = (int64_t)h * D + part * EPL;

  vec qv[NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    qv[t] = vec{};
    if (t < nq)
      qv[t] = *reinterpret_cast<const vec*>(static_cast<const T*>(p.q) +
                                           ((int64_t)b * p.n_new + t0 + t) * rs + col);
  }
  float m[NQ], l[NQ], o[NQ][EPL];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    m[t] = ninf();
    l[t] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[t][e] = 0.f;
  }

  const T* kbase = static_cast<const T*>(p.k) + (int64_t)b * p.cache_rows * rs + col;
  const T* vbase = static_cast<const T*>(p.v) + (int64_t)b * p.cache_rows * rs + col;
  // The last position any query of this workgroup sees fully: a block whose
  // keys all lie at or before it, and inside the range, needs no mask.
  const int64_t all_see = p.cache_idx + t0;
  // The K and V slices of one block of keys (rows past the range are
  // clamped onto its last row: read, then masked).  The cache is streamed
  // once: nontemporal loads (82.7 % of the HBM peak on the 7B-shaped step,
  // against 76.0 % with ordinary loads).
  auto load = [&](int64_t base, vec* kd, vec* vd) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t key = base + u * G + grp;
      const int64_t row = key < ke ? key : ke - 1;
      kd[u] = __builtin_bit_cast(
          vec, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kbase + row * rs)));
      vd[u] = __builtin_bit_cast(
          vec, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vbase + row * rs)));
    }
  };
  // Each block's slices are loaded one block ahead: the next block's loads
  // are in flight while this one is computed.
  vec kn[U], vn[U];
  if (kb < ke) load(kb, kn, vn);
  for (int64_t base = kb; base < ke; base += KB) {
    vec kv[U], vv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kv[u] = kn[u];
      vv[u] = vn[u];
    }
    if (base + KB < ke) load(base + KB, kn, vn);
    const bool full = base + KB <= ke && base + KB - 1 <= all_see;
    float x[NQ][U];
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
#pragma unroll
      for (int u = 0; u < U; ++u) x[t][u] = group_sum<LPR>(dot_share(qv[t], kv[u])) * p.scale_log2;
      if (!full) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t key = base + u * G + grp;
          if (key >= ke || key > p.cache_idx + t0 + t) x[t][u] = ninf();
        }
      }
      float bm = x[t][0];
#pragma unroll
      for (int u = 1; u < U; ++u) bm = fmaxf(bm, x[t][u]);
      // The kept max moves only when a weight would exceed 2^kDecLazy (the
      // group's lanes hold equal logits, so they agree).
      if (bm > m[t] + kDecLazy) {
        const float a = carry_weight(m[t], bm);
        l[t] *= a;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[t][e] *= a;
        m[t] = bm;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // (x = -inf gives 0, also while the carry is still empty)
        const float pr = x[t][u] == ninf() ? 0.f : __builtin_amdgcn_exp2f(x[t][u] - m[t]);
        x[t][u] = pr;
        l[t] += pr;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[EPL];
      to_f32(vv[u], vf);
#pragma unroll
      for (int t = 0; t < NQ; ++t)
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[t][e] = __builtin_fmaf(x[t][u], vf[e], o[t][e]);
    }
  }

  // Fold the wave's groups: lanes LPR, 2 LPR, .. apart hold the same columns.
#pragma unroll
  for (int off = LPR; off < 64; off *= 2) {
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      const float m2 = __shfl_xor(m[t], off), l2 = __shfl_xor(l[t], off);
      const float mn = fmaxf(m[t], m2);
      const float a = carry_weight(m[t], mn), a2 = carry_weight(m2, mn);
      l[t] = l[t] * a + l2 * a2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float o2 = __shfl_xor(o[t][e], off);
        o[t][e] = o[t][e] * a + o2 * a2;
      }
      m[t] = mn;
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[wave][t][part * EPL + e] = o[t][e];
      if (lane == 0) {
        sm_ml[wave][t][0] = m[t];
        sm_ml[wave][t][1] = l[t];
      }
    }
  }
  __syncthreads();

  // Fold the waves: thread (t, c) for query t and EPL columns c.
  const int t = threadIdx.x / LPR, c = threadIdx.x % LPR;
  if (t >= nq) return;
  float mn = ninf();
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) mn = fmaxf(mn, sm_ml[w][t][0]);
  float den = 0.f, num[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) num[e] = 0.f;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) {
    const float a = carry_weight(sm_ml[w][t][0], mn);
    den += sm_ml[w][t][1] * a;
#pragma unroll
    for (int e = 0; e < EPL; ++e) num[e] += sm_o[w][t][c * EPL + e] * a;
  }
  const int tq = t0 + t;
  if (p.key_splits == 1) {
    // The only split: normalise and write out and lse.
    const float inv = den > 0.f ? 1.f / den : 0.f;
    T* orow = static_cast<T*>(p.out) + ((int64_t)b * p.n_new + tq) * rs + (int64_t)h * D + c * EPL;
    if constexpr (std::is_same<T, float>::value) {
      *reinterpret_cast<float4*>(orow) =
          make_float4(num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv);
    } else {
      bf16x8_t ov;
#pragma unroll
      for (int e = 0; e < EPL; ++e) ov[e] = (__bf16)(num[e] * inv);
      *reinterpret_cast<bf16x8_t*>(orow) = ov;
    }
    if (c == 0)
      p.lse[((int64_t)b * p.heads + h) * p.n_new + tq] =
          den > 0.f ? (mn + __builtin_log2f(den)) * 0.69314718055994531f : ninf();
  } else {
    // Partial of this split: [split][b][h][t] rows of D numerator columns
    // and (kept max, denominator).
    const int64_t prow = (((int64_t)split * p.batch + b) * p.heads + h) * p.n_new + tq;
    float* po = p.part_o + prow * D + c * EPL;
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      *reinterpret_cast<float4*>(po + e) = make_float4(num[e], num[e + 1], num[e + 2], num[e + 3]);
    if (c == 0) *reinterpret_cast<float2*>(p.part_ml + 2 * prow) = make_float2(mn, den);
  }
}

// Fold the splits' partials: one thread per (b, h, t) row and 4 columns, in
// one pass over the splits, eight per round trip (their loads issued
// together), the running max moved per batch.
template <typename T>
__global__ __launch_bounds__(256) void decode_combine_kernel(const DecParams p, int head_dim) {
  const int groups = head_dim / 4;
  const int64_t rows = (int64_t)p.batch * p.heads * p.n_new;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= rows * groups) return;
  const int64_t r = tid / groups;  // (b * H + h) * n_new + t
  const int g = (int)(tid % groups);
  float mn = ninf(), den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < p.key_splits; s0 += 8) {
    float2 ml[8];
    float4 o[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t pr = (int64_t)(s0 + u) * rows + r;
      if (s0 + u < p.key_splits) {
        ml[u] = *reinterpret_cast<const float2*>(p.part_ml + 2 * pr);
        o[u] = *reinterpret_cast<const float4*>(p.part_o + pr * head_dim + 4 * g);
      } else {
        ml[u] = make_float2(ninf(), 0.f);
        o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float bm = mn;
#pragma unroll
    for (int u = 0; u < 8; ++u) bm = fmaxf(bm, ml[u].x);
    const float a0 = carry_weight(mn, bm);
    den *= a0;
    num.x *= a0;
    num.y *= a0;
    num.z *= a0;
    num.w *= a0;
    mn = bm;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float a = carry_weight(ml[u].x, mn);
      den += ml[u].y * a;
      num.x += o[u].x * a;
      num.y += o[u].y * a;
      num.z += o[u].z * a;
      num.w += o[u].w * a;
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int64_t t = r % p.n_new, bh = r / p.n_new;
  const int64_t h = bh % p.heads, b = bh / p.heads;
  T* orow = static_cast<T*>(p.out) + ((b * p.n_new + t) * p.heads + h) * head_dim + 4 * g;
  if constexpr (std::is_same<T, float>::value) {
    *reinterpret_cast<float4*>(orow) = make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
  } else {
    orow[0] = (__bf16)(num.x * inv);
    orow[1] = (__bf16)(num.y * inv);
    orow[2] = (__bf16)(num.z * inv);
    orow[3] = (__bf16)(num.w * inv);
  }
  if (g == 0) p.lse[r] = den > 0.f ? (mn + __builtin_log2f(den)) * 0.69314718055994531f : ninf();
}

template <int D, typename T>
void launch_decode_t(const DecParams& p, int nq, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)p.batch * p.heads * p.q_groups * p.key_splits));
  const dim3 block(kDecThreads);
  if (nq == 1)
    hipLaunchKernelGGL((decode_kernel<D, T, 1>), grid, block, 0, s, p);
  else if (nq == 2)
    hipLaunchKernelGGL((decode_kernel<D, T, 2>), grid, block, 0, s, p);
  else if (nq == 4)
    hipLaunchKernelGGL((decode_kernel<D, T, 4>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((decode_kernel<D, T, 8>), grid, block, 0, s, p);
  if (p.key_splits > 1) {
    const int64_t threads = (int64_t)p.batch * p.heads * p.n_new * (D / 4);
    hipLaunchKernelGGL((decode_combine_kernel<T>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, s, p, D);
  }
}

}  // namespace

int launch_decode(const DecParams& p, Dtype dtype, int head_dim, int nq, void* stream, char* err,
                  int errlen) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipGetLastError();  // clear a stale error from earlier work
  (void)e;
  if (dtype == Dtype::BF16 && head_dim == 128)
    launch_decode_t<128, __bf16>(p, nq, s);
  else if (dtype == Dtype::BF16)
    launch_decode_t<64, __bf16>(p, nq, s);
  else if (head_dim == 128)
    launch_decode_t<128, float>(p, nq, s);
  else
    launch_decode_t<64, float>(p, nq, s);
  e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(err, errlen, "decode launch failed: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

}  // namespace ra
