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
// (query, key) pair: for up to a few dozen queries it is bound by HBM
// bandwidth.  Two kernels:
//   * bf16 (decode_mfma_kernel): both products on the matrix cores, a tile
//     of 32 queries per workgroup, each wave walking its own 32-key tiles,
//     K and V rows loaded whole (one load instruction = whole rows) and
//     staged through the wave's LDS (below);
//   * float32 (decode_kernel): the arithmetic on the vector ALUs.  A group
//     of LPR lanes owns one key per step: each lane holds 16 bytes of the
//     key's row and of the value row (whole-row loads), forms its share of
//     q.k for each query and the group sums the shares with DPP row
//     operations; each group keeps, per query, the running max (base 2,
//     moved lazily: only when a logit would exceed it by 2^8, as in the
//     forward), the denominator and its 4 columns of the numerator ("2.
//     数值稳定的注意力计算": the carry and its correction); the groups of a
//     workgroup walk interleaved keys of one contiguous key range, U keys
//     each per iteration, loaded one iteration ahead, and fold their
//     carries at the end (within a wave by lane exchanges, across waves
//     through LDS).
// Both load the cache with nontemporal loads (it is streamed once).
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
#include "ra_decode.h"
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int kDecThreads = 256;  // 4 waves
constexpr int kDecWaves = kDecThreads / 64;
// Largest log2 of a probability weight before the running max must move.
constexpr float kDecLazy = 8.f;

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

// The lane's share of q.k (4 elements).
__device__ __forceinline__ float dot_share(const float4& q, const float4& k) {
  float s = q.x * k.x;
  s = __builtin_fmaf(q.y, k.y, s);
  s = __builtin_fmaf(q.z, k.z, s);
  return __builtin_fmaf(q.w, k.w, s);
}

// Weight of a carry with kept max m under the common max mn (0 for an
// empty carry, whose m is -inf).
__device__ __forceinline__ float carry_weight(float m, float mn) {
  return m == ninf() ? 0.f : __builtin_amdgcn_exp2f(m - mn);
}

// Which (batch, head, query group, split) a workgroup owns.  Workgroup ids
// are dispatched round-robin over the 8 XCDs; the logical index (split
// fastest, then query group) is laid out so that consecutive logical
// indices share an XCD: the query groups of one split, which stream the
// same cache rows at the same time, then meet in that XCD's L2.
struct DecCoord {
  int b, h, qg, split;
};
__device__ __forceinline__ DecCoord dec_coord(const DecParams& p) {
  const int pid = blockIdx.x, n = gridDim.x;
  const int xcd = pid & 7, idx = pid >> 3, cnt = n >> 3, rem = n & 7;
  const int logical =
      xcd < rem ? xcd * (cnt + 1) + idx : rem * (cnt + 1) + (xcd - rem) * cnt + idx;
  const int qg = logical % p.q_groups;
  const int rest = logical / p.q_groups;
  const int split = rest % p.key_splits;
  const int bh = rest / p.key_splits;
  return DecCoord{bh / p.heads, bh % p.heads, qg, split};
}

// float32 inputs.
template <int D, int NQ>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(const DecParams p) {
  using vec = float4;
  constexpr int EPL = 4;                 // elements per lane
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
  const DecCoord wc = dec_coord(p);
  const int b = wc.b, h = wc.h, qg = wc.qg, split = wc.split;
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
      qv[t] = *reinterpret_cast<const vec*>(static_cast<const float*>(p.q) +
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

  const float* kbase = static_cast<const float*>(p.k) + (int64_t)b * p.cache_rows * rs + col;
  const float* vbase = static_cast<const float*>(p.v) + (int64_t)b * p.cache_rows * rs + col;
  // The last position any query of this workgroup sees fully: a block whose
  // keys all lie at or before it, and inside the range, needs no mask.
  const int64_t all_see = p.cache_idx + t0;
  // The K and V slices of one block of keys (rows past the range are
  // clamped onto its last row: read, then masked).  The cache is streamed
  // once: nontemporal loads (with bf16 inputs, which this kernel served
  // first, the 7B-shaped step ran at 82.7 % of the HBM peak with them and
  // 76.0 % without).
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
      const float vf[EPL] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
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
    float* orow = static_cast<float*>(p.out) + ((int64_t)b * p.n_new + tq) * rs + (int64_t)h * D + c * EPL;
    *reinterpret_cast<float4*>(orow) =
        make_float4(num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv);
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

// ---------------------------------------------------------------------------
// bf16: the matrix cores
// ---------------------------------------------------------------------------
//
// On the vector ALUs a bf16 step of more than a few queries is bound by the
// arithmetic (4 D flop per pair), and with one query the matrix-core kernel
// is still the faster (6.91 against 6.70 TB/s on the 7B-shaped step).  It
// keeps the split, carry and partial format of the kernel above and does
// both products on v_mfma_f32_32x32x16_bf16 in the forward's orientation:
// a workgroup holds one tile of 32 queries (Q^T, the B operand, in
// registers), and each of its 4 waves walks every fourth 32-key tile of the
// workgroup's key range on its own:
//   S^T = K Q^T   (keys = M: the A operand read from the wave's LDS copy of
//                 the K tile, lane l holding key l % 32),
//   the carry per query (lane l and l ^ 32 hold query l % 32; the kept max
//   moves lazily, for the whole wave at once, as in the forward),
//   O^T += V^T P^T  (P^T converted in place from the S^T registers; V^T read
//                 with ds_read_b64_tr_b16 from the wave's own LDS copy of the
//                 V tile, laid out as the forward's V tile so that the keys
//                 of each k-slot match those of P^T).
// The next tile's K and V rows are loaded while this one is computed; they
// are written to LDS at the start of their tile (the wave's own LDS
// operations complete in order, so the writes follow the previous tile's
// reads).  The probabilities are rounded to bf16 for the P.V product and the
// denominator sums the rounded values, as in the forward.  At the end the
// waves fold their carries through LDS and write the workgroup's partial
// (or, with one split, out and lse).
//
// SHARE (steps of more than 32 tokens): each wave holds its own tile of 32
// queries instead (4 per workgroup), and the waves share every 32-key tile
// of the workgroup's range: each loads 8 of its rows, writes them into one
// of two LDS stages, and one barrier per tile shows the tile complete and
// every wave done with the stage the next tile refills.  No fold: each
// wave writes its own queries.  Without it, every further tile of 32
// queries streamed the cache again (64 tokens: 3.76 TB/s).

template <int D, bool SHARE>
__global__ __launch_bounds__(kDecThreads, 2) void decode_mfma_kernel(const DecParams p) {
  constexpr int NC = D / 16;   // k-chunks of S^T
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  constexpr int GR = D / 8;    // 16-byte granules per row
  constexpr int TK = 32;       // keys per tile
  constexpr int RPI = 64 / GR; // rows per whole-row load instruction
  constexpr int RW = SHARE ? TK / kDecWaves : TK;  // rows of a tile one wave loads
  constexpr int NV = RW / RPI; // K (and V) loads per lane per tile
  static_assert(NV * RPI == RW, "a wave's rows split into whole instructions");
  constexpr int VT = TK * D;   // bf16 elements of one K or V tile
  // One K and one V tile per wave; reused at the end for the fold (2 x 32 x
  // D floats).
  __shared__ __attribute__((aligned(16))) __bf16 kv_lds[kDecWaves * 2 * VT];
  __shared__ float fold_ml[2][32][2];
  static_assert(kDecWaves * 2 * VT * 2 >= 2 * 32 * D * 4, "fold regions fit the tiles");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lrow = lane & 31, half = lane >> 5;
  const DecCoord wc = dec_coord(p);
  const int b = wc.b, h = wc.h, qg = wc.qg, split = wc.split;
  const int t0 = (SHARE ? qg * kDecWaves + wave : qg) * 32;
  const int nq = min(32, p.n_new - t0);  // (<= 0: a SHARE wave without queries)
  const int64_t kb = (int64_t)split * p.split_keys;
  const int64_t ke = kb + p.split_keys < p.n_keys ? kb + p.split_keys : p.n_keys;
  const int64_t rs = (int64_t)p.heads * D;
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + (int64_t)b * p.cache_rows * rs + (int64_t)h * D;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + (int64_t)b * p.cache_rows * rs + (int64_t)h * D;
  // The wave's own K and V tiles, or (SHARE) stage 0 of the shared ones.
  __bf16* kt = kv_lds + (SHARE ? 0 : wave * 2 * VT);
  __bf16* vt = kt + VT;
  const int row0 = SHARE ? RW * wave : 0;  // the tile rows this wave loads

  // Q^T: lane l holds query t0 + l % 32, d-slots 16 c + 8 (l / 32) .. + 7.
  bf16x8_t qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) qf[c] = bf16x8_t{};
  if (lrow < nq) {
    const __bf16* qrow = static_cast<const __bf16*>(p.q) + ((int64_t)b * p.n_new + t0 + lrow) * rs +
                         (int64_t)h * D + 8 * half;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * c);
  }

  // K and V rows of a tile, whole: lane l loads granule l % GR of row k0 +
  // RPI u + l / GR, so that a load instruction reads RPI whole rows (reading
  // K straight in the A-operand layout, 32 rows x 32 bytes per instruction,
  // held the step at 5.1 TB/s against 6.7 with whole rows).  Rows past the
  // range are clamped onto its last row (read, then masked).
  auto load = [&](int64_t k0, bf16x8_t* kd, bf16x8_t* vd) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int64_t r = k0 + row0 + RPI * u + lane / GR;
      const int64_t rr = r < ke ? r : ke - 1;
      kd[u] = __builtin_bit_cast(bf16x8_t, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
                                               kbase + rr * rs + 8 * (lane % GR))));
      vd[u] = __builtin_bit_cast(bf16x8_t, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
                                               vbase + rr * rs + 8 * (lane % GR))));
    }
  };
  // The K tile in LDS, 16-byte slots: slot(r, g) = (g / 4) 128 + (r / 16) 64
  // + (g % 4) 16 + ((r % 16) ^ (g % 16)).  The A-operand read of 16 lanes
  // (16 rows, one granule) touches 16 slots that differ modulo 16 (every
  // bank once), and so do the 16 lanes of a whole-row write (one row, 16
  // granules; for D = 64, two rows of 8 granules meet twice).
  auto kslot = [](int r, int g) {
    return (g >> 2) * 128 + (r >> 4) * 64 + (g & 3) * 16 + ((r & 15) ^ (g & 15));
  };
  auto kstore = [&](const bf16x8_t* kd) {
#pragma unroll
    for (int u = 0; u < NV; ++u)
      *reinterpret_cast<bf16x8_t*>(kt + 8 * kslot(row0 + RPI * u + lane / GR, lane % GR)) = kd[u];
  };
  // A operand of chunk c: key l % 32, granule 2 c + l / 32.
  auto kread = [&](int c) {
    return *reinterpret_cast<const bf16x8_t*>(kt + 8 * kslot(lrow, 2 * c + half));
  };
  // The V tile in LDS: 32-d block j = g / 4 holds the tile's 32 rows of 32
  // elements, row-major (element (r, d) at 1024 j + 32 r + d % 32).
  auto vstore = [&](const bf16x8_t* vd) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int r = row0 + RPI * u + lane / GR, g = lane % GR;
      *reinterpret_cast<bf16x8_t*>(vt + (TK * 32) * (g >> 2) + 32 * r + 8 * (g & 3)) = vd[u];
    }
  };
  // V^T for 32-d block j and 16-key step cc: a group of 16 lanes reads rows
  // 16 cc + 4 (l / 32) + (l % 16) / 4 (and + 8) at columns 16 ((l / 16) % 2)
  // + 4 (l % 4); the transpose hands lane l, for its column l % 32, keys
  // 16 cc + 4 (l / 32) + 0..3 and + 8 .. + 11: the keys the S^T registers
  // 8 cc .. 8 cc + 7 of the lane hold.
  const int v_rd = 32 * (4 * half + ((lane & 15) >> 2)) + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto vread = [&](int j, int cc) {
    const __bf16* src = vt + v_rd + (TK * 32) * j + 32 * 16 * cc;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)src);
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(src + 256));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16_t acc[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) acc[j] = f32x16_t{};
  float m_run = ninf(), l_run = 0.f;  // l_run: this lane half's keys
  const bf16x2_t one2 = {(__bf16)1.f, (__bf16)1.f};
  const int64_t see = p.cache_idx + t0 + lrow;  // last key this lane's query sees
  const int64_t all_see = p.cache_idx + t0;     // ... that every query of the tile sees

  bf16x8_t kn[NV], vn[NV];
  constexpr int64_t kStep = SHARE ? TK : (int64_t)TK * kDecWaves;
  int64_t k0 = kb + (SHARE ? 0 : (int64_t)TK * wave);
  if (k0 < ke) load(k0, kn, vn);
  for (int it = 0; k0 < ke; k0 += kStep, ++it) {
    if constexpr (SHARE) {
      kt = kv_lds + (it & 1) * 2 * VT;
      vt = kt + VT;
    }
    kstore(kn);
    vstore(vn);
    if constexpr (SHARE) __syncthreads();  // the tile is complete; the other stage is free
    const int64_t k1 = k0 + kStep;
    if (k1 < ke) load(k1, kn, vn);
    if (SHARE && nq <= 0) continue;

    f32x16_t sc = f32x16_t{};
#pragma unroll
    for (int c = 0; c < NC; ++c) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(c), qf[c], sc, 0, 0, 0);
    // Logits (base 2); element i holds key k0 + 8 (i / 4) + 4 half + i % 4.
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = sc[i] * p.scale_log2;
    if (k0 + TK > ke || k0 + TK - 1 > all_see) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t key = k0 + 8 * (i / 4) + 4 * half + i % 4;
        if (key >= ke || key > see) x[i] = ninf();
      }
    }
    float bm = x[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) bm = fmaxf(bm, x[i]);
    bm = pair_max(bm);
    // The kept max moves only when a weight would exceed 2^kDecLazy, for the
    // whole wave at once (one vote).
    if (__builtin_amdgcn_ballot_w64(bm > m_run + kDecLazy) != 0) {
      const float mn = fmaxf(m_run, bm);
      const float a = carry_weight(m_run, mn);
      l_run *= a;
#pragma unroll
      for (int j = 0; j < NDB; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] *= a;
      m_run = mn;
    }
    bf16x8_t pb[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      f32x8_t e;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xi = x[8 * cc + i];
        e[i] = xi == ninf() ? 0.f : __builtin_amdgcn_exp2f(xi - m_run);
      }
      pb[cc] = __builtin_convertvector(e, bf16x8_t);
      // the denominator from the rounded probabilities, as the forward
      float ps = __builtin_amdgcn_fdot2_f32_bf16(pb[cc].s01, one2, l_run, false);
      ps = __builtin_amdgcn_fdot2_f32_bf16(pb[cc].s23, one2, ps, false);
      ps = __builtin_amdgcn_fdot2_f32_bf16(pb[cc].s45, one2, ps, false);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(pb[cc].s67, one2, ps, false);
    }
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread(j, cc), pb[cc], acc[j], 0, 0, 0);
  }
  float l_tot = pair_sum(l_run);

  // Fold the waves: 3 and 2 into 1 and 0, then 1 into 0.  A region holds one
  // wave's O^T as [32 queries][D] floats (its element i of block j at
  // d = 32 j + 8 (i / 4) + 4 half + i % 4).
  float* region = reinterpret_cast<float*>(kv_lds);
  auto put = [&](int slot) {
    float* r = region + slot * 32 * D + lrow * D;
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(r + 32 * j + 8 * g + 4 * half) =
            make_float4(acc[j][4 * g], acc[j][4 * g + 1], acc[j][4 * g + 2], acc[j][4 * g + 3]);
    if (half == 0) {
      fold_ml[slot][lrow][0] = m_run;
      fold_ml[slot][lrow][1] = l_tot;
    }
  };
  auto take = [&](int slot) {
    const float* r = region + slot * 32 * D + lrow * D;
    const float m2 = fold_ml[slot][lrow][0], l2 = fold_ml[slot][lrow][1];
    const float mn = fmaxf(m_run, m2);
    const float a = carry_weight(m_run, mn), a2 = carry_weight(m2, mn);
    l_tot = l_tot * a + l2 * a2;
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 o2 = *reinterpret_cast<const float4*>(r + 32 * j + 8 * g + 4 * half);
        acc[j][4 * g] = acc[j][4 * g] * a + o2.x * a2;
        acc[j][4 * g + 1] = acc[j][4 * g + 1] * a + o2.y * a2;
        acc[j][4 * g + 2] = acc[j][4 * g + 2] * a + o2.z * a2;
        acc[j][4 * g + 3] = acc[j][4 * g + 3] * a + o2.w * a2;
      }
    m_run = mn;
  };
  if constexpr (!SHARE) {
    __syncthreads();  // every wave is done with its K and V tiles
    if (wave >= 2) put(wave - 2);
    __syncthreads();
    if (wave < 2) take(wave);
    __syncthreads();
    if (wave == 1) put(0);
    __syncthreads();
    if (wave != 0) return;
    take(0);
  }
  if (lrow >= nq) return;

  const int tq = t0 + lrow;
  if (p.key_splits == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __bf16* orow = static_cast<__bf16*>(p.out) + ((int64_t)b * p.n_new + tq) * rs + (int64_t)h * D;
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        bf16x4_t ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(acc[j][4 * g + e] * inv);
        *reinterpret_cast<bf16x4_t*>(orow + 32 * j + 8 * g + 4 * half) = ov;
      }
    if (half == 0)
      p.lse[((int64_t)b * p.heads + h) * p.n_new + tq] =
          l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * 0.69314718055994531f : ninf();
  } else {
    const int64_t prow = (((int64_t)split * p.batch + b) * p.heads + h) * p.n_new + tq;
    float* po = p.part_o + prow * D;
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(po + 32 * j + 8 * g + 4 * half) =
            make_float4(acc[j][4 * g], acc[j][4 * g + 1], acc[j][4 * g + 2], acc[j][4 * g + 3]);
    if (half == 0) *reinterpret_cast<float2*>(p.part_ml + 2 * prow) = make_float2(m_run, l_tot);
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

template <typename T>
void launch_combine(const DecParams& p, int head_dim, hipStream_t s) {
  if (p.key_splits > 1) {
    const int64_t threads = (int64_t)p.batch * p.heads * p.n_new * (head_dim / 4);
    hipLaunchKernelGGL((decode_combine_kernel<T>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, s, p, head_dim);
  }
}

template <int D>
void launch_decode_f32(const DecParams& p, int nq, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)p.batch * p.heads * p.q_groups * p.key_splits));
  const dim3 block(kDecThreads);
  if (nq == 1)
    hipLaunchKernelGGL((decode_kernel<D, 1>), grid, block, 0, s, p);
  else if (nq == 2)
    hipLaunchKernelGGL((decode_kernel<D, 2>), grid, block, 0, s, p);
  else if (nq == 4)
    hipLaunchKernelGGL((decode_kernel<D, 4>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((decode_kernel<D, 8>), grid, block, 0, s, p);
  launch_combine<float>(p, D, s);
}

template <int D>
void launch_decode_bf16(const DecParams& p, int nq, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)p.batch * p.heads * p.q_groups * p.key_splits));
  if (nq == 32)
    hipLaunchKernelGGL((decode_mfma_kernel<D, false>), grid, dim3(kDecThreads), 0, s, p);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<D, true>), grid, dim3(kDecThreads), 0, s, p);
  launch_combine<__bf16>(p, D, s);
}

}  // namespace

int launch_decode(const DecParams& p, Dtype dtype, int head_dim, int nq, void* stream, char* err,
                  int errlen) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipGetLastError();  // clear a stale error from earlier work
  (void)e;
  if (dtype == Dtype::BF16 && nq != 32 && nq != 128) {
    snprintf(err, errlen, "bf16 decoding takes 32 or 128 queries per workgroup (got %d)", nq);
    return 1;
  }
  if (dtype == Dtype::BF16 && head_dim == 128)
    launch_decode_bf16<128>(p, nq, s);
  else if (dtype == Dtype::BF16)
    launch_decode_bf16<64>(p, nq, s);
  else if (head_dim == 128)
    launch_decode_f32<128>(p, nq, s);
  else
    launch_decode_f32<64>(p, nq, s);
  e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(err, errlen, "decode launch failed: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

}  // namespace ra
