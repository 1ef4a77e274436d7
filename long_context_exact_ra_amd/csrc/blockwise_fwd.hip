// Blockwise exact-attention forward for one Ring Attention device share,
// written for gfx950 (MI355X, CDNA4).
//
// One workgroup of 4 waves owns 128 query rows of one (batch, head); each
// wave owns 32 of them.  The workgroup walks the N key/value blocks in ring
// order -- step t uses block (r - t) mod N ("Ring Attention with Blockwise
// Transformers for Near-Infinite Context", section 三 "环形注意力算法") --
// and inside a block the keys in tiles of TILE_N.  Tiles are staged through
// double-buffered LDS; the next tile's global loads are issued before the
// current tile is computed, also across block boundaries, which is the
// single-device stand-in for receiving the next block while computing.
//
// Per tile and wave:
//   S^T = K_tile . Q^T on MFMA (keys are the M dimension, queries the N
//         dimension), so each lane holds the logits of one query row;
//   masking (causal block test, segment ids) only on tiles that need it;
//   the online-softmax carry of "从论文到代码：深入理解RingAttention的块注意力
//   计算逻辑", section "2. 数值稳定的注意力计算": new max, correction
//   exp(prev_max - new_max), numerator and denominator rescaled, in the
//   base-2 domain with the 1/sqrt(D) scale folded into log2(e);
//   O^T += V^T . P^T on MFMA with P rounded to the input dtype.
// Whole 32-key sub-tiles whose keys are causally invisible from all 32 rows
// of a wave are skipped, which is the chunk-pair skip of section
// "3. 因果注意力掩码支持" at the kernel's own granularity.
//
// MFMA operand layouts used (wave64, 32x32 output tiles):
//   A[m][k]: lane l holds row m = l % 32, k-slots 8*(l/32) .. +7 (bf16 x16
//            variant) or k = l / 32 (f32 x2 variant);
//   B[k][n]: lane l holds column n = l % 32, the same k-slots;
//   C[m][n]: lane l holds column n = l % 32, rows 8*(i/4) + 4*(l/32) + i%4
//            for i = 0 .. 15.
// The contraction only pairs equal (lane half, slot) positions of A and B,
// so any assignment of keys to k-slots is valid as long as both operands
// use it: P^T is fed straight from the S^T registers and V^T is stored in
// LDS with its keys permuted to match.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <climits>
#include <cstdio>
#include <type_traits>

#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float ninf() { return -__builtin_inff(); }

template <typename T, int D>
struct Tile;

// bf16: 64-key tiles.  K row-major [64][D + 8]; V transposed and permuted
// [D][64 + 8] (slot s of a 16-key group g holds key 16g + 8*((s%8)/4) +
// 4*(s/8) + s%4, so a lane half reads its 8 P.V keys with one 16-byte load).
template <int D>
struct Tile<__bf16, D> {
  static constexpr int N = 64;
  static constexpr int KS = D + 8;   // K row stride (elements)
  static constexpr int VS = N + 8;   // V^T row stride (elements)
  static constexpr int K_ELEMS = N * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int K_LOADS = N * D / 8 / kThreads;    // 16-byte loads per thread
  static constexpr int V_UNITS = (N / 8) * (D / 2) / kThreads;  // 8 keys x 2 dims
};

// f32: 32-key tiles, K and V both row-major with a 4-element pad.
template <int D>
struct Tile<float, D> {
  static constexpr int N = 32;
  static constexpr int KS = D + 4;
  static constexpr int VS = D + 4;
  static constexpr int K_ELEMS = N * KS;
  static constexpr int V_ELEMS = N * VS;
  static constexpr int K_LOADS = N * D / 4 / kThreads;
  static constexpr int V_LOADS = N * D / 4 / kThreads;
};

// Global tile registers in flight between the load and the LDS store.
template <typename T, int D>
struct Staged;

template <int D>
struct Staged<__bf16, D> {
  uint4 k[Tile<__bf16, D>::K_LOADS];
  uint32_t v[Tile<__bf16, D>::V_UNITS][8];
  int32_t seg;
};

template <int D>
struct Staged<float, D> {
  uint4 k[Tile<float, D>::K_LOADS];
  uint4 v[Tile<float, D>::V_LOADS];
  int32_t seg;
};

// Position of the workgroup's current tile in the ring walk.
struct Cursor {
  int t;       // ring step
  int kb;      // key/value block used at this step
  int kt;      // tile index inside the block
  int ntile;   // tiles to visit in this block
  int klen;    // keys to visit in this block (multiple of 32)
  bool valid;
};

__device__ __forceinline__ int block_of_step(int r, int t, int n) {
  int kb = (r - t) % n;
  return kb < 0 ? kb + n : kb;
}

// Keys of block kb that some row of the workgroup (last global row q_last)
// can see, rounded up to whole 32-key sub-tiles.
__device__ __forceinline__ int block_klen(const FwdParams& p, int kb, int64_t q_last) {
  if (p.causal == 0) return p.seq_q;
  const int64_t kend = (q_last / p.causal + 1) * p.causal;  // first invisible key
  int64_t len = kend - (int64_t)kb * p.seq_q;
  if (len <= 0) return 0;
  len = (len + 31) & ~int64_t(31);
  return len > p.seq_q ? p.seq_q : (int)len;
}

template <int TN>
__device__ __forceinline__ void cursor_seek(const FwdParams& p, Cursor& c, int64_t q_last) {
  while (c.t < p.ring_size) {
    c.kb = block_of_step(p.ring_index, c.t, p.ring_size);
    c.klen = block_klen(p, c.kb, q_last);
    c.ntile = (c.klen + TN - 1) / TN;
    if (c.ntile > 0) {
      c.valid = true;
      return;
    }
    ++c.t;
  }
  c.valid = false;
}

template <int TN>
__device__ __forceinline__ void cursor_next(const FwdParams& p, Cursor& c, int64_t q_last) {
  if (++c.kt < c.ntile) return;
  c.kt = 0;
  ++c.t;
  cursor_seek<TN>(p, c, q_last);
}

// ---------------------------------------------------------------------------
// Global -> registers -> LDS staging
// ---------------------------------------------------------------------------

template <typename T, int D>
__device__ __forceinline__ void load_tile(const FwdParams& p, const Cursor& c, int b, int h,
                                          int tid, Staged<T, D>& st) {
  using TL = Tile<T, D>;
  const int64_t row0 = (int64_t)b * p.seq_k + (int64_t)c.kb * p.seq_q + (int64_t)c.kt * TL::N;
  const int64_t rs = (int64_t)p.heads * D;  // row stride (elements)
  const int nvalid = min(TL::N, c.klen - c.kt * TL::N);
  const T* kb = static_cast<const T*>(p.k) + row0 * rs + (int64_t)h * D;
  const T* vb = static_cast<const T*>(p.v) + row0 * rs + (int64_t)h * D;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int u = 0; u < TL::K_LOADS; ++u) {
      const int ci = tid + u * kThreads;
      const int row = ci / (D / 8), col = (ci % (D / 8)) * 8;
      if (row < nvalid)
        st.k[u] = *reinterpret_cast<const uint4*>(kb + row * rs + col);
    }
#pragma unroll
    for (int u = 0; u < TL::V_UNITS; ++u) {
      const int ui = tid + u * kThreads;
      const int dp = ui % (D / 2), unit = ui / (D / 2);
      const int g = unit >> 1, hh = unit & 1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = 16 * g + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (key < nvalid)
          st.v[u][e] = *reinterpret_cast<const uint32_t*>(vb + key * rs + 2 * dp);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < TL::K_LOADS; ++u) {
      const int ci = tid + u * kThreads;
      const int row = ci / (D / 4), col = (ci % (D / 4)) * 4;
      if (row < nvalid) {
        st.k[u] = *reinterpret_cast<const uint4*>(kb + row * rs + col);
        st.v[u] = *reinterpret_cast<const uint4*>(vb + row * rs + col);
      }
    }
  }
  if (p.seg != nullptr && tid < nvalid) st.seg = p.seg[row0 + tid];
}

template <typename T, int D>
__device__ __forceinline__ void store_tile(const Cursor& c, int tid, const Staged<T, D>& st,
                                           T* ks, T* vs, int32_t* segs, bool has_seg) {
  using TL = Tile<T, D>;
  const int nvalid = min(TL::N, c.klen - c.kt * TL::N);
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int u = 0; u < TL::K_LOADS; ++u) {
      const int ci = tid + u * kThreads;
      const int row = ci / (D / 8), col = (ci % (D / 8)) * 8;
      if (row < nvalid) *reinterpret_cast<uint4*>(ks + row * TL::KS + col) = st.k[u];
    }
#pragma unroll
    for (int u = 0; u < TL::V_UNITS; ++u) {
      const int ui = tid + u * kThreads;
      const int dp = ui % (D / 2), unit = ui / (D / 2);
      const int g = unit >> 1, hh = unit & 1;
      if (16 * g < nvalid) {
        // Split the 8 (even d, odd d) pairs into an even-d row and an odd-d row.
        uint4 lo, hi;
        lo.x = (st.v[u][0] & 0xffffu) | (st.v[u][1] << 16);
        lo.y = (st.v[u][2] & 0xffffu) | (st.v[u][3] << 16);
        lo.z = (st.v[u][4] & 0xffffu) | (st.v[u][5] << 16);
        lo.w = (st.v[u][6] & 0xffffu) | (st.v[u][7] << 16);
        hi.x = (st.v[u][0] >> 16) | (st.v[u][1] & 0xffff0000u);
        hi.y = (st.v[u][2] >> 16) | (st.v[u][3] & 0xffff0000u);
        hi.z = (st.v[u][4] >> 16) | (st.v[u][5] & 0xffff0000u);
        hi.w = (st.v[u][6] >> 16) | (st.v[u][7] & 0xffff0000u);
        const int slot = 16 * g + 8 * hh;
        *reinterpret_cast<uint4*>(vs + (2 * dp) * TL::VS + slot) = lo;
        *reinterpret_cast<uint4*>(vs + (2 * dp + 1) * TL::VS + slot) = hi;
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < TL::K_LOADS; ++u) {
      const int ci = tid + u * kThreads;
      const int row = ci / (D / 4), col = (ci % (D / 4)) * 4;
      if (row < nvalid) {
        *reinterpret_cast<uint4*>(ks + row * TL::KS + col) = st.k[u];
        *reinterpret_cast<uint4*>(vs + row * TL::VS + col) = st.v[u];
      }
    }
  }
  if (has_seg && tid < nvalid) segs[tid] = st.seg;
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

template <typename T, int D>
__global__ __launch_bounds__(kThreads, 2) void blockwise_fwd_kernel(const FwdParams p) {
  using TL = Tile<T, D>;
  constexpr int TN = TL::N;
  constexpr int NSUB = TN / 32;     // 32-key sub-tiles per tile
  constexpr int NDB = D / 32;       // 32-wide output blocks of the head dim

  __shared__ __attribute__((aligned(16))) T k_lds[2][TL::K_ELEMS];
  __shared__ __attribute__((aligned(16))) T v_lds[2][TL::V_ELEMS];
  __shared__ int32_t seg_lds[2][TN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 31;   // query row of this lane inside the wave's 32
  const int half = lane >> 5;   // lane half: selects k-slots / C rows

  // Workgroups are dispatched round-robin over the 8 XCDs; remap so that
  // consecutive logical tiles (the query tiles of one head, which stream the
  // same keys and values) run on the same XCD and share its L2.
  int logical;
  {
    const int pid = blockIdx.x, n = p.n_wg;
    const int xcd = pid & 7, idx = pid >> 3, cnt = n >> 3, rem = n & 7;
    logical = xcd < rem ? xcd * (cnt + 1) + idx : rem * (cnt + 1) + (xcd - rem) * cnt + idx;
  }
  // Heavier query tiles (more causal work) first.
  const int qt = p.n_qtiles - 1 - logical % p.n_qtiles;
  const int bh = logical / p.n_qtiles;
  const int h = bh % p.heads;
  const int b = bh / p.heads;

  const int m0 = qt * kBlockM;
  const int m_end = min(m0 + kBlockM, p.seq_q);
  const int qg0 = m0 + wave * 32;           // first row of this wave
  const bool wave_active = qg0 < p.seq_q;   // seq_q is a multiple of 32
  const int64_t qpos_base = (int64_t)p.ring_index * p.seq_q;
  const int64_t wg_q_last = qpos_base + m_end - 1;

  // Causal limits of this wave: a sub-tile starting at key position pk0 has a
  // visible pair iff pk0 < run_lim, and needs no causal mask iff
  // pk0 + 31 < full_lim.
  const int64_t pq_first = qpos_base + qg0, pq_last = pq_first + 31;
  int64_t run_lim = INT64_MAX, full_lim = INT64_MAX, lane_lim = INT64_MAX;
  const int64_t pq_lane = pq_first + lrow;
  if (p.causal > 0) {
    run_lim = (pq_last / p.causal + 1) * p.causal;
    full_lim = (pq_first / p.causal + 1) * p.causal;
    lane_lim = (pq_lane / p.causal + 1) * p.causal;
  }
  const int32_t lane_lim32 = (int32_t)min(lane_lim, (int64_t)p.seq_k);
  const bool has_seg = p.seg != nullptr;
  int32_t seg_q = 0;
  if (has_seg && wave_active) seg_q = p.seg[(int64_t)b * p.seq_k + pq_lane];

  // Q of this wave as the MFMA B operand (queries are the N dimension).
  const int64_t rs = (int64_t)p.heads * D;
  constexpr int QREGS = sizeof(T) == 2 ? D / 16 : D / 2;
  typename std::conditional<sizeof(T) == 2, bf16x8_t, float>::type qf[QREGS];
  if (wave_active) {
    const T* qrow = static_cast<const T*>(p.q) +
                    ((int64_t)b * p.seq_q + qg0 + lrow) * rs + (int64_t)h * D;
#pragma unroll
    for (int c = 0; c < QREGS; ++c) {
      if constexpr (sizeof(T) == 2) {
        const uint4 raw = *reinterpret_cast<const uint4*>(qrow + 16 * c + 8 * half);
        qf[c] = __builtin_bit_cast(bf16x8_t, raw);
      } else {
        qf[c] = qrow[2 * c + half];
      }
    }
  }

  f32x16_t acc[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) acc[j] = f32x16_t{};
  float m_run = ninf();   // running max of the scaled logits (base-2 domain)
  float l_run = 0.f;      // this lane half's part of the denominator

  const int nqc = p.seq_q / p.q_chunk, nkc = p.seq_q / p.k_chunk;

  Cursor cur{0, 0, 0, 0, 0, false};
  cursor_seek<TN>(p, cur, wg_q_last);

  Staged<T, D> st;
  if (cur.valid) {
    load_tile<T, D>(p, cur, b, h, tid, st);
    store_tile<T, D>(cur, tid, st, k_lds[0], v_lds[0], seg_lds[0], has_seg);
  }
  __syncthreads();

  int buf = 0;
  while (cur.valid) {
    Cursor nxt = cur;
    cursor_next<TN>(p, nxt, wg_q_last);
    if (nxt.valid) load_tile<T, D>(p, nxt, b, h, tid, st);

    // ---- per-wave work on the current tile ----
    const int kloc0 = cur.kt * TN;                      // first key in the block
    const int64_t pk_tile = (int64_t)cur.kb * p.seq_q + kloc0;
    bool run[NSUB], mask[NSUB];
    bool any = false;
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
      const int64_t pk0 = pk_tile + 32 * sb;
      run[sb] = wave_active && (kloc0 + 32 * sb < cur.klen) && pk0 < run_lim;
      mask[sb] = has_seg || !(pk0 + 31 < full_lim);
      any |= run[sb];
    }
    if (any) {
      const T* ks = k_lds[buf];
      const T* vs = v_lds[buf];
      const int32_t* sg = seg_lds[buf];
      f32x16_t s[NSUB];
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb) {
        s[sb] = f32x16_t{};
        if (!run[sb]) continue;
        const T* krow = ks + (32 * sb + lrow) * TL::KS;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int c = 0; c < D / 16; ++c) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(krow + 16 * c + 8 * half);
            s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[sb], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int c = 0; c < D / 2; ++c)
            s[sb] = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * c + half], qf[c], s[sb], 0, 0, 0);
        }
      }

      // Mask and row max.  Lane (lrow, half) holds keys
      // kloc0 + 32*sb + 8*(i/4) + 4*half + i%4 of query row lrow.
      float mx = ninf();
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb) {
        if (!run[sb]) {
#pragma unroll
          for (int i = 0; i < 16; ++i) s[sb][i] = ninf();
          continue;
        }
        if (mask[sb]) {
          const int32_t pkb = (int32_t)(pk_tile + 32 * sb) + 4 * half;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int koff = 8 * (i >> 2) + (i & 3);
            bool ok = pkb + koff < lane_lim32;
            if (has_seg) ok = ok && sg[32 * sb + 4 * half + koff] == seg_q;
            if (!ok) s[sb][i] = ninf();
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sb][i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * p.scale_log2);
      const float m_use = m_new == ninf() ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float rowsum = 0.f;
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][i], p.scale_log2, -m_use));
          s[sb][i] = e;
          rowsum += e;
        }
      }
      l_run = l_run * alpha + rowsum;
      m_run = m_new;
#pragma unroll
      for (int j = 0; j < NDB; ++j) acc[j] *= alpha;

      // O^T += V^T . P^T
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb) {
        if (!run[sb]) continue;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const f32x8_t pf = {s[sb][8 * cc + 0], s[sb][8 * cc + 1], s[sb][8 * cc + 2],
                                s[sb][8 * cc + 3], s[sb][8 * cc + 4], s[sb][8 * cc + 5],
                                s[sb][8 * cc + 6], s[sb][8 * cc + 7]};
            const bf16x8_t pb = __builtin_convertvector(pf, bf16x8_t);
#pragma unroll
            for (int j = 0; j < NDB; ++j) {
              const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
                  vs + (32 * j + lrow) * TL::VS + 32 * sb + 16 * cc + 8 * half);
              acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[j], 0, 0, 0);
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const T* vrow = vs + (32 * sb + 8 * (i >> 2) + 4 * half + (i & 3)) * TL::VS;
#pragma unroll
            for (int j = 0; j < NDB; ++j)
              acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * j + lrow], s[sb][i],
                                                           acc[j], 0, 0, 0);
          }
        }
      }

      if (p.run_map != nullptr && lane == 0) {
        const int a = qg0 / p.q_chunk;
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb)
          if (run[sb])
            p.run_map[((int64_t)cur.t * nqc + a) * nkc + (kloc0 + 32 * sb) / p.k_chunk] = 1;
      }
    }

    if (nxt.valid) {
      const int nb = buf ^ 1;
      store_tile<T, D>(nxt, tid, st, k_lds[nb], v_lds[nb], seg_lds[nb], has_seg);
    }
    __syncthreads();
    cur = nxt;
    buf ^= 1;
  }

  // ---- epilogue: out = numerator / denominator, lse = ln(denominator) + max ----
  if (!wave_active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int row = qg0 + lrow;
  T* orow = static_cast<T*>(p.out) + ((int64_t)b * p.seq_q + row) * rs + (int64_t)h * D;
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * j + 8 * g + 4 * half;
      if constexpr (sizeof(T) == 2) {
        typedef float f32x4_t __attribute__((ext_vector_type(4)));
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        const f32x4_t o = {acc[j][4 * g] * inv, acc[j][4 * g + 1] * inv,
                           acc[j][4 * g + 2] * inv, acc[j][4 * g + 3] * inv};
        *reinterpret_cast<bf16x4_t*>(orow + d) = __builtin_convertvector(o, bf16x4_t);
      } else {
        float4 o = make_float4(acc[j][4 * g] * inv, acc[j][4 * g + 1] * inv,
                               acc[j][4 * g + 2] * inv, acc[j][4 * g + 3] * inv);
        *reinterpret_cast<float4*>(orow + d) = o;
      }
    }
  }
  if (half == 0) {
    p.lse[((int64_t)b * p.heads + h) * p.seq_q + row] =
        l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : ninf();
  }
}

__global__ void fill_u8_kernel(uint8_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

template <typename T, int D>
hipError_t launch_typed(const FwdParams& p, hipStream_t s) {
  hipLaunchKernelGGL((blockwise_fwd_kernel<T, D>), dim3(p.n_wg), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int launch_fwd(const FwdParams& p, Dtype dtype, int head_dim, int64_t run_map_bytes,
               void* stream, char* err, int errlen) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipGetLastError();  // clear a stale error from earlier work
  (void)e;
  if (p.run_map != nullptr && run_map_bytes > 0) {
    const int64_t blocks = std::min<int64_t>((run_map_bytes + 255) / 256, 1024);
    hipLaunchKernelGGL(fill_u8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p.run_map,
                       run_map_bytes);
    e = hipGetLastError();
    if (e != hipSuccess) {
      snprintf(err, errlen, "run_map clear launch failed: %s", hipGetErrorString(e));
      return 1;
    }
  }
  if (dtype == Dtype::BF16)
    e = head_dim == 128 ? launch_typed<__bf16, 128>(p, s) : launch_typed<__bf16, 64>(p, s);
  else
    e = head_dim == 128 ? launch_typed<float, 128>(p, s) : launch_typed<float, 64>(p, s);
  if (e != hipSuccess) {
    snprintf(err, errlen, "kernel launch failed: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

}  // namespace ra
