// Blockwise exact-attention forward for one Ring Attention device share,
// written for gfx950 (MI355X, CDNA4).
//
// One workgroup of 4 waves owns 128 query rows of one (batch, head); each
// wave owns 32 of them.  The workgroup walks the N key/value blocks in ring
// order -- step t uses block (r - t) mod N ("Ring Attention with Blockwise
// Transformers for Near-Infinite Context", section 三 "环形注意力算法") --
// and inside a block the keys in tiles.  Tiles are staged through
// double-buffered LDS; the next tile's global loads are issued before the
// current tile is computed, also across block boundaries, which is the
// single-device stand-in for receiving the next block while computing.
//
// Per tile and wave:
//   S^T = K_tile . Q^T on MFMA (keys are the M dimension, queries the N
//         dimension), so each lane holds the logits of one query row;
//   masking (causal block test, segment ids) only on sub-tiles that need it;
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
// use it: P^T is fed straight from the S^T registers, and V^T is gathered
// with the same key-to-slot assignment.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <climits>
#include <cstdio>

#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kThreads = 256;
constexpr float kLn2 = 0.69314718055994530942f;
// Buffer resource word 3 for gfx9 raw (untyped) buffer access.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ float ninf() { return -__builtin_inff(); }

// A raw buffer descriptor over [base, base + bytes).  Both are uniform across
// the wave; readfirstlane makes that explicit so the descriptor lives in
// scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((hi << 32) | lo), 0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), kRsrcWord3);
}

// ---------------------------------------------------------------------------
// Work decomposition shared by both kernels
// ---------------------------------------------------------------------------

// Which (batch, head, query tile) a workgroup owns.  Workgroups are
// dispatched round-robin over the 8 XCDs; the remap puts consecutive logical
// tiles -- the query tiles of one head, which stream the same keys and
// values -- on the same XCD so they share its L2.  Heavier query tiles (more
// causal work) come first.
struct WgCoord {
  int b, h, m0;
};

__device__ __forceinline__ WgCoord wg_coord(const FwdParams& p) {
  const int pid = blockIdx.x, n = p.n_wg;
  const int xcd = pid & 7, idx = pid >> 3, cnt = n >> 3, rem = n & 7;
  const int logical =
      xcd < rem ? xcd * (cnt + 1) + idx : rem * (cnt + 1) + (xcd - rem) * cnt + idx;
  const int qt = p.n_qtiles - 1 - logical % p.n_qtiles;
  const int bh = logical / p.n_qtiles;
  // The values are workgroup-uniform; say so, so that addresses and buffer
  // descriptors derived from them stay in scalar registers.
  return WgCoord{__builtin_amdgcn_readfirstlane(bh / p.heads),
                 __builtin_amdgcn_readfirstlane(bh % p.heads),
                 __builtin_amdgcn_readfirstlane(qt * kBlockM)};
}

// Position of the workgroup's current tile in the ring walk.
struct Cursor {
  int t;       // ring step
  int kb;      // key/value block used at this step
  int kt;      // tile index inside the block
  int ntile;   // tiles to visit in this block
  int klen;    // keys to visit in this block (multiple of 32)
  int valid;   // int, not bool: no padding bytes to copy around
};

// kend: first key position no row of the workgroup can see (INT64_MAX when
// non-causal).  The keys of block kb to visit are those before kend, rounded
// up to whole 32-key sub-tiles.
__device__ __forceinline__ int block_klen(const FwdParams& p, int kb, int64_t kend) {
  const int64_t len = kend - (int64_t)kb * p.seq_q;
  if (len <= 0) return 0;
  if (len >= p.seq_q) return p.seq_q;
  const int l32 = ((int)len + 31) & ~31;
  return l32 > p.seq_q ? p.seq_q : l32;
}

template <int TN>
__device__ __forceinline__ void cursor_seek(const FwdParams& p, Cursor& c, int64_t kend) {
#pragma clang loop vectorize(disable) unroll(disable)
  while (c.t < p.ring_size) {
    // Ring order: step t uses block (r - t) mod N.
    c.kb = p.ring_index - c.t;
    if (c.kb < 0) c.kb += p.ring_size;
    c.klen = block_klen(p, c.kb, kend);
    c.ntile = (c.klen + TN - 1) / TN;
    if (c.ntile > 0) {
      c.valid = 1;
      return;
    }
    ++c.t;
  }
  c.valid = 0;
}

template <int TN>
__device__ __forceinline__ void cursor_next(const FwdParams& p, Cursor& c, int64_t kend) {
  if (++c.kt < c.ntile) return;
  c.kt = 0;
  ++c.t;
  cursor_seek<TN>(p, c, kend);
}

// Per-wave causal limits: a 32-key sub-tile starting at key position pk0
// holds a visible pair iff pk0 < run_lim, and needs no causal mask iff
// pk0 + 31 < full_lim; key position pk is visible from this lane's row iff
// pk < lane_lim.
struct WaveLimits {
  int64_t run_lim, full_lim;
  int32_t lane_lim;
};

__device__ __forceinline__ WaveLimits wave_limits(const FwdParams& p, int64_t pq_first,
                                                  int lrow) {
  WaveLimits w{INT64_MAX, INT64_MAX, p.seq_k};
  if (p.causal > 0) {
    const int64_t c = p.causal;
    w.run_lim = ((pq_first + 31) / c + 1) * c;
    w.full_lim = (pq_first / c + 1) * c;
    w.lane_lim = (int32_t)std::min<int64_t>(((pq_first + lrow) / c + 1) * c, p.seq_k);
  }
  return w;
}

__device__ __forceinline__ int64_t wg_kend(const FwdParams& p, int m0) {
  if (p.causal == 0) return INT64_MAX;
  const int64_t q_last = (int64_t)p.ring_index * p.seq_q + std::min(m0 + kBlockM, p.seq_q) - 1;
  return (q_last / p.causal + 1) * p.causal;
}

__device__ __forceinline__ void write_run_map(const FwdParams& p, int t, int qg0, int key0) {
  const int nqc = p.seq_q / p.q_chunk, nkc = p.seq_q / p.k_chunk;
  p.run_map[((int64_t)t * nqc + qg0 / p.q_chunk) * nkc + key0 / p.k_chunk] = 1;
}

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------
//
// 64-key tiles.  LDS per stage: K row-major [64][D + 8] (the 16-byte pad
// spreads the A-operand reads of 8 consecutive rows over all banks), V
// row-major [64][D + 16] read with ds_read_b64_tr_b16, and 64 segment ids.
// Within each 16-lane group that instruction hands destination lane i,
// element e the element i % 4 of source lane 4e + i / 4.  A lane of group g
// therefore sources row base + (lane % 16) / 4 at column
// 16 * (g % 2) + 4 * (lane % 4) and receives, for its own column
// (lane % 32), the 4 consecutive rows base .. base + 3: exactly four k-slots
// of the P.V A operand V^T.
//
// Global loads are bounds-checked buffer loads: each thread's byte offsets
// inside a tile are fixed, only the (scalar) tile base changes, and rows past
// the tile's valid length read as zero.

template <int D>
struct Bf16Cfg {
  static constexpr int TN = 64;
  static constexpr int KS = D + 8;
  static constexpr int VS = D + 16;
  static constexpr int GR = D / 8;                    // 16-byte granules per row
  static constexpr int LOADS = TN * GR / kThreads;    // per thread per tensor
  static_assert(LOADS * kThreads == TN * GR, "tile must split evenly");
};

// Softmax/accumulator state of one wave (32 query rows, one per lane pair).
template <int D>
struct Bf16Wave {
  static constexpr int NDB = D / 32;
  f32x16_t acc[NDB];
  float m_run;   // running max of the scaled logits (base-2 domain)
  float l_run;   // this lane half's part of the denominator
};

// One 64-key tile for one wave.  MASKED selects the general path: any of the
// two 32-key sub-tiles may be skipped (run[sb] false) or need the causal /
// segment mask; otherwise both run unmasked, straight-line.
template <int D, bool MASKED, bool SEG>
__device__ __forceinline__ void bf16_tile(Bf16Wave<D>& w, const bf16x8_t* qf,
                                          const __bf16* ks, const __bf16* vs,
                                          const int32_t* sg, int lrow, int half, int vrd,
                                          bool run0, bool run1, bool mask0, bool mask1,
                                          int32_t pk_tile,
                                          int32_t lane_lim, int32_t seg_q, float scale_log2) {
  using C = Bf16Cfg<D>;
  constexpr int NDB = D / 32;

  // S^T = K . Q^T
  f32x16_t s[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    s[sb] = f32x16_t{};
    if (MASKED && !(sb ? run1 : run0)) continue;
    const __bf16* krow = ks + (32 * sb + lrow) * C::KS + 8 * half;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(krow + 16 * c);
      s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[sb], 0, 0, 0);
    }
  }

  // Mask and row max.  Lane (lrow, half) holds keys
  // pk_tile + 32*sb + 8*(i/4) + 4*half + i%4 of query row lrow.
  if (MASKED) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int32_t pkb = pk_tile + 32 * sb + 4 * half;
      const bool r = sb ? run1 : run0, m = sb ? mask1 : mask0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int koff = 8 * (i >> 2) + (i & 3);
        bool ok = r && (!m || pkb + koff < lane_lim);
        if (SEG) ok = ok && sg[32 * sb + 4 * half + koff] == seg_q;
        s[sb][i] = ok ? s[sb][i] : ninf();
      }
    }
  }
  float mx = ninf();
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sb][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(w.m_run, mx * scale_log2);
  // Rescale only when some row's max grew: otherwise the correction
  // exp(prev_max - new_max) is exactly 1 for every row.
  if (__builtin_amdgcn_ballot_w64(m_new > w.m_run) != 0) {
    const float alpha = m_new == ninf() ? 1.f : __builtin_amdgcn_exp2f(w.m_run - m_new);
#pragma unroll
    for (int j = 0; j < NDB; ++j) w.acc[j] *= alpha;
    w.l_run *= alpha;
    w.m_run = m_new;
  }
  const float m_use = MASKED && w.m_run == ninf() ? 0.f : w.m_run;
  float rowsum = 0.f;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][i], scale_log2, -m_use));
      s[sb][i] = e;
      rowsum += e;
    }
  }
  w.l_run += rowsum;

  // O^T += V^T . P^T
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    if (MASKED && !(sb ? run1 : run0)) continue;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const f32x8_t pf = {s[sb][8 * cc + 0], s[sb][8 * cc + 1], s[sb][8 * cc + 2],
                          s[sb][8 * cc + 3], s[sb][8 * cc + 4], s[sb][8 * cc + 5],
                          s[sb][8 * cc + 6], s[sb][8 * cc + 7]};
      const bf16x8_t pb = __builtin_convertvector(pf, bf16x8_t);
      const __bf16* vsrc = vs + vrd + (32 * sb + 16 * cc) * C::VS;
#pragma unroll
      for (int j = 0; j < NDB; ++j) {
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vsrc + 32 * j));
        const i16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vsrc + 8 * C::VS + 32 * j));
        const bf16x8_t a =
            __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        w.acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, w.acc[j], 0, 0, 0);
      }
    }
  }
}

template <int D, bool SEG>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(const FwdParams p) {
  using C = Bf16Cfg<D>;
  constexpr int TN = C::TN;
  constexpr int NDB = D / 32;

  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][TN * C::KS];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[2][TN * C::VS];
  __shared__ int32_t seg_lds[2][SEG ? TN : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 31;
  const int half = lane >> 5;

  const WgCoord wc = wg_coord(p);
  const int b = wc.b, h = wc.h, m0 = wc.m0;
  const int qg0 = m0 + wave * 32;
  const bool wave_active = qg0 < p.seq_q;
  const int64_t pq_first = (int64_t)p.ring_index * p.seq_q + qg0;
  const WaveLimits lim = wave_limits(p, pq_first, lrow);
  const int64_t kend = wg_kend(p, m0);
  int32_t seg_q = 0;
  if (SEG && wave_active) seg_q = p.seg[(int64_t)b * p.seq_k + pq_first + lrow];

  const int64_t rs = (int64_t)p.heads * D;            // row stride (elements)
  const uint32_t rs_bytes = (uint32_t)(rs * 2);

  // Q of this wave as the MFMA B operand (queries are the N dimension).
  bf16x8_t qf[D / 16];
  if (wave_active) {
    const __bf16* qrow = static_cast<const __bf16*>(p.q) +
                         ((int64_t)b * p.seq_q + qg0 + lrow) * rs + (int64_t)h * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      qf[c] = __builtin_bit_cast(bf16x8_t,
                                 *reinterpret_cast<const uint4*>(qrow + 16 * c + 8 * half));
  }

  // Fixed per-thread offsets of the cooperative tile loads.
  uint32_t goff[C::LOADS];
  int kst[C::LOADS], vst[C::LOADS];
#pragma unroll
  for (int u = 0; u < C::LOADS; ++u) {
    const int ci = tid + u * kThreads;
    const int row = ci / C::GR, g = ci % C::GR;
    goff[u] = (uint32_t)row * rs_bytes + (uint32_t)g * 16u;
    kst[u] = row * C::KS + g * 8;
    vst[u] = row * C::VS + g * 8;
  }
  // Source address of this lane's transposing V reads (see above).
  const int vrd = (4 * half + ((lane & 15) >> 2)) * C::VS + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  Bf16Wave<D> w;
#pragma unroll
  for (int j = 0; j < NDB; ++j) w.acc[j] = f32x16_t{};
  w.m_run = ninf();
  w.l_run = 0.f;

  const __bf16* kbase0 = static_cast<const __bf16*>(p.k) + (int64_t)b * p.seq_k * rs + (int64_t)h * D;
  const __bf16* vbase0 = static_cast<const __bf16*>(p.v) + (int64_t)b * p.seq_k * rs + (int64_t)h * D;
  const int32_t* sbase0 = SEG ? p.seg + (int64_t)b * p.seq_k : nullptr;

  u32x4_t kreg[C::LOADS], vreg[C::LOADS];
  int32_t sreg = 0;
  auto load_tile = [&](const Cursor& c) {
    const int64_t row0 = (int64_t)c.kb * p.seq_q + (int64_t)c.kt * TN;
    const int nvalid = std::min(TN, c.klen - c.kt * TN);
    const uint32_t bytes = (uint32_t)nvalid * rs_bytes;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase0 + row0 * rs, bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase0 + row0 * rs, bytes);
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      kreg[u] = __builtin_amdgcn_raw_buffer_load_b128(kr, goff[u], 0, 0);
      vreg[u] = __builtin_amdgcn_raw_buffer_load_b128(vr, goff[u], 0, 0);
    }
    if (SEG && tid < TN) {
      const __amdgpu_buffer_rsrc_t sr = make_rsrc(sbase0 + row0, (uint32_t)nvalid * 4u);
      sreg = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(sr, tid * 4, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      *reinterpret_cast<u32x4_t*>(&k_lds[buf][kst[u]]) = kreg[u];
      *reinterpret_cast<u32x4_t*>(&v_lds[buf][vst[u]]) = vreg[u];
    }
    if (SEG && tid < TN) seg_lds[buf][tid] = sreg;
  };

  Cursor cur{0, 0, 0, 0, 0, 0};
  cursor_seek<TN>(p, cur, kend);
  if (cur.valid) {
    load_tile(cur);
    store_tile(0);
  }
  __syncthreads();

  int buf = 0;
  while (cur.valid) {
    Cursor nxt = cur;
    cursor_next<TN>(p, nxt, kend);
    if (nxt.valid) load_tile(nxt);

    const int kloc0 = cur.kt * TN;
    const int64_t pk_tile = (int64_t)cur.kb * p.seq_q + kloc0;
    const bool run0 = wave_active && pk_tile < lim.run_lim;
    const bool run1 = wave_active && (kloc0 + 32 < cur.klen) && pk_tile + 32 < lim.run_lim;
    const bool mask0 = SEG || !(pk_tile + 31 < lim.full_lim);
    const bool mask1 = SEG || !(pk_tile + 63 < lim.full_lim);
    if (run0 || run1) {
      const int32_t* sg = SEG ? seg_lds[buf] : nullptr;
      if (!SEG && run0 && run1 && !mask0 && !mask1)
        bf16_tile<D, false, false>(w, qf, k_lds[buf], v_lds[buf], sg, lrow, half, vrd, true, true,
                                   false, false, (int32_t)pk_tile, lim.lane_lim, seg_q,
                                   p.scale_log2);
      else
        bf16_tile<D, true, SEG>(w, qf, k_lds[buf], v_lds[buf], sg, lrow, half, vrd, run0, run1,
                                mask0, mask1, (int32_t)pk_tile, lim.lane_lim, seg_q,
                                p.scale_log2);
      if (p.run_map != nullptr && lane == 0) {
        if (run0) write_run_map(p, cur.t, qg0, kloc0);
        if (run1) write_run_map(p, cur.t, qg0, kloc0 + 32);
      }
    }

    if (nxt.valid) store_tile(buf ^ 1);
    __syncthreads();
    cur = nxt;
    buf ^= 1;
  }

  // ---- epilogue: out = numerator / denominator, lse = ln(denominator) + max ----
  if (!wave_active) return;
  const float l_tot = w.l_run + __shfl_xor(w.l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int row = qg0 + lrow;
  __bf16* orow = static_cast<__bf16*>(p.out) + ((int64_t)b * p.seq_q + row) * rs + (int64_t)h * D;
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      typedef float f32x4_t __attribute__((ext_vector_type(4)));
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      const f32x4_t o = {w.acc[j][4 * g] * inv, w.acc[j][4 * g + 1] * inv,
                         w.acc[j][4 * g + 2] * inv, w.acc[j][4 * g + 3] * inv};
      *reinterpret_cast<bf16x4_t*>(orow + 32 * j + 8 * g + 4 * half) =
          __builtin_convertvector(o, bf16x4_t);
    }
  }
  if (half == 0)
    p.lse[((int64_t)b * p.heads + h) * p.seq_q + row] =
        l_tot > 0.f ? (w.m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : ninf();
}

// ---------------------------------------------------------------------------
// fp32 kernel
// ---------------------------------------------------------------------------
//
// 32-key tiles, K and V row-major in LDS with a 4-element pad, fp32 MFMA
// v_mfma_f32_32x32x2_f32 (one k-slot per lane half).  The P.V A operand is
// V^T: lane (d, half) reads V[key][d] for the key its P^T slot holds.

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_f32_kernel(const FwdParams p) {
  constexpr int TN = 32;
  constexpr int KS = D + 4;
  constexpr int NDB = D / 32;
  constexpr int LOADS = TN * D / 4 / kThreads;

  __shared__ __attribute__((aligned(16))) float k_lds[2][TN * KS];
  __shared__ __attribute__((aligned(16))) float v_lds[2][TN * KS];
  __shared__ int32_t seg_lds[2][TN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 31;
  const int half = lane >> 5;

  const WgCoord wc = wg_coord(p);
  const int b = wc.b, h = wc.h, m0 = wc.m0;
  const int qg0 = m0 + wave * 32;
  const bool wave_active = qg0 < p.seq_q;
  const int64_t pq_first = (int64_t)p.ring_index * p.seq_q + qg0;
  const WaveLimits lim = wave_limits(p, pq_first, lrow);
  const int64_t kend = wg_kend(p, m0);
  const bool has_seg = p.seg != nullptr;
  int32_t seg_q = 0;
  if (has_seg && wave_active) seg_q = p.seg[(int64_t)b * p.seq_k + pq_first + lrow];

  const int64_t rs = (int64_t)p.heads * D;
  float qf[D / 2];
  if (wave_active) {
    const float* qrow = static_cast<const float*>(p.q) +
                        ((int64_t)b * p.seq_q + qg0 + lrow) * rs + (int64_t)h * D;
#pragma unroll
    for (int c = 0; c < D / 2; ++c) qf[c] = qrow[2 * c + half];
  }

  f32x16_t acc[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) acc[j] = f32x16_t{};
  float m_run = ninf();
  float l_run = 0.f;

  const float* kbase0 = static_cast<const float*>(p.k) + (int64_t)b * p.seq_k * rs + (int64_t)h * D;
  const float* vbase0 = static_cast<const float*>(p.v) + (int64_t)b * p.seq_k * rs + (int64_t)h * D;

  float4 kreg[LOADS], vreg[LOADS];
  int32_t sreg = 0;
  auto load_tile = [&](const Cursor& c) {
    const int64_t row0 = (int64_t)c.kb * p.seq_q + (int64_t)c.kt * TN;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int ci = tid + u * kThreads;
      const int row = ci / (D / 4), col = (ci % (D / 4)) * 4;
      kreg[u] = *reinterpret_cast<const float4*>(kbase0 + (row0 + row) * rs + col);
      vreg[u] = *reinterpret_cast<const float4*>(vbase0 + (row0 + row) * rs + col);
    }
    if (has_seg && tid < TN) sreg = p.seg[(int64_t)b * p.seq_k + row0 + tid];
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int ci = tid + u * kThreads;
      const int row = ci / (D / 4), col = (ci % (D / 4)) * 4;
      *reinterpret_cast<float4*>(&k_lds[buf][row * KS + col]) = kreg[u];
      *reinterpret_cast<float4*>(&v_lds[buf][row * KS + col]) = vreg[u];
    }
    if (has_seg && tid < TN) seg_lds[buf][tid] = sreg;
  };

  Cursor cur{0, 0, 0, 0, 0, 0};
  cursor_seek<TN>(p, cur, kend);
  if (cur.valid) {
    load_tile(cur);
    store_tile(0);
  }
  __syncthreads();

  int buf = 0;
  while (cur.valid) {
    Cursor nxt = cur;
    cursor_next<TN>(p, nxt, kend);
    if (nxt.valid) load_tile(nxt);

    const int kloc0 = cur.kt * TN;
    const int64_t pk0 = (int64_t)cur.kb * p.seq_q + kloc0;
    const bool run = wave_active && pk0 < lim.run_lim;
    const bool mask = has_seg || !(pk0 + 31 < lim.full_lim);
    if (run) {
      const float* ks = k_lds[buf];
      const float* vs = v_lds[buf];
      const int32_t* sg = seg_lds[buf];
      f32x16_t s = f32x16_t{};
      const float* krow = ks + lrow * KS + half;
#pragma unroll
      for (int c = 0; c < D / 2; ++c)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * c], qf[c], s, 0, 0, 0);

      if (mask) {
        const int32_t pkb = (int32_t)pk0 + 4 * half;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int koff = 8 * (i >> 2) + (i & 3);
          bool ok = pkb + koff < lim.lane_lim;
          if (has_seg) ok = ok && sg[4 * half + koff] == seg_q;
          if (!ok) s[i] = ninf();
        }
      }
      float mx = ninf();
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * p.scale_log2);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
        const float alpha = m_new == ninf() ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int j = 0; j < NDB; ++j) acc[j] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == ninf() ? 0.f : m_run;
      float rowsum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], p.scale_log2, -m_use));
        rowsum += s[i];
      }
      l_run += rowsum;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float* vrow = vs + (8 * (i >> 2) + 4 * half + (i & 3)) * KS;
#pragma unroll
        for (int j = 0; j < NDB; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * j + lrow], s[i], acc[j], 0, 0, 0);
      }
      if (p.run_map != nullptr && lane == 0) write_run_map(p, cur.t, qg0, kloc0);
    }

    if (nxt.valid) store_tile(buf ^ 1);
    __syncthreads();
    cur = nxt;
    buf ^= 1;
  }

  if (!wave_active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int row = qg0 + lrow;
  float* orow = static_cast<float*>(p.out) + ((int64_t)b * p.seq_q + row) * rs + (int64_t)h * D;
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      *reinterpret_cast<float4*>(orow + 32 * j + 8 * g + 4 * half) =
          make_float4(acc[j][4 * g] * inv, acc[j][4 * g + 1] * inv, acc[j][4 * g + 2] * inv,
                      acc[j][4 * g + 3] * inv);
    }
  }
  if (half == 0)
    p.lse[((int64_t)b * p.heads + h) * p.seq_q + row] =
        l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : ninf();
}

__global__ void fill_u8_kernel(uint8_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
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
  const dim3 grid(p.n_wg), block(kThreads);
  if (dtype == Dtype::BF16) {
    const bool seg = p.seg != nullptr;
    if (head_dim == 128) {
      if (seg)
        hipLaunchKernelGGL((fwd_bf16_kernel<128, true>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((fwd_bf16_kernel<128, false>), grid, block, 0, s, p);
    } else {
      if (seg)
        hipLaunchKernelGGL((fwd_bf16_kernel<64, true>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((fwd_bf16_kernel<64, false>), grid, block, 0, s, p);
    }
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, s, p);
    else
      hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, s, p);
  }
  e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(err, errlen, "kernel launch failed: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

}  // namespace ra
