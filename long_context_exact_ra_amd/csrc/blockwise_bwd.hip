// Backward of the blockwise exact attention for one Ring Attention device
// share, written for gfx950 (MI355X, CDNA4), bf16 inputs.
//
// The pages pair the ring forward with a backward pass but print no
// backward equations ("Ring Attention with Blockwise Transformers for
// Near-Infinite Context", section 三, the self-attention equation; the
// blockwise code of "从论文到代码：深入理解RingAttention的块注意力计算逻辑").
// These kernels compute the exact derivatives of the attention definition,
// with p_ij recomputed from the forward's lse:
//
//   delta_i = <dout_i, out_i>
//   p_ij    = exp(scale <q_i, k_j> - lse_i)        (0 where j is invisible)
//   ds_ij   = p_ij (<dout_i, v_j> - delta_i)
//   dq_i    = scale sum_j ds_ij k_j
//   dk_j    = scale sum_i ds_ij q_i,   dv_j = sum_i p_ij dout_i
//
// Three launches (four with key splits, below):
//   bwd_delta_kernel   delta (one pass over dout and out);
//   bwd_dq_kernel      query-stationary, like the forward: a workgroup owns
//                      256 query rows and walks the key tiles in the
//                      forward's order (the local block last), K and V tiles
//                      arriving by buffer-to-LDS DMA through a 4-stage ring;
//   bwd_dkdv_kernel    key-stationary: a workgroup owns 256 keys (K of each
//                      wave in registers, V resident in LDS) and streams the
//                      query tiles that can see them (Q, dout, segment ids,
//                      lse and delta) through two LDS stages.
// With key splits (small shares, whose query tiles leave compute units
// idle), the dq kernel's workgroups each walk one run of the key tiles and
// write their addend to dq into a workspace; a fourth launch,
// bwd_dq_sum_kernel, adds them in split order.
// Both main kernels recompute the scores and dp, so a visible pair costs
// 7 matrix products here against the 5 of the algorithm; every result is
// written exactly once (no atomics), so dk and dv of keys no local query
// sees come out as 0.
//
// MFMA orientation (v_mfma_f32_32x32x16_bf16; A[m][k] lane l row m = l % 32,
// k-slots 8 (l / 32) .. +7; B[k][n] lane l column n = l % 32; C[m][n] lane l
// column n = l % 32, rows 8 (i / 4) + 4 (l / 32) + i % 4):
//   dq kernel:   S^T = K Q^T and dP^T = V dO^T (keys = M, queries = N), so
//                a lane holds one query row and its lse and delta are
//                per-lane scalars; dQ^T += K^T dS^T takes dS^T straight from
//                the C registers and K^T from transposing LDS reads of the
//                same K tile, with the same key-to-slot assignment.
//   dkdv kernel: S = Q K^T and dP = dO V^T (queries = M, keys = N), so a
//                lane holds one key; dV^T += dO^T P and dK^T += Q^T dS take P
//                and dS from the C registers and dO^T, Q^T from transposing
//                LDS reads of the Q and dO tiles.
// All tiles use one LDS layout (16-byte slots, r = row, g = 16-byte granule
// of the row): slot(r, g) = (g / 4) * 256 + (r / 16) * 64 + (g % 4) * 16 +
// ((r % 16) ^ (4 * (g % 4))), read as rows by ds_read_b128 and as columns by
// ds_read_b64_tr_b16.  LDS has 64 four-byte banks, so 16 consecutive slots
// (256 bytes) cover every bank once.  A row read (16 lanes: 16 rows, one
// granule) and a column read (32 lanes: 4 rows x 4 granules of a quad) each
// touch 16 slots that differ modulo 16, so neither has bank conflicts; the
// XOR of the row's bits 2-3 with the granule is what makes the column read
// conflict-free (without it, the 4 rows of a column read hit the same 4 of
// the 16 bank groups four times each).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <climits>
#include <cstdio>
#include <type_traits>

#include "ra_device.h"
#include "ra_internal.h"
#include "ra_lds.h"

namespace ra {
namespace {

constexpr int kWaves = 8;                 // waves per workgroup (both main kernels)
constexpr int kThreadsBwd = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

// The layout's arithmetic (slot map, DMA lane map, row and column read
// offsets) lives in ra_lds.h, where tests/lds_check.cpp checks it on the
// host against the MFMA operand layout and the LDS banks.
__device__ __forceinline__ uint32_t tile_lane_off(int lane, uint32_t rs_bytes) {
  return (uint32_t)lds::bwd_dma_row(lane) * rs_bytes + 16u * (uint32_t)lds::bwd_dma_gran(lane);
}
__device__ __forceinline__ int row_rd(int lane) { return lds::bwd_row_rd(lane); }
__device__ __forceinline__ constexpr int row_rd_c(int rd, int c) { return lds::bwd_row_rd_c(rd, c); }
__device__ __forceinline__ constexpr int row_off(int c, int blk) { return lds::bwd_row_off(c, blk); }
__device__ __forceinline__ int col_rd(int lane) { return lds::bwd_col_rd(lane); }
__device__ __forceinline__ constexpr int col_off(int jb, int rb) { return lds::bwd_col_off(jb, rb); }

__device__ __forceinline__ bf16x8_t col_operand(const __bf16* tile, int rd, int jb, int rb) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(tile + rd + col_off(jb, rb)));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4_t*)(tile + lds::bwd_col_hi(rd) + col_off(jb, rb)));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bf16x8_t row_operand(const __bf16* tile, int rd, int c, int blk) {
  return *reinterpret_cast<const bf16x8_t*>(tile + row_rd_c(rd, c) + row_off(c, blk));
}

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// s_waitcnt lgkmcnt(0): this wave's LDS writes have completed (gfx9
// encoding; vmcnt and expcnt not waited).  A barrier alone does not wait for
// them on gfx950, so writes that other waves read after a barrier wait here
// first.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// ---------------------------------------------------------------------------
// delta_i = <dout_i, out_i>
// ---------------------------------------------------------------------------

// 16 lanes per row of D = 128 (8 for D = 64), 8 values each (T: __bf16 or
// float, the input dtype; the sum is float32).
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const BwdParams bp) {
  constexpr int LPR = D / 8;  // lanes per row
  const FwdParams& p = bp.f;
  const int64_t rows = (int64_t)p.batch * p.seq_q * p.heads;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const T* o = static_cast<const T*>(bp.out) + row * D + part * 8;
    const T* g = static_cast<const T*>(bp.dout) + row * D + part * 8;
    if constexpr (std::is_same<T, __bf16>::value) {
      const bf16x8_t ov = *reinterpret_cast<const bf16x8_t*>(o);
      const bf16x8_t gv = *reinterpret_cast<const bf16x8_t*>(g);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = __builtin_fmaf((float)ov[i], (float)gv[i], acc);
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float4 ov = *reinterpret_cast<const float4*>(o + 4 * u);
        const float4 gv = *reinterpret_cast<const float4*>(g + 4 * u);
        acc = __builtin_fmaf(ov.x, gv.x, acc);
        acc = __builtin_fmaf(ov.y, gv.y, acc);
        acc = __builtin_fmaf(ov.z, gv.z, acc);
        acc = __builtin_fmaf(ov.w, gv.w, acc);
      }
    }
  }
#pragma unroll
  for (int m = LPR / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < rows && part == 0) {
    // row = (b * Lq + i) * H + h  ->  delta[b][h][i]
    const int64_t h = row % p.heads, bi = row / p.heads;
    const int64_t b = bi / p.seq_q, i = bi % p.seq_q;
    bp.delta[(b * p.heads + h) * p.seq_q + i] = acc;
  }
}

// ---------------------------------------------------------------------------
// dq kernel (query-stationary)
// ---------------------------------------------------------------------------

template <int D, bool SEG>
struct DqStage {
  static constexpr int ELEMS = 64 * D;  // bf16 per 64-row tensor tile
  static constexpr int STAGE = 2 * ELEMS + (SEG ? 128 : 0);
  static constexpr int NPT = 2 * (64 * D / 8 / 64 / kWaves) + (SEG ? 1 : 0);  // DMA per wave
};

struct DqWave {
  int lane, lrow, half, wave, qg0, k_rd, t_rd;
  bool active;
  int32_t seg_q;
  SegRange qseg;  // id range of the wave's queries
  int64_t kend;
  const char* kbase0;
  const char* vbase0;
  const int32_t* sbase0;
  uint32_t rs_bytes, k_lane;
};

// One key tile: S^T, dP^T, dS^T and dQ^T += K^T dS^T.
template <int D, bool SEG, bool STRIPED>
__device__ __forceinline__ void dq_tile(const FwdParams& p, const DqWave& w, const WaveLimits& lim,
                                        const TileInfo& ti, const bf16x8_t* qf,
                                        const bf16x8_t* dof, float lse2, const f32x16_t& ndlt,
                                        f32x16_t* acc, const __bf16* kst, const __bf16* vst,
                                        const int32_t* sg) {
  constexpr int NDB = D / 32;
  TileFlags f = tile_flags<SEG, STRIPED>(ti, lim);
  if (SEG) {
    // Halves whose key ids miss the queries' id range hold no visible pair.
    const uint32_t ok = seg_overlap_halves(sg, w.lane, w.qseg);
    f.run0 = f.run0 && (ok & 1u);
    f.run1 = f.run1 && (ok & 2u);
    // Halves whose keys and queries all carry one id need no id test.
    f.seg0 = !(ok & 4u);
    f.seg1 = !(ok & 8u);
  }
  if (!(f.run0 || f.run1)) return;
  // dp starts from -delta (each lane holds one query row), so the MFMAs
  // deliver dP - delta directly.
  f32x16_t s[2], dp[2];
  // Without segment ids (registers to spare), each MFMA's LDS operand is
  // read two MFMAs ahead (fenced), so an MFMA does not wait on the read
  // issued just before it.
  constexpr bool kPrefetch = !SEG;
  if constexpr (kPrefetch) {
    constexpr int NM = 2 * 2 * (D / 16);  // MFMAs (sb, c, S or dP)
    auto rread = [&](int n) {
      const int sb = n / (D / 8), c = (n / 2) % (D / 16);
      return row_operand((n & 1) ? vst : kst, w.k_rd, c, sb);
    };
    bf16x8_t o[3];
    o[0] = rread(0);
    o[1] = rread(1);
#pragma unroll
    for (int n = 0; n < NM; ++n) {
      if (n + 2 < NM) o[(n + 2) % 3] = rread(n + 2);
      __builtin_amdgcn_sched_barrier(0);
      const int sb = n / (D / 8), c = (n / 2) % (D / 16);
      if (n & 1)
        dp[sb] = mfma(o[n % 3], dof[c], c == 0 ? ndlt : dp[sb]);
      else
        s[sb] = mfma(o[n % 3], qf[c], c == 0 ? f32x16_t{} : s[sb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = mfma(row_operand(kst, w.k_rd, 0, sb), qf[0], f32x16_t{});
      dp[sb] = mfma(row_operand(vst, w.k_rd, 0, sb), dof[0], ndlt);
#pragma unroll
      for (int c = 1; c < D / 16; ++c) {
        s[sb] = mfma(row_operand(kst, w.k_rd, c, sb), qf[c], s[sb]);
        dp[sb] = mfma(row_operand(vst, w.k_rd, c, sb), dof[c], dp[sb]);
      }
    }
  }
  // With segment ids every tile takes the masked path (a second, unmasked
  // path would not fit the register budget); single-id halves skip only the
  // id compare there.
  const bool masked = SEG || !(f.run0 && f.run1) || f.mask0 || f.mask1;
  if (masked) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const bool r = sb ? f.run1 : f.run0, m = sb ? f.mask1 : f.mask0;
      const int32_t nvis = !r ? 0 : m ? lim.lane_lim - (f.pk + 32 * sb + 4 * w.half) : 32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int koff = 8 * (i >> 2) + (i & 3);
        bool ok = koff < nvis;
        if (SEG && (sb ? f.seg1 : f.seg0)) ok = ok && sg[32 * sb + 4 * w.half + koff] == w.seg_q;
        s[sb][i] = ok ? s[sb][i] : ninf();
      }
    }
  }
  bf16x8_t dsb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x8_t d;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = 8 * (q & 1) + i;
      const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[q >> 1][e], p.scale_log2, -lse2));
      d[i] = pr * dp[q >> 1][e];
    }
    dsb[q] = __builtin_convertvector(d, bf16x8_t);
  }
  if constexpr (kPrefetch) {
    constexpr int NM = 4 * NDB;  // MFMAs (k-step 2 sb + cc, j)
    auto cread = [&](int n) { return col_operand(kst, w.t_rd, n % NDB, n / NDB); };
    bf16x8_t o[3];
    o[0] = cread(0);
    o[1] = cread(1);
#pragma unroll
    for (int n = 0; n < NM; ++n) {
      if (n + 2 < NM) o[(n + 2) % 3] = cread(n + 2);
      __builtin_amdgcn_sched_barrier(0);
      acc[n % NDB] = mfma(o[n % 3], dsb[n / NDB], acc[n % NDB]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int j = 0; j < NDB; ++j)
          acc[j] = mfma(col_operand(kst, w.t_rd, j, 2 * sb + cc), dsb[2 * sb + cc], acc[j]);
  }
}

template <int D, bool SEG, bool STRIPED>
__global__ __launch_bounds__(kThreadsBwd, 1) void bwd_dq_kernel(const BwdParams bp) {
  using St = DqStage<D, SEG>;
  constexpr int NDB = D / 32, NPT = St::NPT;
  const FwdParams& p = bp.f;
  __shared__ __attribute__((aligned(16))) __bf16 st0[St::STAGE], st1[St::STAGE], st2[St::STAGE],
      st3[St::STAGE];
  __bf16* const stg[4] = {st0, st1, st2, st3};

  DqWave w;
  w.lane = threadIdx.x & 63;
  w.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  w.lrow = w.lane & 31;
  w.half = w.lane >> 5;
  // With key splits: one workgroup per run of each query tile's walk, as in
  // the forward (a workgroup past the runs exits).
  const WgCoord wc = p.split_wgs > 0 ? wg_coord_runs<kBlockMBf16, 64, STRIPED>(p)
                                     : wg_coord<kBlockMBf16>(p);
  if (wc.split < 0) return;
  const int b = wc.b, h = wc.h, m0 = wc.m0;
  w.qg0 = m0 + w.wave * 32;
  w.active = w.qg0 < p.seq_q;
  // Storage row of the wave's first query (segment ids) and its query
  // coordinate (causal limits; the local row under striped placement).
  const int64_t pq_first = (int64_t)p.ring_index * p.seq_q + w.qg0;
  const WaveLimits lim = wave_limits(p, STRIPED ? w.qg0 : pq_first, w.lrow, w.active);
  w.kend = wg_kend<kBlockMBf16, STRIPED>(p, m0);
  // With key splits this workgroup walks only its run of the key tiles; a
  // surplus split of a short walk adds nothing to dq.
  const SplitRange sr = split_range<64, STRIPED>(
      p, wc.split, w.kend, wg_kend<kBlockMBf16, STRIPED>(p, (p.n_qtiles - 1) * kBlockMBf16));
  if (sr.idle) {
    if (w.active) {
      float* drow = bp.dq_part + (int64_t)wc.split * p.batch * p.seq_q * p.heads * D +
                    ((int64_t)b * p.seq_q + w.qg0 + w.lrow) * ((int64_t)p.heads * D) +
                    (int64_t)h * D;
#pragma unroll
      for (int j = 0; j < NDB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(drow + 32 * j + 8 * g + 4 * w.half) =
              make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  w.seg_q = 0;
  if (SEG && w.active) w.seg_q = p.seg[(int64_t)b * p.seq_k + pq_first + w.lrow];
  w.qseg = SegRange{0, 0};
  if (SEG) w.qseg = wave_range(w.seg_q);
  // Segment ids: mark the key tiles whose ids can meet the workgroup's.
  __shared__ uint8_t smask[SEG ? kSegMaskSlots : 1];
  __shared__ int32_t wg_ids[2 * kWaves];
  const uint8_t* smask_p = nullptr;
  if (SEG && p.ring_size * seg_mask_tpb(p) <= kSegMaskSlots) {
    if (w.lane == 0) {
      wg_ids[2 * w.wave] = w.active ? w.qseg.lo : INT32_MAX;
      wg_ids[2 * w.wave + 1] = w.active ? w.qseg.hi : INT32_MIN;
    }
    __syncthreads();
    SegRange wr{INT32_MAX, INT32_MIN};
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      wr.lo = min(wr.lo, wg_ids[2 * i]);
      wr.hi = max(wr.hi, wg_ids[2 * i + 1]);
    }
    build_seg_mask(p, p.seg + (int64_t)b * p.seq_k, wr, STRIPED ? INT64_MAX : w.kend, smask,
                   (int)threadIdx.x, kThreadsBwd);
    __syncthreads();
    smask_p = smask;
  }
  const int64_t rs = (int64_t)p.heads * D;
  w.rs_bytes = (uint32_t)(rs * 2);
  w.kbase0 = static_cast<const char*>(p.k) + ((int64_t)b * p.seq_k * rs + (int64_t)h * D) * 2;
  w.vbase0 = static_cast<const char*>(p.v) + ((int64_t)b * p.seq_k * rs + (int64_t)h * D) * 2;
  w.sbase0 = SEG ? p.seg + (int64_t)b * p.seq_k : nullptr;
  w.k_lane = tile_lane_off(w.lane, w.rs_bytes);
  w.k_rd = row_rd(w.lane);
  w.t_rd = col_rd(w.lane);

  // Q^T and dO^T of this wave as B operands; the row's lse (base 2) and delta.
  bf16x8_t qf[D / 16], dof[D / 16];
  float lse2 = 0.f, dlt = 0.f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    qf[c] = bf16x8_t{};
    dof[c] = bf16x8_t{};
  }
  if (w.active) {
    const int64_t roff = ((int64_t)b * p.seq_q + w.qg0 + w.lrow) * rs + (int64_t)h * D;
    const __bf16* qrow = static_cast<const __bf16*>(p.q) + roff;
    const __bf16* grow = static_cast<const __bf16*>(bp.dout) + roff;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      qf[c] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * c + 8 * w.half);
      dof[c] = *reinterpret_cast<const bf16x8_t*>(grow + 16 * c + 8 * w.half);
    }
    const int64_t li = ((int64_t)b * p.heads + h) * p.seq_q + w.qg0 + w.lrow;
    lse2 = bp.lse[li];
    dlt = bp.delta[li];
  }
  // These loads stay in flight while the prologue's K/V DMA is issued (a
  // workgroup of a short walk would otherwise pay both latencies in turn);
  // their values are first used after the prologue's wait.  The compiler
  // does not count the DMA (inline asm), so it waits for every load there.

  f32x16_t acc[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) acc[j] = f32x16_t{};

  // Tiles 0, 1, 2 in flight; tile i is read in step i, tile i+3 is fetched
  // into the stage of tile i-1 at the start of step i.
  TileInfo ti[4];
  Cursor ic{0, 0, 0, 0, 0, 0, 0};
  cursor_seek<64, STRIPED>(p, ic, w.kend);
  cursor_to<64, STRIPED>(p, ic, w.kend, sr.begin);
  auto fetch = [&](int s) {
    if (SEG && smask_p != nullptr) cursor_skip_masked<64, STRIPED>(p, ic, w.kend, smask_p);
    if (ic.pos >= sr.end) ic.valid = 0;
    ti[s] = tile_info<64, STRIPED>(p, ic);
    if (ic.valid) {
      __bf16* d = stg[s];
      issue_tile<D, kWaves, SEG>(ti[s], w.kbase0, w.vbase0, w.sbase0, w.rs_bytes, w.wave, w.lane,
                                 w.k_lane, w.k_lane, d, d + St::ELEMS,
                                 reinterpret_cast<int32_t*>(d + 2 * St::ELEMS));
      cursor_next<64, STRIPED>(p, ic, w.kend);
    }
  };
  fetch(0);
  fetch(1);
  fetch(2);
  // Tile 0 must have landed for every wave before step 0 reads it.
  if (ti[2].valid)
    wait_vm<2 * NPT>();
  else if (ti[1].valid)
    wait_vm<NPT>();
  else
    wait_vm<0>();
  stage_barrier();
  // (The empty asm keeps the compiler from hoisting the uses, and its wait
  // for the loads, above the DMA.)
  asm volatile("" : "+v"(lse2), "+v"(dlt));
  lse2 *= kLog2e;
  f32x16_t ndlt;
#pragma unroll
  for (int i = 0; i < 16; ++i) ndlt[i] = -dlt;

  auto step = [&](auto PHc) -> bool {
    constexpr int PH = decltype(PHc)::value;
    constexpr int S0 = PH, S1 = (PH + 1) & 3;
    fetch((PH + 3) & 3);
    if (w.active)
      dq_tile<D, SEG, STRIPED>(p, w, lim, ti[S0], qf, dof, lse2, ndlt, acc, stg[S0], stg[S0] + St::ELEMS,
                      reinterpret_cast<const int32_t*>(stg[S0] + 2 * St::ELEMS));
    // Tile i+1 must have landed (for every wave) before the next step.
    if (ti[S1].valid) {
      if (ti[(PH + 3) & 3].valid)
        wait_vm<2 * NPT>();
      else if (ti[(PH + 2) & 3].valid)
        wait_vm<NPT>();
      else
        wait_vm<0>();
    }
    stage_barrier();
    return ti[S1].valid;
  };
  if (ti[0].valid) {
    for (;;) {
      if (!step(std::integral_constant<int, 0>{})) break;
      if (!step(std::integral_constant<int, 1>{})) break;
      if (!step(std::integral_constant<int, 2>{})) break;
      if (!step(std::integral_constant<int, 3>{})) break;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  if (!w.active) return;
  const float scale = p.scale_log2 / kLog2e;
  // A split writes its addend to dq into its own slice of the workspace.
  float* const dst =
      bp.dq_part != nullptr
          ? bp.dq_part + (int64_t)wc.split * p.batch * p.seq_q * p.heads * D
          : bp.dq;
  float* drow = dst + ((int64_t)b * p.seq_q + w.qg0 + w.lrow) * rs + (int64_t)h * D;
#pragma unroll
  for (int j = 0; j < NDB; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(drow + 32 * j + 8 * g + 4 * w.half) =
          make_float4(acc[j][4 * g] * scale, acc[j][4 * g + 1] * scale,
                      acc[j][4 * g + 2] * scale, acc[j][4 * g + 3] * scale);
}

// ---------------------------------------------------------------------------
// dk / dv kernel (key-stationary)
// ---------------------------------------------------------------------------

template <int D, bool SEG>
struct KvLds {
  static constexpr int ELEMS = 64 * D;                     // one 64-row tile
  static constexpr int VRES = kBlockNBwd / 64 * ELEMS;     // resident V, 4 tiles
  // A query stage: Q tile, dO tile, then 64 segment ids, 64 lse, 64 delta.
  static constexpr int QSTAGE = 2 * ELEMS + 3 * 128;
};

// Which (batch, head, key tile) a workgroup owns: consecutive key tiles of
// one head (which stream the same queries) share an XCD; earlier key tiles,
// seen by more queries under a causal mask, come first.
__device__ __forceinline__ WgCoord kv_coord(const BwdParams& bp) {
  const int pid = blockIdx.x, n = bp.n_wg_kv;
  const int xcd = pid & 7, idx = pid >> 3, cnt = n >> 3, rem = n & 7;
  const int logical =
      xcd < rem ? xcd * (cnt + 1) + idx : rem * (cnt + 1) + (xcd - rem) * cnt + idx;
  const int kt = logical % bp.n_ktiles;
  const int bh = logical / bp.n_ktiles;
  return WgCoord{__builtin_amdgcn_readfirstlane(bh / bp.f.heads),
                 __builtin_amdgcn_readfirstlane(bh % bp.f.heads),
                 __builtin_amdgcn_readfirstlane(kt * kBlockNBwd)};
}

template <int D, bool SEG, bool STRIPED>
__global__ __launch_bounds__(kThreadsBwd, 1) void bwd_dkdv_kernel(const BwdParams bp) {
  using L = KvLds<D, SEG>;
  constexpr int NDB = D / 32;
  // Operand reads ahead of the MFMAs need registers that the segment-id
  // variants do not have (they spill): those keep the reads next to their
  // MFMAs.  On the 7B share the read-ahead makes the kernel 2.7 % faster.
  constexpr bool kPrefetch = !SEG;
  const FwdParams& p = bp.f;
  __shared__ __attribute__((aligned(16))) __bf16 vres[L::VRES];
  __shared__ __attribute__((aligned(16))) __bf16 qs[2 * L::QSTAGE];  // two query stages

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 31, half = lane >> 5;
  const WgCoord wc = kv_coord(bp);
  const int b = wc.b, h = wc.h, k0 = wc.m0;
  const int kw0 = k0 + 32 * wave;          // first key of this wave
  const bool active = kw0 < p.seq_k;       // seq_k is a multiple of 32
  const int key = kw0 + lrow;              // this lane's key
  const int64_t rs = (int64_t)p.heads * D;
  const uint32_t rs_bytes = (uint32_t)(rs * 2);
  const uint32_t lane_off = tile_lane_off(lane, rs_bytes);
  const int r_rd = row_rd(lane), t_rd = col_rd(lane);
  const int32_t qrow0 = p.ring_index * p.seq_q;  // storage row of local row 0
  // Query coordinate of local row 0: its global position (contiguous), 0
  // (striped: the coordinate is the local row itself).
  const int32_t qpos0 = STRIPED ? 0 : qrow0;

  const KeyThresholds kth = key_thresholds<STRIPED>(p, kw0, lrow);
  const int64_t c = p.causal;
  const int32_t thr = kth.lane, thr_first = kth.first, thr_last = kth.last;
  const int32_t seg_k = SEG && active ? p.seg[(int64_t)b * p.seq_k + key] : 0;
  const SegRange kseg = SEG ? wave_range(seg_k) : SegRange{0, 0};  // the wave's key ids

  // K^T of this wave as the B operand of S = Q K^T.
  bf16x8_t kf[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) kf[cc] = bf16x8_t{};
  if (active) {
    const __bf16* krow = static_cast<const __bf16*>(p.k) +
                         ((int64_t)b * p.seq_k + key) * rs + (int64_t)h * D;
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc)
      kf[cc] = *reinterpret_cast<const bf16x8_t*>(krow + 16 * cc + 8 * half);
  }

  // The workgroup's V rows, resident in LDS for the whole walk.
  const char* vbase0 = static_cast<const char*>(p.v) + ((int64_t)b * p.seq_k * rs + (int64_t)h * D) * 2;
  const int kend = std::min(p.seq_k, k0 + kBlockNBwd);
#pragma unroll
  for (int t = 0; t < kBlockNBwd / 64; ++t)
    issue_rows<D, kWaves>(TileInfo{k0 + 64 * t, kend, 0, 0, 1, 0}, vbase0, rs_bytes, wave, lane_off,
                          vres + t * L::ELEMS);
  __builtin_amdgcn_s_waitcnt(0);
  // The resident V is kept negated: dp starts from delta (read from the
  // query stage straight into the accumulators), so the MFMAs deliver
  // delta - dout.v_j and no subtraction per pair is left.  Each wave flips
  // the sign bits of the 16-byte slots its own DMA wrote (lane l of DMA
  // instruction j wrote slot 64 j + l); the walk's first barrier orders
  // these writes before any read.
  {
    constexpr int DPW = 64 * D / 8 / 64 / kWaves;  // DMA instructions per wave and tile
#pragma unroll
    for (int t = 0; t < kBlockNBwd / 64; ++t)
#pragma unroll
      for (int u = 0; u < DPW; ++u) {
        u32x4_t* slot = reinterpret_cast<u32x4_t*>(vres + t * L::ELEMS + (wave * DPW + u) * 512 + 8 * lane);
        *slot = *slot ^ 0x80008000u;
      }
    wait_lds();
  }

  // Query rows that can see any key of the workgroup: [q_lo, Lq).
  int q_lo = first_query_row<STRIPED>(p, k0, kBlockNBwd, qpos0);
  q_lo &= ~63;
  const int n_qt = (p.seq_q - q_lo + 63) / 64;

  const char* qbase0 = static_cast<const char*>(p.q) + ((int64_t)b * p.seq_q * rs + (int64_t)h * D) * 2;
  const char* gbase0 = static_cast<const char*>(bp.dout) + ((int64_t)b * p.seq_q * rs + (int64_t)h * D) * 2;
  const int32_t* sbase0 = SEG ? p.seg + (int64_t)b * p.seq_k + qrow0 : nullptr;
  const float* lbase = bp.lse + ((int64_t)b * p.heads + h) * p.seq_q;
  const float* dbase = bp.delta + ((int64_t)b * p.heads + h) * p.seq_q;

  // Per wave, the DMA of a stage is its share of the Q and dO tiles (and
  // ids): kQDma instructions, issued after the lse (wave 0) or delta (wave 1).
  constexpr int kQDma = 2 * (64 * D / 8 / 64 / kWaves) + (SEG ? 1 : 0);
  auto fetch = [&](int qt, int s) {
    const int q0 = q_lo + 64 * qt;
    __bf16* d = qs + s * L::QSTAGE;
    const int nvalid = std::min(64, p.seq_q - q0);
    if (wave == 0)
      dma_b32(lds_addr(d + 2 * L::ELEMS + 128), (uint32_t)lane * 4u,
              rsrc_words(lbase + q0, (uint32_t)nvalid * 4u));
    if (wave == 1)
      dma_b32(lds_addr(d + 2 * L::ELEMS + 256), (uint32_t)lane * 4u,
              rsrc_words(dbase + q0, (uint32_t)nvalid * 4u));
    issue_tile<D, kWaves, SEG>(TileInfo{q0, p.seq_q, 0, 0, 1, 0}, qbase0, gbase0, sbase0, rs_bytes,
                               wave, lane, lane_off, lane_off, d, d + L::ELEMS,
                               reinterpret_cast<int32_t*>(d + 2 * L::ELEMS));
  };
  // Wave 0, which fetched the stage's 64 lse, rewrites them as
  // -lse log2(e), the exponent's offset, once per query tile instead of once
  // per pair.  Its lse DMA must have landed (DMA completes in issue order,
  // so the kQDma issued after it may still be in flight), and the rewrite
  // completes before the barrier after which the stage is read.
  auto prep_lse = [&](int s) {
    if (wave != 0) return;
    wait_vm<kQDma>();
    float* l = reinterpret_cast<float*>(qs + s * L::QSTAGE + 2 * L::ELEMS + 128);
    l[lane] = l[lane] * -kLog2e;
    wait_lds();
  };

  // Segment ids: list the query tiles whose id range meets the id range of
  // the workgroup's keys (exact: disjoint ranges share no id); the walk
  // fetches only those.  Wave 0 tests 64 tiles per round, one per lane, and
  // appends the hits in order.
  constexpr int kQList = 2048;
  __shared__ int16_t qlist[SEG ? kQList : 1];
  __shared__ int32_t wg_ids[2 * kWaves + 1];
  int n_run = n_qt;
  bool use_list = false;
  if (SEG && n_qt <= kQList) {
    if (lane == 0) {
      wg_ids[2 * wave] = active ? kseg.lo : INT32_MAX;
      wg_ids[2 * wave + 1] = active ? kseg.hi : INT32_MIN;
    }
    __syncthreads();
    if (wave == 0) {
      SegRange kr{INT32_MAX, INT32_MIN};
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        kr.lo = min(kr.lo, wg_ids[2 * i]);
        kr.hi = max(kr.hi, wg_ids[2 * i + 1]);
      }
      int n = 0;
      for (int t0 = 0; t0 < n_qt; t0 += 64) {
        const int t = t0 + lane;
        bool hit = false;
        if (t < n_qt) {
          const int q0 = q_lo + 64 * t;
          const int nq = std::min(64, p.seq_q - q0);
          int32_t lo = INT32_MAX, hi = INT32_MIN;
#pragma unroll
          for (int j = 0; j < 64; ++j) {
            if (j < nq) {
              const int32_t v = sbase0[q0 + j];
              lo = min(lo, v);
              hi = max(hi, v);
            }
          }
          hit = hi >= kr.lo && lo <= kr.hi;
        }
        const uint64_t m = __builtin_amdgcn_ballot_w64(hit);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (hit) qlist[n + below] = (int16_t)t;
        n += __builtin_popcountll(m);
      }
      if (lane == 0) wg_ids[2 * kWaves] = n;
    }
    __syncthreads();
    n_run = __builtin_amdgcn_readfirstlane(wg_ids[2 * kWaves]);
    use_list = true;
  }
  auto tile_of = [&](int i) -> int {
    return use_list ? __builtin_amdgcn_readfirstlane((int)qlist[i]) : i;
  };

  f32x16_t dk[NDB], dv[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
    dk[j] = f32x16_t{};
    dv[j] = f32x16_t{};
  }

  if (n_run > 0) {
    fetch(tile_of(0), 0);
    prep_lse(0);
  }
  // One barrier per query tile: after it, tile qt has landed for every wave
  // (each waited for its own share, the only DMA in flight) and every wave
  // is done with the previous tile, so the next tile's DMA may refill that
  // stage.
  for (int it = 0; it < n_run; ++it) {
    const int qt = tile_of(it);
    const int s = it & 1;
    wait_vm<0>();
    wait_lds();  // this wave's reads of the previous tile have completed
    stage_barrier();
    if (it + 1 < n_run) fetch(tile_of(it + 1), s ^ 1);

    const __bf16* qt_t = qs + s * L::QSTAGE;
    const __bf16* gt_t = qt_t + L::ELEMS;
    const int32_t* sg = reinterpret_cast<const int32_t*>(qt_t + 2 * L::ELEMS);
    const float* lse_t = reinterpret_cast<const float*>(qt_t + 2 * L::ELEMS + 128);
    const float* dlt_t = reinterpret_cast<const float*>(qt_t + 2 * L::ELEMS + 256);
    const int q0 = q_lo + 64 * qt;
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      // The next stage's lse, between the two halves: its DMA has had half
      // a tile step, and the other wave of the SIMD runs meanwhile.
      if (qh == 1 && it + 1 < n_run) prep_lse(s ^ 1);
      const int qb = q0 + 32 * qh;  // local row of the block's first query
      // Does the block hold a visible pair, and is every pair visible?
      const int qlast = std::min(qb + 31, p.seq_q - 1);
      const bool rows_in = qb < p.seq_q;
      bool run = active && rows_in && (c == 0 || qpos0 + qlast >= thr_first);
      // With segment ids: does every pair of the block carry one id?
      bool uni = !SEG;
      if (SEG && run) {
        // Query blocks whose ids miss the keys' id range hold no visible pair.
        const SegRange qr = half_range(sg[32 * qh + lrow]);
        run = __builtin_amdgcn_readfirstlane((int)(qr.hi >= kseg.lo && qr.lo <= kseg.hi)) != 0;
        uni = __builtin_amdgcn_readfirstlane(
                  (int)(qr.lo == qr.hi && kseg.lo == kseg.hi && qr.lo == kseg.lo)) != 0;
      }
      const bool full = uni && qb + 31 < p.seq_q && (c == 0 || qpos0 + qb >= thr_last);
      if (!run) continue;

      f32x16_t sc = f32x16_t{}, dp;
      // dp = delta of the lane's 16 query rows (rows 8 (e / 4) + 4 half + e % 4).
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 d4 = *reinterpret_cast<const float4*>(dlt_t + 32 * qh + 8 * g + 4 * half);
        dp[4 * g] = d4.x;
        dp[4 * g + 1] = d4.y;
        dp[4 * g + 2] = d4.z;
        dp[4 * g + 3] = d4.w;
      }
      auto vread = [&](int cc) {
        return *reinterpret_cast<const bf16x8_t*>(vres + (wave >> 1) * L::ELEMS +
                                                  row_rd_c(r_rd, cc) + row_off(cc, wave & 1));
      };
      if constexpr (kPrefetch) {
        // Operands one step ahead: the reads of step cc + 1 are issued
        // before the MFMAs of step cc (fenced), so an MFMA does not wait on
        // the read issued just before it.
        bf16x8_t oq[2], og[2], ov[2];
        oq[0] = row_operand(qt_t, r_rd, 0, qh);
        og[0] = row_operand(gt_t, r_rd, 0, qh);
        ov[0] = vread(0);
#pragma unroll
        for (int cc = 0; cc < D / 16; ++cc) {
          if (cc + 1 < D / 16) {
            oq[(cc + 1) & 1] = row_operand(qt_t, r_rd, cc + 1, qh);
            og[(cc + 1) & 1] = row_operand(gt_t, r_rd, cc + 1, qh);
            ov[(cc + 1) & 1] = vread(cc + 1);
          }
          __builtin_amdgcn_sched_barrier(0);
          sc = mfma(oq[cc & 1], kf[cc], sc);
          dp = mfma(og[cc & 1], ov[cc & 1], dp);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < D / 16; ++cc) {
          const bf16x8_t vop = vread(cc);
          sc = mfma(row_operand(qt_t, r_rd, cc, qh), kf[cc], sc);
          dp = mfma(row_operand(gt_t, r_rd, cc, qh), vop, dp);
        }
      }
      // The 16 query rows of this lane: 8 (e / 4) + 4 half + e % 4; p and
      // ds overwrite the scores and dp in place.
      const int32_t lo = thr == INT32_MIN ? INT32_MIN : thr - (qpos0 + qb);
      const int32_t hi = p.seq_q - qb;
      // Without segment ids, two copies of the softmax: fully visible blocks
      // (nearly all of a long share) skip the per-pair visibility test,
      // which, merged into one path with a select, costs two compares, three
      // mask operations and a select per pair.  The segment-id kernels have
      // no registers for the second copy and keep the merged path.
      auto softmax = [&](auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 l4 = *reinterpret_cast<const float4*>(lse_t + 32 * qh + 8 * g + 4 * half);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * g + i;
            // lv = -lse log2(e), rewritten in the stage by prep_lse.
            float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], p.scale_log2, lv[i]));
            // (Without segment ids the masked copy runs only when !full.)
            if (MASKED && (!SEG || !full)) {
              const int off = 8 * g + 4 * half + i;
              bool ok = off >= lo && off < hi;
              if (SEG && !uni) ok = ok && sg[32 * qh + off] == seg_k;
              pr = ok ? pr : 0.f;
            }
            sc[e] = pr;
            dp[e] = -pr * dp[e];  // p (dout.v_j - delta): dp holds delta - dout.v_j
          }
        }
      };
      if (!SEG && full)
        softmax(std::false_type{});
      else
        softmax(std::true_type{});
      bf16x8_t pb[2], db[2];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        f32x8_t a, d;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          a[i] = sc[8 * cc + i];
          d[i] = dp[8 * cc + i];
        }
        pb[cc] = __builtin_convertvector(a, bf16x8_t);
        db[cc] = __builtin_convertvector(d, bf16x8_t);
      }
      if constexpr (kPrefetch) {
        // Column operands two MFMAs ahead (fenced), as above.
        constexpr int NM = 4 * NDB;  // MFMAs (cc, j, dV or dK)
        auto cread = [&](int n) {
          const int cc = n / (2 * NDB), j = (n / 2) % NDB;
          return col_operand((n & 1) ? qt_t : gt_t, t_rd, j, 2 * qh + cc);
        };
        bf16x8_t oc[3];
        oc[0] = cread(0);
        oc[1] = cread(1);
#pragma unroll
        for (int n = 0; n < NM; ++n) {
          if (n + 2 < NM) oc[(n + 2) % 3] = cread(n + 2);
          __builtin_amdgcn_sched_barrier(0);
          const int cc = n / (2 * NDB), j = (n / 2) % NDB;
          if (n & 1)
            dk[j] = mfma(oc[n % 3], db[cc], dk[j]);
          else
            dv[j] = mfma(oc[n % 3], pb[cc], dv[j]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int j = 0; j < NDB; ++j) {
            dv[j] = mfma(col_operand(gt_t, t_rd, j, 2 * qh + cc), pb[cc], dv[j]);
            dk[j] = mfma(col_operand(qt_t, t_rd, j, 2 * qh + cc), db[cc], dk[j]);
          }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  if (!active) return;
  const float scale = p.scale_log2 / kLog2e;
  const int64_t roff = ((int64_t)b * p.seq_k + key) * rs + (int64_t)h * D;
#pragma unroll
  for (int j = 0; j < NDB; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * j + 8 * g + 4 * half;
      *reinterpret_cast<float4*>(bp.dk + roff + d) =
          make_float4(dk[j][4 * g] * scale, dk[j][4 * g + 1] * scale, dk[j][4 * g + 2] * scale,
                      dk[j][4 * g + 3] * scale);
      *reinterpret_cast<float4*>(bp.dv + roff + d) =
          make_float4(dv[j][4 * g], dv[j][4 * g + 1], dv[j][4 * g + 2], dv[j][4 * g + 3]);
    }
}

// The dQ and dK/dV kernels of one configuration.
// dq = the sum of the splits' addends, four values per thread, in split
// order (deterministic).  Only the runs of the value's query tile hold an
// addend (the dq grid has one workgroup per run); their count comes from the
// same walk lengths as the workgroup mapping.  row4: float4s per query row
// (heads * head_dim / 4).  BM, TN: the dq kernel's query rows per
// workgroup and keys per tile (bf16: 256 and 64; float32: 128 and 32).
template <int BM, int TN, bool STRIPED>
__global__ __launch_bounds__(256) void bwd_dq_sum_kernel(const BwdParams bp, int64_t n4,
                                                         int32_t row4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const FwdParams& p = bp.f;
  int nsplit = p.key_splits;
  const walk::Share sh = share_of<BM, TN, STRIPED>(p);
  // Guard: the dq grid the host launched must hold exactly the runs counted
  // here (the same functions); otherwise dq[0] is poisoned rather than
  // summing slots that no workgroup wrote.
  if (i == 0 && p.split_wgs > 0 && walk::split_wgs(sh, p.key_splits) != p.split_wgs) {
    reinterpret_cast<uint32_t*>(bp.dq)[0] = 0x7fc00000u;  // NaN
    return;
  }
  // Walks only grow with the query tile: when tile 0 (uniform arithmetic)
  // takes all key_splits runs, every tile does.
  if (p.split_wgs > 0 && walk::qtile_runs(sh, p.key_splits, 0) < p.key_splits) {
    const int q = n4 <= INT32_MAX ? (int)((uint32_t)i / (uint32_t)row4 % (uint32_t)p.seq_q)
                                  : (int)(i / row4 % p.seq_q);
    nsplit = walk::qtile_runs(sh, p.key_splits, q / BM);
  }
  const float4* part = reinterpret_cast<const float4*>(bp.dq_part);
  float4 acc = part[i];
  for (int s = 1; s < nsplit; ++s) {
    const float4 v = part[(int64_t)s * n4 + i];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  reinterpret_cast<float4*>(bp.dq)[i] = acc;
}

template <int D, bool SEG, bool STRIPED>
void launch_main(dim3 qgrid, dim3 kgrid, dim3 block, hipStream_t s, const BwdParams& bp) {
  hipLaunchKernelGGL((bwd_dq_kernel<D, SEG, STRIPED>), qgrid, block, 0, s, bp);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, SEG, STRIPED>), kgrid, block, 0, s, bp);
}

}  // namespace

int launch_bwd(const BwdParams& bp, Dtype dtype, int head_dim, void* stream, char* err,
               int errlen) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipGetLastError();  // clear a stale error from earlier work
  (void)e;
  const FwdParams& p = bp.f;
  const bool seg = p.seg != nullptr;
  const bool f32 = dtype == Dtype::F32;
  const int64_t rows = (int64_t)p.batch * p.seq_q * p.heads;
  const int64_t lanes = rows * (head_dim / 8);
  const dim3 dgrid((unsigned)((lanes + 255) / 256));
  if (head_dim == 128 && f32)
    hipLaunchKernelGGL((bwd_delta_kernel<128, float>), dgrid, dim3(256), 0, s, bp);
  else if (head_dim == 128)
    hipLaunchKernelGGL((bwd_delta_kernel<128, __bf16>), dgrid, dim3(256), 0, s, bp);
  else if (f32)
    hipLaunchKernelGGL((bwd_delta_kernel<64, float>), dgrid, dim3(256), 0, s, bp);
  else
    hipLaunchKernelGGL((bwd_delta_kernel<64, __bf16>), dgrid, dim3(256), 0, s, bp);
  const dim3 block(kThreadsBwd);
  const dim3 qgrid((unsigned)p.n_wg), kgrid((unsigned)bp.n_wg_kv);
  const bool str = p.striped != 0;
  if (f32) {
    launch_bwd_f32_main(bp, head_dim, stream);
  } else if (head_dim == 128) {
    if (seg)
      str ? launch_main<128, true, true>(qgrid, kgrid, block, s, bp)
          : launch_main<128, true, false>(qgrid, kgrid, block, s, bp);
    else
      str ? launch_main<128, false, true>(qgrid, kgrid, block, s, bp)
          : launch_main<128, false, false>(qgrid, kgrid, block, s, bp);
  } else {
    if (seg)
      str ? launch_main<64, true, true>(qgrid, kgrid, block, s, bp)
          : launch_main<64, true, false>(qgrid, kgrid, block, s, bp);
    else
      str ? launch_main<64, false, true>(qgrid, kgrid, block, s, bp)
          : launch_main<64, false, false>(qgrid, kgrid, block, s, bp);
  }
  if (bp.dq_part != nullptr) {
    const int64_t n4 = rows * head_dim / 4;
    const int32_t row4 = bp.f.heads * head_dim / 4;
    const dim3 sgrid((unsigned)((n4 + 255) / 256));
    if (f32 && str)
      hipLaunchKernelGGL((bwd_dq_sum_kernel<kBlockMF32, 32, true>), sgrid, dim3(256), 0, s, bp,
                         n4, row4);
    else if (f32)
      hipLaunchKernelGGL((bwd_dq_sum_kernel<kBlockMF32, 32, false>), sgrid, dim3(256), 0, s, bp,
                         n4, row4);
    else if (str)
      hipLaunchKernelGGL((bwd_dq_sum_kernel<kBlockMBf16, 64, true>), sgrid, dim3(256), 0, s, bp,
                         n4, row4);
    else
      hipLaunchKernelGGL((bwd_dq_sum_kernel<kBlockMBf16, 64, false>), sgrid, dim3(256), 0, s, bp,
                         n4, row4);
  }
  e = hipGetLastError();
  if (e != hipSuccess) {
    std::snprintf(err, errlen, "backward launch failed: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

}  // namespace ra
