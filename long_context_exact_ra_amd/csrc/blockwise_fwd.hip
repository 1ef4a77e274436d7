// Blockwise exact-attention forward for one Ring Attention device share,
// written for gfx950 (MI355X, CDNA4).
//
// A workgroup owns a tile of query rows of one (batch, head) (256 rows = 8
// waves for bf16, 128 rows = 4 waves for fp32); each wave owns 32 of them.  The workgroup walks the N key/value blocks
// (the ring of "Ring Attention with Blockwise Transformers for
// Near-Infinite Context", section 三 "环形注意力算法", visits block (r - t)
// mod N at step t; on one device all blocks are resident and the fold order
// is free, so the walk takes the ring order with the local block moved to
// the end, which keeps the workgroups of a head in step) and inside a block
// the keys in tiles.  Tiles are staged through LDS and
// fetched ahead of use, also across block boundaries, which is the
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
// With key splits (shares whose query tiles alone leave compute units
// idle), a query tile has several workgroups, each walking one run of the
// tile's key walk and writing its partial max, numerator and denominator;
// combine_splits_kernel folds them into out and lse with the same carry.
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
#include <mutex>

#include "ra_device.h"
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int kThreads = 256;
// Largest log2 of a probability weight before the running max must move.
constexpr float kLazyMax = 8.f;

// ---------------------------------------------------------------------------
// Key splits: partial results and their combination
// ---------------------------------------------------------------------------
//
// A split's workgroup ends with the unnormalised numerator of each of its
// rows (float32), the max it kept (base 2) and its denominator.  Folding the
// splits is the same carry as folding blocks ("2. 数值稳定的注意力计算"): with
// M the largest kept max, out = sum_s 2^(m_s - M) num_s / sum_s 2^(m_s - M)
// den_s and lse = (M + log2 of that denominator) ln 2.

__device__ __forceinline__ int64_t part_row(const FwdParams& p, int split, int b, int h, int row) {
  return (((int64_t)split * p.batch + b) * p.heads + h) * p.seq_q + row;
}

// This lane's half of row `row`: acc[j][4g + e] is column 32j + 8g + 4half + e.
template <int NDB>
__device__ __forceinline__ void write_partial(const FwdParams& p, int split, int b, int h, int row,
                                              int half, const f32x16_t* acc, float m_run,
                                              float l_tot) {
  constexpr int D = NDB * 32;
  const int64_t pr = part_row(p, split, b, h, row);
  float* po = p.part_o + pr * D;
#pragma unroll
  for (int j = 0; j < NDB; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(po + 32 * j + 8 * g + 4 * half) =
          make_float4(acc[j][4 * g], acc[j][4 * g + 1], acc[j][4 * g + 2], acc[j][4 * g + 3]);
  if (half == 0) *reinterpret_cast<float2*>(p.part_ml + 2 * pr) = make_float2(m_run, l_tot);
}

// The partial of a split that has no run (an idle workgroup): denominator 0,
// so the combine skips the slot and never reads its numerator.
__device__ __forceinline__ void write_empty_partial(const FwdParams& p, int split, int b, int h,
                                                    int row) {
  *reinterpret_cast<float2*>(p.part_ml + 2 * part_row(p, split, b, h, row)) =
      make_float2(ninf(), 0.f);
}

// One thread per (row, 4 columns); rows in [b][h][i] order, as lse.  The
// splits are folded eight at a time with a running max, so that the loads
// of eight splits are in flight together; a split without a visible key
// (denominator 0) gets weight 0, and its numerator (unwritten if the split
// was idle) is not used.  Under the exact grid a query tile's slots past
// its run count are empty by construction, so only its runs are read (the
// count comes from the same walk lengths as the workgroup mapping;
// BM and TN are the forward kernel's rows per workgroup and keys per tile).
template <typename T, int BM, int TN, bool STRIPED>
__global__ void combine_splits_kernel(const FwdParams p, int head_dim) {
  const int groups = head_dim / 4;
  const int64_t rows = (int64_t)p.batch * p.heads * p.seq_q;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= rows * groups) return;
  const int64_t r = tid / groups;
  const int g = (int)(tid % groups);
  const int64_t i = r % p.seq_q, bh = r / p.seq_q;
  int nsplit = p.key_splits;
  if (p.split_wgs > 0) {
    const walk::Share sh = share_of<BM, TN, STRIPED>(p);
    nsplit = walk::qtile_runs(sh, p.key_splits, (int)i / BM);
    // Guard: the grid the host launched must hold exactly the runs counted
    // here (the same functions, so this holds unless the parameters are
    // inconsistent); otherwise row 0's lse is poisoned rather than folding
    // slots that no workgroup wrote.
    if (tid == 0 && walk::split_wgs(sh, p.key_splits) != p.split_wgs) {
      // (the NaN bit pattern, stored as an integer: this source is built
      // without NaN semantics)
      reinterpret_cast<uint32_t*>(p.lse)[0] = 0x7fc00000u;
      return;
    }
  }
  float mmax = ninf(), den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float2 ml[8];
    float4 o[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t pr = (int64_t)(s0 + u) * rows + r;
      if (s0 + u < nsplit) {
        ml[u] = *reinterpret_cast<const float2*>(p.part_ml + 2 * pr);
        o[u] = *reinterpret_cast<const float4*>(p.part_o + pr * head_dim + 4 * g);
      } else {
        ml[u] = make_float2(ninf(), 0.f);
        o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float cm = mmax;
#pragma unroll
    for (int u = 0; u < 8; ++u) cm = ml[u].y > 0.f ? fmaxf(cm, ml[u].x) : cm;
    // Nothing folded yet (mmax = -inf) means den and num are still 0.
    const float sc = mmax == ninf() ? 0.f : __builtin_amdgcn_exp2f(mmax - cm);
    den *= sc;
    num.x *= sc;
    num.y *= sc;
    num.z *= sc;
    num.w *= sc;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (!(ml[u].y > 0.f)) continue;
      const float w = __builtin_amdgcn_exp2f(ml[u].x - cm);
      den += w * ml[u].y;
      num.x += w * o[u].x;
      num.y += w * o[u].y;
      num.z += w * o[u].z;
      num.w += w * o[u].w;
    }
    mmax = cm;
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int64_t b = bh / p.heads, h = bh % p.heads;
  T* o = static_cast<T*>(p.out) + ((b * p.seq_q + i) * p.heads + h) * head_dim + 4 * g;
  o[0] = (T)(num.x * inv);
  o[1] = (T)(num.y * inv);
  o[2] = (T)(num.z * inv);
  o[3] = (T)(num.w * inv);
  if (g == 0) p.lse[r] = den > 0.f ? (mmax + __builtin_amdgcn_logf(den)) * kLn2 : ninf();
}

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------
//
// 8 waves, 256 query rows per workgroup, one workgroup per CU.  64-key tiles
// flow through a ring of 4 LDS stages filled by bounds-checked
// buffer-to-LDS DMA (buffer_load_dwordx4 ... lds) issued 3 tiles ahead, so
// the fetch of a tile overlaps two tiles of compute and needs no staging
// registers.  Keys past a block's visible length read as zero.  The loop is
// unrolled over the ring so that every stage is a distinct LDS object; the
// per-wave waits on the DMA are explicit vmcnt counts.
//
// A DMA instruction writes 64 lanes x 16 bytes contiguously, so the LDS
// layouts are chosen for the reads (all in 16-byte slots, g = the 16-byte
// granule of a row, r = the row = key):
//   K: slot(r, g) = (g / 4) * 256 + (r / 16) * 64 + (g % 4) * 16 + r % 16.
//      The QK^T A operand of 16 consecutive lanes (16 rows, one granule) is
//      then 256 contiguous bytes, and its address is a per-lane base plus a
//      compile-time offset.
//   V: slot(r, g) = (g / 4) * 256 + r * 4 + g % 4.  A ds_read_b64_tr_b16 of
//      32 lanes (4 rows x 64 contiguous bytes) is then 256 contiguous bytes.
// Within each 16-lane group ds_read_b64_tr_b16 hands destination lane i,
// element e the element i % 4 of source lane 4e + i / 4; a lane of group g
// sources row base + (lane % 16) / 4 at column 16 * (g % 2) + 4 * (lane % 4)
// and so receives, for its own column lane % 32, rows base .. base + 3: four
// k-slots of the P.V A operand V^T.
//
// Software pipeline per tile i (tile i+1's keys already in LDS):
//   S_next = K_{i+1} . Q^T   (MFMA)      -- independent of --
//   softmax carry on S_cur = tile i (VALU),
//   O^T += V_i^T . P_i^T     (MFMA),
// with the two products interleaved MFMA by MFMA (step_ilv).  On gfx950 a
// SIMD does not run VALU work of one wave under the MFMAs of another, and
// LDS operand reads cost issue time too, so the step is laid out to spread
// the K reads, the (half-rate) transposing V reads and the exponentials
// evenly between the MFMAs rather than to hide one phase behind another.

// Softmax/accumulator state of one wave (32 query rows, one per lane pair).
template <int D>
struct Bf16Wave {
  static constexpr int NDB = D / 32;
  f32x16_t acc[NDB];
  float m_run;     // running max of the scaled logits (base-2 domain)
  // This lane half's part of the denominator, as four running sums (one per
  // group of 8 probabilities of a tile), so that no per-tile sum has to be
  // started from zero and folded in.
  float l_run[4];
};

template <int D>
struct PipeCfg {
  static constexpr int kWaves = kBlockMBf16 / 32;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int TN = 64;                 // keys per tile
  static constexpr int GR = D / 8;              // 16-byte granules per row
  static constexpr int SLOTS = TN * GR;         // 16-byte slots per tensor tile
  static constexpr int ELEMS = SLOTS * 8;       // bf16 elements per tensor tile
  static constexpr int DPW = SLOTS / 64 / kWaves;  // 1 KiB DMA per wave per tensor
  static_assert(DPW * 64 * kWaves == SLOTS, "tile must split evenly over the waves");
};

// S^T = K . Q^T for the two 32-key halves of a tile.
template <int D>
__device__ __forceinline__ void qk_tile(f32x16_t* s, const bf16x8_t* qf, const __bf16* kst,
                                        int k_rd) {
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    s[sb] = f32x16_t{};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
          kst + k_rd + 2048 * (c >> 1) + 256 * (c & 1) + 1024 * sb);
      s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[sb], 0, 0, 0);
    }
  }
}

// Mask the logits of a tile in place and return this lane's max over them.
// A half may be skipped (run false: all -inf) or need the causal / segment
// mask.  Element i of a half sits at key offset 8 * (i / 4) + i % 4 from the
// lane's first key, so the causal test of a whole half reduces to one
// per-lane count of visible keys.
template <bool SEG>
__device__ __forceinline__ float mask_max(f32x16_t* s, const int32_t* sg, int half,
                                          const TileFlags& f, int32_t lane_lim, int32_t seg_q) {
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const bool r = sb ? f.run1 : f.run0, m = sb ? f.mask1 : f.mask0;
    // Keys at offsets below nvis are causally visible from this lane's row.
    const int32_t nvis = !r ? 0 : m ? lane_lim - (f.pk + 32 * sb + 4 * half) : 32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int koff = 8 * (i >> 2) + (i & 3);
      bool ok = koff < nvis;
      if (SEG && (sb ? f.seg1 : f.seg0)) ok = ok && sg[32 * sb + 4 * half + koff] == seg_q;
      s[sb][i] = ok ? s[sb][i] : ninf();
    }
  }
  // Independent partial maxima keep the dependency chains short.
  float mp[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) mp[k] = fmaxf(s[k >> 1][8 * (k & 1)], s[k >> 1][8 * (k & 1) + 1]);
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int i = 2; i < 8; ++i) mp[k] = fmaxf(mp[k], s[k >> 1][8 * (k & 1) + i]);
  return fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
}

// Fold a tile's row max into the carry ("2. 数值稳定的注意力计算"): rescale a
// row's numerator and denominator by exp(prev_max - new_max) and move its
// max.  The max is moved only when some row of the wave would see a weight
// above 2^kLazyMax otherwise; until then the rows keep their previous max and
// their weights exp(s - max) stay below 2^kLazyMax, exact in fp32 and bf16.
// The result is the same softmax (numerator and denominator share the max,
// and lse uses the max actually kept); rescaling becomes rare after the first
// tiles.
template <int D>
__device__ __forceinline__ void carry_max(Bf16Wave<D>& w, float mx, float scale_log2) {
  constexpr int NDB = D / 32;
  mx = pair_max(mx);
  const float m_new = fmaxf(w.m_run, mx * scale_log2);
  if (__builtin_amdgcn_ballot_w64(m_new > w.m_run + kLazyMax) != 0) {
    const float alpha = m_new == ninf() ? 1.f : __builtin_amdgcn_exp2f(w.m_run - m_new);
#pragma unroll
    for (int j = 0; j < NDB; ++j) w.acc[j] *= alpha;
#pragma unroll
    for (int g = 0; g < 4; ++g) w.l_run[g] *= alpha;
    w.m_run = m_new;
  }
}


// One step with the QK^T MFMAs of tile i+1 and the P.V MFMAs of tile i
// interleaved one to one, so that the K reads (plain) and the V reads
// (transposing, half rate) are spread over the whole step, and the
// exponentials of tile i feed the P.V MFMAs group by group.  QK MFMA 0 is
// issued first, with the first group's exponentials behind it; then slot t
// issues QK MFMA t+1, the LDS reads of the K operand three and the V
// operand two MFMAs ahead, P.V MFMA t and its share of the exponentials, so
// that each MFMA is followed by independent work that the wave issues while
// the matrix core runs it.  The row max of each half of tile i+1 is taken
// as soon as its QK MFMAs are in flight.  `mid` runs at slot 2: the caller
// issues the next tile's DMA there, so that its scalar work (cursor,
// descriptors) runs beside the matrix cores instead of delaying the first
// MFMAs of both waves of a SIMD after the barrier (2.9-3.8 % faster on the
// 7B-shaped share than issuing it at the start of the step; slots 0, 1, 3
// and 5 were measured slower).  The running sums and maxima are pinned with
// empty asm so that the compiler does not sink them behind the last MFMA.
// Returns this lane's max over tile i+1 (unmasked).
template <int D, typename Mid>
__device__ __forceinline__ float step_ilv(Bf16Wave<D>& w, f32x16_t* s_cur, f32x16_t* s_next,
                                          const bf16x8_t* qf, const __bf16* kst,
                                          const __bf16* vst, int k_rd, int v_rd,
                                          float scale_log2, Mid&& mid) {
  constexpr int NDB = D / 32, NC = D / 16, N = D / 8;  // N QK and N P.V MFMAs
  const float m_use = w.m_run == ninf() ? 0.f : w.m_run;
  const bf16x2_t one2 = {(__bf16)1.f, (__bf16)1.f};
  auto kread = [&](int t) -> bf16x8_t {
    const int sb = t / NC, c = t % NC;
    return *reinterpret_cast<const bf16x8_t*>(kst + k_rd + 2048 * (c >> 1) + 256 * (c & 1) +
                                              1024 * sb);
  };
  auto vread = [&](int t) -> bf16x8_t {
    const int q = t / NDB, j = t % NDB, sb = q >> 1, cc = q & 1;
    const __bf16* src = vst + v_rd + 2048 * j + 32 * (32 * sb + 16 * cc);
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)src);
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(src + 256));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  bf16x8_t pb[4];
  f32x8_t e;
  auto exp_part = [&](int q, int i0, int n) {
#pragma unroll
    for (int i = i0; i < i0 + n; ++i)
      e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[q >> 1][8 * (q & 1) + i], scale_log2, -m_use));
  };
  auto finish_pb = [&](int q) {
    pb[q] = __builtin_convertvector(e, bf16x8_t);
    float ps = __builtin_amdgcn_fdot2_f32_bf16(pb[q].s01, one2, w.l_run[q], false);
    ps = __builtin_amdgcn_fdot2_f32_bf16(pb[q].s23, one2, ps, false);
    ps = __builtin_amdgcn_fdot2_f32_bf16(pb[q].s45, one2, ps, false);
    w.l_run[q] = __builtin_amdgcn_fdot2_f32_bf16(pb[q].s67, one2, ps, false);
    // keep the sum in its slot: unpinned, it is sunk past the mask branch,
    // behind the last MFMA
    asm volatile("" : "+v"(w.l_run[q]));
  };
  auto make_pb = [&](int q) {
    exp_part(q, 0, 8);
    finish_pb(q);
  };
  bf16x8_t ka[3], va[3];
  ka[0] = kread(0);
  ka[1] = kread(1);
  va[0] = vread(0);
  va[1] = vread(1);
  s_next[0] = f32x16_t{};
  s_next[1] = f32x16_t{};
  // QK MFMA 0 first: the first group's exponentials run behind it.
  s_next[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[0], s_next[0], 0, 0, 0);
  ka[2] = kread(2);
  make_pb(0);
  float mp0 = ninf(), mp1 = ninf();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < N; ++t) {
    // QK MFMA t+1 leads P.V MFMA t by one slot
    if (t + 1 < N) {
      const int u = t + 1, sb = u / NC, c = u % NC;
      s_next[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[u % 3], qf[c], s_next[sb], 0, 0, 0);
    }
    if (t + 3 < N) ka[(t + 3) % 3] = kread(t + 3);
    if (t + 2 < N) va[(t + 2) % 3] = vread(t + 2);
    __builtin_amdgcn_sched_barrier(0);
    {
      const int q = t / NDB, j = t % NDB;
      w.acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t % 3], pb[q], w.acc[j], 0, 0, 0);
    }
    // the probabilities of the next group, a share per slot, ready before
    // its first P.V MFMA
    if (t / NDB + 1 < 4) {
      constexpr int PER = 8 / NDB;
      exp_part(t / NDB + 1, (t % NDB) * PER, PER);
      if (t % NDB == NDB - 1) finish_pb(t / NDB + 1);
    }
    if (t == 2) {
      __builtin_amdgcn_sched_barrier(0);
      mid();
      __builtin_amdgcn_sched_barrier(0);
    }
    // the max over the first half of tile i+1, complete after QK MFMA NC-1
    if (t == N - 3) {
      float a = fmaxf(s_next[0][0], s_next[0][1]), b = fmaxf(s_next[0][8], s_next[0][9]);
#pragma unroll
      for (int i = 2; i < 8; ++i) {
        a = fmaxf(a, s_next[0][i]);
        b = fmaxf(b, s_next[0][8 + i]);
      }
      mp0 = fmaxf(a, b);
      asm volatile("" : "+v"(mp0));
    }
    // and over the second half, behind the last P.V MFMA
    if (t == N - 1) {
      float a = fmaxf(s_next[1][0], s_next[1][1]), b = fmaxf(s_next[1][8], s_next[1][9]);
#pragma unroll
      for (int i = 2; i < 8; ++i) {
        a = fmaxf(a, s_next[1][i]);
        b = fmaxf(b, s_next[1][8 + i]);
      }
      mp1 = fmaxf(a, b);
      asm volatile("" : "+v"(mp1));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  return fmaxf(mp0, mp1);
}

// Everything one wave carries through the ring walk.
template <int D>
struct PipeState {
  Bf16Wave<D> w;
  // Logits of tiles i and i+1 in two buffers whose roles alternate from
  // step to step (even steps: tile i in buffer 0), so no step copies them.
  f32x16_t s[2][2];
  // The tile held by each LDS stage; stage indices are compile-time
  // constants in the unrolled loop, so these stay in fixed registers.
  TileInfo ti[4];
  Cursor ic;  // the next tile to fetch
  // With segment ids: per stage, which 32-key halves of its tile share an id
  // range with the wave's queries (bit 0, bit 1).
  uint32_t segok[4];
};

struct PipeConst {
  const char* kbase0;
  const char* vbase0;
  const int32_t* sbase0;
  uint32_t rs_bytes;
  int wave, lane, lrow, half, qg0;
  bool wave_active;
  uint32_t k_lane, v_lane;
  int k_rd, v_rd;
  int64_t kend;
  int pos_end;  // walk position where this workgroup's key split ends
  int32_t seg_q;
  SegRange qseg;  // id range of the wave's queries
  // With segment ids: the workgroup's tile mask in LDS, or nullptr (walk
  // every causally visible tile).
  const uint8_t* smask;
};

// Record the tile under the fetch cursor (past the tiles the segment mask
// leaves out) as the content of stage S, start its DMA and advance the
// cursor.
template <int D, bool SEG, bool STRIPED, int S>
__device__ __forceinline__ void fetch_next(const FwdParams& p, const PipeConst& k,
                                           PipeState<D>& st, __bf16* const* ks,
                                           __bf16* const* vs, int32_t* const* ss) {
  if (SEG && k.smask != nullptr)
    cursor_skip_masked<PipeCfg<D>::TN, STRIPED>(p, st.ic, k.kend, k.smask);
  if (st.ic.pos >= k.pos_end) st.ic.valid = 0;
  st.ti[S] = tile_info<PipeCfg<D>::TN, STRIPED>(p, st.ic);
  if (st.ic.valid) {
    issue_tile<D, PipeCfg<D>::kWaves, SEG>(st.ti[S], k.kbase0, k.vbase0, k.sbase0, k.rs_bytes,
                                           k.wave, k.lane, k.k_lane, k.v_lane, ks[S], vs[S],
                                           ss[S]);
    cursor_next<PipeCfg<D>::TN, STRIPED>(p, st.ic, k.kend);
  }
}

// One pipeline step: tile i lives in stage PH, tile i+1 in stage PH+1, the
// DMA for tile i+3 goes into stage PH+3 (all mod 4).  Returns whether a next
// tile exists.
template <int D, bool SEG, bool STRIPED, int PH>
__device__ __forceinline__ bool pipe_step(const FwdParams& p, const PipeConst& k,
                                          const WaveLimits& lim, const bf16x8_t* qf,
                                          PipeState<D>& st, __bf16* const* ks,
                                          __bf16* const* vs, int32_t* const* ss) {
  constexpr int NPT = 2 * PipeCfg<D>::DPW + (SEG ? 1 : 0);  // DMA per wave per tile
  constexpr int S0 = PH, S1 = (PH + 1) & 3, S2 = (PH + 2) & 3, S3 = (PH + 3) & 3;
  // The DMA of tile i+3 into stage S3 (read last in step i-1, before the
  // barrier that ended it) is issued inside the MFMA block, where its
  // scalar work runs beside the matrix cores.
  auto fetch = [&]() { fetch_next<D, SEG, STRIPED, S3>(p, k, st, ks, vs, ss); };

  TileFlags f0 = tile_flags<SEG, STRIPED>(st.ti[S0], lim);
  TileFlags f1 = tile_flags<SEG, STRIPED>(st.ti[S1], lim);

  // Tile i (logits in s_cur, already masked and max-folded): probabilities and
  // P.V.  Tile i+1: logits and row max.  Both 32-key halves of both tiles
  // are always computed, so this is one straight-line block for every step;
  // a half without a visible pair is masked to -inf and contributes exactly 0
  // (its keys in LDS are real keys or zeros, never undefined).  The debug
  // run map (the causal decisions) is written first, so that no branch splits
  // the block.
  f32x16_t* const s_cur = st.s[PH & 1];
  f32x16_t* const s_next = st.s[(PH + 1) & 1];
  if (p.run_map != nullptr && k.lane == 0) {
    const TileInfo& t0 = st.ti[S0];
    const int kloc0 = t0.pk - t0.kb * p.seq_q;
    if (f0.run0) write_run_map(p, t0.kb, k.qg0, kloc0);
    if (f0.run1) write_run_map(p, t0.kb, k.qg0, kloc0 + 32);
  }
  if (SEG) {
    // Halves whose key ids miss the queries' id range hold no visible pair.
    f0.run0 = f0.run0 && (st.segok[S0] & 1u);
    f0.run1 = f0.run1 && (st.segok[S0] & 2u);
    const uint32_t ok1 = seg_overlap_halves(ss[S1], k.lane, k.qseg);
    st.segok[S1] = ok1;
    f1.run0 = f1.run0 && (ok1 & 1u);
    f1.run1 = f1.run1 && (ok1 & 2u);
    // Halves whose keys and queries all carry one id need no id test.
    f1.seg0 = !(ok1 & 4u);
    f1.seg1 = !(ok1 & 8u);
    f1.mask0 = f1.mask0 || f1.seg0;
    f1.mask1 = f1.mask1 || f1.seg1;
  }
  float mx = ninf();
  const bool any0 = f0.run0 || f0.run1, any1 = f1.run0 || f1.run1;
  if (any0 || any1) {
    mx = step_ilv<D>(st.w, s_cur, s_next, qf, ks[S1], vs[S0], k.k_rd, k.v_rd, p.scale_log2,
                     fetch);
    if (!(f1.run0 && f1.run1) || f1.mask0 || f1.mask1) {
      // Keep this a real branch: if-converted, the mask would run on every
      // step.  An empty volatile asm cannot be speculated.  The masked max
      // never exceeds the unmasked one; taking the smaller of the two keeps
      // the unmasked max used on both paths, so it stays in the block above,
      // between the P.V MFMAs.
      asm volatile("");
      mx = fminf(mx, mask_max<SEG>(s_next, ss[S1], k.half, f1, lim.lane_lim, k.seg_q));
    }
  } else {
    fetch();
    s_next[0] = f32x16_t{} - __builtin_inff();
    s_next[1] = s_next[0];
  }
  if (k.wave_active) carry_max<D>(st.w, mx, p.scale_log2);

  // Tile i+2 must have landed (for every wave) before the next step reads it.
  if (st.ti[S2].valid) {
    if (st.ti[S3].valid)
      wait_vm<NPT>();
    else
      wait_vm<0>();
  }
  stage_barrier();
  return st.ti[S1].valid;
}

template <int D, bool SEG, bool STRIPED>
__global__ __launch_bounds__(PipeCfg<D>::kThreads, 1) void fwd_bf16_kernel(const FwdParams p) {
  using C = PipeCfg<D>;
  constexpr int NDB = D / 32;

  // One LDS object per stage (K tile, V tile, then the segment ids), so that
  // the compiler can tell the DMA into one stage from the reads of another.
  constexpr int STAGE = 2 * C::ELEMS + (SEG ? 128 : 0);
  __shared__ __attribute__((aligned(16))) __bf16 st0[STAGE], st1[STAGE], st2[STAGE], st3[STAGE];
  __bf16* const ks[4] = {st0, st1, st2, st3};
  __bf16* const vs[4] = {st0 + C::ELEMS, st1 + C::ELEMS, st2 + C::ELEMS, st3 + C::ELEMS};
  int32_t* const ss[4] = {reinterpret_cast<int32_t*>(st0 + 2 * C::ELEMS),
                          reinterpret_cast<int32_t*>(st1 + 2 * C::ELEMS),
                          reinterpret_cast<int32_t*>(st2 + 2 * C::ELEMS),
                          reinterpret_cast<int32_t*>(st3 + 2 * C::ELEMS)};

  PipeConst k;
  k.lane = threadIdx.x & 63;
  k.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  k.lrow = k.lane & 31;
  k.half = k.lane >> 5;

  const WgCoord wc = p.split_wgs > 0 ? wg_coord_runs<kBlockMBf16, C::TN, STRIPED>(p)
                                     : wg_coord<kBlockMBf16>(p);
  if (wc.split < 0) return;
  const int b = wc.b, h = wc.h, m0 = wc.m0;
  k.qg0 = m0 + k.wave * 32;
  k.wave_active = k.qg0 < p.seq_q;
  // Storage row of the wave's first query (segment ids) and its query
  // coordinate (causal limits; the local row under striped placement).
  const int64_t pq_first = (int64_t)p.ring_index * p.seq_q + k.qg0;
  const WaveLimits lim = wave_limits(p, STRIPED ? k.qg0 : pq_first, k.lrow, k.wave_active);
  k.kend = wg_kend<kBlockMBf16, STRIPED>(p, m0);
  const SplitRange sr = split_range<C::TN, STRIPED>(
      p, wc.split, k.kend, wg_kend<kBlockMBf16, STRIPED>(p, (p.n_qtiles - 1) * kBlockMBf16));
  if (sr.idle) {
    // A surplus split of a short walk: its partial holds no key.
    if (k.wave_active && k.half == 0) write_empty_partial(p, wc.split, b, h, k.qg0 + k.lrow);
    return;
  }
  k.pos_end = sr.end;
  k.seg_q = 0;
  if (SEG && k.wave_active) k.seg_q = p.seg[(int64_t)b * p.seq_k + pq_first + k.lrow];
  k.qseg = SegRange{0, 0};
  if (SEG) k.qseg = wave_range(k.seg_q);
  // Segment ids: mark the tiles whose ids can meet the workgroup's (not
  // with the debug run map, which records every causal decision).
  __shared__ uint8_t smask[SEG ? kSegMaskSlots : 1];
  __shared__ int32_t wg_ids[2 * C::kWaves];
  k.smask = nullptr;
  if (SEG && p.run_map == nullptr && p.ring_size * seg_mask_tpb(p) <= kSegMaskSlots) {
    if (k.lane == 0) {
      wg_ids[2 * k.wave] = k.wave_active ? k.qseg.lo : INT32_MAX;
      wg_ids[2 * k.wave + 1] = k.wave_active ? k.qseg.hi : INT32_MIN;
    }
    __syncthreads();
    SegRange wr{INT32_MAX, INT32_MIN};
#pragma unroll
    for (int w = 0; w < C::kWaves; ++w) {
      wr.lo = min(wr.lo, wg_ids[2 * w]);
      wr.hi = max(wr.hi, wg_ids[2 * w + 1]);
    }
    build_seg_mask(p, p.seg + (int64_t)b * p.seq_k, wr, STRIPED ? INT64_MAX : k.kend, smask,
                   (int)threadIdx.x, C::kThreads);
    __syncthreads();
    k.smask = smask;
  }

  const int64_t rs = (int64_t)p.heads * D;
  k.rs_bytes = (uint32_t)(rs * 2);
  k.kbase0 = static_cast<const char*>(p.k) + ((int64_t)b * p.seq_k * rs + (int64_t)h * D) * 2;
  k.vbase0 = static_cast<const char*>(p.v) + ((int64_t)b * p.seq_k * rs + (int64_t)h * D) * 2;
  k.sbase0 = SEG ? p.seg + (int64_t)b * p.seq_k : nullptr;
  k.k_lane = (uint32_t)(k.lane & 15) * k.rs_bytes + 16u * (uint32_t)(k.lane >> 4);
  k.v_lane = (uint32_t)(k.lane >> 2) * k.rs_bytes + 16u * (uint32_t)(k.lane & 3);
  k.k_rd = 512 * (k.lrow >> 4) + 128 * k.half + 8 * (k.lrow & 15);
  {
    const int g = k.lane >> 4, j16 = k.lane & 15;
    k.v_rd = 32 * (4 * (g >> 1) + (j16 >> 2)) + 16 * (g & 1) + 4 * (j16 & 3);
  }

  // Q of this wave as the MFMA B operand (queries are the N dimension).
  bf16x8_t qf[D / 16];
  if (k.wave_active) {
    const __bf16* qrow = static_cast<const __bf16*>(p.q) +
                         ((int64_t)b * p.seq_q + k.qg0 + k.lrow) * rs + (int64_t)h * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      qf[c] = __builtin_bit_cast(bf16x8_t,
                                 *reinterpret_cast<const uint4*>(qrow + 16 * c + 8 * k.half));
  }
  // The Q (and segment id) loads stay in flight while the prologue's K/V
  // DMA is issued: a workgroup of a short walk would otherwise pay both
  // latencies in turn.  The compiler does not count the DMA (inline asm),
  // so it waits for every load before the first use of Q (the prologue's
  // QK, by when tiles 0-2 are due anyway).

  PipeState<D> st;
#pragma unroll
  for (int j = 0; j < NDB; ++j) st.w.acc[j] = f32x16_t{};
  st.w.m_run = ninf();
#pragma unroll
  for (int g = 0; g < 4; ++g) st.w.l_run[g] = 0.f;

  // Prologue: tiles 0, 1, 2 in flight, the cursor on tile 3.
  st.ic = Cursor{0, 0, 0, 0, 0, 0, 0};
  cursor_seek<C::TN, STRIPED>(p, st.ic, k.kend);
  cursor_to<C::TN, STRIPED>(p, st.ic, k.kend, sr.begin);
  fetch_next<D, SEG, STRIPED, 0>(p, k, st, ks, vs, ss);
  fetch_next<D, SEG, STRIPED, 1>(p, k, st, ks, vs, ss);
  fetch_next<D, SEG, STRIPED, 2>(p, k, st, ks, vs, ss);
  // Tiles 0 and 1 must have landed: tile 1 is read by the first step's QK.
  constexpr int NPT = 2 * C::DPW + (SEG ? 1 : 0);
  if (st.ti[2].valid)
    wait_vm<NPT>();
  else
    wait_vm<0>();
  stage_barrier();
  if (SEG) st.segok[0] = seg_overlap_halves(ss[0], k.lane, k.qseg);
  if (st.ti[0].valid && k.wave_active) {
    TileFlags f = tile_flags<SEG, STRIPED>(st.ti[0], lim);
    if (SEG) {
      f.run0 = f.run0 && (st.segok[0] & 1u);
      f.run1 = f.run1 && (st.segok[0] & 2u);
      f.seg0 = !(st.segok[0] & 4u);
      f.seg1 = !(st.segok[0] & 8u);
    }
    qk_tile<D>(st.s[0], qf, ks[0], k.k_rd);
    const float mx = mask_max<SEG>(st.s[0], ss[0], k.half, f, lim.lane_lim, k.seg_q);
    carry_max<D>(st.w, mx, p.scale_log2);
  }

  if (st.ti[0].valid) {
    for (;;) {
      if (!pipe_step<D, SEG, STRIPED, 0>(p, k, lim, qf, st, ks, vs, ss)) break;
      if (!pipe_step<D, SEG, STRIPED, 1>(p, k, lim, qf, st, ks, vs, ss)) break;
      if (!pipe_step<D, SEG, STRIPED, 2>(p, k, lim, qf, st, ks, vs, ss)) break;
      if (!pipe_step<D, SEG, STRIPED, 3>(p, k, lim, qf, st, ks, vs, ss)) break;
    }
  }

  // ---- epilogue: out = numerator / denominator, lse = ln(denominator) + max ----
  if (!k.wave_active) return;
  const float l_tot =
      pair_sum((st.w.l_run[0] + st.w.l_run[1]) + (st.w.l_run[2] + st.w.l_run[3]));
  const int row = k.qg0 + k.lrow;
  if (p.part_o != nullptr) {
    write_partial<NDB>(p, wc.split, b, h, row, k.half, st.w.acc, st.w.m_run, l_tot);
    // With an exact grid no workgroup holds the slots past this tile's runs.
    if (p.split_wgs > 0 && wc.split == sr.runs - 1 && k.half == 0)
      for (int u = sr.runs; u < p.key_splits; ++u) write_empty_partial(p, u, b, h, row);
    return;
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  __bf16* orow = static_cast<__bf16*>(p.out) + ((int64_t)b * p.seq_q + row) * rs + (int64_t)h * D;
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      typedef float f32x4_t __attribute__((ext_vector_type(4)));
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      const f32x4_t o = {st.w.acc[j][4 * g] * inv, st.w.acc[j][4 * g + 1] * inv,
                         st.w.acc[j][4 * g + 2] * inv, st.w.acc[j][4 * g + 3] * inv};
      *reinterpret_cast<bf16x4_t*>(orow + 32 * j + 8 * g + 4 * k.half) =
          __builtin_convertvector(o, bf16x4_t);
    }
  }
  if (k.half == 0)
    p.lse[((int64_t)b * p.heads + h) * p.seq_q + row] =
        l_tot > 0.f ? (st.w.m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : ninf();
}

// ---------------------------------------------------------------------------
// fp32 kernel
// ---------------------------------------------------------------------------
//
// 32-key tiles, K and V row-major in LDS with a 4-element pad, fp32 MFMA
// v_mfma_f32_32x32x2_f32 (one k-slot per lane half).  The P.V A operand is
// V^T: lane (d, half) reads V[key][d] for the key its P^T slot holds.

template <int D, bool STRIPED>
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

  const WgCoord wc =
      p.split_wgs > 0 ? wg_coord_runs<kBlockMF32, 32, STRIPED>(p) : wg_coord<kBlockMF32>(p);
  if (wc.split < 0) return;
  const int b = wc.b, h = wc.h, m0 = wc.m0;
  const int qg0 = m0 + wave * 32;
  const bool wave_active = qg0 < p.seq_q;
  const int64_t pq_first = (int64_t)p.ring_index * p.seq_q + qg0;
  const WaveLimits lim = wave_limits(p, STRIPED ? qg0 : pq_first, lrow, wave_active);
  const int64_t kend = wg_kend<kBlockMF32, STRIPED>(p, m0);
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

  const SplitRange sr = split_range<TN, STRIPED>(
      p, wc.split, kend, wg_kend<kBlockMF32, STRIPED>(p, (p.n_qtiles - 1) * kBlockMF32));
  if (sr.idle) {
    if (wave_active && half == 0) write_empty_partial(p, wc.split, b, h, qg0 + lrow);
    return;
  }
  Cursor cur{0, 0, 0, 0, 0, 0, 0};
  cursor_seek<TN, STRIPED>(p, cur, kend);
  cursor_to<TN, STRIPED>(p, cur, kend, sr.begin);
  if (cur.pos >= sr.end) cur.valid = 0;
  if (cur.valid) {
    load_tile(cur);
    store_tile(0);
  }
  __syncthreads();

  int buf = 0;
  while (cur.valid) {
    Cursor nxt = cur;
    cursor_next<TN, STRIPED>(p, nxt, kend);
    if (nxt.pos >= sr.end) nxt.valid = 0;
    if (nxt.valid) load_tile(nxt);

    const int kloc0 = cur.kt * TN;
    const int32_t pk0 = block_vbase<STRIPED>(p, cur.kb) + kloc0;  // key coordinate
    const bool run = pk0 < lim.run_lim;
    const bool mask = has_seg || pk0 >= lim.mask_lim;
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
        const int32_t pkb = pk0 + 4 * half;
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
      if (p.run_map != nullptr && lane == 0) write_run_map(p, cur.kb, qg0, kloc0);
    }

    if (nxt.valid) store_tile(buf ^ 1);
    __syncthreads();
    cur = nxt;
    buf ^= 1;
  }

  if (!wave_active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const int row = qg0 + lrow;
  if (p.part_o != nullptr) {
    write_partial<NDB>(p, wc.split, b, h, row, half, acc, m_run, l_tot);
    if (p.split_wgs > 0 && wc.split == sr.runs - 1 && half == 0)
      for (int u = sr.runs; u < p.key_splits; ++u) write_empty_partial(p, u, b, h, row);
    return;
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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

template <int D>
void launch_bf16(bool seg, bool striped, dim3 grid, dim3 block, hipStream_t s,
                 const FwdParams& p) {
  if (seg) {
    if (striped)
      hipLaunchKernelGGL((fwd_bf16_kernel<D, true, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<D, true, false>), grid, block, 0, s, p);
  } else {
    if (striped)
      hipLaunchKernelGGL((fwd_bf16_kernel<D, false, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<D, false, false>), grid, block, 0, s, p);
  }
}

}  // namespace

// Scratch of ra_blockwise_attn_fwd_split_noalloc (the split partials of
// callers that cannot allocate).  In host code `scratch` names a host-side
// stand-in, not device memory: kernels only ever get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[kFwdScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};
}  // namespace

int fwd_scratch(void** ptr, char* err, int errlen) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) {
    snprintf(err, errlen, "no usable current device (%s, device %d)", hipGetErrorString(e), dev);
    return 1;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      snprintf(err, errlen, "hipGetSymbolAddress of the scratch array failed on device %d: %s",
               dev, hipGetErrorString(e));
      return 1;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

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
  const dim3 grid(p.n_wg);
  if (dtype == Dtype::BF16) {
    const dim3 block(PipeCfg<128>::kThreads);
    const bool seg = p.seg != nullptr, str = p.striped != 0;
    if (head_dim == 128)
      launch_bf16<128>(seg, str, grid, block, s, p);
    else
      launch_bf16<64>(seg, str, grid, block, s, p);
  } else {
    const dim3 block(kThreads);
    const bool str = p.striped != 0;
    if (head_dim == 128) {
      if (str)
        hipLaunchKernelGGL((fwd_f32_kernel<128, true>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((fwd_f32_kernel<128, false>), grid, block, 0, s, p);
    } else {
      if (str)
        hipLaunchKernelGGL((fwd_f32_kernel<64, true>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((fwd_f32_kernel<64, false>), grid, block, 0, s, p);
    }
  }
  e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(err, errlen, "kernel launch failed: %s", hipGetErrorString(e));
    return 1;
  }
  if (p.part_o != nullptr) {
    const int64_t threads = (int64_t)p.batch * p.heads * p.seq_q * (head_dim / 4);
    const dim3 cgrid((unsigned)((threads + 255) / 256));
    const bool str = p.striped != 0;
    if (dtype == Dtype::BF16) {
      if (str)
        hipLaunchKernelGGL((combine_splits_kernel<__bf16, kBlockMBf16, 64, true>), cgrid,
                           dim3(256), 0, s, p, head_dim);
      else
        hipLaunchKernelGGL((combine_splits_kernel<__bf16, kBlockMBf16, 64, false>), cgrid,
                           dim3(256), 0, s, p, head_dim);
    } else {
      if (str)
        hipLaunchKernelGGL((combine_splits_kernel<float, kBlockMF32, 32, true>), cgrid,
                           dim3(256), 0, s, p, head_dim);
      else
        hipLaunchKernelGGL((combine_splits_kernel<float, kBlockMF32, 32, false>), cgrid,
                           dim3(256), 0, s, p, head_dim);
    }
    e = hipGetLastError();
    if (e != hipSuccess) {
      snprintf(err, errlen, "split combine launch failed: %s", hipGetErrorString(e));
      return 1;
    }
  }
  return 0;
}

}  // namespace ra
