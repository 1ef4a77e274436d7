// Backward of one ring share for float32 inputs: the same gradients as the
// bf16 kernels (blockwise_bwd.hip), computed in float32 throughout on
// v_mfma_f32_32x32x2_f32.  The pages say the ring code carries a backward
// pass for its forward ("从论文到代码：深入理解RingAttention的块注意力计算逻辑":
// the file holds forward and backward) and run their multi-device example
// in float32 ("多设备分布式计算"); the derivative is that of the attention
// definition ("Ring Attention with Blockwise Transformers for Near-Infinite
// Context", section 三, 自注意力):
//   p_ij  = exp(q_i.k_j / sqrt(D) - lse_i) on visible pairs, 0 elsewhere,
//   dv_j  = sum_i p_ij dout_i,
//   ds_ij = p_ij (dout_i.v_j - delta_i),   delta_i = dout_i.out_i,
//   dq_i  = sum_j ds_ij k_j / sqrt(D),      dk_j = sum_i ds_ij q_i / sqrt(D).
//
// Two kernels, both 4 waves x 32 rows with 32-row tiles staged through
// registers into double-buffered LDS (row-major, 4-float pad), like the
// float32 forward; they serve the float32 workloads and edge shapes, not
// speed.
//   bwd_dq_f32_kernel (query-stationary, the forward's walk, masks and key
//     splits): S^T = K Q^T and dP^T = V dO^T with keys = M, so a lane holds
//     one query row (its lse and delta are scalars); dQ^T += K^T dS^T.
//   bwd_dkdv_f32_kernel (key-stationary, 128 keys per workgroup, K and V of
//     the lane's key in registers): S = Q K^T and dP = dO V^T with keys = N,
//     so a lane holds one key; dV^T += dO^T P and dK^T += Q^T dS.
// v_mfma_f32_32x32x2_f32: A[m][k] lane l row m = l % 32, k = l / 32; B[k][n]
// lane l column n = l % 32, k = l / 32; C[m][n] lane l column n = l % 32,
// rows 8 (i / 4) + 4 (l / 32) + i % 4 of register i.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <climits>

#include "ra_device.h"
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int kThreadsF32 = 256;  // 4 waves
constexpr int kTileF32 = 32;      // rows per staged tile
constexpr float kLog2eF = 1.4426950408889634f;

__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row of register i's element in a 32 x 32 C block, for lane half `half`.
__device__ __forceinline__ constexpr int c_row(int i, int half) {
  return 8 * (i >> 2) + 4 * half + (i & 3);
}

// Stage a 32-row tile of a [rows, H*D] float32 tensor (rows from row0,
// rows at or past `nrows` as zeros) through registers.
template <int D>
struct RowTile {
  static constexpr int KS = D + 4;
  static constexpr int LOADS = kTileF32 * D / 4 / kThreadsF32;
  float4 reg[LOADS];

  __device__ __forceinline__ void load(const float* base, int64_t rs, int64_t row0, int64_t nrows,
                                       int tid) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int ci = tid + u * kThreadsF32;
      const int row = ci / (D / 4), col = (ci % (D / 4)) * 4;
      reg[u] = row0 + row < nrows
                   ? *reinterpret_cast<const float4*>(base + (row0 + row) * rs + col)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ void store(float* lds, int tid) const {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int ci = tid + u * kThreadsF32;
      const int row = ci / (D / 4), col = (ci % (D / 4)) * 4;
      *reinterpret_cast<float4*>(&lds[row * KS + col]) = reg[u];
    }
  }
};

// ---------------------------------------------------------------------------
// dq (query-stationary)
// ---------------------------------------------------------------------------

template <int D, bool STRIPED>
__global__ __launch_bounds__(kThreadsF32, 1) void bwd_dq_f32_kernel(const BwdParams bp) {
  constexpr int TN = kTileF32, KS = D + 4, NDB = D / 32;
  const FwdParams& p = bp.f;
  __shared__ __attribute__((aligned(16))) float k_lds[2][TN * KS];
  __shared__ __attribute__((aligned(16))) float v_lds[2][TN * KS];
  __shared__ int32_t seg_lds[2][TN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 31;
  const int half = lane >> 5;

  const WgCoord wc =
      p.split_wgs > 0 ? wg_coord_runs<kBlockMF32, TN, STRIPED>(p) : wg_coord<kBlockMF32>(p);
  if (wc.split < 0) return;
  const int b = wc.b, h = wc.h, m0 = wc.m0;
  const int qg0 = m0 + wave * 32;
  const bool wave_active = qg0 < p.seq_q;
  const int64_t pq_first = (int64_t)p.ring_index * p.seq_q + qg0;
  const WaveLimits lim = wave_limits(p, STRIPED ? qg0 : pq_first, lrow, wave_active);
  const int64_t kend = wg_kend<kBlockMF32, STRIPED>(p, m0);
  const bool has_seg = p.seg != nullptr;
  const int64_t rs = (int64_t)p.heads * D;
  const int row = qg0 + lrow;
  float* const dst = bp.dq_part != nullptr
                         ? bp.dq_part + (int64_t)wc.split * p.batch * p.seq_q * rs
                         : bp.dq;
  float* const drow = dst + ((int64_t)b * p.seq_q + row) * rs + (int64_t)h * D;

  const SplitRange sr = split_range<TN, STRIPED>(
      p, wc.split, kend, wg_kend<kBlockMF32, STRIPED>(p, (p.n_qtiles - 1) * kBlockMF32));
  if (sr.idle) {
    // A split with no run adds nothing to dq.
    if (wave_active)
#pragma unroll
      for (int j = 0; j < NDB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(drow + 32 * j + 8 * g + 4 * half) =
              make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }

  // Q^T and dO^T of this lane's row as B operands; its lse (base 2) and delta.
  float qf[D / 2], gf[D / 2];
  float lse2 = 0.f, dlt = 0.f;
  int32_t seg_q = 0;
#pragma unroll
  for (int c = 0; c < D / 2; ++c) qf[c] = gf[c] = 0.f;
  if (wave_active) {
    const int64_t roff = ((int64_t)b * p.seq_q + row) * rs + (int64_t)h * D;
    const float* qrow = static_cast<const float*>(p.q) + roff;
    const float* grow = static_cast<const float*>(bp.dout) + roff;
#pragma unroll
    for (int c = 0; c < D / 2; ++c) {
      qf[c] = qrow[2 * c + half];
      gf[c] = grow[2 * c + half];
    }
    const int64_t li = ((int64_t)b * p.heads + h) * p.seq_q + row;
    lse2 = bp.lse[li] * kLog2eF;
    dlt = bp.delta[li];
    if (has_seg) seg_q = p.seg[(int64_t)b * p.seq_k + pq_first + lrow];
  }

  f32x16_t acc[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) acc[j] = f32x16_t{};

  const float* kbase0 = static_cast<const float*>(p.k) + (int64_t)b * p.seq_k * rs + (int64_t)h * D;
  const float* vbase0 = static_cast<const float*>(p.v) + (int64_t)b * p.seq_k * rs + (int64_t)h * D;
  RowTile<D> kt, vt;
  int32_t sreg = 0;
  auto load_tile = [&](const Cursor& c) {
    const int64_t row0 = (int64_t)c.kb * p.seq_q + (int64_t)c.kt * TN;
    kt.load(kbase0, rs, row0, p.seq_k, tid);
    vt.load(vbase0, rs, row0, p.seq_k, tid);
    if (has_seg && tid < TN) sreg = p.seg[(int64_t)b * p.seq_k + row0 + tid];
  };
  auto store_tile = [&](int buf) {
    kt.store(k_lds[buf], tid);
    vt.store(v_lds[buf], tid);
    if (has_seg && tid < TN) seg_lds[buf][tid] = sreg;
  };

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

    const int32_t pk0 = block_vbase<STRIPED>(p, cur.kb) + cur.kt * TN;  // key coordinate
    if (pk0 < lim.run_lim) {
      const float* ks = k_lds[buf];
      const float* vs = v_lds[buf];
      const int32_t* sg = seg_lds[buf];
      // S^T = K Q^T and dP^T - delta = V dO^T - delta (keys = M).
      f32x16_t s = f32x16_t{}, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) dp[i] = -dlt;
      const float* krow = ks + lrow * KS + half;
      const float* vrow = vs + lrow * KS + half;
#pragma unroll
      for (int c = 0; c < D / 2; ++c) {
        s = mfma_f32(krow[2 * c], qf[c], s);
        dp = mfma_f32(vrow[2 * c], gf[c], dp);
      }
      const bool mask = has_seg || pk0 >= lim.mask_lim;
      f32x16_t ds;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int koff = c_row(i, half);
        bool ok = true;
        if (mask) {
          ok = pk0 + koff < lim.lane_lim;
          if (has_seg) ok = ok && sg[koff] == seg_q;
        }
        const float pr = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], p.scale_log2, -lse2)) : 0.f;
        ds[i] = pr * dp[i];
      }
      // dQ^T += K^T dS^T: A = K^T (d = M), register i's pair of keys.
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float* kr = ks + c_row(i, half) * KS + lrow;
#pragma unroll
        for (int j = 0; j < NDB; ++j) acc[j] = mfma_f32(kr[32 * j], ds[i], acc[j]);
      }
    }

    if (nxt.valid) store_tile(buf ^ 1);
    __syncthreads();
    cur = nxt;
    buf ^= 1;
  }

  if (!wave_active) return;
  const float scale = p.scale_log2 / kLog2eF;
#pragma unroll
  for (int j = 0; j < NDB; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(drow + 32 * j + 8 * g + 4 * half) =
          make_float4(acc[j][4 * g] * scale, acc[j][4 * g + 1] * scale,
                      acc[j][4 * g + 2] * scale, acc[j][4 * g + 3] * scale);
}

// ---------------------------------------------------------------------------
// dk / dv (key-stationary)
// ---------------------------------------------------------------------------

template <int D, bool STRIPED>
__global__ __launch_bounds__(kThreadsF32, 1) void bwd_dkdv_f32_kernel(const BwdParams bp) {
  constexpr int TQ = kTileF32, KS = D + 4, NDB = D / 32;
  const FwdParams& p = bp.f;
  __shared__ __attribute__((aligned(16))) float q_lds[2][TQ * KS];
  __shared__ __attribute__((aligned(16))) float g_lds[2][TQ * KS];
  __shared__ float lse_lds[2][TQ], dlt_lds[2][TQ];
  __shared__ int32_t seg_lds[2][TQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 31;
  const int half = lane >> 5;

  // Workgroup -> (batch, head, 128-key tile): consecutive key tiles of one
  // head (which stream the same queries) share an XCD.
  const int pid = blockIdx.x, n = bp.n_wg_kv;
  const int xcd = pid & 7, idx = pid >> 3, cnt = n >> 3, rem = n & 7;
  const int logical =
      xcd < rem ? xcd * (cnt + 1) + idx : rem * (cnt + 1) + (xcd - rem) * cnt + idx;
  const int bh = logical / bp.n_ktiles;
  const int b = bh / p.heads, h = bh % p.heads;
  const int k0 = (logical % bp.n_ktiles) * kBlockNBwdF32;
  const int kw0 = k0 + 32 * wave;  // first key of this wave
  const bool active = kw0 < p.seq_k;
  const int key = kw0 + lrow;
  const int64_t rs = (int64_t)p.heads * D;
  const int32_t qrow0 = p.ring_index * p.seq_q;   // storage row of local row 0
  const int32_t qpos0 = STRIPED ? 0 : qrow0;      // its query coordinate
  const int64_t c = p.causal;
  const KeyThresholds kth = key_thresholds<STRIPED>(p, kw0, lrow);
  const bool has_seg = p.seg != nullptr;
  const int32_t seg_k = has_seg && active ? p.seg[(int64_t)b * p.seq_k + key] : 0;

  // K^T and V^T of this lane's key as B operands.
  float kf[D / 2], vf[D / 2];
#pragma unroll
  for (int cc = 0; cc < D / 2; ++cc) kf[cc] = vf[cc] = 0.f;
  if (active) {
    const int64_t koff = ((int64_t)b * p.seq_k + key) * rs + (int64_t)h * D;
    const float* krow = static_cast<const float*>(p.k) + koff;
    const float* vrow = static_cast<const float*>(p.v) + koff;
#pragma unroll
    for (int cc = 0; cc < D / 2; ++cc) {
      kf[cc] = krow[2 * cc + half];
      vf[cc] = vrow[2 * cc + half];
    }
  }

  const int q_lo = first_query_row<STRIPED>(p, k0, kBlockNBwdF32, qpos0) & ~(TQ - 1);
  const int n_qt = (p.seq_q - q_lo + TQ - 1) / TQ;

  const float* qbase0 = static_cast<const float*>(p.q) + (int64_t)b * p.seq_q * rs + (int64_t)h * D;
  const float* gbase0 =
      static_cast<const float*>(bp.dout) + (int64_t)b * p.seq_q * rs + (int64_t)h * D;
  const float* lbase = bp.lse + ((int64_t)b * p.heads + h) * p.seq_q;
  const float* dbase = bp.delta + ((int64_t)b * p.heads + h) * p.seq_q;
  RowTile<D> qt_r, gt_r;
  float lreg = 0.f, dreg = 0.f;
  int32_t sreg = 0;
  auto load_tile = [&](int t) {
    const int q0 = q_lo + TQ * t;
    qt_r.load(qbase0, rs, q0, p.seq_q, tid);
    gt_r.load(gbase0, rs, q0, p.seq_q, tid);
    if (tid < TQ && q0 + tid < p.seq_q) {
      lreg = lbase[q0 + tid] * kLog2eF;
      dreg = dbase[q0 + tid];
      if (has_seg) sreg = p.seg[(int64_t)b * p.seq_k + qrow0 + q0 + tid];
    }
  };
  auto store_tile = [&](int buf) {
    qt_r.store(q_lds[buf], tid);
    gt_r.store(g_lds[buf], tid);
    if (tid < TQ) {
      lse_lds[buf][tid] = lreg;
      dlt_lds[buf][tid] = dreg;
      seg_lds[buf][tid] = sreg;
    }
  };

  f32x16_t dk[NDB], dv[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) dk[j] = dv[j] = f32x16_t{};

  if (n_qt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int t = 0; t < n_qt; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_qt) load_tile(t + 1);
    const int q0 = q_lo + TQ * t;
    const int qlast = std::min(q0 + TQ - 1, p.seq_q - 1);
    if (active && (c == 0 || qpos0 + qlast >= kth.first)) {
      const float* qs = q_lds[buf];
      const float* gs = g_lds[buf];
      // S = Q K^T and dP = dO V^T (keys = N): lane = key, 16 query rows.
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
      const float* qrow = qs + lrow * KS + half;
      const float* grow = gs + lrow * KS + half;
#pragma unroll
      for (int cc = 0; cc < D / 2; ++cc) {
        s = mfma_f32(qrow[2 * cc], kf[cc], s);
        dp = mfma_f32(grow[2 * cc], vf[cc], dp);
      }
      f32x16_t pv, dsv;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = c_row(i, half);
        bool ok = q0 + qi < p.seq_q && (c == 0 || qpos0 + q0 + qi >= kth.lane);
        if (has_seg) ok = ok && seg_lds[buf][qi] == seg_k;
        const float pr =
            ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], p.scale_log2, -lse_lds[buf][qi])) : 0.f;
        pv[i] = pr;
        dsv[i] = pr * (dp[i] - dlt_lds[buf][qi]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS: A = dO^T, Q^T (d = M).
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = c_row(i, half);
        const float* gr = gs + qi * KS + lrow;
        const float* qr = qs + qi * KS + lrow;
#pragma unroll
        for (int j = 0; j < NDB; ++j) {
          dv[j] = mfma_f32(gr[32 * j], pv[i], dv[j]);
          dk[j] = mfma_f32(qr[32 * j], dsv[i], dk[j]);
        }
      }
    }
    if (t + 1 < n_qt) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!active) return;
  const float scale = p.scale_log2 / kLog2eF;
  const int64_t roff = ((int64_t)b * p.seq_k + key) * rs + (int64_t)h * D;
  float* dkrow = bp.dk + roff;
  float* dvrow = bp.dv + roff;
#pragma unroll
  for (int j = 0; j < NDB; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * j + 8 * g + 4 * half;
      *reinterpret_cast<float4*>(dkrow + d) =
          make_float4(dk[j][4 * g] * scale, dk[j][4 * g + 1] * scale, dk[j][4 * g + 2] * scale,
                      dk[j][4 * g + 3] * scale);
      *reinterpret_cast<float4*>(dvrow + d) =
          make_float4(dv[j][4 * g], dv[j][4 * g + 1], dv[j][4 * g + 2], dv[j][4 * g + 3]);
    }
}

template <int D, bool STRIPED>
void launch_f32(const BwdParams& bp, hipStream_t s) {
  const dim3 block(kThreadsF32);
  hipLaunchKernelGGL((bwd_dq_f32_kernel<D, STRIPED>), dim3((unsigned)bp.f.n_wg), block, 0, s, bp);
  hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, STRIPED>), dim3((unsigned)bp.n_wg_kv), block, 0, s,
                     bp);
}

}  // namespace

void launch_bwd_f32_main(const BwdParams& bp, int head_dim, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool str = bp.f.striped != 0;
  if (head_dim == 128 && str)
    launch_f32<128, true>(bp, s);
  else if (head_dim == 128)
    launch_f32<128, false>(bp, s);
  else if (str)
    launch_f32<64, true>(bp, s);
  else
    launch_f32<64, false>(bp, s);
}

}  // namespace ra
