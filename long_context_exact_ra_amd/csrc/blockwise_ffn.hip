// Blockwise feedforward of the Blockwise Transformer on MI355X (gfx950):
// y = max(0, x W1 + b1) W2 + b2 ("Ring Attention with Blockwise Transformers
// for Near-Infinite Context", section 三 "核心公式"), computed one sequence
// chunk at a time ("Blockwise Feedforward网络详解", sections "核心技术原理"
// and "技术实现细节"), so the hidden activations of only one chunk
// (chunk x ffn values) exist at any time, in a caller-provided workspace.
//
// Both products are dense GEMMs, Y = act(X W + b) with X [M, K], W [K, N],
// Y [M, N] row-major bf16, fp32 accumulation, the bias added in fp32, then
// (first product) the ReLU, then one rounding to bf16.  One kernel,
// gemm_bias_kernel, serves both; a chunk is two launches:
//   H = relu(X_chunk W1 + b1)   into the bf16 workspace   (M = chunk, K = hidden, N = ffn)
//   Y_chunk = H W2 + b2         into the chunk's rows of y (M = chunk, K = ffn, N = hidden)
//
// The kernel computes Y^T = W^T X^T on v_mfma_f32_32x32x16_bf16 (n = the
// MFMA's M dimension, m its N dimension), so a lane of an accumulator holds
// one row m of Y and runs of 4 consecutive columns n: the epilogue stores 8
// contiguous bytes per lane.  A workgroup owns a 256 x BN tile of Y (BN =
// 256, or 128 when the 256-wide grid would not fill the compute units) with 4 waves,
// each owning a 128 x (BN / 2) quarter: 4 x (BN / 64) accumulators of 32 x
// 32, up to 256 float32 per lane (the accumulation registers).
//
// K is walked in stages of 32.  X and W stage tiles flow through a ring of
// 5 LDS stages (160 KB for 256 x 256 tiles) filled by bounds-checked
// buffer-to-LDS DMA (buffer_load_dwordx4 ... lds) four stages ahead; rows
// past M (X) and past K (W) read as zero, so ragged M and K need no special
// path (columns past N compute values that are never stored).  Layouts
// (16-byte slots; g = the 16-byte granule of a row):
//   X stage, 256 rows m x 4 granules: slot(m, g) = (m / 16) * 64 + g * 16 +
//     m % 16.  A DMA instruction (64 lanes x 16 bytes) fills 16 rows x 4
//     granules; the X^T operand of 16 consecutive lanes (16 rows, one
//     granule: 8 consecutive k of each row) is 256 contiguous bytes, one
//     ds_read_b128.
//   W stage, 32 rows k x BN / 8 granules, row-major with the granules of row
//     k permuted: slot k * BN / 8 + j holds granule j ^ 4 (k % 4).  A DMA
//     instruction fetches whole rows (64 lanes, BN / 8 per row); two
//     ds_read_b64_tr_b16 (gfx950's transposing LDS read) give each lane 8
//     consecutive k of its own column n, the W^T operand, with no transpose
//     in registers.  Half a wave of one transposing read touches 4 rows x 4
//     granules of a quad; a row is a multiple of 256 bytes (the 64 four-byte
//     banks), so without the permutation the 4 rows would hit the same 4 of
//     the 16 bank groups; XORing the granule's quad bits with the row puts
//     them in 4 different quads, every bank once.
// Both operands assign the 16 k of an MFMA step to the k-slots the same
// way (lane half h takes k = 8 h .. 8 h + 7), so the contraction is exact.
// Workgroups are numbered so that consecutive tiles of one column block
// (which share W) run on the same XCD and share its L2.
//
// Measured on the 7B-shaped feedforward (32768 tokens, hidden 4096, ffn
// 16384, chunks of 2048): the data movement into LDS, not the LDS reads or
// the barriers, separates this kernel from hipBLASLt's (timing variants
// with the DMA removed ran 40 % faster, with the transposing reads replaced
// by plain ones no faster); issuing each stage's DMA spread over the MFMAs,
// whole W rows per instruction and a fifth stage gained 3 %.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstdio>
#include <mutex>

#include "ra_device.h"
#include "ra_internal.h"
#include "ra_lds.h"

namespace ra {
namespace {

constexpr int kGemmWaves = 4;
constexpr int kGemmThreads = 64 * kGemmWaves;
constexpr int kBK = 32;    // k per LDS stage
constexpr int kStages = 5;

// A BM x BN tile per workgroup, 4 waves in a 2 x 2 layout, each owning a
// (BM / 2) x (BN / 2) quarter: MB 32-row blocks x NB 32-column blocks.
template <int BM, int BN>
struct GemmCfg {
  static constexpr int WM = BM / 2, WN = BN / 2;  // rows / columns per wave
  static constexpr int MB = WM / 32, NB = WN / 32;
  static constexpr int X_ELEMS = BM * kBK;   // bf16 per X stage tile
  static constexpr int W_ELEMS = kBK * BN;   // bf16 per W stage tile
  static constexpr int STAGE = X_ELEMS + W_ELEMS;
  static constexpr int X_DMA = BM / 16 / kGemmWaves;       // DMA instructions per wave
  static constexpr int W_DMA = kBK * BN / 512 / kGemmWaves;
  static constexpr int NPT = X_DMA + W_DMA;                // per wave per stage
  static_assert(X_DMA * 16 * kGemmWaves == BM && W_DMA * 512 * kGemmWaves == kBK * BN,
                "stage tiles must split evenly over the waves");
};

struct GemmArgs {
  const __bf16* x;     // [M, K]
  const __bf16* w;     // [K, N]
  const __bf16* bias;  // [N]
  __bf16* y;           // [M, N]
  int32_t m, n, k;
  int32_t tiles_m, tiles_n;
};

// Issue this wave's share of the DMA of K-stage kt into LDS stage `st`.
template <int BM, int BN>
__device__ __forceinline__ void gemm_fetch(const GemmArgs& a, int m0, int n0, int kt, __bf16* st,
                                           int wave, int lane) {
  using C = GemmCfg<BM, BN>;
  const int k0 = kt * kBK;
  // X rows [0, M) of the chunk: rows past M read as zero.
  const i32x4_t xr = rsrc_words(a.x, (uint32_t)a.m * (uint32_t)a.k * 2u);
  // W rows [k0, K): rows past K read as zero.
  const i32x4_t wr = rsrc_words(a.w + (int64_t)k0 * a.n, (uint32_t)(a.k - k0) * (uint32_t)a.n * 2u);
#pragma unroll
  for (int u = 0; u < C::X_DMA; ++u) {
    const int i = wave * C::X_DMA + u;  // 16 rows of the tile
    const uint32_t off = (uint32_t)(m0 + 16 * i + (lane & 15)) * (uint32_t)a.k * 2u +
                         (uint32_t)(k0 + 8 * (lane >> 4)) * 2u;
    dma_b128(lds_addr(st + i * 512), off, xr);
  }
  // W: whole rows of the stage tile per instruction (BN / 8 lanes per row);
  // slot k * (BN / 8) + j of the stage holds granule j ^ 4 (k % 4) of row k.
  constexpr int GPR = BN / 8;          // granules per row
  constexpr int RPI = 64 / GPR;        // rows per DMA instruction
#pragma unroll
  for (int u = 0; u < C::W_DMA; ++u) {
    const int i = wave * C::W_DMA + u;
    const int k = RPI * i + lane / GPR;
    const int g = lds::gemm_w_gran(k, lane % GPR);
    const uint32_t off = (uint32_t)k * (uint32_t)a.n * 2u + (uint32_t)(n0 + 8 * g) * 2u;
    dma_b128(lds_addr(st + C::X_ELEMS + i * 512), off, wr);
  }
}

// One of this wave's NPT DMA instructions of K-stage kt (u < X_DMA: X,
// else W), the same as gemm_fetch issues them.
template <int BM, int BN>
__device__ __forceinline__ void gemm_fetch_one(const GemmArgs& a, int m0, int n0, int kt,
                                               __bf16* st, int wave, int lane, int u) {
  using C = GemmCfg<BM, BN>;
  const int k0 = kt * kBK;
  if (u < C::X_DMA) {
    const i32x4_t xr = rsrc_words(a.x, (uint32_t)a.m * (uint32_t)a.k * 2u);
    const int i = wave * C::X_DMA + u;
    const uint32_t off = (uint32_t)(m0 + 16 * i + (lane & 15)) * (uint32_t)a.k * 2u +
                         (uint32_t)(k0 + 8 * (lane >> 4)) * 2u;
    dma_b128(lds_addr(st + i * 512), off, xr);
  } else {
    const i32x4_t wr =
        rsrc_words(a.w + (int64_t)k0 * a.n, (uint32_t)(a.k - k0) * (uint32_t)a.n * 2u);
    constexpr int GPR = BN / 8, RPI = 64 / GPR;
    const int i = wave * C::W_DMA + (u - C::X_DMA);
    const int k = RPI * i + lane / GPR;
    const int g = lds::gemm_w_gran(k, lane % GPR);
    const uint32_t off = (uint32_t)k * (uint32_t)a.n * 2u + (uint32_t)(n0 + 8 * g) * 2u;
    dma_b128(lds_addr(st + C::X_ELEMS + i * 512), off, wr);
  }
}

// Wait until at most `pending` (0 or 1) later stages of this wave are still
// in flight (explicit counts: the DMA is invisible to the compiler).
template <int NPT>
__device__ __forceinline__ void gemm_wait(int pending) {
  if (pending >= 1)
    wait_vm<NPT>();
  else
    wait_vm<0>();
}

// The operands of one 16-k step of a stage: W^T of the wave's NB column
// blocks (two transposing reads each) and X^T of its MB row blocks.
template <int BM, int BN>
struct Operands {
  bf16x8_t w[GemmCfg<BM, BN>::NB], x[GemmCfg<BM, BN>::MB];
};

template <int BM, int BN>
__device__ __forceinline__ void read_operands(Operands<BM, BN>& o, const __bf16* st,
                                              const int (&w_rd)[GemmCfg<BM, BN>::NB], int x_rd,
                                              int ks) {
  using C = GemmCfg<BM, BN>;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    // rows ks*16 .. of the swizzled row-major W stage (the lane's base
    // w_rd[nb] holds its row and swizzled granule; the rest is a constant)
    const __bf16* src = st + w_rd[nb] + ks * 16 * BN;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)src);
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(src + 4 * BN));
    o.w[nb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
    o.x[mb] = *reinterpret_cast<const bf16x8_t*>(st + x_rd + mb * 1024 + ks * 256);
}

// acc[nb * MB + mb]: the accumulator of column block nb, row block mb.
template <int BM, int BN>
__device__ __forceinline__ void mma_step(f32x16_t* acc, const Operands<BM, BN>& o) {
  using C = GemmCfg<BM, BN>;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
      acc[nb * C::MB + mb] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.w[nb], o.x[mb], acc[nb * C::MB + mb], 0, 0, 0);
}

// The same with hook(j) after MFMA j (fenced, so the hook's instructions
// sit between the MFMAs).
template <int BM, int BN, typename Hook>
__device__ __forceinline__ void mma_step_hook(f32x16_t* acc, const Operands<BM, BN>& o,
                                              Hook&& hook) {
  using C = GemmCfg<BM, BN>;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      acc[nb * C::MB + mb] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.w[nb], o.x[mb], acc[nb * C::MB + mb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      hook(nb * C::MB + mb);
      __builtin_amdgcn_sched_barrier(0);
    }
}

// Pipeline per stage kt (two 16-k steps): the operands of step 0 are already
// in registers (read in the previous iteration); read those of step 1, run
// step 0's MFMAs; then the stage barrier -- stage kt + 1 has landed for
// every wave and every wave is done with stage kt - 1 -- the reads of stage
// kt + 1's step 0, and step 1's MFMAs with the DMA of stage kt + 4 (into
// stage kt - 1's place) spread between them.  Operand reads thus run one
// step ahead of the MFMAs, also across the barrier, and no stage starts by
// waiting on LDS.
template <int BM, int BN, bool RELU>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bias_kernel(const GemmArgs a) {
  using C = GemmCfg<BM, BN>;
  __shared__ __attribute__((aligned(16))) __bf16 lds[kStages * C::STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Tile of this workgroup: consecutive logical ids share an XCD (ids are
  // dispatched round-robin over the 8 XCDs) and, m-fastest, a column block.
  const int pid = blockIdx.x, nwg = a.tiles_m * a.tiles_n;
  const int xcd = pid & 7, idx = pid >> 3, cnt = nwg >> 3, rem = nwg & 7;
  const int logical =
      xcd < rem ? xcd * (cnt + 1) + idx : rem * (cnt + 1) + (xcd - rem) * cnt + idx;
  const int tm = __builtin_amdgcn_readfirstlane(logical % a.tiles_m);
  const int tn = __builtin_amdgcn_readfirstlane(logical / a.tiles_m);
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm = (wave & 1) * C::WM, wn = (wave >> 1) * C::WN;  // the wave's quarter

  // Per-lane parts of the operand addresses (bf16 elements).
  const int l32 = lane & 31, h = lane >> 5;
  const int x_rd = ((l32 >> 4) * 64 + h * 16 + (lane & 15)) * 8 + (wm / 16) * 512;
  // W: with g16 = lane / 16 and j16 = lane % 16, the lane reads row kr =
  // 8 (g16 / 2) + j16 / 4 (+ ks * 16, + 4 for the second read; kr % 4 =
  // j16 / 4 either way) at column wn + 32 nb + 16 (g16 % 2) + 4 (j16 % 4):
  // granule gc = (wn + 32 nb) / 8 + 2 (g16 % 2) + (j16 % 4) / 2, stored at
  // slot kr * BN / 8 + (gc ^ 4 (kr % 4)).  The XOR touches the bits of gc
  // that nb sets, so each nb has its own base.
  int w_rd[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) w_rd[nb] = C::X_ELEMS + lds::gemm_w_rd(lane, wn, nb, BN);

  f32x16_t acc[C::NB * C::MB];
#pragma unroll
  for (int i = 0; i < C::NB * C::MB; ++i) acc[i] = f32x16_t{};

  const int nk = (a.k + kBK - 1) / kBK;
  // Prologue: stages 0 .. 3 in flight; stage 0 landed; its step-0 operands.
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < nk) gemm_fetch<BM, BN>(a, m0, n0, s, lds + s * C::STAGE, wave, lane);
  {
    const int pend = nk - 1 < 3 ? nk - 1 : 3;
    if (pend >= 3)
      wait_vm<3 * C::NPT>();
    else if (pend == 2)
      wait_vm<2 * C::NPT>();
    else if (pend == 1)
      wait_vm<C::NPT>();
    else
      wait_vm<0>();
  }
  stage_barrier();
  Operands<BM, BN> op0, op1;
  read_operands<BM, BN>(op0, lds, w_rd, x_rd, 0);

  // Every stage but the last; the loop body has no branch around the
  // barrier, so the compiler's LDS waits stay exact (LDS reads complete in
  // order: a conservative wait on an earlier read would also wait for the
  // next stage's reads issued after it).  cur / nxt: LDS stages of kt and
  // kt + 1 (mod 5).
  int cur = 0;
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const int nxt = cur == kStages - 1 ? 0 : cur + 1;
    const int prv = cur == 0 ? kStages - 1 : cur - 1;  // stage of kt - 1 = kt + 4
    read_operands<BM, BN>(op1, lds + cur * C::STAGE, w_rd, x_rd, 1);
    mma_step<BM, BN>(acc, op0);
    // Stage kt + 1 must have landed (stages kt + 1 .. kt + 3, as far as
    // issued, are in flight here).
    {
      const int pend = nk - kt - 2 < 2 ? nk - kt - 2 : 2;
      if (pend >= 2)
        wait_vm<2 * C::NPT>();
      else if (pend == 1)
        wait_vm<C::NPT>();
      else
        wait_vm<0>();
    }
    stage_barrier();
    read_operands<BM, BN>(op0, lds + nxt * C::STAGE, w_rd, x_rd, 0);
    // the DMA of stage kt + 4, spread over the MFMAs
    const bool dma = kt + 4 < nk;
    __bf16* const dst = lds + prv * C::STAGE;
    // (instruction u after MFMA u * MFMAs / NPT: every instruction once)
    mma_step_hook<BM, BN>(acc, op1, [&](int j) {
      constexpr int M = C::NB * C::MB;
#pragma unroll
      for (int u = 0; u < C::NPT; ++u)
        if (u * M / C::NPT == j && dma) gemm_fetch_one<BM, BN>(a, m0, n0, kt + 4, dst, wave, lane, u);
    });
    cur = nxt;
  }
  read_operands<BM, BN>(op1, lds + cur * C::STAGE, w_rd, x_rd, 1);
  mma_step<BM, BN>(acc, op0);
  mma_step<BM, BN>(acc, op1);

  // Epilogue: + bias (fp32), ReLU, one rounding to bf16.  Lane: row m,
  // columns n .. n + 3 of each group of four.
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int n = n0 + wn + nb * 32 + 8 * gi + 4 * h;
      if (n >= a.n) continue;  // N is a multiple of 8: n .. n + 3 are all in or all out
      const bf16x4_t bv = *reinterpret_cast<const bf16x4_t*>(a.bias + n);
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const int m = m0 + wm + mb * 32 + l32;
        if (m >= a.m) continue;
        f32x4_t o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = acc[nb * C::MB + mb][4 * gi + e] + (float)bv[e];
          if (RELU) v = v > 0.f ? v : 0.f;
          o[e] = v;
        }
        *reinterpret_cast<bf16x4_t*>(a.y + (int64_t)m * a.n + n) = __builtin_convertvector(o, bf16x4_t);
      }
    }
  }
}

// Compute units of the current device, looked up once per device.
std::mutex g_cu_mu;
int g_cus[64] = {};

int compute_units(int dev) {
  if (dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(g_cu_mu);
  if (g_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    g_cus[dev] = n;
  }
  return g_cus[dev];
}

template <int BM, int BN>
void launch_gemm(const GemmArgs& a0, bool relu, hipStream_t s) {
  GemmArgs a = a0;
  a.tiles_m = (a.m + BM - 1) / BM;
  a.tiles_n = (a.n + BN - 1) / BN;
  const dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(kGemmThreads);
  if (relu)
    hipLaunchKernelGGL((gemm_bias_kernel<BM, BN, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gemm_bias_kernel<BM, BN, false>), grid, block, 0, s, a);
}

int gemm_bias(const __bf16* x, const __bf16* w, const __bf16* bias, __bf16* y, int64_t m,
              int64_t n, int64_t k, bool relu, int cus, hipStream_t s) {
  const GemmArgs a{x, w, bias, y, (int32_t)m, (int32_t)n, (int32_t)k, 0, 0};
  // 256 x 256 tiles when they fill the compute units, else 256 x 128.
  if (((m + 255) / 256) * ((n + 255) / 256) >= cus)
    launch_gemm<256, 256>(a, relu, s);
  else
    launch_gemm<256, 128>(a, relu, s);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

int launch_ffn(const FfnParams& p, void* stream, char* err, int errlen) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    std::snprintf(err, errlen, "hipGetDevice failed");
    return 1;
  }
  const int cus = compute_units(dev);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error from earlier work
  const int64_t H = p.hidden, F = p.ffn, C = p.chunk;
  const __bf16* x = static_cast<const __bf16*>(p.x);
  const __bf16* w1 = static_cast<const __bf16*>(p.w1);
  const __bf16* b1 = static_cast<const __bf16*>(p.b1);
  const __bf16* w2 = static_cast<const __bf16*>(p.w2);
  const __bf16* b2 = static_cast<const __bf16*>(p.b2);
  __bf16* y = static_cast<__bf16*>(p.y);
  __bf16* hid = static_cast<__bf16*>(p.workspace);
  for (int64_t b = 0; b < p.batch; ++b) {
    for (int64_t c0 = 0; c0 < p.seq; c0 += C) {
      const int64_t row = b * p.seq + c0;
      // H = relu(X W1 + b1) into the chunk workspace, then Y = H W2 + b2
      // into the chunk's rows of y.
      if (gemm_bias(x + row * H, w1, b1, hid, C, F, H, true, cus, s) ||
          gemm_bias(hid, w2, b2, y + row * H, C, H, F, false, cus, s)) {
        std::snprintf(err, errlen, "feedforward launch failed: %s",
                      hipGetErrorString(hipGetLastError()));
        return 1;
      }
    }
  }
  return 0;
}

}  // namespace ra
