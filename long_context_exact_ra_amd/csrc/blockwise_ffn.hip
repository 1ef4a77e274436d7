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
// K is walked in stages of 32 (two MFMA steps of 16).  X arrives in pair
// stages of 64 k through a ring of 3 LDS slots, W in stages of 32 k through
// a ring of 4 (160 KB for 256 x 256 tiles), filled by bounds-checked
// buffer-to-LDS DMA (buffer_load_dwordx4 ... lds) about four stages ahead;
// rows past M (X) and past K (W) read as zero, so ragged M and K need no
// special path (columns past N compute values that are never stored).  The
// X pair is what makes the DMA fast: a DMA instruction then fetches 8 whole
// 128-byte rows of X, where 16 half rows (a 32-deep stage) move at about
// 18 bytes per clock and compute unit, less than a third of the rate of
// whole lines, and held the kernel to 834 TFLOP/s on the 7B-shaped shape.
// Layouts (16-byte slots; g = the 16-byte granule of a row):
//   X pair stage, 256 rows m x 8 granules: slot(m, g) = (m / 8) * 64 +
//     (g ^ ((m / 8) % 2)) * 8 + m % 8.  A DMA instruction (64 lanes x 16
//     bytes) fills 8 rows x 8 granules; the X^T operand of 16 consecutive
//     lanes (16 rows, one granule: 8 consecutive k of each row) is one
//     ds_read_b128 touching every bank once (the odd blocks' granule
//     permutation puts the second 8 rows on the other half of the banks).
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
// the barriers, separated this kernel from hipBLASLt's (timing variants
// with the DMA removed ran 40 % faster, with the transposing reads replaced
// by plain ones no faster), and within it the half-line X fetches.

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
constexpr int kBK = 32;     // k per MFMA stage (two 16-k steps)
constexpr int kXSlots = 3;  // X pair stages (64 k each) in LDS
constexpr int kWSlots = 4;  // W stages (32 k each) in LDS

// A BM x BN tile per workgroup, 4 waves in a 2 x 2 layout, each owning a
// (BM / 2) x (BN / 2) quarter: MB 32-row blocks x NB 32-column blocks.
template <int BM, int BN>
struct GemmCfg {
  static constexpr int WM = BM / 2, WN = BN / 2;  // rows / columns per wave
  static constexpr int MB = WM / 32, NB = WN / 32;
  static constexpr int X_PAIR = BM * 2 * kBK;     // bf16 per X pair stage (64 k)
  static constexpr int W_ELEMS = kBK * BN;        // bf16 per W stage
  static constexpr int LDS = kXSlots * X_PAIR + kWSlots * W_ELEMS;
  static constexpr int XH = BM / 8 / 2 / kGemmWaves;  // X DMA per wave: half a pair
  static constexpr int W_DMA = kBK * BN / 512 / kGemmWaves;
  static constexpr int NPT = XH + W_DMA;              // DMA per wave per iteration
  static_assert(XH * 8 * 2 * kGemmWaves == BM && W_DMA * 512 * kGemmWaves == kBK * BN,
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

// The per-lane parts of this wave's DMA source offsets, fixed for the
// whole walk: X piece u of pair half h reads row m0 + 8 i + lane % 8 of the
// tile at granule (lane / 8) ^ (i % 2) (i = (BM / 16) h + XH wave + u); the
// half adds BM / 2 rows (i changes by BM / 16, an even number, so the
// granule does not) and each pair q adds 128 q bytes, both scalars.  W
// piece u reads row k = RPI i + lane / GPR of the stage (i = W_DMA wave +
// u) at granule gemm_w_gran(k, lane % GPR) of the tile's columns.
template <int BM, int BN>
struct DmaLanes {
  uint32_t x[GemmCfg<BM, BN>::XH], w[GemmCfg<BM, BN>::W_DMA];
};

template <int BM, int BN>
__device__ __forceinline__ DmaLanes<BM, BN> dma_lanes(const GemmArgs& a, int m0, int n0, int wave,
                                                      int lane) {
  using C = GemmCfg<BM, BN>;
  DmaLanes<BM, BN> d;
  static_assert((BM / 16) % 2 == 0, "the pair halves share the granule permutation");
#pragma unroll
  for (int u = 0; u < C::XH; ++u) {
    const int i = wave * C::XH + u;
    d.x[u] = (uint32_t)(m0 + lds::gemm_x_dma_row(lane, i)) * (uint32_t)a.k * 2u +
             16u * (uint32_t)lds::gemm_x_dma_gran(lane, i);
  }
  constexpr int GPR = BN / 8, RPI = 64 / GPR;  // granules per row, rows per instruction
#pragma unroll
  for (int u = 0; u < C::W_DMA; ++u) {
    const int i = wave * C::W_DMA + u;
    const int k = RPI * i + lane / GPR;
    d.w[u] = (uint32_t)k * (uint32_t)a.n * 2u +
             (uint32_t)(n0 + 8 * lds::gemm_w_gran(k, lane % GPR)) * 2u;
  }
  return d;
}

// One iteration's DMA group, its scalars computed once: half h of X pair q
// (k 64 q .. 64 q + 63) into the LDS pair slot at byte address xs, and W
// stage kt (k 32 kt .. 32 kt + 31) into the stage slot at ws.  X rows past
// M and W rows past K read as zero (buffer bounds).
struct DmaGroup {
  bool x_ok, w_ok;
  uint32_t xs, ws;  // LDS byte addresses of this wave's first pieces
  uint32_t xadd;    // 128 q + the half's BM / 2 rows
  i32x4_t wr;       // W rows [32 kt, K)
};

template <int BM, int BN>
__device__ __forceinline__ void dma_issue(const DmaGroup& g, const DmaLanes<BM, BN>& d,
                                          const i32x4_t& xr, int u) {
  using C = GemmCfg<BM, BN>;
  if (u < C::XH) {
    if (g.x_ok) dma_b128(g.xs + 1024u * u, d.x[u] + g.xadd, xr);
  } else {
    if (g.w_ok) dma_b128(g.ws + 1024u * (u - C::XH), d.w[u - C::XH], g.wr);
  }
}

// The operands of one 16-k step: W^T of the wave's NB column blocks (two
// transposing reads each) and X^T of its MB row blocks.
template <int BM, int BN>
struct Operands {
  bf16x8_t w[GemmCfg<BM, BN>::NB], x[GemmCfg<BM, BN>::MB];
};

// Step ks of the 32-k stage held by W stage `ws` and half sp of X pair `xs`.
template <int BM, int BN>
__device__ __forceinline__ void read_operands(Operands<BM, BN>& o, const __bf16* xs,
                                              const __bf16* ws,
                                              const int (&w_rd)[GemmCfg<BM, BN>::NB], int x_rd,
                                              int sp, int ks) {
  using C = GemmCfg<BM, BN>;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    // rows ks*16 .. of the swizzled row-major W stage (the lane's base
    // w_rd[nb] holds its row and swizzled granule; the rest is a constant)
    const __bf16* src = ws + w_rd[nb] + ks * 16 * BN;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)src);
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(src + 4 * BN));
    o.w[nb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
    o.x[mb] = *reinterpret_cast<const bf16x8_t*>(xs + x_rd + mb * 2048 + sp * 256 + ks * 128);
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

// Floor division by 2 (for the prologue's negative iteration numbers).
__device__ __forceinline__ constexpr int half_floor(int v) { return v >= 0 ? v / 2 : -((1 - v) / 2); }

// Iteration j's DMA group: W stage j + 4 (into the slot of stage j, whose
// reads are done after iteration j's barrier) and half (j + 1) % 2 of X pair
// q = floor((j + 1) / 2) + 2 (into the slot of pair q - 3, also done).  Each
// group is XH + W_DMA instructions per wave while the stages exist, so a
// stage's data is complete once every group but the last two has landed.
// Pipeline per iteration kt (stage kt's two 16-k steps): the operands of
// step 0 are already in registers (read in the previous iteration); read
// those of step 1, run step 0's MFMAs; then the stage barrier -- stage
// kt + 1 has landed for every wave and every wave is done with stage kt --
// the reads of stage kt + 1's step 0, and step 1's MFMAs with the group's
// DMA spread between them.  Operand reads thus run one step ahead of the
// MFMAs, also across the barrier, and no stage starts by waiting on LDS.
template <int BM, int BN, bool RELU>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bias_kernel(const GemmArgs a) {
  using C = GemmCfg<BM, BN>;
  __shared__ __attribute__((aligned(16))) __bf16 lds[C::LDS];
  __bf16* const xbase = lds;                          // kXSlots X pair stages
  __bf16* const wbase = lds + kXSlots * C::X_PAIR;    // kWSlots W stages

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
  const int x_rd = lds::gemm_x_rd(lane, wm);
  // W: with g16 = lane / 16 and j16 = lane % 16, the lane reads row kr =
  // 8 (g16 / 2) + j16 / 4 (+ ks * 16, + 4 for the second read; kr % 4 =
  // j16 / 4 either way) at column wn + 32 nb + 16 (g16 % 2) + 4 (j16 % 4):
  // granule gc = (wn + 32 nb) / 8 + 2 (g16 % 2) + (j16 % 4) / 2, stored at
  // slot kr * BN / 8 + (gc ^ 4 (kr % 4)).  The XOR touches the bits of gc
  // that nb sets, so each nb has its own base.
  int w_rd[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) w_rd[nb] = lds::gemm_w_rd(lane, wn, nb, BN);

  f32x16_t acc[C::NB * C::MB];
#pragma unroll
  for (int i = 0; i < C::NB * C::MB; ++i) acc[i] = f32x16_t{};

  const int nk = (a.k + kBK - 1) / kBK;
  auto xslot = [&](int q) { return xbase + (q % kXSlots) * C::X_PAIR; };
  auto wslot = [&](int kt) { return wbase + (kt % kWSlots) * C::W_ELEMS; };
  const DmaLanes<BM, BN> dl = dma_lanes<BM, BN>(a, m0, n0, wave, lane);
  const i32x4_t xr = rsrc_words(a.x, (uint32_t)a.m * (uint32_t)a.k * 2u);
  // Iteration j's group (stages past K are not fetched).
  auto make_group = [&](int j) {
    DmaGroup g;
    const int q = half_floor(j + 1) + 2, kt = j + 4, h = (j + 1) & 1;
    g.x_ok = 2 * q < nk;
    g.w_ok = kt < nk && kt >= 0;
    g.xs = lds_addr(xslot(q)) + 1024u * (uint32_t)((BM / 16) * h + wave * C::XH);
    g.ws = lds_addr(wslot(kt)) + 1024u * (uint32_t)(wave * C::W_DMA);
    g.xadd = 128u * (uint32_t)q + (uint32_t)h * (uint32_t)(BM / 2) * (uint32_t)a.k * 2u;
    const int k0 = g.w_ok ? kt * kBK : 0;
    g.wr = rsrc_words(a.w + (int64_t)k0 * a.n, (uint32_t)(a.k - k0) * (uint32_t)a.n * 2u);
    return g;
  };
  // Prologue: the groups of iterations -5 .. -1 (W stages 0 .. 3, X pairs 0
  // and 1, half of pair 2); stage 0 complete once the first two have landed.
#pragma unroll
  for (int j = -5; j < 0; ++j) {
    const DmaGroup g = make_group(j);
#pragma unroll
    for (int u = 0; u < C::NPT; ++u) dma_issue<BM, BN>(g, dl, xr, u);
  }
  if (nk > 4)
    wait_vm<3 * C::NPT>();
  else
    wait_vm<0>();
  stage_barrier();
  Operands<BM, BN> op0, op1;
  read_operands<BM, BN>(op0, xslot(0), wslot(0), w_rd, x_rd, 0, 0);

  // Every stage but the last; the loop body has no branch around the
  // barrier, so the compiler's LDS waits stay exact (LDS reads complete in
  // order: a conservative wait on an earlier read would also wait for the
  // next stage's reads issued after it).
  for (int kt = 0; kt + 1 < nk; ++kt) {
    read_operands<BM, BN>(op1, xslot(kt >> 1), wslot(kt), w_rd, x_rd, kt & 1, 1);
    mma_step<BM, BN>(acc, op0);
    // Stage kt + 1 must have landed: the groups of iterations kt - 2 and
    // kt - 1 may still be in flight (all complete near the end of K).
    if (kt + 4 < nk)
      wait_vm<2 * C::NPT>();
    else
      wait_vm<0>();
    // This wave's reads of stage kt (issued before the MFMAs above) have
    // completed: after the barrier the DMA may overwrite its slots.  (The
    // barrier's fence waits only after it.)
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    stage_barrier();
    read_operands<BM, BN>(op0, xslot((kt + 1) >> 1), wslot(kt + 1), w_rd, x_rd, (kt + 1) & 1, 0);
    // this iteration's group, spread over the MFMAs (instruction u after
    // MFMA u * MFMAs / NPT: every instruction once)
    const DmaGroup g = make_group(kt);
    mma_step_hook<BM, BN>(acc, op1, [&](int jm) {
      constexpr int M = C::NB * C::MB;
#pragma unroll
      for (int u = 0; u < C::NPT; ++u)
        if (u * M / C::NPT == jm) dma_issue<BM, BN>(g, dl, xr, u);
    });
  }
  read_operands<BM, BN>(op1, xslot((nk - 1) >> 1), wslot(nk - 1), w_rd, x_rd, (nk - 1) & 1, 1);
  mma_step<BM, BN>(acc, op0);
  mma_step<BM, BN>(acc, op1);
  // (Every DMA group issued was waited for by the last iteration's wait.)

  // Epilogue: + bias (fp32), ReLU, one rounding to bf16.  Lane: row m,
  // columns n .. n + 3 of each group of four.
  const int l32 = lane & 31, h = lane >> 5;
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
