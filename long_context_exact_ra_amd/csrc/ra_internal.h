// Internal interface between the host-side C ABI (ra_host.cpp, plain C++)
// and the HIP side (blockwise_fwd.hip, blockwise_bwd.hip, blockwise_ffn.hip).
// Not installed, not part of the ABI.
#pragma once

#include <stdint.h>

namespace ra {

// Everything the forward kernel needs, validated and derived on the host.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seg;   // [B, S] or nullptr
  void* out;
  float* lse;
  uint8_t* run_map;     // [N][Lq/qc][Lq/kc] or nullptr
  int64_t causal;       // effective causal block size; 0 = non-causal
  int32_t seq_q;        // Lq
  int32_t seq_k;        // S = N * Lq
  int32_t q_chunk;
  int32_t k_chunk;
  int32_t batch;
  int32_t heads;
  int32_t ring_size;
  int32_t ring_index;
  int32_t n_qtiles;     // query tiles per (batch, head)
  int32_t n_wg;         // workgroups in the grid
  float scale_log2;     // log2(e) / sqrt(head_dim)
  int32_t striped;      // 1: striped placement (causal is then in key coordinates)
  // Striped placement: blocks kb >= stripe_hi have key coordinates from 1
  // (walk::striped_causal); the host sets it for contiguous calls too.
  int32_t stripe_hi;
  // Key splits (>= 1).  With more than one, every query tile's key walk is
  // cut into key_splits runs, one workgroup each; they write partial
  // results and a combine kernel folds them into out and lse.
  int32_t key_splits;
  float* part_o;        // [key_splits][B][H][Lq][D] unnormalised numerators
  float* part_ml;       // [key_splits][B][H][Lq][2] (kept max, base 2; denominator)
  // Forward with key splits: workgroups per (batch, head), one per run of
  // each query tile's walk (0: key_splits workgroups per query tile).
  int32_t split_wgs;
};

enum class Dtype : int { BF16 = 0, F32 = 1 };

// Query rows per workgroup: 8 waves x 32 rows for bf16, 4 waves x 32 rows
// for fp32.
constexpr int kBlockMBf16 = 256;
constexpr int kBlockMF32 = 128;
inline int block_rows(Dtype d) { return d == Dtype::BF16 ? kBlockMBf16 : kBlockMF32; }

// Everything the backward kernels need: the forward's parameters (q, k, v,
// segment ids, masks and sizes; out/lse/run_map of FwdParams unused) plus
// the forward outputs, the upstream gradient and the gradient outputs.
struct BwdParams {
  FwdParams f;
  const void* out;      // [B, Lq, H, D], the input dtype
  const float* lse;     // [B, H, Lq]
  const void* dout;     // [B, Lq, H, D], the input dtype
  float* dq;            // [B, Lq, H, D]
  float* dk;            // [B, S, H, D]
  float* dv;            // [B, S, H, D]
  float* delta;         // [B, H, Lq]
  // With key splits (f.key_splits > 1): the splits' addends to dq,
  // [key_splits][B, Lq, H, D]; a sum kernel writes dq.  Otherwise nullptr.
  float* dq_part;
  int32_t n_ktiles;     // key tiles (bwd_key_block keys) per (batch, head) of the dK/dV kernel
  int32_t n_wg_kv;      // workgroups of the dK/dV kernel
};

// Keys per workgroup of the dK/dV kernel (bf16: 8 waves x 32 keys; float32:
// 4 waves x 32 keys).
constexpr int kBlockNBwd = 256;
constexpr int kBlockNBwdF32 = 128;
inline int bwd_key_block(Dtype d) { return d == Dtype::BF16 ? kBlockNBwd : kBlockNBwdF32; }

// Enqueue the backward on `stream`; same conventions as launch_fwd.
int launch_bwd(const BwdParams& p, Dtype dtype, int head_dim, void* stream, char* err,
               int errlen);

// The float32 dq and dK/dV kernels (blockwise_bwd_f32.hip), enqueued by
// launch_bwd after the delta kernel.
void launch_bwd_f32_main(const BwdParams& p, int head_dim, void* stream);

// The blockwise feedforward: y = max(0, x W1 + b1) W2 + b2, chunk by chunk.
struct FfnParams {
  const void* x;     // [batch, seq, hidden] bf16
  const void* w1;    // [hidden, ffn] bf16
  const void* b1;    // [ffn] bf16
  const void* w2;    // [ffn, hidden] bf16
  const void* b2;    // [hidden] bf16
  void* y;           // [batch, seq, hidden] bf16
  void* workspace;   // [chunk, ffn] bf16: one chunk's hidden activations
  int64_t batch, seq, hidden, ffn, chunk;
};

// Enqueue the feedforward on `stream`; same conventions as launch_fwd.
int launch_ffn(const FfnParams& p, void* stream, char* err, int errlen);

// The no-allocation forward's scratch: a file-scope device array of the
// forward's source, one copy per GPU, held until the process ends.
constexpr int64_t kFwdScratchBytes = 64LL << 20;

// Device address of the current device's scratch array (looked up once per
// device with hipGetSymbolAddress, then cached).  Returns 0 on success,
// otherwise writes a message into err and returns nonzero.
int fwd_scratch(void** ptr, char* err, int errlen);

// Enqueue the forward on `stream` (a hipStream_t).  Returns 0 on success,
// otherwise writes a message into err (size errlen) and returns nonzero.
int launch_fwd(const FwdParams& p, Dtype dtype, int head_dim, int64_t run_map_bytes,
               void* stream, char* err, int errlen);

}  // namespace ra
