// Blockwise feedforward of the Blockwise Transformer on MI355X:
// y = max(0, x W1 + b1) W2 + b2 ("Ring Attention with Blockwise Transformers
// for Near-Infinite Context", section 三 "核心公式"), computed one sequence
// chunk at a time ("Blockwise Feedforward网络详解", sections "核心技术原理"
// and "技术实现细节"), so the hidden activations of only one chunk
// (chunk x ffn values) exist at any time, in a caller-provided workspace.
//
// Both products are plain dense GEMMs on the bf16 matrix cores with fp32
// accumulation, run by hipBLASLt with fused epilogues: bias + ReLU into the
// bf16 workspace for the first, bias into y for the second.  Row-major
// operands are passed as their column-major transposes, so no data moves:
//   H^T [ffn x chunk]    = W1^T [ffn x hidden] . X^T [hidden x chunk]
//   Y^T [hidden x chunk] = W2^T [hidden x ffn] . H^T [ffn x chunk]
// with each bias indexed by the row of the column-major result.

#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>
#include <stdint.h>

#include <cstdio>
#include <map>
#include <mutex>
#include <tuple>

#include "ra_internal.h"

namespace ra {
namespace {

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;
// Algorithm chosen by the heuristic for (device, m, n, k, epilogue).
std::map<std::tuple<int, int64_t, int64_t, int64_t, int>, hipblasLtMatmulAlgo_t> g_algos;

const char* status_name(hipblasStatus_t s) {
  switch (s) {
    case HIPBLAS_STATUS_SUCCESS: return "success";
    case HIPBLAS_STATUS_NOT_INITIALIZED: return "not initialized";
    case HIPBLAS_STATUS_ALLOC_FAILED: return "allocation failed";
    case HIPBLAS_STATUS_INVALID_VALUE: return "invalid value";
    case HIPBLAS_STATUS_ARCH_MISMATCH: return "arch mismatch";
    case HIPBLAS_STATUS_EXECUTION_FAILED: return "execution failed";
    case HIPBLAS_STATUS_NOT_SUPPORTED: return "not supported";
    default: return "error";
  }
}

// RAII holders for the per-call descriptors.
struct Desc {
  hipblasLtMatmulDesc_t d = nullptr;
  ~Desc() { if (d) hipblasLtMatmulDescDestroy(d); }
};
struct Layout {
  hipblasLtMatrixLayout_t l = nullptr;
  ~Layout() { if (l) hipblasLtMatrixLayoutDestroy(l); }
};
struct Pref {
  hipblasLtMatmulPreference_t p = nullptr;
  ~Pref() { if (p) hipblasLtMatmulPreferenceDestroy(p); }
};

#define RA_LT(call)                                                                    \
  do {                                                                                 \
    hipblasStatus_t st_ = (call);                                                      \
    if (st_ != HIPBLAS_STATUS_SUCCESS) {                                               \
      std::snprintf(err, errlen, "hipBLASLt %s: %s", #call, status_name(st_));         \
      return 1;                                                                        \
    }                                                                                  \
  } while (0)

int handle_for(int dev, hipblasLtHandle_t* h, char* err, int errlen) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_handles.find(dev);
  if (it != g_handles.end()) {
    *h = it->second;
    return 0;
  }
  hipblasLtHandle_t nh = nullptr;
  RA_LT(hipblasLtCreate(&nh));
  g_handles[dev] = nh;
  *h = nh;
  return 0;
}

// D [m x n, column-major, ld m] = A [m x k, ld m] . B [k x n, ld k] + bias[m]
// (then ReLU when `relu`), bf16 in and out, fp32 accumulation.
int gemm_bias(hipblasLtHandle_t h, int dev, int64_t m, int64_t n, int64_t k, const void* A,
              const void* B, void* D, const void* bias, bool relu, hipStream_t stream, char* err,
              int errlen) {
  Desc desc;
  RA_LT(hipblasLtMatmulDescCreate(&desc.d, HIPBLAS_COMPUTE_32F, HIP_R_32F));
  const hipblasOperation_t op = HIPBLAS_OP_N;
  RA_LT(hipblasLtMatmulDescSetAttribute(desc.d, HIPBLASLT_MATMUL_DESC_TRANSA, &op, sizeof(op)));
  RA_LT(hipblasLtMatmulDescSetAttribute(desc.d, HIPBLASLT_MATMUL_DESC_TRANSB, &op, sizeof(op)));
  const hipblasLtEpilogue_t epi = relu ? HIPBLASLT_EPILOGUE_RELU_BIAS : HIPBLASLT_EPILOGUE_BIAS;
  RA_LT(hipblasLtMatmulDescSetAttribute(desc.d, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi)));
  RA_LT(hipblasLtMatmulDescSetAttribute(desc.d, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias,
                                        sizeof(bias)));
  const hipDataType bias_type = HIP_R_16BF;
  RA_LT(hipblasLtMatmulDescSetAttribute(desc.d, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bias_type,
                                        sizeof(bias_type)));
  Layout la, lb, ld;
  RA_LT(hipblasLtMatrixLayoutCreate(&la.l, HIP_R_16BF, (uint64_t)m, (uint64_t)k, m));
  RA_LT(hipblasLtMatrixLayoutCreate(&lb.l, HIP_R_16BF, (uint64_t)k, (uint64_t)n, k));
  RA_LT(hipblasLtMatrixLayoutCreate(&ld.l, HIP_R_16BF, (uint64_t)m, (uint64_t)n, m));

  hipblasLtMatmulAlgo_t algo;
  const auto key = std::make_tuple(dev, m, n, k, relu ? 1 : 0);
  bool have = false;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_algos.find(key);
    if (it != g_algos.end()) {
      algo = it->second;
      have = true;
    }
  }
  if (!have) {
    Pref pref;
    RA_LT(hipblasLtMatmulPreferenceCreate(&pref.p));
    const uint64_t ws = 0;  // algorithms that need no library workspace
    RA_LT(hipblasLtMatmulPreferenceSetAttribute(pref.p, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                &ws, sizeof(ws)));
    hipblasLtMatmulHeuristicResult_t res[1];
    int n_res = 0;
    RA_LT(hipblasLtMatmulAlgoGetHeuristic(h, desc.d, la.l, lb.l, ld.l, ld.l, pref.p, 1, res,
                                          &n_res));
    if (n_res < 1) {
      std::snprintf(err, errlen, "hipBLASLt found no algorithm for %lld x %lld x %lld",
                    (long long)m, (long long)n, (long long)k);
      return 1;
    }
    algo = res[0].algo;
    std::lock_guard<std::mutex> lk(g_mu);
    g_algos[key] = algo;
  }
  const float alpha = 1.f, beta = 0.f;
  RA_LT(hipblasLtMatmul(h, desc.d, &alpha, A, la.l, B, lb.l, &beta, D, ld.l, D, ld.l, &algo,
                        nullptr, 0, stream));
  return 0;
}

}  // namespace

int launch_ffn(const FfnParams& p, void* stream, char* err, int errlen) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    std::snprintf(err, errlen, "hipGetDevice failed");
    return 1;
  }
  hipblasLtHandle_t h = nullptr;
  if (handle_for(dev, &h, err, errlen) != 0) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t H = p.hidden, F = p.ffn, C = p.chunk;
  const __bf16* x = static_cast<const __bf16*>(p.x);
  __bf16* y = static_cast<__bf16*>(p.y);
  for (int64_t b = 0; b < p.batch; ++b) {
    for (int64_t c0 = 0; c0 < p.seq; c0 += C) {
      const int64_t row = b * p.seq + c0;
      // H^T = relu(W1^T X^T + b1) into the chunk workspace
      if (gemm_bias(h, dev, F, C, H, p.w1, x + row * H, p.workspace, p.b1, true, s, err, errlen))
        return 1;
      // Y^T = W2^T H^T + b2 into the chunk's rows of y
      if (gemm_bias(h, dev, H, C, F, p.w2, p.workspace, y + row * H, p.b2, false, s, err, errlen))
        return 1;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    std::snprintf(err, errlen, "feedforward launch failed: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

}  // namespace ra
