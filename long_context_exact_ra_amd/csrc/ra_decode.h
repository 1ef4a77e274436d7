// Internal interface of the decoding step between the host-side C ABI
// (ra_host.cpp) and its kernels (blockwise_decode.hip).  Kept apart from
// ra_internal.h, which the forward kernel's source includes.  Not
// installed, not part of the ABI.
#pragma once

#include <stdint.h>

#include "ra_internal.h"

namespace ra {

// One decoding step over a KV cache (blockwise_decode.hip).
struct DecParams {
  const void* q;        // [B, n_new, H, D], the input dtype
  const void* k;        // [B, cache_rows, H, D]
  const void* v;        // [B, cache_rows, H, D]
  void* out;            // [B, n_new, H, D], the input dtype
  float* lse;           // [B, H, n_new]
  // With key_splits > 1: [key_splits][B][H][n_new][D] numerators and
  // [key_splits][B][H][n_new][2] (kept max, base 2; denominator).
  float* part_o;
  float* part_ml;
  int64_t cache_idx;    // position of the first new token
  int64_t cache_rows;   // rows of the cache tensors
  int64_t n_keys;       // cache rows read: cache_idx + n_new
  int64_t split_keys;   // keys per split
  int32_t batch;
  int32_t heads;
  int32_t n_new;
  int32_t key_splits;
  int32_t q_groups;     // workgroups per (batch, head, split) along the queries
  float scale_log2;     // log2(e) / sqrt(head_dim)
};

// Enqueue a decoding step (nq: queries per workgroup: 32 or 128 for bf16,
// on the matrix cores; 1, 2, 4 or 8 for float32, on the vector ALUs); same
// conventions as launch_fwd.
int launch_decode(const DecParams& p, Dtype dtype, int head_dim, int nq, void* stream, char* err,
                  int errlen);

}  // namespace ra
