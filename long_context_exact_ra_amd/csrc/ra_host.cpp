// Host side of the C ABI declared in include/ra_attn.h: argument
// validation, the ring-step planner and error reporting.  Plain C++; device
// work is delegated to ra::launch_fwd (blockwise_fwd.hip), ra::launch_bwd
// (blockwise_bwd.hip) and ra::launch_ffn (blockwise_ffn.hip).

#include "ra_attn.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "ra_decode.h"
#include "ra_internal.h"
#include "ra_walk.h"

namespace {

thread_local char g_err[512];

ra_status_t fail(ra_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_err[0] = '\0'; }

constexpr int64_t kInt32Max = 2147483647LL;

// The kernels move tensor rows in 16-byte vectors (loads, buffer-to-LDS DMA,
// stores) and ids, lse and delta as 4-byte words.
inline bool aligned(const void* ptr, uintptr_t bytes) {
  return (reinterpret_cast<uintptr_t>(ptr) & (bytes - 1)) == 0;
}

// Checks shared by the forward and the planner.  `kernel_chunks` adds the
// kernels' requirement that chunks are multiples of their 32-row sub-tiles.
ra_status_t check_ring(int64_t causal_block_size, int64_t q_chunk, int64_t k_chunk,
                       int64_t seq_q, int32_t ring_size, int32_t ring_index,
                       bool kernel_chunks) {
  if (ring_size < 1) return fail(RA_E_INVALID, "ring_size must be >= 1 (got %d)", ring_size);
  if (ring_index < 0 || ring_index >= ring_size)
    return fail(RA_E_INVALID, "ring_index %d outside [0, %d)", ring_index, ring_size);
  if (causal_block_size < 0)
    return fail(RA_E_INVALID, "causal_block_size must be >= 0 (got %lld)",
                (long long)causal_block_size);
  if (seq_q < 0) return fail(RA_E_INVALID, "seq_q must be >= 0 (got %lld)", (long long)seq_q);
  if (q_chunk <= 0 || k_chunk <= 0)
    return fail(RA_E_INVALID, "q_chunk and k_chunk must be positive (got %lld, %lld)",
                (long long)q_chunk, (long long)k_chunk);
  // The blockwise scheme splits a block with integer division
  // ("1. 分块处理机制"): the chunk sizes have to divide the block length.
  if (seq_q % q_chunk != 0 || seq_q % k_chunk != 0)
    return fail(RA_E_INVALID, "q_chunk %lld and k_chunk %lld must divide seq_q %lld",
                (long long)q_chunk, (long long)k_chunk, (long long)seq_q);
  if (seq_q * (int64_t)ring_size > kInt32Max)
    return fail(kernel_chunks ? RA_E_UNSUPPORTED : RA_E_INVALID,
                "ring_size * seq_q = %lld exceeds 2^31 - 1 positions",
                (long long)(seq_q * (int64_t)ring_size));
  if (kernel_chunks && (q_chunk % 32 != 0 || k_chunk % 32 != 0))
    return fail(RA_E_UNSUPPORTED, "q_chunk %lld and k_chunk %lld must be multiples of 32",
                (long long)q_chunk, (long long)k_chunk);
  return RA_OK;
}

// The chunk-pair run test of "3. 因果注意力掩码支持": the pair runs iff it
// holds at least one causally visible pair, i.e. the causal block of the
// pair's last query is not before the causal block of its first key.
inline bool pair_runs(int64_t c, int64_t last_q, int64_t first_k) {
  return c == 0 || last_q / c >= first_k / c;
}

}  // namespace

extern "C" {

const char* ra_last_error(void) { return g_err; }

// "+<id>": the first 16 hex digits of the SHA-256 of the device sources the
// library was built from (set by the build script), so a measurement can be
// tied to the exact kernel that produced it.
#ifndef RA_BUILD_ID
#define RA_BUILD_ID "unknown"
#endif
const char* ra_version(void) { return "0.1.0+" RA_BUILD_ID; }

ra_status_t ra_blockwise_plan_placed(int64_t causal_block_size, int64_t q_chunk,
                                     int64_t k_chunk, int64_t seq_q, int32_t ring_size,
                                     int32_t ring_index, ra_placement_t placement,
                                     int32_t* kv_block_of_step, uint8_t* run_bits,
                                     int64_t* n_run_chunk_pairs) {
  clear_error();
  ra_status_t st = check_ring(causal_block_size, q_chunk, k_chunk, seq_q, ring_size,
                              ring_index, false);
  if (st != RA_OK) return st;
  if (placement != RA_PLACE_CONTIGUOUS && placement != RA_PLACE_STRIPED)
    return fail(RA_E_INVALID, "unknown placement %d", (int)placement);
  if (kv_block_of_step == nullptr) return fail(RA_E_INVALID, "kv_block_of_step is NULL");
  const bool striped = placement == RA_PLACE_STRIPED;
  const int64_t nq = seq_q / q_chunk, nk = seq_q / k_chunk, N = ring_size;
  int64_t n_run = 0;
  for (int32_t t = 0; t < ring_size; ++t) {
    // Ring order: at outer step t the device uses block (index - t) mod N.
    const int32_t kb = ((ring_index - t) % ring_size + ring_size) % ring_size;
    kv_block_of_step[t] = kb;
    for (int64_t a = 0; a < nq; ++a) {
      // Position of the chunk's last query row, (a + 1) * q_chunk - 1.
      const int64_t i_last = (a + 1) * q_chunk - 1;
      const int64_t last_q = striped ? i_last * N + ring_index : ring_index * seq_q + i_last;
      for (int64_t b = 0; b < nk; ++b) {
        // Position of the chunk's first key, row b * k_chunk of block kb.
        const int64_t j0 = b * k_chunk;
        const int64_t first_k = striped ? j0 * N + kb : (int64_t)kb * seq_q + j0;
        const bool run = pair_runs(causal_block_size, last_q, first_k);
        n_run += run;
        if (run_bits) run_bits[((int64_t)t * nq + a) * nk + b] = run ? 1 : 0;
      }
    }
  }
  if (n_run_chunk_pairs) *n_run_chunk_pairs = n_run;
  return RA_OK;
}

ra_status_t ra_blockwise_plan(int64_t causal_block_size, int64_t q_chunk, int64_t k_chunk,
                              int64_t seq_q, int32_t ring_size, int32_t ring_index,
                              int32_t* kv_block_of_step, uint8_t* run_bits,
                              int64_t* n_run_chunk_pairs) {
  return ra_blockwise_plan_placed(causal_block_size, q_chunk, k_chunk, seq_q, ring_size,
                                  ring_index, RA_PLACE_CONTIGUOUS, kv_block_of_step, run_bits,
                                  n_run_chunk_pairs);
}

}  // extern "C"

namespace {

// Validation and derived parameters shared by the forward and the backward.
// Returns RA_OK with `empty` set for a valid call that has nothing to do.
ra_status_t prepare(const void* q, const void* k, const void* v, const int32_t* segment_ids,
                    int64_t causal_block_size, int64_t q_chunk, int64_t k_chunk,
                    int32_t ring_size, int32_t ring_index, ra_placement_t placement,
                    int64_t batch, int64_t seq_q, int64_t heads, int64_t head_dim,
                    ra_dtype_t dtype, ra::FwdParams& p, bool& empty) {
  empty = false;
  if (placement != RA_PLACE_CONTIGUOUS && placement != RA_PLACE_STRIPED)
    return fail(RA_E_INVALID, "unknown placement %d", (int)placement);
  if (batch < 0 || heads < 0)
    return fail(RA_E_INVALID, "batch and heads must be >= 0 (got %lld, %lld)",
                (long long)batch, (long long)heads);
  if (head_dim <= 0) return fail(RA_E_INVALID, "head_dim must be positive");
  ra_status_t st = check_ring(causal_block_size, q_chunk, k_chunk, seq_q, ring_size,
                              ring_index, true);
  if (st != RA_OK) return st;
  // A causal block at least as long as the whole sequence puts every
  // position in block 0: every key is visible, exactly as without a mask.
  const int64_t seq_k = seq_q * ring_size;
  const int64_t causal = causal_block_size >= seq_k ? 0 : causal_block_size;
  // Striped placement: the kernels test visibility on key coordinates
  // (walk::striped_causal), which exist when the causal block divides the
  // ring size or is a multiple of it.
  const ra::walk::StripedCausal sc = ra::walk::striped_causal(causal, ring_size, ring_index);
  const bool striped = placement == RA_PLACE_STRIPED;
  if (striped && !sc.ok)
    return fail(RA_E_UNSUPPORTED,
                "striped placement supports a causal_block_size that divides ring_size or is a "
                "multiple of it (got %lld with ring_size %d)",
                (long long)causal_block_size, ring_size);
  if (dtype != RA_BF16 && dtype != RA_F32)
    return fail(RA_E_UNSUPPORTED, "dtype %d is not supported (RA_BF16, RA_F32)", (int)dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(RA_E_UNSUPPORTED, "head_dim %lld is not supported (64, 128)",
                (long long)head_dim);
  if (batch == 0 || seq_q == 0 || heads == 0) {
    empty = true;
    return RA_OK;
  }
  if (!q || !k || !v) return fail(RA_E_INVALID, "q, k and v must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
    return fail(RA_E_INVALID, "q, k and v must be 16-byte aligned");
  if (segment_ids && !aligned(segment_ids, 4))
    return fail(RA_E_INVALID, "segment_ids must be 4-byte aligned");
  if (heads * head_dim > (1LL << 24))
    return fail(RA_E_UNSUPPORTED, "heads * head_dim = %lld exceeds 2^24",
                (long long)(heads * head_dim));
  const ra::Dtype dt = dtype == RA_BF16 ? ra::Dtype::BF16 : ra::Dtype::F32;
  const int64_t bm = ra::block_rows(dt);
  const int64_t n_qtiles = (seq_q + bm - 1) / bm;
  const int64_t n_wg = batch * heads * n_qtiles;
  if (n_wg > kInt32Max || batch > kInt32Max)
    return fail(RA_E_UNSUPPORTED, "grid of %lld workgroups is too large", (long long)n_wg);

  p = ra::FwdParams{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.seg = segment_ids;
  p.causal = striped ? sc.causal : causal;
  p.striped = striped ? 1 : 0;
  p.stripe_hi = striped ? sc.stripe_hi : ring_index + 1;
  p.seq_q = (int32_t)seq_q;
  p.seq_k = (int32_t)seq_k;
  p.q_chunk = (int32_t)q_chunk;
  p.k_chunk = (int32_t)k_chunk;
  p.batch = (int32_t)batch;
  p.heads = (int32_t)heads;
  p.ring_size = ring_size;
  p.ring_index = ring_index;
  p.n_qtiles = (int32_t)n_qtiles;
  p.n_wg = (int32_t)n_wg;
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
  p.key_splits = 1;
  return RA_OK;
}

// Largest number of key splits a call accepts.
constexpr int32_t kMaxKeySplits = 64;

// The walk terms of a prepared call (the kernels build the same from the
// parameters they receive).
ra::walk::Share share_of(const ra::FwdParams& p, int64_t bm, int64_t tn) {
  return ra::walk::Share{p.seq_q,      p.ring_size, p.ring_index, p.causal,    p.striped != 0,
                         (int32_t)bm, (int32_t)tn, p.stripe_hi};
}

// Workgroups per (batch, head) of a launch with P key splits: the runs of
// every query tile's walk, counted by the same functions the kernels map
// workgroups with (ra_walk.h).
int64_t split_wgs_host(int32_t P, const ra::FwdParams& p, int64_t bm, int64_t tn) {
  return ra::walk::split_wgs(share_of(p, bm, tn), P);
}

int64_t split_workspace_bytes(int64_t batch, int64_t seq_q, int64_t heads, int64_t head_dim,
                              int32_t key_splits) {
  if (key_splits <= 1 || batch <= 0 || seq_q <= 0 || heads <= 0 || head_dim <= 0) return 0;
  return (int64_t)key_splits * batch * heads * seq_q * (head_dim + 2) * 4;
}

}  // namespace

extern "C" {

ra_status_t ra_blockwise_attn_fwd_split(const void* q, const void* k, const void* v,
                                        const int32_t* segment_ids, int64_t causal_block_size,
                                        int64_t q_chunk, int64_t k_chunk, int32_t ring_size,
                                        int32_t ring_index, ra_placement_t placement,
                                        int64_t batch, int64_t seq_q, int64_t heads,
                                        int64_t head_dim, ra_dtype_t dtype, void* out,
                                        float* lse, uint8_t* run_map, int32_t key_splits,
                                        void* workspace, int64_t workspace_bytes,
                                        void* stream) {
  clear_error();
  if (key_splits < 1 || key_splits > kMaxKeySplits)
    return fail(RA_E_INVALID, "key_splits %d outside [1, %d]", key_splits, kMaxKeySplits);
  ra::FwdParams p;
  bool empty = false;
  ra_status_t st = prepare(q, k, v, segment_ids, causal_block_size, q_chunk, k_chunk, ring_size,
                           ring_index, placement, batch, seq_q, heads, head_dim, dtype, p, empty);
  if (st != RA_OK || empty) return st;
  if (!out || !lse) return fail(RA_E_INVALID, "out and lse must be non-NULL");
  if (!aligned(out, 16) || !aligned(lse, 4))
    return fail(RA_E_INVALID, "out must be 16-byte and lse 4-byte aligned");
  if (key_splits > 1) {
    const int64_t need = split_workspace_bytes(batch, seq_q, heads, head_dim, key_splits);
    if (!workspace) return fail(RA_E_INVALID, "key_splits %d needs a workspace", key_splits);
    if (!aligned(workspace, 16)) return fail(RA_E_INVALID, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
      return fail(RA_E_INVALID, "workspace of %lld bytes is smaller than the %lld required",
                  (long long)workspace_bytes, (long long)need);
    // One workgroup per run of every query tile's walk (heavier walks are
    // cut into more runs), none idle.
    const int64_t bm = ra::block_rows(dtype == RA_BF16 ? ra::Dtype::BF16 : ra::Dtype::F32);
    const int64_t wgs = split_wgs_host(key_splits, p, bm, dtype == RA_BF16 ? 64 : 32);
    const int64_t n_wg = batch * heads * wgs;
    if (n_wg > kInt32Max || wgs > kInt32Max)
      return fail(RA_E_UNSUPPORTED, "grid of %lld workgroups is too large", (long long)n_wg);
    p.n_wg = (int32_t)n_wg;
    p.split_wgs = (int32_t)wgs;
    p.key_splits = key_splits;
    p.part_o = static_cast<float*>(workspace);
    p.part_ml = p.part_o + (int64_t)key_splits * batch * heads * seq_q * head_dim;
  }
  p.out = out;
  p.lse = lse;
  p.run_map = run_map;
  const int64_t map_bytes =
      run_map ? (int64_t)ring_size * (seq_q / q_chunk) * (seq_q / k_chunk) : 0;
  const ra::Dtype dt = dtype == RA_BF16 ? ra::Dtype::BF16 : ra::Dtype::F32;
  char err[256];
  if (ra::launch_fwd(p, dt, (int)head_dim, map_bytes, stream, err, (int)sizeof(err)) != 0)
    return fail(RA_E_HIP, "%s", err);
  return RA_OK;
}

int64_t ra_blockwise_attn_fwd_split_workspace_bytes(int64_t batch, int64_t seq_q, int64_t heads,
                                                     int64_t head_dim, int32_t key_splits) {
  return split_workspace_bytes(batch, seq_q, heads, head_dim, key_splits);
}

ra_status_t ra_blockwise_attn_fwd_split_noalloc(
    const void* q, const void* k, const void* v, const int32_t* segment_ids,
    int64_t causal_block_size, int64_t q_chunk, int64_t k_chunk, int32_t ring_size,
    int32_t ring_index, ra_placement_t placement, int64_t batch, int64_t seq_q, int64_t heads,
    int64_t head_dim, ra_dtype_t dtype, void* out, float* lse, uint8_t* run_map,
    int32_t key_splits, void* stream) {
  clear_error();
  // The partials live in the library's fixed scratch; larger calls are
  // refused before anything touches the GPU.
  const int64_t need = split_workspace_bytes(batch, seq_q, heads, head_dim, key_splits);
  if (need > ra::kFwdScratchBytes)
    return fail(RA_E_UNSUPPORTED,
                "key_splits %d over batch %lld x heads %lld x seq_q %lld needs %lld bytes of "
                "split partials; the no-allocation forward's scratch holds %lld",
                key_splits, (long long)batch, (long long)heads, (long long)seq_q,
                (long long)need, (long long)ra::kFwdScratchBytes);
  void* scratch = nullptr;
  char err[256];
  if (ra::fwd_scratch(&scratch, err, (int)sizeof(err)) != 0) return fail(RA_E_HIP, "%s", err);
  return ra_blockwise_attn_fwd_split(q, k, v, segment_ids, causal_block_size, q_chunk, k_chunk,
                                     ring_size, ring_index, placement, batch, seq_q, heads,
                                     head_dim, dtype, out, lse, run_map, key_splits, scratch,
                                     ra::kFwdScratchBytes, stream);
}

int32_t ra_blockwise_attn_fwd_key_splits(int64_t batch, int64_t seq_q, int64_t heads,
                                         ra_dtype_t dtype, int64_t causal_block_size,
                                         int32_t ring_size, int32_t ring_index,
                                         ra_placement_t placement, int32_t compute_units) {
  if (batch <= 0 || seq_q <= 0 || heads <= 0 || compute_units <= 0 || ring_size < 1 ||
      ring_index < 0 || ring_index >= ring_size || (dtype != RA_BF16 && dtype != RA_F32) ||
      (placement != RA_PLACE_CONTIGUOUS && placement != RA_PLACE_STRIPED))
    return 1;
  const int64_t bm = ra::block_rows(dtype == RA_BF16 ? ra::Dtype::BF16 : ra::Dtype::F32);
  const int64_t n_qtiles = (seq_q + bm - 1) / bm;
  const int64_t n_wg = batch * heads * n_qtiles;
  if (n_wg >= compute_units) return 1;
  // The largest P whose runs (every query tile's walk cut into runs of
  // about the longest walk's n_max / P tiles, one workgroup each) fit one
  // workgroup per compute unit -- a second dispatch round costs more than
  // shorter runs save --
  // with at least 4 tiles per run of the longest walk (fewer did not pay in
  // timings of the small causal share).
  const int64_t seq_k = seq_q * ring_size;
  const bool striped = placement == RA_PLACE_STRIPED;
  const int64_t c = causal_block_size >= seq_k ? 0 : causal_block_size;
  const ra::walk::StripedCausal sc = ra::walk::striped_causal(c, ring_size, ring_index);
  if (striped && !sc.ok) return 1;  // such calls are refused anyway
  ra::FwdParams p{};
  p.seq_q = (int32_t)seq_q;
  p.ring_size = ring_size;
  p.ring_index = ring_index;
  p.causal = striped ? sc.causal : c;
  p.striped = striped ? 1 : 0;
  p.stripe_hi = striped ? sc.stripe_hi : ring_index + 1;
  const int64_t tn = dtype == RA_BF16 ? 64 : 32;
  const int64_t n_max64 = ra::walk::qtile_walk(share_of(p, bm, 64), (int32_t)n_qtiles - 1);
  int64_t best = 1;
  for (int32_t P = 2; P <= std::min<int64_t>(kMaxKeySplits, n_max64 / 4); ++P) {
    const int64_t wgs = split_wgs_host(P, p, bm, tn);
    if (batch * heads * wgs > compute_units) break;
    best = P;
  }
  return (int32_t)best;
}

ra_status_t ra_blockwise_attn_fwd_placed(const void* q, const void* k, const void* v,
                                         const int32_t* segment_ids, int64_t causal_block_size,
                                         int64_t q_chunk, int64_t k_chunk, int32_t ring_size,
                                         int32_t ring_index, ra_placement_t placement,
                                         int64_t batch, int64_t seq_q, int64_t heads,
                                         int64_t head_dim, ra_dtype_t dtype, void* out,
                                         float* lse, uint8_t* run_map, void* stream) {
  return ra_blockwise_attn_fwd_split(q, k, v, segment_ids, causal_block_size, q_chunk, k_chunk,
                                     ring_size, ring_index, placement, batch, seq_q, heads,
                                     head_dim, dtype, out, lse, run_map, 1, nullptr, 0, stream);
}

ra_status_t ra_blockwise_attn_fwd_ex(const void* q, const void* k, const void* v,
                                     const int32_t* segment_ids, int64_t causal_block_size,
                                     int64_t q_chunk, int64_t k_chunk, int32_t ring_size,
                                     int32_t ring_index, int64_t batch, int64_t seq_q,
                                     int64_t heads, int64_t head_dim, ra_dtype_t dtype,
                                     void* out, float* lse, uint8_t* run_map, void* stream) {
  return ra_blockwise_attn_fwd_placed(q, k, v, segment_ids, causal_block_size, q_chunk, k_chunk,
                                      ring_size, ring_index, RA_PLACE_CONTIGUOUS, batch, seq_q,
                                      heads, head_dim, dtype, out, lse, run_map, stream);
}

ra_status_t ra_blockwise_attn_bwd_split(const void* q, const void* k, const void* v,
                                        const int32_t* segment_ids, int64_t causal_block_size,
                                        int64_t q_chunk, int64_t k_chunk, int32_t ring_size,
                                        int32_t ring_index, ra_placement_t placement,
                                        int64_t batch, int64_t seq_q, int64_t heads,
                                        int64_t head_dim, ra_dtype_t dtype, const void* out,
                                        const float* lse, const void* dout, float* dq,
                                        float* dk, float* dv, float* delta, int32_t key_splits,
                                        void* workspace, int64_t workspace_bytes,
                                        void* stream) {
  clear_error();
  if (key_splits < 1 || key_splits > kMaxKeySplits)
    return fail(RA_E_INVALID, "key_splits %d outside [1, %d]", key_splits, kMaxKeySplits);
  ra::BwdParams bp{};
  bool empty = false;
  ra_status_t st = prepare(q, k, v, segment_ids, causal_block_size, q_chunk, k_chunk, ring_size,
                           ring_index, placement, batch, seq_q, heads, head_dim, dtype, bp.f,
                           empty);
  if (st != RA_OK || empty) return st;
  const ra::Dtype dt = dtype == RA_BF16 ? ra::Dtype::BF16 : ra::Dtype::F32;
  if (!out || !lse || !dout || !dq || !dk || !dv || !delta)
    return fail(RA_E_INVALID, "out, lse, dout, dq, dk, dv and delta must be non-NULL");
  if (!aligned(out, 16) || !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) ||
      !aligned(dv, 16) || !aligned(lse, 4) || !aligned(delta, 4))
    return fail(RA_E_INVALID,
                "out, dout, dq, dk and dv must be 16-byte aligned, lse and delta 4-byte");
  if (key_splits > 1) {
    const int64_t need = ra_blockwise_attn_bwd_split_workspace_bytes(batch, seq_q, heads,
                                                                      head_dim, key_splits);
    if (!workspace) return fail(RA_E_INVALID, "key_splits %d needs a workspace", key_splits);
    if (!aligned(workspace, 16)) return fail(RA_E_INVALID, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
      return fail(RA_E_INVALID, "workspace of %lld bytes is smaller than the %lld required",
                  (long long)workspace_bytes, (long long)need);
    // The dq kernel: one workgroup per run of every query tile's walk, as in
    // the forward (and with the forward's tiles of the dtype).
    const int64_t wgs =
        split_wgs_host(key_splits, bp.f, ra::block_rows(dt), dt == ra::Dtype::BF16 ? 64 : 32);
    const int64_t n_wg = batch * heads * wgs;
    if (n_wg > kInt32Max || wgs > kInt32Max)
      return fail(RA_E_UNSUPPORTED, "grid of %lld workgroups is too large", (long long)n_wg);
    bp.f.n_wg = (int32_t)n_wg;
    bp.f.split_wgs = (int32_t)wgs;
    bp.f.key_splits = key_splits;
    bp.dq_part = static_cast<float*>(workspace);
  }
  bp.out = out;
  bp.lse = lse;
  bp.dout = dout;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  bp.delta = delta;
  const int64_t n_ktiles = ((int64_t)bp.f.seq_k + ra::bwd_key_block(dt) - 1) / ra::bwd_key_block(dt);
  const int64_t n_wg_kv = batch * heads * n_ktiles;
  if (n_wg_kv > kInt32Max)
    return fail(RA_E_UNSUPPORTED, "grid of %lld workgroups is too large", (long long)n_wg_kv);
  bp.n_ktiles = (int32_t)n_ktiles;
  bp.n_wg_kv = (int32_t)n_wg_kv;
  char err[256];
  if (ra::launch_bwd(bp, dt, (int)head_dim, stream, err, (int)sizeof(err)) != 0)
    return fail(RA_E_HIP, "%s", err);
  return RA_OK;
}

int64_t ra_blockwise_attn_bwd_split_workspace_bytes(int64_t batch, int64_t seq_q, int64_t heads,
                                                     int64_t head_dim, int32_t key_splits) {
  if (key_splits <= 1 || batch <= 0 || seq_q <= 0 || heads <= 0 || head_dim <= 0) return 0;
  return (int64_t)key_splits * batch * seq_q * heads * head_dim * 4;
}

ra_status_t ra_blockwise_attn_bwd_placed(const void* q, const void* k, const void* v,
                                         const int32_t* segment_ids, int64_t causal_block_size,
                                         int64_t q_chunk, int64_t k_chunk, int32_t ring_size,
                                         int32_t ring_index, ra_placement_t placement,
                                         int64_t batch, int64_t seq_q, int64_t heads,
                                         int64_t head_dim, ra_dtype_t dtype, const void* out,
                                         const float* lse, const void* dout, float* dq,
                                         float* dk, float* dv, float* delta, void* stream) {
  return ra_blockwise_attn_bwd_split(q, k, v, segment_ids, causal_block_size, q_chunk, k_chunk,
                                     ring_size, ring_index, placement, batch, seq_q, heads,
                                     head_dim, dtype, out, lse, dout, dq, dk, dv, delta, 1,
                                     nullptr, 0, stream);
}

ra_status_t ra_blockwise_attn_bwd(const void* q, const void* k, const void* v,
                                  const int32_t* segment_ids, int64_t causal_block_size,
                                  int64_t q_chunk, int64_t k_chunk, int32_t ring_size,
                                  int32_t ring_index, int64_t batch, int64_t seq_q,
                                  int64_t heads, int64_t head_dim, ra_dtype_t dtype,
                                  const void* out, const float* lse, const void* dout,
                                  float* dq, float* dk, float* dv, float* delta, void* stream) {
  return ra_blockwise_attn_bwd_placed(q, k, v, segment_ids, causal_block_size, q_chunk, k_chunk,
                                      ring_size, ring_index, RA_PLACE_CONTIGUOUS, batch, seq_q,
                                      heads, head_dim, dtype, out, lse, dout, dq, dk, dv, delta,
                                      stream);
}

int64_t ra_blockwise_ffn_workspace_bytes(int64_t chunk_size, int64_t ffn_hidden) {
  if (chunk_size <= 0 || ffn_hidden <= 0) return 0;
  return chunk_size * ffn_hidden * 2;
}

ra_status_t ra_blockwise_ffn(const void* x, const void* w1, const void* b1, const void* w2,
                             const void* b2, int64_t batch, int64_t seq, int64_t hidden,
                             int64_t ffn_hidden, int64_t chunk_size, ra_dtype_t dtype, void* y,
                             void* workspace, int64_t workspace_bytes, void* stream) {
  clear_error();
  if (batch < 0 || seq < 0)
    return fail(RA_E_INVALID, "batch and seq must be >= 0 (got %lld, %lld)", (long long)batch,
                (long long)seq);
  if (hidden <= 0 || ffn_hidden <= 0)
    return fail(RA_E_INVALID, "hidden and ffn_hidden must be positive (got %lld, %lld)",
                (long long)hidden, (long long)ffn_hidden);
  if (chunk_size <= 0) return fail(RA_E_INVALID, "chunk_size must be positive");
  // The sequence is cut with an exact reshape into chunks.
  if (seq % chunk_size != 0)
    return fail(RA_E_INVALID, "chunk_size %lld must divide seq %lld", (long long)chunk_size,
                (long long)seq);
  if (dtype != RA_BF16)
    return fail(RA_E_UNSUPPORTED, "the feedforward takes bf16 inputs only");
  // The GEMM kernel moves rows in 16-byte vectors and addresses each operand
  // with 32-bit byte offsets.
  if (hidden % 8 != 0 || ffn_hidden % 8 != 0)
    return fail(RA_E_UNSUPPORTED, "hidden %lld and ffn_hidden %lld must be multiples of 8",
                (long long)hidden, (long long)ffn_hidden);
  if (hidden * ffn_hidden * 2 > 4294967295LL || chunk_size * hidden * 2 > 4294967295LL ||
      chunk_size * ffn_hidden * 2 > 4294967295LL)
    return fail(RA_E_UNSUPPORTED, "an operand of the feedforward exceeds 4 GiB");
  if (batch == 0 || seq == 0) return RA_OK;
  if (!x || !w1 || !b1 || !w2 || !b2 || !y || !workspace)
    return fail(RA_E_INVALID, "x, w1, b1, w2, b2, y and workspace must be non-NULL");
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(y, 16) ||
      !aligned(workspace, 16) || !aligned(b1, 8) || !aligned(b2, 8))
    return fail(RA_E_INVALID,
                "x, w1, w2, y and workspace must be 16-byte aligned, b1 and b2 8-byte aligned");
  const int64_t need = ra_blockwise_ffn_workspace_bytes(chunk_size, ffn_hidden);
  if (workspace_bytes < need)
    return fail(RA_E_INVALID, "workspace of %lld bytes is smaller than the %lld required",
                (long long)workspace_bytes, (long long)need);
  ra::FfnParams p{x, w1, b1, w2, b2, y, workspace, batch, seq, hidden, ffn_hidden, chunk_size};
  char err[256];
  if (ra::launch_ffn(p, stream, err, (int)sizeof(err)) != 0) return fail(RA_E_HIP, "%s", err);
  return RA_OK;
}

}  // extern "C"

namespace {

// Decoding: queries per workgroup.  bf16 steps run on the matrix cores, 32
// queries per workgroup up to 32 new tokens (even one query leaves the step
// bound by HBM), 128 beyond (4 query tiles sharing each key tile); float32
// steps on the vector ALUs, 1, 2, 4 or 8 queries per workgroup (their
// carries in registers).
constexpr int32_t kMaxDecodeSplits = 1024;
constexpr int64_t kMaxDecodeNew = 256;

int decode_nq(int64_t n_new, bool bf16) {
  if (bf16) return n_new <= 32 ? 32 : 128;
  return n_new <= 1 ? 1 : n_new <= 2 ? 2 : n_new <= 4 ? 4 : 8;
}

}  // namespace

extern "C" {

int64_t ra_attn_decode_workspace_bytes(int64_t batch, int64_t n_new, int64_t heads,
                                       int64_t head_dim, int32_t key_splits) {
  if (key_splits <= 1 || batch <= 0 || n_new <= 0 || heads <= 0 || head_dim <= 0) return 0;
  return (int64_t)key_splits * batch * heads * n_new * (head_dim + 2) * 4;
}

int32_t ra_attn_decode_key_splits(int64_t batch, int64_t n_new, int64_t heads, int64_t cache_idx,
                                  int32_t compute_units) {
  if (batch <= 0 || n_new <= 0 || heads <= 0 || cache_idx < 0 || compute_units <= 0) return 1;
  // Shapes no launch could take (the products below would overflow): 1.
  if (batch > kInt32Max || heads > kInt32Max || batch * heads > kInt32Max || n_new > kInt32Max ||
      cache_idx > (1LL << 48))
    return 1;
  const int nq = decode_nq(n_new, true);
  const int64_t per_split = batch * heads * ((n_new + nq - 1) / nq);
  const int64_t n_keys = cache_idx + n_new;
  // About eight workgroups per compute unit (each is 4 waves of modest
  // register use), and at least 1024 keys per split; down to 512 keys per
  // split while the grid would not give every compute unit a workgroup.
  int64_t P = (8LL * compute_units + per_split - 1) / per_split;
  int64_t cap = (n_keys + 1023) / 1024;
  if (per_split * cap < compute_units)
    cap = std::max(cap, std::min<int64_t>((n_keys + 511) / 512,
                                          (compute_units + per_split - 1) / per_split));
  P = std::min<int64_t>(P, cap);
  P = std::min<int64_t>(P, kMaxDecodeSplits);
  return (int32_t)std::max<int64_t>(P, 1);
}

ra_status_t ra_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                           int64_t cache_idx, int64_t cache_rows, int64_t batch, int64_t n_new,
                           int64_t heads, int64_t head_dim, ra_dtype_t dtype, int32_t key_splits,
                           void* workspace, int64_t workspace_bytes, void* out, float* lse,
                           void* stream) {
  clear_error();
  if (batch < 0 || heads < 0 || n_new < 0)
    return fail(RA_E_INVALID, "batch, heads and n_new must be >= 0 (got %lld, %lld, %lld)",
                (long long)batch, (long long)heads, (long long)n_new);
  if (head_dim <= 0) return fail(RA_E_INVALID, "head_dim must be positive");
  if (cache_idx < 0) return fail(RA_E_INVALID, "cache_idx must be >= 0 (got %lld)", (long long)cache_idx);
  // (written so that no sum can overflow: cache_idx and cache_rows may be any int64)
  if (cache_rows < n_new || cache_idx > cache_rows - n_new)
    return fail(RA_E_INVALID, "cache_idx %lld + n_new %lld exceeds the %lld cache rows",
                (long long)cache_idx, (long long)n_new, (long long)cache_rows);
  if (key_splits < 1 || key_splits > kMaxDecodeSplits)
    return fail(RA_E_INVALID, "key_splits %d outside [1, %d]", key_splits, kMaxDecodeSplits);
  if (dtype != RA_BF16 && dtype != RA_F32)
    return fail(RA_E_UNSUPPORTED, "dtype %d is not supported (RA_BF16, RA_F32)", (int)dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(RA_E_UNSUPPORTED, "head_dim %lld is not supported (64, 128)", (long long)head_dim);
  if (n_new > kMaxDecodeNew)
    return fail(RA_E_UNSUPPORTED,
                "n_new %lld exceeds %lld (a longer step is a prefill: use the blockwise forward)",
                (long long)n_new, (long long)kMaxDecodeNew);
  if (heads * head_dim > (1LL << 24))
    return fail(RA_E_UNSUPPORTED, "heads * head_dim = %lld exceeds 2^24",
                (long long)(heads * head_dim));
  if (batch == 0 || heads == 0 || n_new == 0) return RA_OK;
  if (!q || !k_cache || !v_cache || !out || !lse)
    return fail(RA_E_INVALID, "q, k_cache, v_cache, out and lse must be non-NULL");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(lse, 4))
    return fail(RA_E_INVALID, "q, k_cache, v_cache and out must be 16-byte aligned, lse 4-byte");
  const int nq = decode_nq(n_new, dtype == RA_BF16);
  const int64_t q_groups = (n_new + nq - 1) / nq;
  const int64_t n_wg = batch * heads * q_groups * key_splits;
  if (n_wg > kInt32Max || batch * heads * n_new * head_dim / 4 / 256 > kInt32Max)
    return fail(RA_E_UNSUPPORTED, "grid of %lld workgroups is too large", (long long)n_wg);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (key_splits > 1) {
    const int64_t need = ra_attn_decode_workspace_bytes(batch, n_new, heads, head_dim, key_splits);
    if (!workspace) return fail(RA_E_INVALID, "key_splits %d needs a workspace", key_splits);
    if (!aligned(workspace, 16)) return fail(RA_E_INVALID, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
      return fail(RA_E_INVALID, "workspace of %lld bytes is smaller than the %lld required",
                  (long long)workspace_bytes, (long long)need);
    part_o = static_cast<float*>(workspace);
    part_ml = part_o + key_splits * batch * heads * n_new * head_dim;
  }
  const int64_t n_keys = cache_idx + n_new;
  int64_t split_keys = (n_keys + key_splits - 1) / key_splits;
  split_keys = (split_keys + 63) / 64 * 64;
  ra::DecParams p{q, k_cache, v_cache, out, lse, part_o, part_ml, cache_idx, cache_rows, n_keys,
                  split_keys, (int32_t)batch, (int32_t)heads, (int32_t)n_new, key_splits,
                  (int32_t)q_groups, (float)(1.4426950408889634 / std::sqrt((double)head_dim))};
  char err[256];
  if (ra::launch_decode(p, dtype == RA_BF16 ? ra::Dtype::BF16 : ra::Dtype::F32, (int)head_dim, nq,
                        stream, err, (int)sizeof(err)) != 0)
    return fail(RA_E_HIP, "%s", err);
  return RA_OK;
}

ra_status_t ra_blockwise_attn_fwd(const void* q, const void* k, const void* v,
                                  const int32_t* segment_ids, int64_t causal_block_size,
                                  int64_t q_chunk, int64_t k_chunk, int32_t ring_size,
                                  int32_t ring_index, int64_t batch, int64_t seq_q,
                                  int64_t heads, int64_t head_dim, ra_dtype_t dtype,
                                  void* out, float* lse, void* stream) {
  return ra_blockwise_attn_fwd_ex(q, k, v, segment_ids, causal_block_size, q_chunk, k_chunk,
                                  ring_size, ring_index, batch, seq_q, heads, head_dim, dtype,
                                  out, lse, nullptr, stream);
}

}  // extern "C"
