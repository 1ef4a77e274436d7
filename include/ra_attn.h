/*
 * ra_attn.h -- C ABI of the blockwise exact-attention forward of Ring
 * Attention for AMD MI355X (gfx950).
 *
 * What is computed.  One device's share of Ring Attention: the local query
 * block Q_r (ring position r of N) attends to all N key/value blocks (the
 * ring visits the block (r - t) mod N at outer step t; on one device every
 * block is resident and the library folds them in that order with the local
 * block r moved to the end) with a
 * running max / numerator / denominator carry that is rescaled per block
 * ("Ring Attention with Blockwise Transformers for Near-Infinite Context",
 * section 三: the self-attention equation, "分块注意力", "环形注意力算法"
 * and "排列不变性"; the carry update and chunk skipping of
 * "从论文到代码：深入理解RingAttention的块注意力计算逻辑", sections
 * "2. 数值稳定的注意力计算" and "3. 因果注意力掩码支持").  The result is
 * exact softmax(Q K^T / sqrt(D)) V over the visible keys:
 *
 *   query row i has global position pq = r * Lq + i, key j has position j;
 *   key j is visible from row i iff
 *     (causal_block_size == 0 or floor(pq / c) >= floor(j / c))   and
 *     (segment_ids == NULL or segment_ids[b][pq] == segment_ids[b][j]).
 *
 * Tensor layouts (row-major, contiguous, element strides implied):
 *   q, out   [batch, seq_q, heads, head_dim]             dtype
 *   k, v     [batch, ring_size * seq_q, heads, head_dim]  dtype, all N
 *            blocks in global order (block kb = rows kb*seq_q .. +seq_q-1)
 *   segment_ids [batch, ring_size * seq_q] int32, or NULL
 *   lse      [batch, heads, seq_q] float32, natural log of the softmax
 *            denominator (log-sum-exp of the scaled logits over visible keys)
 *
 * Arithmetic: logits, the running max, the denominator and the numerator
 * are float32.  bf16 inputs multiply on bf16 matrix cores with float32
 * accumulation; the probabilities are rounded to bf16 (round to nearest
 * even), and both the P.V product and the denominator use the rounded
 * values, so out is an exact convex combination of the rows of V (up to the
 * float32 accumulation).
 * out is rounded to the input dtype.  A query row with no visible key gets
 * out = 0 and lse = -inf.  q, k and v must be finite: NaN or infinite
 * inputs give unspecified results.
 *
 * Alignment: q, k, v, out (and the backward's dout, dq, dk, dv and the
 * split workspaces) must be 16-byte aligned; segment_ids, lse and delta
 * 4-byte aligned.  Misaligned pointers are rejected with RA_E_INVALID.
 *
 * Ownership and synchronisation: all pointers except those marked "host"
 * are device pointers allocated by the caller; the library allocates no
 * device memory and keeps no pointer after a call returns (its only device
 * memory is the fixed scratch array of ra_blockwise_attn_fwd_split_noalloc,
 * part of its code object).  Work is enqueued
 * on `stream` (a hipStream_t; NULL = the default stream) and the call
 * returns after the launch; the caller synchronises.  Calls are thread-safe.
 *
 * Errors: every entry point returns a status; nothing throws or aborts
 * across the ABI.  Argument errors are detected on the host before any
 * device work is enqueued.  ra_last_error() describes the last failure on
 * the calling thread.
 */
#ifndef RA_ATTN_H
#define RA_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_OK = 0,
  RA_E_INVALID = 1,     /* malformed argument (null pointer, bad size, ...)   */
  RA_E_UNSUPPORTED = 2, /* well-formed but outside what the kernels handle    */
  RA_E_HIP = 3          /* the HIP runtime reported an error at launch        */
} ra_status_t;

typedef enum { RA_BF16 = 0, RA_F32 = 1 } ra_dtype_t;

/* Which global positions a device's block holds (see
 * ra_blockwise_attn_fwd_placed). */
typedef enum { RA_PLACE_CONTIGUOUS = 0, RA_PLACE_STRIPED = 1 } ra_placement_t;

/*
 * ra_blockwise_attn_fwd -- the forward of one ring position.
 *
 *   q, k, v, segment_ids, out, lse: see the layouts above.
 *   causal_block_size: 0 = non-causal; 1 = token-level causal; c > 1 =
 *       block-causal with blocks of c positions ("3. 因果注意力掩码支持").
 *   q_chunk, k_chunk: query / key chunk sizes of the blockwise scheme
 *       ("1. 分块处理机制"); both must divide seq_q and be multiples of 32.
 *       A key chunk of a KV block is skipped for a query chunk when no pair
 *       in the two chunks is causally visible.
 *   ring_size N >= 1, ring_index r in [0, N).
 *   batch, seq_q (= Lq, the local block length), heads >= 0; a zero size
 *       is a valid empty call.  head_dim in {64, 128}.
 *
 * Returns RA_E_INVALID for null required pointers, negative sizes,
 * ring_index outside [0, ring_size), causal_block_size < 0, non-positive
 * chunks or chunks that do not divide seq_q; RA_E_UNSUPPORTED for other
 * head_dim, dtype, chunks not a multiple of 32 or sizes beyond the index
 * range of the kernels; RA_E_HIP if the launch fails.
 */
ra_status_t ra_blockwise_attn_fwd(const void* q, const void* k, const void* v,
                                  const int32_t* segment_ids,
                                  int64_t causal_block_size, int64_t q_chunk,
                                  int64_t k_chunk, int32_t ring_size,
                                  int32_t ring_index, int64_t batch,
                                  int64_t seq_q, int64_t heads,
                                  int64_t head_dim, ra_dtype_t dtype,
                                  void* out, float* lse, void* stream);

/*
 * ra_blockwise_attn_fwd_ex -- the same forward, additionally recording the
 * chunk-pair skip decisions the kernel took.
 *
 *   run_map: device bytes [ring_size][seq_q / q_chunk][seq_q / k_chunk] in
 *       ring-step order, or NULL.  The library clears it and the kernel sets
 *       run_map[t][a][b] = 1 when it folded into the softmax carry of query
 *       chunk a a 32-key part of key chunk b (block of ring step t) that
 *       holds at least one visible pair.  Parts without a visible pair are
 *       never folded in: a 64-key tile with none is skipped outright, and
 *       inside a processed tile such a part is masked to exactly zero weight.
 *       The map records the causal decisions: segment ids never enter it
 *       (parts whose key ids miss every id of the part's queries are also
 *       skipped, but are recorded as the causal test decides).
 *       Intended for debugging and parity checks; it costs extra stores.
 *
 * Errors as for ra_blockwise_attn_fwd.
 */
ra_status_t ra_blockwise_attn_fwd_ex(const void* q, const void* k,
                                     const void* v, const int32_t* segment_ids,
                                     int64_t causal_block_size, int64_t q_chunk,
                                     int64_t k_chunk, int32_t ring_size,
                                     int32_t ring_index, int64_t batch,
                                     int64_t seq_q, int64_t heads,
                                     int64_t head_dim, ra_dtype_t dtype,
                                     void* out, float* lse, uint8_t* run_map,
                                     void* stream);

/*
 * ra_blockwise_attn_fwd_placed -- the forward under a chosen placement of
 * the sequence on the ring.
 *
 * The review of "Ring Attention with Blockwise Transformers for
 * Near-Infinite Context" (sections 六 and 七) notes that causal attention
 * leaves contiguous blocks unbalanced -- device r holds about (r + 1/2)
 * blocks of visible pairs -- and names Striped Attention's striped
 * partition as the fix, for causal attention only.  Reading taken here:
 *
 *   RA_PLACE_CONTIGUOUS: block r holds positions r*Lq .. r*Lq + Lq - 1
 *       (ra_blockwise_attn_fwd);
 *   RA_PLACE_STRIPED: block r holds positions r, r + N, r + 2N, ...: query
 *       row i has position pq = i*N + r and storage row kb*Lq + j of k, v
 *       and segment_ids holds position j*N + kb.
 *
 * The visibility rule is unchanged: it compares positions (causal) and the
 * segment ids stored with the query's row (r*Lq + i) and the key's row
 * (segment_ids stay in storage order).  Under striped placement every
 * device holds N*Lq*(Lq+1)/2 - Lq*(N-1-r) visible pairs (token causal).
 * Striped placement serves the causal blocks c that divide N (the mask is
 * then token causal between local indices, with the keys of blocks kb >=
 * (floor(r/c) + 1) c counted one index later) and those that are multiples
 * of N (block causal with blocks of c/N local indices); other c have no
 * such form.  Layouts, arithmetic and outputs are those of
 * ra_blockwise_attn_fwd; run_map is that of ra_blockwise_attn_fwd_ex (a
 * chunk pair runs iff it holds a visible pair under the placement; its
 * first index is the ring step (r - kb) mod N).
 *
 * Errors as for ra_blockwise_attn_fwd_ex, plus RA_E_INVALID for an unknown
 * placement and RA_E_UNSUPPORTED for RA_PLACE_STRIPED with an effective
 * causal_block_size c > 0 that neither divides ring_size nor is a multiple
 * of it (a causal block at least as long as the sequence counts as 0).
 */
ra_status_t ra_blockwise_attn_fwd_placed(const void* q, const void* k,
                                         const void* v, const int32_t* segment_ids,
                                         int64_t causal_block_size, int64_t q_chunk,
                                         int64_t k_chunk, int32_t ring_size,
                                         int32_t ring_index, ra_placement_t placement,
                                         int64_t batch, int64_t seq_q, int64_t heads,
                                         int64_t head_dim, ra_dtype_t dtype,
                                         void* out, float* lse, uint8_t* run_map,
                                         void* stream);

/*
 * ra_blockwise_attn_fwd_split -- the forward with each query tile's walk
 * over the keys cut into key_splits runs that run in parallel.
 *
 * A small share (few heads, a short local block) gives the forward fewer
 * query tiles than the GPU has compute units, and each tile walks all its
 * keys alone.  Because the softmax carry folds key blocks in any order and
 * grouping with the same result (review of "Ring Attention with Blockwise
 * Transformers for Near-Infinite Context", section 三 "排列不变性", and the
 * carry of "2. 数值稳定的注意力计算"), the walk can be cut: the longest
 * walk of the share (its last query tile's) into key_splits runs, a query
 * tile whose walk has n of the longest walk's n_max tiles into
 * ceil(key_splits n / n_max) runs, so that runs are about equally long.
 * Split s of a tile folds the s-th of its equal runs (walk order, skips and
 * masks unchanged) into its own max, numerator and denominator, one
 * workgroup per run (the grid holds exactly the runs; the slots of a tile's
 * surplus splits are marked empty), and a second kernel folds the splits
 * into out and lse with the same carry.
 *
 *   key_splits: 1 .. 64; 1 is exactly ra_blockwise_attn_fwd_placed (the
 *       workspace may then be NULL).
 *   workspace: device memory of at least
 *       ra_blockwise_attn_fwd_split_workspace_bytes(...) bytes, owned by
 *       the caller, used as scratch during the call (float32 partial
 *       numerators [key_splits][batch][heads][seq_q][head_dim], then
 *       [key_splits][batch][heads][seq_q][2] kept maxima and denominators);
 *       its contents on entry do not matter.  Two calls sharing a workspace
 *       must be ordered on one stream.
 *   Everything else as for ra_blockwise_attn_fwd_placed, including run_map
 *   (the union of the splits' decisions is the unsplit map).
 *
 * The result equals the unsplit forward up to float32 rounding of the
 * fold (the probabilities a split rounds to bf16 are taken against its
 * own kept max).  Errors as for ra_blockwise_attn_fwd_placed, plus
 * RA_E_INVALID for key_splits outside [1, 64], or key_splits > 1 with a
 * NULL workspace or one smaller than required.
 */
ra_status_t ra_blockwise_attn_fwd_split(const void* q, const void* k,
                                        const void* v, const int32_t* segment_ids,
                                        int64_t causal_block_size, int64_t q_chunk,
                                        int64_t k_chunk, int32_t ring_size,
                                        int32_t ring_index, ra_placement_t placement,
                                        int64_t batch, int64_t seq_q, int64_t heads,
                                        int64_t head_dim, ra_dtype_t dtype,
                                        void* out, float* lse, uint8_t* run_map,
                                        int32_t key_splits, void* workspace,
                                        int64_t workspace_bytes, void* stream);

/* Workspace bytes ra_blockwise_attn_fwd_split needs: key_splits * batch *
 * heads * seq_q * (head_dim + 2) * 4; 0 when key_splits <= 1 or a size is
 * not positive.  Host-only. */
int64_t ra_blockwise_attn_fwd_split_workspace_bytes(int64_t batch, int64_t seq_q,
                                                     int64_t heads, int64_t head_dim,
                                                     int32_t key_splits);

/*
 * ra_blockwise_attn_fwd_split_noalloc -- ra_blockwise_attn_fwd_split for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the split partials
 * go to a scratch array that the library holds itself, so the call takes no
 * workspace and calls no hipMalloc, hipFree or other allocating routine.
 *
 *   The scratch is a device array of 64 MiB (67108864 bytes) in the library's
 *   code object: each GPU the library runs on holds one copy until the
 *   process ends.  Its device address is looked up on the first call on each
 *   device (the current device; `stream` must belong to it).  Calls whose
 *   partials, ra_blockwise_attn_fwd_split_workspace_bytes(batch, seq_q,
 *   heads, head_dim, key_splits) bytes, exceed 64 MiB return
 *   RA_E_UNSUPPORTED before any GPU work.  Nothing in the scratch has to
 *   start at zero (every slot a call reads is written by that call first).
 *   All calls on one GPU share its scratch: calls that may overlap on one
 *   GPU (on different streams, or from several threads without ordering)
 *   race; order them on one stream.
 *
 * Arguments, results and other errors as for ra_blockwise_attn_fwd_split
 * without the workspace; RA_E_HIP also when the scratch's address cannot be
 * obtained.
 */
ra_status_t ra_blockwise_attn_fwd_split_noalloc(const void* q, const void* k,
                                                const void* v, const int32_t* segment_ids,
                                                int64_t causal_block_size, int64_t q_chunk,
                                                int64_t k_chunk, int32_t ring_size,
                                                int32_t ring_index, ra_placement_t placement,
                                                int64_t batch, int64_t seq_q, int64_t heads,
                                                int64_t head_dim, ra_dtype_t dtype,
                                                void* out, float* lse, uint8_t* run_map,
                                                int32_t key_splits, void* stream);

/* A key split count for a share: 1 when the unsplit grid (batch * heads *
 * ceil(seq_q / rows per workgroup) workgroups, 256 rows for RA_BF16, 128
 * for RA_F32) already fills compute_units; otherwise the most splits whose
 * runs (one workgroup each, over every query tile and head of the batch)
 * fit one workgroup per compute unit, at most one per 4
 * key tiles of 64 keys of the longest walk (the share's last query tile's:
 * its blocks' keys up to its causal limit), and at most 64.  The dq kernel
 * of ra_blockwise_attn_bwd_split launches the same runs (the forward's
 * query rows per workgroup and key tiles of the dtype: 256 rows and 64
 * keys for RA_BF16, 128 and 32 for RA_F32), so the count serves the
 * backward as well.
 * Host-only; invalid arguments give 1. */
int32_t ra_blockwise_attn_fwd_key_splits(int64_t batch, int64_t seq_q, int64_t heads,
                                         ra_dtype_t dtype, int64_t causal_block_size,
                                         int32_t ring_size, int32_t ring_index,
                                         ra_placement_t placement, int32_t compute_units);

/*
 * ra_blockwise_attn_bwd -- the gradients of one ring position's share.
 *
 * For the forward of ra_blockwise_attn_fwd with the same q, k, v,
 * segment_ids and masks, and an upstream gradient dout of its output,
 * computes the gradients of sum(dout * out).  The pages pair the ring
 * forward with a backward pass but print no backward equations; these are
 * the exact derivatives of the attention definition ("Ring Attention with
 * Blockwise Transformers for Near-Infinite Context", section 三, the
 * self-attention equation): with p_ij the softmax weights of the forward,
 *   delta_i = sum_d dout_i,d * out_i,d,
 *   ds_ij   = p_ij * (dout_i . v_j - delta_i),
 *   dq_i    = (1/sqrt(D)) sum_j ds_ij k_j,
 *   dk_j    = (1/sqrt(D)) sum_i ds_ij q_i,   dv_j = sum_i p_ij dout_i.
 *
 *   out, lse: the forward's outputs for these inputs (layouts as above);
 *       p_ij is recomputed from q, k and lse.
 *   dout: [batch, seq_q, heads, head_dim] dtype.
 *   dq: [batch, seq_q, heads, head_dim] float32, written.
 *   dk, dv: [batch, ring_size * seq_q, heads, head_dim] float32, written:
 *       this share's contribution to the gradients of all N key/value
 *       blocks (in the ring, the addend this device puts into the dK/dV
 *       blocks as they pass); keys that no local query sees get 0.
 *   delta: [batch, heads, seq_q] float32, written (the row terms above).
 *
 * Arithmetic: the scores, p and ds are float32.  RA_BF16: p and ds are
 * rounded to bf16 (round to nearest even) as operands of the bf16 matrix
 * products, which accumulate in float32.  RA_F32: every operand stays
 * float32 (float32 matrix products).
 *
 * Errors as for ra_blockwise_attn_fwd, plus RA_E_INVALID for a null out,
 * lse, dout, dq, dk, dv or delta.  Ownership, streams and threading as
 * for the forward.
 */
ra_status_t ra_blockwise_attn_bwd(const void* q, const void* k, const void* v,
                                  const int32_t* segment_ids,
                                  int64_t causal_block_size, int64_t q_chunk,
                                  int64_t k_chunk, int32_t ring_size,
                                  int32_t ring_index, int64_t batch,
                                  int64_t seq_q, int64_t heads,
                                  int64_t head_dim, ra_dtype_t dtype,
                                  const void* out, const float* lse,
                                  const void* dout, float* dq, float* dk,
                                  float* dv, float* delta, void* stream);

/*
 * ra_blockwise_attn_bwd_placed -- ra_blockwise_attn_bwd under a placement
 * of the sequence on the ring (see ra_blockwise_attn_fwd_placed): the
 * gradients of that placement's forward, with segment_ids, dk and dv in
 * storage order.  Errors as for ra_blockwise_attn_bwd, plus RA_E_INVALID for
 * an unknown placement and RA_E_UNSUPPORTED for RA_PLACE_STRIPED with an
 * effective causal_block_size that neither divides ring_size nor is a
 * multiple of it (as for ra_blockwise_attn_fwd_placed).
 */
ra_status_t ra_blockwise_attn_bwd_placed(const void* q, const void* k,
                                         const void* v, const int32_t* segment_ids,
                                         int64_t causal_block_size, int64_t q_chunk,
                                         int64_t k_chunk, int32_t ring_size,
                                         int32_t ring_index, ra_placement_t placement,
                                         int64_t batch, int64_t seq_q, int64_t heads,
                                         int64_t head_dim, ra_dtype_t dtype,
                                         const void* out, const float* lse,
                                         const void* dout, float* dq, float* dk,
                                         float* dv, float* delta, void* stream);

/*
 * ra_blockwise_attn_bwd_split -- the backward with the query tiles' walks
 * over the keys cut into key_splits runs, as in ra_blockwise_attn_fwd_split.
 *
 * dq_i is a sum over the visible keys of terms that the forward's lse and
 * delta fix completely, so it splits over any partition of the keys: each
 * run's workgroup writes its addend to dq into the workspace, and a last
 * kernel adds the addends in split order (deterministic: no atomics).  dk,
 * dv and delta are computed as by ra_blockwise_attn_bwd_placed.
 *
 *   key_splits: 1 .. 64; 1 is exactly ra_blockwise_attn_bwd_placed (the
 *       workspace may then be NULL).
 *   workspace: device memory of at least
 *       ra_blockwise_attn_bwd_split_workspace_bytes(...) bytes, owned by
 *       the caller (float32 [key_splits][batch][seq_q][heads][head_dim]);
 *       its contents on entry do not matter.  Two calls sharing a workspace
 *       must be ordered on one stream.
 *   Everything else as for ra_blockwise_attn_bwd_placed.
 *
 * Errors as for ra_blockwise_attn_bwd_placed, plus RA_E_INVALID for
 * key_splits outside [1, 64], or key_splits > 1 with a NULL workspace or
 * one smaller than required.
 */
ra_status_t ra_blockwise_attn_bwd_split(const void* q, const void* k,
                                        const void* v, const int32_t* segment_ids,
                                        int64_t causal_block_size, int64_t q_chunk,
                                        int64_t k_chunk, int32_t ring_size,
                                        int32_t ring_index, ra_placement_t placement,
                                        int64_t batch, int64_t seq_q, int64_t heads,
                                        int64_t head_dim, ra_dtype_t dtype,
                                        const void* out, const float* lse,
                                        const void* dout, float* dq, float* dk,
                                        float* dv, float* delta, int32_t key_splits,
                                        void* workspace, int64_t workspace_bytes,
                                        void* stream);

/* Workspace bytes ra_blockwise_attn_bwd_split needs: key_splits * batch *
 * seq_q * heads * head_dim * 4; 0 when key_splits <= 1 or a size is not
 * positive.  Host-only.  ra_blockwise_attn_fwd_key_splits gives a split
 * count for the backward too (its dq kernel has the forward's grid). */
int64_t ra_blockwise_attn_bwd_split_workspace_bytes(int64_t batch, int64_t seq_q,
                                                     int64_t heads, int64_t head_dim,
                                                     int32_t key_splits);

/*
 * ra_blockwise_ffn -- the feedforward of the Blockwise Transformer, one
 * sequence chunk at a time.
 *
 *   y = max(0, x W1 + b1) W2 + b2     ("Ring Attention with Blockwise
 *   Transformers for Near-Infinite Context", section 三, the feedforward
 *   equation), applied to the chunks [c * chunk, (c + 1) * chunk) of every
 *   sequence in order, so that only one chunk's hidden activations exist at
 *   a time ("Blockwise Feedforward网络详解", sections "核心技术原理" and
 *   "技术实现细节").
 *
 *   x, y:  [batch, seq, hidden] bf16, row-major, device.
 *   w1:    [hidden, ffn] bf16;  b1: [ffn] bf16;
 *   w2:    [ffn, hidden] bf16;  b2: [hidden] bf16 (row-major, device).
 *   chunk_size: rows of a sequence per chunk; must divide seq.
 *   workspace: device memory of at least
 *       ra_blockwise_ffn_workspace_bytes(chunk_size, ffn) bytes (the bf16
 *       hidden activations of one chunk); contents are overwritten.
 *
 * Arithmetic: bf16 inputs on the matrix cores with float32 accumulation;
 * each bias is added in float32; the hidden activation is rounded to bf16
 * (round to nearest even) after the ReLU, between the two products; y is
 * rounded to bf16.  Both products run in the library's own GEMM kernel
 * with the bias (and ReLU) fused into its epilogue.
 *
 * Alignment: x, w1, w2, y and the workspace 16-byte, b1 and b2 8-byte.
 *
 * Returns RA_E_INVALID for null or misaligned pointers, non-positive sizes,
 * a chunk size that does not divide seq or a workspace smaller than
 * required; RA_E_UNSUPPORTED for RA_F32, for hidden or ffn_hidden not a
 * multiple of 8, or an operand (w1, w2, one chunk of x, y or of the hidden
 * activations) of more than 4 GiB; RA_E_HIP if a launch fails.  A call with
 * batch == 0 or seq == 0 is a valid no-op.
 */
int64_t ra_blockwise_ffn_workspace_bytes(int64_t chunk_size, int64_t ffn_hidden);

ra_status_t ra_blockwise_ffn(const void* x, const void* w1, const void* b1,
                             const void* w2, const void* b2, int64_t batch,
                             int64_t seq, int64_t hidden, int64_t ffn_hidden,
                             int64_t chunk_size, ra_dtype_t dtype, void* y,
                             void* workspace, int64_t workspace_bytes,
                             void* stream);

/*
 * ra_attn_decode -- one incremental-decoding step over a KV cache.
 *
 * The pages name an inference cache index, cache_idx, among the ring
 * forward's arguments and tie inference to incremental decoding with a KV
 * cache ("RingAttention与传统注意力机制对比为什么它是大语言模型的终极解决
 * 方案", sections "3. 推理成本显著降低" and "关键参数配置";
 * "从论文到代码：深入理解RingAttention的块注意力计算逻辑", section
 * "RingAttention的算法原理"); they print no decoding code.  Reading taken
 * here: cache_idx is the number of tokens already in the cache; the step's
 * n_new query tokens have positions cache_idx .. cache_idx + n_new - 1 and
 * the caller has already written their keys and values into those cache
 * rows.  Query t attends to cache rows 0 .. cache_idx + t (token causal,
 * "3. 因果注意力掩码支持"), exact softmax(q K^T / sqrt(D)) V:
 *
 *   q, out            [batch, n_new, heads, head_dim]       dtype
 *   k_cache, v_cache  [batch, cache_rows, heads, head_dim]  dtype; rows
 *                     0 .. cache_idx + n_new - 1 are read, later rows never
 *   lse               [batch, heads, n_new] float32 (natural log)
 *
 * The cache rows are folded in key_splits contiguous ranges, one workgroup
 * each; with key_splits > 1 the workgroups write their partial carries
 * (kept max, denominator, unnormalised numerator) into `workspace`, at
 * least ra_attn_decode_workspace_bytes(...) bytes of device memory whose
 * contents are overwritten, and a second kernel folds them (the fold of the
 * ring's per-block partials; the order of the fold changes only rounding).
 * key_splits == 1 needs no workspace (NULL allowed).
 *
 * Arithmetic: float32 logits, max, denominator and numerator.  bf16 inputs
 * multiply on the bf16 matrix cores with float32 accumulation, and the
 * probabilities are rounded to bf16 for the P.V product with the
 * denominator summing the rounded values (as the forward); float32 inputs
 * are computed in float32 throughout.  out is rounded to the input dtype.
 * Inputs must be finite.
 *
 * Alignment: q, k_cache, v_cache, out and workspace 16-byte, lse 4-byte.
 *
 * Returns RA_E_INVALID for negative sizes or cache_idx, cache_idx + n_new >
 * cache_rows, key_splits outside [1, 1024], null or misaligned pointers or
 * a short workspace; RA_E_UNSUPPORTED for head_dim other than 64 or 128,
 * a dtype other than RA_BF16 / RA_F32, n_new > 256 (a prefill: use the
 * blockwise forward), heads * head_dim > 2^24 or a grid too large;
 * RA_E_HIP if a launch fails.  batch, heads or n_new == 0 is a valid
 * no-op.
 */
int64_t ra_attn_decode_workspace_bytes(int64_t batch, int64_t n_new, int64_t heads,
                                       int64_t head_dim, int32_t key_splits);

/* The library's key-split count for a decoding step on a GPU with
 * compute_units compute units: about eight workgroups per compute unit and
 * at least 1024 cache rows per split (512 while fewer workgroups than
 * compute units would result), in [1, 1024].  Host only; 1 for
 * non-positive arguments. */
int32_t ra_attn_decode_key_splits(int64_t batch, int64_t n_new, int64_t heads,
                                  int64_t cache_idx, int32_t compute_units);

ra_status_t ra_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                           int64_t cache_idx, int64_t cache_rows, int64_t batch,
                           int64_t n_new, int64_t heads, int64_t head_dim,
                           ra_dtype_t dtype, int32_t key_splits, void* workspace,
                           int64_t workspace_bytes, void* out, float* lse,
                           void* stream);

/*
 * ra_blockwise_plan -- host-only: the ring order and the chunk-pair skip
 * decisions for one ring position, without touching a GPU.
 *
 *   kv_block_of_step: host int32 [ring_size]; entry t = (ring_index - t) mod
 *       ring_size, the block used at ring step t ("环形注意力算法").
 *   run_bits: host bytes [ring_size][seq_q / q_chunk][seq_q / k_chunk], or
 *       NULL; 1 = the chunk pair runs (below or on the causal diagonal).
 *   n_run_chunk_pairs: host, optional; the number of ones in run_bits.
 *
 * Validation as for ra_blockwise_attn_fwd (chunks need not be multiples of
 * 32 here).  Returns RA_OK or RA_E_INVALID.
 */
ra_status_t ra_blockwise_plan(int64_t causal_block_size, int64_t q_chunk,
                              int64_t k_chunk, int64_t seq_q,
                              int32_t ring_size, int32_t ring_index,
                              int32_t* kv_block_of_step, uint8_t* run_bits,
                              int64_t* n_run_chunk_pairs);

/*
 * ra_blockwise_plan_placed -- ra_blockwise_plan under a placement (see
 * ra_blockwise_attn_fwd_placed).  Under RA_PLACE_STRIPED the chunk pair
 * (a, b) of the block kb used at step t runs iff its last query, position
 * ((a+1)*q_chunk - 1)*N + r, sees its first key, position b*k_chunk*N + kb
 * (positions grow with the local index inside a block, so this is the test
 * for any visible pair).  Any causal_block_size is accepted here.  Returns
 * RA_OK or RA_E_INVALID (also for an unknown placement).
 */
ra_status_t ra_blockwise_plan_placed(int64_t causal_block_size, int64_t q_chunk,
                                     int64_t k_chunk, int64_t seq_q,
                                     int32_t ring_size, int32_t ring_index,
                                     ra_placement_t placement,
                                     int32_t* kv_block_of_step, uint8_t* run_bits,
                                     int64_t* n_run_chunk_pairs);

/* Text of the last error on the calling thread ("" if none).  The pointer
 * stays valid until the next ra_* call on the same thread. */
const char* ra_last_error(void);

/* Library version as "major.minor.patch+build" (static storage); build is
 * the first 16 hex digits of the SHA-256 of the device sources the library
 * was compiled from. */
const char* ra_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_ATTN_H */
