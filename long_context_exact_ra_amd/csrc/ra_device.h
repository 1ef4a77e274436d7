// Device-side building blocks shared by the forward and backward kernels of
// the blockwise ring-attention library (gfx950): work decomposition, the
// ring walk (and its cut into key splits), causal limits, buffer-to-LDS DMA
// and the per-tile visibility tests.  Internal; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <climits>

#include "ra_internal.h"
#include "ra_walk.h"

// Everything here has internal linkage: each kernel source that includes
// the header gets its own inlined copy.
namespace ra {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;


constexpr float kLn2 = 0.69314718055994530942f;
// Buffer resource word 3 for gfx9 raw (untyped) buffer access.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ float ninf() { return -__builtin_inff(); }

// ---------------------------------------------------------------------------
// Work decomposition shared by both kernels
// ---------------------------------------------------------------------------

// Which (batch, head, query tile) a workgroup owns.  Workgroups are
// dispatched round-robin over the 8 XCDs; the remap puts consecutive logical
// tiles -- the query tiles of one head, which stream the same keys and
// values -- on the same XCD so they share its L2.  Heavier query tiles (more
// causal work) come first.
// With key splits, split s of a query tile walks only the s-th of
// key_splits equal runs of the tile's key walk; the splits of one head sit
// next to each other, split-major, so that the query tiles walking the same
// key range share an XCD.
struct WgCoord {
  int b, h, m0, split;
};

template <int BM>
__device__ __forceinline__ WgCoord wg_coord(const FwdParams& p) {
  const int pid = blockIdx.x, n = p.n_wg;
  const int xcd = pid & 7, idx = pid >> 3, cnt = n >> 3, rem = n & 7;
  const int logical =
      xcd < rem ? xcd * (cnt + 1) + idx : rem * (cnt + 1) + (xcd - rem) * cnt + idx;
  const int per_bh = p.n_qtiles * p.key_splits;
  const int bh = logical / per_bh, in_bh = logical % per_bh;
  const int qt = p.n_qtiles - 1 - in_bh % p.n_qtiles;
  // The values are workgroup-uniform; say so, so that addresses and buffer
  // descriptors derived from them stay in scalar registers.
  return WgCoord{__builtin_amdgcn_readfirstlane(bh / p.heads),
                 __builtin_amdgcn_readfirstlane(bh % p.heads),
                 __builtin_amdgcn_readfirstlane(qt * BM),
                 __builtin_amdgcn_readfirstlane(in_bh / p.n_qtiles)};
}

// Position of the workgroup's current tile in the ring walk.
struct Cursor {
  int t;       // ring step
  int kb;      // key/value block used at this step
  int kt;      // tile index inside the block
  int ntile;   // tiles to visit in this block
  int klen;    // keys to visit in this block (multiple of 32)
  int valid;   // int, not bool: no padding bytes to copy around
  int pos;     // index of the current tile in the whole walk
  // Striped placement: keys to visit in every block kb <= r and kb > r
  // (the walk's limit is fixed, and a block's count depends only on which
  // side of r it lies); set by cursor_seek.
  int klen_lo, klen_hi;
};

// Key coordinates.  Causal tests compare a key coordinate with a limit
// derived from the query rows.  Contiguous placement: the coordinate of key
// j of block kb is its global position kb * Lq + j, the same as its storage
// row.  Striped placement (position j * N + kb): the coordinate is j + [kb
// >= stripe_hi] and query row i's is i, with p.causal the causal block in
// coordinates (walk::striped_causal: token causal when the mask's block
// divides N, j + [kb > r] <= i for c = 1; block causal on the local indices
// when N divides it).  Either way the coordinate of block kb's first key is
// block_vbase and coordinates grow by one per key inside a block.
template <bool STRIPED>
__device__ __forceinline__ int32_t block_vbase(const FwdParams& p, int kb) {
  return walk::block_vbase(p.seq_q, p.stripe_hi, STRIPED, kb);
}

// kend: first key coordinate no row of the workgroup can see (INT64_MAX when
// non-causal).  The keys of block kb to visit are those before kend, rounded
// up to whole 32-key sub-tiles.
template <bool STRIPED>
__device__ __forceinline__ int block_klen(const FwdParams& p, int kb, int64_t kend) {
  return walk::block_klen(p.seq_q, block_vbase<STRIPED>(p, kb), kend);
}

// The walk over the keys.  Contiguous placement: block by block, the tiles
// of a block in order, the blocks in ring order rotated by one so that the
// local block comes last: walk step t uses block (r - 1 - t) mod N, i.e.
// r - 1, .., 0, N - 1, .., r + 1, then r.  Under a causal mask the local
// (diagonal) block is the only one whose visible length differs between the
// query tiles of a head; walked first, it would start the workgroups of a
// head at different offsets in the blocks that follow, and they would stop
// sharing those blocks' key tiles in L2 (the 7B-shaped share fetched 280 GB
// from HBM per launch that way, 161 GB with the local block last).
// Striped placement: every block is a causal triangle of the same shape, so
// the workgroups of a head, whose query tiles see different numbers of keys
// per block, would drift apart block by block and stop sharing the key tiles
// they stream through L2.  There the walk is tile-major instead -- tile kt
// of every block in ring order, then tile kt + 1 -- which keeps them in
// step until each runs out of keys.  The softmax carry does not depend on
// the order in which keys are folded in.
// Striped walk: the first visited tile at or after (kt, t).  The steps of a
// round visit the blocks kb < stripe_hi first (steps t < stripe_hi: blocks
// r, r - 1, .., 0, then stripe_hi - 1, .., r + 1), then the shifted ones
// (N - 1 down to stripe_hi); with stripe_hi = r + 1 (token causal, no mask)
// this is the ring order, step t using block (r - t) mod N.  Unshifted
// blocks hold ceil(klen_lo / TN) tiles, shifted ones ceil(klen_hi / TN) <=
// that, so within round kt every step t < stripe_hi is visited, a later
// step only while kt is below the smaller count, and the walk ends with the
// larger count.
template <int TN>
__device__ __forceinline__ void striped_settle(const FwdParams& p, Cursor& c) {
  const int n_lo = (c.klen_lo + TN - 1) / TN, n_hi = (c.klen_hi + TN - 1) / TN;
  if (c.t >= p.ring_size || (c.t >= p.stripe_hi && c.kt >= n_hi)) {
    c.t = 0;
    ++c.kt;
  }
  if (c.kt >= n_lo) {
    c.valid = 0;
    return;
  }
  if (c.t < p.stripe_hi) {
    c.kb = p.ring_index - c.t;
    if (c.kb < 0) c.kb += p.stripe_hi;
  } else {
    c.kb = p.ring_size - 1 + p.stripe_hi - c.t;
  }
  c.klen = c.t < p.stripe_hi ? c.klen_lo : c.klen_hi;
  c.ntile = c.t < p.stripe_hi ? n_lo : n_hi;
  c.valid = 1;
}

template <int TN, bool STRIPED = false>
__device__ __forceinline__ void cursor_seek(const FwdParams& p, Cursor& c, int64_t kend) {
  if (STRIPED) {
    c.klen_lo = block_klen<true>(p, 0, kend);
    c.klen_hi = p.stripe_hi < p.ring_size ? block_klen<true>(p, p.stripe_hi, kend) : 0;
    striped_settle<TN>(p, c);
    return;
  }
#pragma clang loop vectorize(disable) unroll(disable)
  while (c.t < p.ring_size) {
    // Walk step t: block (r - 1 - t) mod N (the local block last).
    c.kb = p.ring_index - 1 - c.t;
    if (c.kb < 0) c.kb += p.ring_size;
    c.klen = block_klen<STRIPED>(p, c.kb, kend);
    c.ntile = (c.klen + TN - 1) / TN;
    if (c.ntile > 0) {
      c.valid = 1;
      return;
    }
    ++c.t;
  }
  c.valid = 0;
}

template <int TN, bool STRIPED = false>
__device__ __forceinline__ void cursor_next(const FwdParams& p, Cursor& c, int64_t kend) {
  ++c.pos;
  if (STRIPED) {
    ++c.t;
    striped_settle<TN>(p, c);
    return;
  }
  if (++c.kt < c.ntile) return;
  c.kt = 0;
  ++c.t;
  cursor_seek<TN, STRIPED>(p, c, kend);
}

// Key splits: the run [begin, end) of the workgroup's walk that its split
// covers.  key_splits is the number of runs of the longest walk (the last
// query tile's: causal limits only grow with the row); a query tile whose
// walk is shorter is cut into proportionally fewer runs, ceil(key_splits n
// / n_max), so that every run has about the same number of tiles; its
// surplus splits are idle (with the exact grid of wg_coord_runs no
// workgroup holds one, and the tile's last run marks their slots empty;
// the backward's uniform grid keeps idle workgroups).  A walk's length is the sum of
// its blocks' tile counts (a loop over the ring blocks, or a closed form
// under striped placement), paid only when the share is split (small
// grids).  Without splits the run is the whole walk.
struct SplitRange {
  int begin, end;
  int idle;  // this split has no run: the workgroup writes an empty partial
  int runs;  // runs of this query tile's walk
};

// Striped placement: a block's tile count depends only on whether kb > r
// (its key coordinates start at 1 instead of 0).  Blocks kb <= r are ring
// steps t = 0 .. r, blocks kb > r steps t = r + 1 .. N - 1.
struct StripedCounts {
  int lo, hi;  // tiles of each block kb <= r / kb > r
};

template <int TN, bool STRIPED>
__device__ __forceinline__ int64_t walk_tiles(const FwdParams& p, int64_t kend) {
  return walk::walk_tiles(p.seq_q, p.ring_size, p.stripe_hi, STRIPED, TN, kend);
}

// Runs of a walk of n tiles when the longest walk (n_max tiles) takes
// key_splits of them; the host sizes the grid with the same function.
__device__ __forceinline__ int split_runs(const FwdParams& p, int64_t n, int64_t n_max) {
  return walk::split_runs(p.key_splits, n, n_max);
}

template <int BM, int TN, bool STRIPED>
__device__ __forceinline__ walk::Share share_of(const FwdParams& p) {
  return walk::Share{p.seq_q, p.ring_size, p.ring_index, p.causal, STRIPED, BM, TN, p.stripe_hi};
}

// kend_max: the walk limit of the share's last query tile.
template <int TN, bool STRIPED>
__device__ __forceinline__ SplitRange split_range(const FwdParams& p, int split, int64_t kend,
                                                  int64_t kend_max) {
  if (p.key_splits <= 1) return SplitRange{0, INT_MAX, 0, 1};
  const int64_t n = walk_tiles<TN, STRIPED>(p, kend);
  const int runs = split_runs(p, n, walk_tiles<TN, STRIPED>(p, kend_max));
  if (split >= runs) return SplitRange{0, 0, 1, runs};
  return SplitRange{(int)(n * split / runs), (int)(n * (split + 1) / runs), 0, runs};
}

// Move a freshly sought cursor to walk position `pos` (the first tile of
// its split).  Contiguous walk: block by block.  Striped walk (tile kt of
// every block that has one, in ring order, then kt + 1): every round below
// the smaller tile count visits all N blocks, the rounds above it only the
// blocks with the larger count, which are consecutive ring steps.
template <int TN, bool STRIPED>
__device__ __forceinline__ void cursor_to(const FwdParams& p, Cursor& c, int64_t kend, int pos) {
  if (!STRIPED) {
#pragma clang loop vectorize(disable) unroll(disable)
    while (c.valid && c.pos + (c.ntile - c.kt) <= pos) {
      c.pos += c.ntile - c.kt;
      c.kt = 0;
      ++c.t;
      cursor_seek<TN, false>(p, c, kend);
    }
    if (c.valid && c.pos < pos) {
      c.kt += pos - c.pos;
      c.pos = pos;
    }
    return;
  }
  if (!c.valid || pos <= c.pos) return;
  const StripedCounts sc{(c.klen_lo + TN - 1) / TN, (c.klen_hi + TN - 1) / TN};
  const int n_lo = p.stripe_hi, n_hi = p.ring_size - p.stripe_hi;
  const int full = min(sc.lo, sc.hi);
  const int64_t in_full = (int64_t)full * p.ring_size;
  int kt, t;
  if (pos < in_full) {
    kt = pos / p.ring_size;
    t = pos % p.ring_size;
  } else {
    // Rounds full .. max - 1 visit only the blocks with the larger count.
    const bool lo_longer = sc.lo > sc.hi;
    const int cnt = lo_longer ? n_lo : n_hi;
    const int64_t rest = pos - in_full;
    if (cnt == 0 || rest >= (int64_t)cnt * (max(sc.lo, sc.hi) - full)) {
      c.valid = 0;
      c.pos = pos;
      return;
    }
    kt = full + (int)(rest / cnt);
    t = (int)(rest % cnt) + (lo_longer ? 0 : n_lo);
  }
  c.kt = kt;
  c.t = t;
  c.pos = pos;
  striped_settle<TN>(p, c);
}

// A wave-uniform 64-bit value that the compiler computed in vector registers
// (64-bit division has no scalar form), moved back to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Per-wave causal limits as 32-bit key coordinates (every coordinate is
// below 2^31 - 1, and tiles start at multiples of 32 inside a block).  For
// the 32-key sub-tile starting at key coordinate pk0:
//   it holds a visible pair for some row of the wave iff pk0 < run_lim;
//   it needs the per-element causal test iff pk0 >= mask_lim;
// and key position pk is visible from this lane's row iff pk < lane_lim.
// A wave without rows gets run_lim = INT32_MIN: none of its tiles run.
struct WaveLimits {
  int32_t run_lim, mask_lim, lane_lim;
};

__device__ __forceinline__ int32_t clamp_i32(int64_t x) {
  return (int32_t)std::min<int64_t>(x, INT32_MAX);
}

// pq_first: the query coordinate of the wave's first row -- its global
// position (contiguous) or its local row (striped, token causal).
__device__ __forceinline__ WaveLimits wave_limits(const FwdParams& p, int64_t pq_first,
                                                  int lrow, bool wave_active) {
  WaveLimits w{INT32_MAX, INT32_MAX, p.seq_k};
  if (p.causal > 0) {
    const int64_t c = p.causal;
    // First key position no row of the wave can see, and first key position
    // that some row of the wave cannot see.
    const int64_t run_end = ((pq_first + 31) / c + 1) * c;
    const int64_t full_end = (pq_first / c + 1) * c;
    w.run_lim = clamp_i32(uniform64(run_end));
    w.mask_lim = clamp_i32(uniform64(full_end)) - 31;
    w.lane_lim = (int32_t)std::min<int64_t>(((pq_first + lrow) / c + 1) * c, p.seq_k);
  }
  if (!wave_active) w.run_lim = INT32_MIN;
  return w;
}

// Key-stationary backward: the causal threshold of a key (query
// coordinates >= it see the key) for the lane's key kw0 + lrow of a wave
// whose 32 keys start at storage row kw0, and the wave's smallest and
// largest thresholds (INT32_MIN when non-causal).  Contiguous: floor(pk /
// c) c for the key's position pk.  Striped: key j of block kb has
// coordinate j + [kb >= stripe_hi] and is seen from local rows i with
// floor(i / c) >= floor(coordinate / c) (c in coordinates; c = 1: i >= j +
// [kb > r]).  The 32 keys of a wave lie in one block (Lq is a multiple of
// 32).
struct KeyThresholds {
  int32_t lane, first, last;
};

template <bool STRIPED>
__device__ __forceinline__ KeyThresholds key_thresholds(const FwdParams& p, int kw0, int lrow) {
  const int64_t c = p.causal;
  KeyThresholds t{INT32_MIN, INT32_MIN, INT32_MIN};
  const int key = kw0 + lrow;
  if (c > 0 && STRIPED) {
    const int kb = kw0 / p.seq_q;
    const int32_t sh = (kb >= p.stripe_hi ? 1 : 0) - kb * p.seq_q;
    const int32_t cc = (int32_t)c;
    t.lane = (key + sh) / cc * cc;
    t.first = __builtin_amdgcn_readfirstlane((kw0 + sh) / cc * cc);
    t.last = __builtin_amdgcn_readfirstlane((kw0 + 31 + sh) / cc * cc);
  } else if (c > 0) {
    t.lane = (int32_t)(((int64_t)key / c) * c);
    t.first = (int32_t)uniform64(((int64_t)kw0 / c) * c);
    t.last = (int32_t)uniform64(((int64_t)(kw0 + 31) / c) * c);
  }
  return t;
}

// The first local query row that can see any of the keys [k0, k0 + nkeys)
// of a key-stationary workgroup (Lq when none can); qpos0 is the query
// coordinate of local row 0 (0 under striped placement).  Striped: the
// smallest threshold is that of the first key, unless the keys run into
// the next block, whose first key's threshold is at most 1.
template <bool STRIPED>
__device__ __forceinline__ int first_query_row(const FwdParams& p, int k0, int nkeys,
                                               int32_t qpos0) {
  const int64_t c = p.causal;
  int q_lo = 0;
  if (c > 0 && STRIPED) {
    const int kb = k0 / p.seq_q;
    const int j0 = k0 - kb * p.seq_q;
    const int32_t cc = (int32_t)c;
    q_lo = j0 + nkeys <= p.seq_q ? (j0 + (kb >= p.stripe_hi ? 1 : 0)) / cc * cc : 0;
    q_lo = q_lo >= p.seq_q ? p.seq_q : q_lo;
  } else if (c > 0) {
    const int64_t t0 = ((int64_t)k0 / c) * c - qpos0;
    q_lo = t0 <= 0 ? 0 : (t0 >= p.seq_q ? p.seq_q : (int)t0);
  }
  return q_lo;
}

// The walk limit of the workgroup whose query tile starts at local row m0.
template <int BM, bool STRIPED = false>
__device__ __forceinline__ int64_t wg_kend(const FwdParams& p, int m0) {
  return uniform64(walk::tile_kend(p.causal, p.seq_q, p.ring_index, STRIPED, m0, BM));
}

// Forward with key splits: the grid holds split_wgs workgroups per (batch,
// head), one per run of each query tile's walk (split_runs of it, heavier
// tiles first), so that no workgroup is idle.  The host counts the same
// runs with the same walk lengths.  A workgroup beyond the runs (which a
// count mismatch would cause) gets split -1 and must exit without writing.
template <int BM, int TN, bool STRIPED>
__device__ __forceinline__ WgCoord wg_coord_runs(const FwdParams& p) {
  const int pid = blockIdx.x, n = p.n_wg;
  const int xcd = pid & 7, idx = pid >> 3, cnt = n >> 3, rem = n & 7;
  const int logical =
      xcd < rem ? xcd * (cnt + 1) + idx : rem * (cnt + 1) + (xcd - rem) * cnt + idx;
  const int bh = __builtin_amdgcn_readfirstlane(logical / p.split_wgs);
  const int in_bh = __builtin_amdgcn_readfirstlane(logical % p.split_wgs);
  const walk::Share sh = share_of<BM, TN, STRIPED>(p);
  const int64_t n_max = walk::qtile_walk(sh, p.n_qtiles - 1);
  int qt = -1, split = -1, first = 0;
#pragma clang loop vectorize(disable) unroll(disable)
  for (int t = p.n_qtiles - 1; t >= 0; --t) {
    const int runs = walk::split_runs(p.key_splits, walk::qtile_walk(sh, t), n_max);
    if (in_bh < first + runs) {
      qt = t;
      split = in_bh - first;
      break;
    }
    first += runs;
  }
  return WgCoord{__builtin_amdgcn_readfirstlane(bh / p.heads),
                 __builtin_amdgcn_readfirstlane(bh % p.heads),
                 __builtin_amdgcn_readfirstlane(qt < 0 ? 0 : qt * BM),
                 __builtin_amdgcn_readfirstlane(split)};
}

// Debug run map, in ring-step order: block kb arrives at step (r - kb) mod N
// (the walk itself may visit the blocks in another order).
__device__ __forceinline__ void write_run_map(const FwdParams& p, int kb, int qg0, int key0) {
  const int nqc = p.seq_q / p.q_chunk, nkc = p.seq_q / p.k_chunk;
  const int t = p.ring_index - kb + (kb > p.ring_index ? p.ring_size : 0);
  p.run_map[((int64_t)t * nqc + qg0 / p.q_chunk) * nkc + key0 / p.k_chunk] = 1;
}


// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (gfx9 encoding; expcnt and lgkmcnt not waited).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor words (base, stride 0, num_records, gfx9 word 3),
// wave-uniform and in scalar registers.
__device__ __forceinline__ i32x4_t rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = kRsrcWord3;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Bounds-checked buffer-to-LDS DMA of 16 (4) bytes per lane: lane l's bytes
// land at LDS address lds + 16 * l (4 * l); lanes whose offset is outside
// the descriptor write zeros.  Issued as inline asm on purpose: the compiler
// then does not track these LDS writes (its conservative tracking would add
// waits for all outstanding DMA before unrelated LDS reads); completion is
// enforced by the explicit vmcnt waits and barriers of the pipeline.
__device__ __forceinline__ void dma_b128(uint32_t lds, uint32_t voff, i32x4_t rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc));
}
__device__ __forceinline__ void dma_b32(uint32_t lds, uint32_t voff, i32x4_t rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc));
}

// Workgroup barrier publishing the LDS tiles written by DMA.  The LDS-only
// acquire fence keeps the compiler from reusing or hoisting LDS reads across
// it (it does not see the DMA writes) and costs only an LDS wait.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A tile in flight: the storage row of its first key in K and V, the end
// of the rows to visit in its block, its ring step and block, and vsh = key
// coordinate - storage row (0 for contiguous placement).  A tile with
// valid == 0 is past the end of the walk.
struct TileInfo {
  int32_t pk, end, t, kb, valid, vsh;
};

template <int TN, bool STRIPED = false>
__device__ __forceinline__ TileInfo tile_info(const FwdParams& p, const Cursor& c) {
  const int32_t base = c.kb * p.seq_q;
  const int32_t vsh = STRIPED ? block_vbase<true>(p, c.kb) - base : 0;
  return TileInfo{base + c.kt * TN, base + c.klen, c.t, c.kb, c.valid, vsh};
}

// Per-wave view of one tile: which 32-key halves have a visible pair and
// which need the causal or segment mask; pk is the key coordinate of the
// tile's first key.
struct TileFlags {
  bool run0, run1, mask0, mask1;
  // With segment ids: whether a half needs the per-element id test (set by
  // the caller from the ids in LDS; true until then).
  bool seg0, seg1;
  int32_t pk;
};

template <bool SEG, bool STRIPED = false>
__device__ __forceinline__ TileFlags tile_flags(const TileInfo& ti, const WaveLimits& lim) {
  TileFlags f;
  const int32_t pk = STRIPED ? ti.pk + ti.vsh : ti.pk;
  f.pk = pk;
  f.run0 = ti.valid && pk < lim.run_lim;
  f.run1 = ti.valid && ti.pk + 32 < ti.end && pk + 32 < lim.run_lim;
  f.mask0 = pk >= lim.mask_lim;
  f.mask1 = pk + 32 >= lim.mask_lim;
  f.seg0 = f.seg1 = SEG;
  return f;
}


// The two lanes holding one query row are l and l ^ 32.  Swapping the lane
// halves of x with itself leaves both values of the pair in every lane.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}


// Segment-id ranges.  When every key id of a tile lies outside the id range
// of a wave's queries (or the reverse), the tile holds no visible pair
// whatever the labelling, and skipping it changes nothing.  Packed documents
// then cost their within-document work instead of the whole causal triangle.
struct SegRange {
  int32_t lo, hi;
};

// [min, max] of x over each 32-lane half of the wave (the same in every lane
// of a half).
__device__ __forceinline__ SegRange half_range(int32_t x) {
  int32_t mn = x, mx = x;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    mn = min(mn, __shfl_xor(mn, o));
    mx = max(mx, __shfl_xor(mx, o));
  }
  return SegRange{mn, mx};
}

// [min, max] of x over the whole wave, wave-uniform.
__device__ __forceinline__ SegRange wave_range(int32_t x) {
  SegRange r = half_range(x);
  r.lo = min(r.lo, __shfl_xor(r.lo, 32));
  r.hi = max(r.hi, __shfl_xor(r.hi, 32));
  return SegRange{__builtin_amdgcn_readfirstlane(r.lo), __builtin_amdgcn_readfirstlane(r.hi)};
}

// Bit h (h = 0, 1) set iff the ids of the 32 keys sg[32h .. 32h + 31] of a
// 64-key tile in LDS overlap the range q; bit 2 + h set iff those keys and
// the queries all carry one and the same id, so that every pair of the half
// passes the id test.  Keys past the end of a block read as id 0, which can
// only widen a range.
__device__ __forceinline__ uint32_t seg_overlap_halves(const int32_t* sg, int lane, SegRange q) {
  const SegRange k = half_range(sg[lane]);
  const uint64_t b = __builtin_amdgcn_ballot_w64(k.hi >= q.lo && k.lo <= q.hi);
  const uint64_t u = __builtin_amdgcn_ballot_w64(k.lo == k.hi && q.lo == q.hi && k.lo == q.lo);
  return (uint32_t)(b & 1u) | ((uint32_t)(b >> 32) & 1u) << 1 | ((uint32_t)(u & 1u) << 2) |
         ((uint32_t)(u >> 32) & 1u) << 3;
}

// Workgroup-level tile mask for segment ids.  Before its walk a workgroup
// marks, for every 64-key tile slot (kb, kt) of the share (slot kb * TPB +
// kt, TPB = tiles per block), whether the tile's key ids overlap the id
// range of its queries; the walk then steps over unmarked tiles without
// fetching them.  Exact for any labelling, like the per-half test: disjoint
// ranges share no id.  The mask lives in LDS and is used only when the
// share has at most kSegMaskSlots slots.
constexpr int kSegMaskSlots = 8192;

__device__ __forceinline__ int seg_mask_tpb(const FwdParams& p) { return (p.seq_q + 63) / 64; }

// Fill mask[0 .. N * TPB) cooperatively, one slot per thread (tid of
// nthreads), so that every id load of the workgroup is in flight at once;
// keys past the end of a block take no part.  seg_b: the ids of one batch
// entry in storage order.  Slots of keys at or past kend_row (the first
// storage row no query of the workgroup can reach, for contiguous
// placement; the whole share otherwise) are left unmarked without reading
// their ids.
__device__ __forceinline__ void build_seg_mask(const FwdParams& p, const int32_t* seg_b,
                                               SegRange q, int64_t kend_row, uint8_t* mask,
                                               int tid, int nthreads) {
  const int tpb = seg_mask_tpb(p);
  const int n = p.ring_size * tpb;
  for (int t = tid; t < n; t += nthreads) {
    const int kb = t / tpb, kt = t - kb * tpb;
    const int64_t row0 = (int64_t)kb * p.seq_q + 64 * kt;
    const int nk = row0 < kend_row ? min(64, p.seq_q - 64 * kt) : 0;
    int32_t lo = INT32_MAX, hi = INT32_MIN;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      if (j < nk) {
        const int32_t v = seg_b[row0 + j];
        lo = min(lo, v);
        hi = max(hi, v);
      }
    }
    mask[t] = (nk > 0 && hi >= q.lo && lo <= q.hi) ? 1 : 0;
  }
}

// Advance the cursor past tiles the mask leaves unmarked.
template <int TN, bool STRIPED>
__device__ __forceinline__ void cursor_skip_masked(const FwdParams& p, Cursor& c, int64_t kend,
                                                   const uint8_t* mask) {
  static_assert(TN == 64, "the mask has one slot per 64-key tile");
  const int tpb = seg_mask_tpb(p);
#pragma clang loop vectorize(disable) unroll(disable)
  while (c.valid && __builtin_amdgcn_readfirstlane((int)mask[c.kb * tpb + c.kt]) == 0)
    cursor_next<TN, STRIPED>(p, c, kend);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Issue this wave's share of the DMA of one 64-row tile of two row-major
// tensors A and B (rows of rs_bytes bytes, D bf16 values used per row) and,
// when SEG, of the tile's 64 segment ids.  The WAVES waves of the workgroup
// split the tile: each DMA instruction moves 64 lanes x 16 bytes = 16 rows x
// 64 bytes, which lane l takes from row l % 16 (a_lane) or l / 4 (b_lane) of
// its 16-row group; a_lane / b_lane select the LDS layout of each tensor.
template <int D, int WAVES, bool SEG>
__device__ __forceinline__ void issue_tile(const TileInfo& ti, const char* abase0,
                                           const char* bbase0, const int32_t* sbase0,
                                           uint32_t rs_bytes, int wave, int lane, uint32_t a_lane,
                                           uint32_t b_lane, __bf16* ad, __bf16* bd, int32_t* sd) {
  constexpr int TN = 64, SLOTS = TN * D / 8, DPW = SLOTS / 64 / WAVES, SL = 64 / WAVES;
  static_assert(DPW * 64 * WAVES == SLOTS, "tile must split evenly over the waves");
  const int nvalid = std::min(TN, ti.end - ti.pk);
  const uint32_t bytes = (uint32_t)nvalid * rs_bytes;
  const uint64_t off = (uint64_t)(uint32_t)ti.pk * rs_bytes;
  const i32x4_t ar = rsrc_words(abase0 + off, bytes);
  const i32x4_t br = rsrc_words(bbase0 + off, bytes);
#pragma unroll
  for (int u = 0; u < DPW; ++u) {
    const int j = wave * DPW + u;
    const uint32_t joff = (uint32_t)(j & 3) * 16u * rs_bytes + 64u * (uint32_t)(j >> 2);
    dma_b128(lds_addr(ad + j * 512), a_lane + joff, ar);
    dma_b128(lds_addr(bd + j * 512), b_lane + joff, br);
  }
  if (SEG) {
    const i32x4_t sr = rsrc_words(sbase0 + ti.pk, (uint32_t)nvalid * 4u);
    if (lane < SL) dma_b32(lds_addr(sd + SL * wave), (uint32_t)(SL * wave + lane) * 4u, sr);
  }
}

// The same for one tensor: this wave's share of a 64-row tile of a
// row-major tensor, rows past ti.end read as zeros.
template <int D, int WAVES>
__device__ __forceinline__ void issue_rows(const TileInfo& ti, const char* base0,
                                           uint32_t rs_bytes, int wave, uint32_t lane_off,
                                           __bf16* dst) {
  constexpr int TN = 64, SLOTS = TN * D / 8, DPW = SLOTS / 64 / WAVES;
  static_assert(DPW * 64 * WAVES == SLOTS, "tile must split evenly over the waves");
  const int nvalid = std::min(TN, ti.end - ti.pk);
  const uint32_t bytes = nvalid > 0 ? (uint32_t)nvalid * rs_bytes : 0u;
  const i32x4_t r = rsrc_words(base0 + (uint64_t)(uint32_t)ti.pk * rs_bytes, bytes);
#pragma unroll
  for (int u = 0; u < DPW; ++u) {
    const int j = wave * DPW + u;
    const uint32_t joff = (uint32_t)(j & 3) * 16u * rs_bytes + 64u * (uint32_t)(j >> 2);
    dma_b128(lds_addr(dst + j * 512), lane_off + joff, r);
  }
}

}  // namespace
}  // namespace ra
