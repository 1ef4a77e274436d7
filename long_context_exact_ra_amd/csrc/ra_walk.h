// The length of a query tile's walk over the keys and its cut into key-split
// runs: one definition, compiled into the host side of the C ABI (grid
// sizes, the split count) and into the kernels (the workgroup mapping, the
// combine and the dq sum), so that the number of workgroups the host
// launches and the number of runs the kernels map them to can never come
// from two different formulas.  Plain constexpr functions of integers: HIP
// makes them callable from host and device code alike, and g++ compiles
// them for the host side.  Internal; not part of the C ABI.
//
// Terms.  A query tile (bm local rows from m0) of ring position r visits, in
// every key/value block, the keys up to its causal limit, rounded up to whole
// 32-key sub-tiles, in tiles of tn keys ("3. 因果注意力掩码支持" skips the
// rest).  Key coordinates: contiguous placement, key j of block kb has
// coordinate kb * Lq + j and query row i has coordinate r * Lq + i.  Striped
// placement (query row i of device r at position i * N + r, key j of block
// kb at j * N + kb): query row i has coordinate i and key j of block kb has
// coordinate j + [kb >= stripe_hi], with the causal block c' below
// (striped_causal), so that floor(i N + r, c) >= floor(j N + kb, c) holds
// exactly when floor(i / c') >= floor((j + [kb >= stripe_hi]) / c').
#pragma once

#include <stdint.h>

namespace ra {
namespace walk {

constexpr int64_t kNoLimit = INT64_MAX;

// Striped placement with causal block c (0 < c < N Lq), in coordinates.
//  * c divides N: floor((i N + r) / c) = i N / c + floor(r / c), so key j of
//    block kb is visible from row i iff i > j, or i = j and floor(kb / c) <=
//    floor(r / c): token causal (c' = 1) on the coordinates i and j + [kb >=
//    stripe_hi] with stripe_hi = (floor(r / c) + 1) c.  c = 1 gives the
//    token-causal rule j + [kb > r] <= i.
//  * N divides c: floor((i N + r) / c) = floor(i / (c / N)) because r < N,
//    and the same for keys: block causal with c' = c / N on the local
//    indices, the same in every block (stripe_hi = N: no shift).
//  * Any other c mixes the two and has no such form: not supported.
// c = 0 (no mask): c' = 0, and the shift of blocks kb > r is kept (it only
// orders the walk).
struct StripedCausal {
  int64_t causal;     // c' (0: no mask)
  int32_t stripe_hi;  // blocks kb >= stripe_hi have coordinates from 1
  bool ok;            // c is 0, divides N or is a multiple of N
};

constexpr StripedCausal striped_causal(int64_t c, int32_t ring_size, int32_t ring_index) {
  if (c <= 0) return StripedCausal{0, ring_index + 1, true};
  if (c <= ring_size) {
    if (ring_size % c != 0) return StripedCausal{0, 0, false};
    return StripedCausal{1, (int32_t)((ring_index / c + 1) * c), true};
  }
  if (c % ring_size != 0) return StripedCausal{0, 0, false};
  return StripedCausal{c / ring_size, ring_size, true};
}

// First key coordinate no row of the query tile [m0, m0 + bm) can see
// (kNoLimit when non-causal; c is the effective causal block size, below
// seq_k whenever it is not 0).  32-bit division: the last row's coordinate
// and c are below 2^31.
constexpr int64_t tile_kend(int64_t c, int32_t seq_q, int32_t ring_index, bool striped,
                            int32_t m0, int32_t bm) {
  if (c == 0) return kNoLimit;
  const int32_t last_row = (m0 + bm < seq_q ? m0 + bm : seq_q) - 1;
  const uint32_t q_last = (uint32_t)((striped ? 0 : ring_index * seq_q) + last_row);
  const uint32_t cc = (uint32_t)c;
  return ((int64_t)(q_last / cc) + 1) * cc;
}

// Coordinate of block kb's first key (stripe_hi: striped placement only).
constexpr int32_t block_vbase(int32_t seq_q, int32_t stripe_hi, bool striped, int32_t kb) {
  return striped ? (kb >= stripe_hi ? 1 : 0) : kb * seq_q;
}

// Keys of a block (first key at coordinate vbase) before kend, rounded up
// to whole 32-key sub-tiles and capped at the block length.
constexpr int32_t block_klen(int32_t seq_q, int64_t vbase, int64_t kend) {
  const int64_t len = kend == kNoLimit ? seq_q : kend - vbase;
  if (len <= 0) return 0;
  if (len >= seq_q) return seq_q;
  const int32_t l32 = ((int32_t)len + 31) & ~31;
  return l32 > seq_q ? seq_q : l32;
}

constexpr int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

// Tiles of tn keys in the walk up to kend, in closed form.  Contiguous:
// the blocks before kend / Lq are whole, the next one is cut at kend, the
// rest are empty.  Striped: blocks kb < stripe_hi (stripe_hi of them) and
// kb >= stripe_hi (N - stripe_hi) each have one count.
constexpr int64_t walk_tiles(int32_t seq_q, int32_t ring_size, int32_t stripe_hi, bool striped,
                             int32_t tn, int64_t kend) {
  if (striped) {
    const int32_t lo = ceil_div(block_klen(seq_q, 0, kend), tn);
    const int32_t hi = ceil_div(block_klen(seq_q, 1, kend), tn);
    return (int64_t)stripe_hi * lo + (int64_t)(ring_size - stripe_hi) * hi;
  }
  const int32_t full = ceil_div(seq_q, tn);
  if (kend >= (int64_t)ring_size * seq_q) return (int64_t)ring_size * full;
  const int32_t nfull = (int32_t)kend / seq_q;  // kend < N Lq < 2^31
  return (int64_t)nfull * full +
         ceil_div(block_klen(seq_q, (int64_t)nfull * seq_q, kend), tn);
}

// Runs of a walk of n tiles when the share's longest walk (n_max tiles, its
// last query tile's: causal limits only grow with the row) takes P runs:
// ceil(P n / n_max), between 1 and P, so that runs are about equally long.
constexpr int32_t split_runs(int32_t P, int64_t n, int64_t n_max) {
  const int64_t runs = n_max > 0 ? ((int64_t)P * n + n_max - 1) / n_max : 1;
  return (int32_t)(runs < 1 ? 1 : (runs > P ? P : runs));
}

// Everything the run count of one query tile depends on.
struct Share {
  int32_t seq_q, ring_size, ring_index;
  int64_t causal;  // effective causal block size (striped: c' in coordinates), 0 = none
  bool striped;
  int32_t bm, tn;     // rows per query tile, keys per key tile
  int32_t stripe_hi;  // striped placement: the first shifted block
};

constexpr int32_t n_qtiles(const Share& s) { return ceil_div(s.seq_q, s.bm); }

constexpr int64_t qtile_walk(const Share& s, int32_t qt) {
  return walk_tiles(s.seq_q, s.ring_size, s.stripe_hi, s.striped, s.tn,
                    tile_kend(s.causal, s.seq_q, s.ring_index, s.striped, qt * s.bm, s.bm));
}

// Runs of query tile qt with P key splits.
constexpr int32_t qtile_runs(const Share& s, int32_t P, int32_t qt) {
  return split_runs(P, qtile_walk(s, qt), qtile_walk(s, n_qtiles(s) - 1));
}

// Workgroups per (batch, head) of a split launch: the runs of every query
// tile.  The kernels map workgroup w of a head to (query tile, split) by
// counting the same runs from the last (heaviest) tile down.
constexpr int64_t split_wgs(const Share& s, int32_t P) {
  int64_t w = 0;
  for (int32_t qt = 0; qt < n_qtiles(s); ++qt) w += qtile_runs(s, P, qt);
  return w;
}

}  // namespace walk
}  // namespace ra
