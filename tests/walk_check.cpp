// CPU check of the walk lengths and key-split run counts (csrc/ra_walk.h)
// that the host sizes grids with and the kernels map workgroups with.
//
//  * Every block's visited key count (block_klen) and a query tile's walk
//    length (walk_tiles, a closed form) against brute force from the
//    visibility definition: in block kb, the tile visits the keys up to the
//    last one that its last row sees (rows further on see at least as much:
//    floor(pq / c) grows with pq), rounded up to whole 32-key sub-tiles, in
//    tiles of tn keys.
//  * The run counts: between 1 and P, P for the longest walk, never
//    decreasing from one query tile to the next (the dq sum relies on it),
//    and the kernels' mapping of a head's workgroups (from the last query
//    tile down) hitting every (tile, run) exactly once for split_wgs
//    workgroups.
// Exit status 0 = every check passed.

#include <cstdint>
#include <cstdio>
#include <vector>

#include "ra_walk.h"

namespace w = ra::walk;

static long g_checks = 0, g_fail = 0;
#define CHECK(cond, ...)                                 \
  do {                                                   \
    ++g_checks;                                          \
    if (!(cond)) {                                       \
      if (g_fail < 20) {                                 \
        std::printf("FAILED line %d: %s | ", __LINE__, #cond); \
        std::printf(__VA_ARGS__);                        \
        std::printf("\n");                               \
      }                                                  \
      ++g_fail;                                          \
    }                                                    \
  } while (0)

// Is the key of local index j in block kb visible from local query row i?
// c = 0: no causal mask.  Positions as the placements define them.
static bool visible(int64_t Lq, int64_t N, int64_t r, bool striped, int64_t c, int64_t i,
                    int64_t kb, int64_t j) {
  if (c == 0) return true;
  const int64_t pq = striped ? i * N + r : r * Lq + i;
  const int64_t pk = striped ? j * N + kb : kb * Lq + j;
  return pq / c >= pk / c;
}

static int64_t brute_klen(int64_t Lq, int64_t N, int64_t r, bool striped, int64_t c,
                          int64_t last_row, int64_t kb) {
  int64_t last = -1;
  for (int64_t j = 0; j < Lq; ++j)
    if (visible(Lq, N, r, striped, c, last_row, kb, j)) last = j;
  if (last < 0) return 0;
  const int64_t l32 = (last + 1 + 31) / 32 * 32;
  return l32 < Lq ? l32 : Lq;
}

int main() {
  const int32_t seqs[] = {32, 64, 96, 160, 256, 288, 512};
  const int32_t rings[] = {1, 2, 3, 5, 8};
  long configs = 0;
  for (int32_t Lq : seqs)
    for (int32_t N : rings)
      for (int32_t r = 0; r < N; ++r)
        for (int striped = 0; striped < 2; ++striped) {
          const int64_t S = (int64_t)Lq * N;
          std::vector<int64_t> cs = {0, 1};
          for (int64_t c : std::vector<int64_t>{2, 3, 4, 5, 8, 10, 37, 64, 100, (int64_t)Lq,
                                                3 * (int64_t)Lq / 2, 2 * (int64_t)N, 4 * (int64_t)N,
                                                (int64_t)Lq * N / 2, S - 1, S, 2 * S})
            cs.push_back(c);
          for (int64_t c_raw : cs) {
            // the host passes c >= S as "no mask"
            const int64_t c0 = c_raw >= S ? 0 : c_raw;
            // Striped placement: the causal block in key coordinates, for
            // the blocks that have one (c divides N or is a multiple of it).
            const w::StripedCausal sc = w::striped_causal(c0, N, r);
            const bool supported = c0 == 0 || N % c0 == 0 || c0 % N == 0;
            CHECK(!striped || sc.ok == supported, "striped_causal ok N %d c %lld", N,
                  (long long)c0);
            if (striped && !sc.ok) continue;
            const int64_t c = striped ? sc.causal : c0;
            const int32_t shi = striped ? sc.stripe_hi : r + 1;
            CHECK(shi > r && shi <= N, "stripe_hi %d r %d N %d", shi, r, N);
            for (int32_t bm : {128, 256})
              for (int32_t tn : {32, 64}) {
                ++configs;
                const w::Share sh{Lq, N, r, c, striped != 0, bm, tn, shi};
                const int32_t nq = w::n_qtiles(sh);
                CHECK(nq == (Lq + bm - 1) / bm, "n_qtiles");
                std::vector<int64_t> walks(nq);
                for (int32_t qt = 0; qt < nq; ++qt) {
                  const int32_t m0 = qt * bm;
                  const int64_t last_row = std::min<int64_t>(m0 + bm, Lq) - 1;
                  const int64_t kend = w::tile_kend(c, Lq, r, striped != 0, m0, bm);
                  int64_t n_bf = 0;
                  for (int32_t kb = 0; kb < N; ++kb) {
                    const int64_t bf = brute_klen(Lq, N, r, striped != 0, c_raw, last_row, kb);
                    const int32_t got =
                        w::block_klen(Lq, w::block_vbase(Lq, shi, striped != 0, kb), kend);
                    CHECK(got == bf, "Lq %d N %d r %d striped %d c %lld bm %d qt %d kb %d: %d vs %lld",
                          Lq, N, r, striped, (long long)c_raw, bm, qt, kb, got, (long long)bf);
                    n_bf += (bf + tn - 1) / tn;
                  }
                  walks[qt] = w::qtile_walk(sh, qt);
                  CHECK(walks[qt] == n_bf, "walk Lq %d N %d r %d striped %d c %lld bm %d tn %d qt %d: %lld vs %lld",
                        Lq, N, r, striped, (long long)c_raw, bm, tn, qt, (long long)walks[qt],
                        (long long)n_bf);
                  CHECK(walks[qt] == w::walk_tiles(Lq, N, shi, striped != 0, tn, kend), "walk");
                }
                for (int32_t P = 1; P <= 64; P = P < 16 ? P + 1 : P * 2) {
                  int32_t prev = 0;
                  for (int32_t qt = 0; qt < nq; ++qt) {
                    const int32_t runs = w::qtile_runs(sh, P, qt);
                    CHECK(runs >= 1 && runs <= P, "runs %d P %d", runs, P);
                    CHECK(runs >= prev, "runs decrease at qt %d", qt);
                    prev = runs;
                  }
                  if (walks[nq - 1] > 0) CHECK(w::qtile_runs(sh, P, nq - 1) == P, "longest walk");
                  // The kernels' mapping of workgroup index -> (tile, split),
                  // counting runs from the last query tile down.
                  const int64_t wgs = w::split_wgs(sh, P);
                  std::vector<int> hit(wgs, 0);
                  for (int64_t in_bh = 0; in_bh < wgs; ++in_bh) {
                    int qt = -1, split = -1;
                    int64_t first = 0;
                    for (int32_t t = nq - 1; t >= 0; --t) {
                      const int32_t runs = w::qtile_runs(sh, P, t);
                      if (in_bh < first + runs) {
                        qt = t;
                        split = (int)(in_bh - first);
                        break;
                      }
                      first += runs;
                    }
                    CHECK(qt >= 0 && split >= 0 && split < w::qtile_runs(sh, P, qt),
                          "workgroup %lld unmapped", (long long)in_bh);
                    // position of (qt, split) in the head's run list
                    int64_t pos = split;
                    for (int32_t t = nq - 1; t > qt; --t) pos += w::qtile_runs(sh, P, t);
                    if (pos >= 0 && pos < wgs) ++hit[pos];
                  }
                  for (int64_t i = 0; i < wgs; ++i) CHECK(hit[i] == 1, "run %lld hit %d times",
                                                          (long long)i, hit[i]);
                }
              }
          }
        }
  std::printf("%ld configurations, %ld checks: %ld failure(s)\n", configs, g_checks, g_fail);
  return g_fail == 0 ? 0 : 1;
}
