// CPU check of the LDS layouts that are read both as rows and transposed
// (long_context_exact_ra_amd/csrc/ra_lds.h): every lane of every operand
// read receives the tile elements the MFMA operand layout asks for, the DMA
// puts every (row, granule) where the readers look for it, and every read
// touches each of the 64 four-byte banks exactly once per cycle.
//
// Hardware facts used (gfx950):
//  * v_mfma_f32_32x32x16_bf16: operand lane l holds row (A) or column (B)
//    l % 32 and the 8 consecutive k of k-slot group l / 32.
//  * ds_read_b128: 16 lanes per cycle; ds_read_b64_tr_b16: 32 lanes per
//    cycle, and within each group of 16 lanes, destination lane i, element e
//    receives element i % 4 of the 4 that source lane 4 e + i / 4 addresses.
//  * buffer_load_dwordx4 ... lds: lane l of a DMA instruction writes 16
//    bytes at LDS slot base + l.
// Exit status 0 = every check passed.

#include <cstdint>
#include <cstdio>
#include <map>
#include <set>
#include <utility>
#include <vector>

#include "ra_lds.h"

namespace l = ra::lds;

static long g_checks = 0, g_fail = 0;
#define CHECK(cond, ...)                                         \
  do {                                                           \
    ++g_checks;                                                  \
    if (!(cond)) {                                               \
      if (g_fail < 20) {                                         \
        std::printf("FAILED line %d: %s | ", __LINE__, #cond);  \
        std::printf(__VA_ARGS__);                                \
        std::printf("\n");                                       \
      }                                                          \
      ++g_fail;                                                  \
    }                                                            \
  } while (0)

// Banks (4-byte words mod 64) touched by reads of `bytes` each at the given
// byte addresses: every bank exactly once?
static bool covers_all_banks_once(const std::vector<int>& byte_addr, int bytes) {
  std::vector<int> n(64, 0);
  for (int a : byte_addr)
    for (int w = 0; w < bytes / 4; ++w) ++n[(a / 4 + w) % 64];
  for (int b = 0; b < 64; ++b)
    if (n[b] != 1) return false;
  return true;
}

// Element of a transposing read: what destination lane `lane` gets as its
// element e (0..3), given each lane's element offset `src` of its 4-element
// read.  Returns the element offset read.
static int tr_element(const std::vector<int>& src, int lane, int e) {
  const int g = lane / 16, i = lane % 16;
  const int s = 16 * g + 4 * e + i / 4;
  return src[s] + i % 4;
}

static void check_bwd(int D) {
  const int G = D / 8;  // granules per row
  // slot -> (row, granule), and the layout is a bijection
  std::map<int, std::pair<int, int>> at;
  for (int r = 0; r < 64; ++r)
    for (int g = 0; g < G; ++g) {
      const int s = l::bwd_slot(r, g);
      CHECK(s >= 0 && s < 64 * G, "slot range D %d r %d g %d", D, r, g);
      CHECK(at.count(s) == 0, "slot %d used twice", s);
      at[s] = {r, g};
    }
  // element offset -> (row, column)
  auto elem = [&](int e) {
    const auto rg = at.at(e / 8);
    return std::make_pair(rg.first, rg.second * 8 + e % 8);
  };
  // DMA: instruction j fills slots 64 j .. + 63 with rows 16 (j % 4) .. of
  // granule quad j / 4; lane l loads (row, granule) = dma_row, dma_gran.
  for (int j = 0; j < 64 * G / 64; ++j)
    for (int lane = 0; lane < 64; ++lane) {
      const int r = 16 * (j & 3) + l::bwd_dma_row(lane), g = 4 * (j >> 2) + l::bwd_dma_gran(lane);
      CHECK(l::bwd_slot(r, g) == 64 * j + lane, "dma D %d j %d lane %d", D, j, lane);
    }
  // Row operand: lane l, k-step c, 32-row block blk -> row 32 blk + l % 32,
  // columns 16 c + 8 (l / 32) + 0..7.
  for (int c = 0; c < D / 16; ++c)
    for (int blk = 0; blk < 2; ++blk) {
      std::vector<int> addr(64);
      for (int lane = 0; lane < 64; ++lane) {
        const int e0 = l::bwd_row_rd_c(l::bwd_row_rd(lane), c) + l::bwd_row_off(c, blk);
        CHECK(e0 % 8 == 0, "row read not slot aligned");
        for (int k = 0; k < 8; ++k) {
          const auto rc = elem(e0 + k);
          CHECK(rc.first == 32 * blk + lane % 32 && rc.second == 16 * c + 8 * (lane / 32) + k,
                "row operand D %d c %d blk %d lane %d k %d", D, c, blk, lane, k);
        }
        addr[lane] = 2 * e0;
      }
      for (int q = 0; q < 4; ++q)
        CHECK(covers_all_banks_once(std::vector<int>(addr.begin() + 16 * q, addr.begin() + 16 * q + 16), 16),
              "row read banks D %d c %d blk %d quarter %d", D, c, blk, q);
    }
  // Column operand: lane l, 32-column block jb, 16-row block rb -> column
  // 32 jb + l % 32 and, for its k-slots s = 0..7 (low read 0..3, high
  // 4..7), tile rows 16 rb + 8 (s / 4) + 4 (l / 32) + s % 4: the order in
  // which the other operand of these products (P or dS, converted from the
  // C registers of the score MFMA, whose lane half h holds rows 8 (i / 4) +
  // 4 h + i % 4) presents the same rows, so the contraction pairs them.
  for (int jb = 0; jb < D / 32; ++jb)
    for (int rb = 0; rb < 4; ++rb)
      for (int hi = 0; hi < 2; ++hi) {
        std::vector<int> src(64), addr(64);
        for (int lane = 0; lane < 64; ++lane) {
          const int rd = l::bwd_col_rd(lane);
          src[lane] = (hi ? l::bwd_col_hi(rd) : rd) + l::bwd_col_off(jb, rb);
          CHECK(src[lane] % 4 == 0, "column read not 8-byte aligned");
          addr[lane] = 2 * src[lane];
        }
        for (int lane = 0; lane < 64; ++lane)
          for (int e = 0; e < 4; ++e) {
            const auto rc = elem(tr_element(src, lane, e));
            CHECK(rc.second == 32 * jb + lane % 32 &&
                      rc.first == 16 * rb + 8 * hi + 4 * (lane / 32) + e,
                  "column operand D %d jb %d rb %d hi %d lane %d e %d: row %d col %d", D, jb, rb,
                  hi, lane, e, rc.first, rc.second);
          }
        for (int h = 0; h < 2; ++h)
          CHECK(covers_all_banks_once(std::vector<int>(addr.begin() + 32 * h, addr.begin() + 32 * h + 32), 8),
                "column read banks D %d jb %d rb %d hi %d half %d", D, jb, rb, hi, h);
      }
}

// The GEMM's W stage: 32 rows k x BN columns; slot k * BN / 8 + j holds
// granule gemm_w_gran(k, j).  A DMA instruction fetches whole rows: lane l
// writes slot base + l, i.e. row k = RPI i + l / GPR, slot j = l % GPR.
static void check_gemm_w(int BN) {
  const int GPR = BN / 8;
  auto elem = [&](int e) {  // element offset -> (k, column)
    const int s = e / 8, k = s / GPR, j = s % GPR;
    return std::make_pair(k, 8 * l::gemm_w_gran(k, j) + e % 8);
  };
  // the permutation of each row is a bijection
  for (int k = 0; k < 32; ++k) {
    std::set<int> seen;
    for (int j = 0; j < GPR; ++j) seen.insert(l::gemm_w_gran(k, j));
    CHECK((int)seen.size() == GPR && *seen.begin() == 0 && *seen.rbegin() == GPR - 1,
          "W permutation BN %d k %d", BN, k);
    for (int j = 0; j < GPR; ++j)
      CHECK(l::gemm_w_gran(k, l::gemm_w_gran(k, j)) == j, "W permutation not an involution");
  }
  const int WN = BN / 2, NB = WN / 32;
  for (int wq = 0; wq < 2; ++wq) {
    const int wn = wq * WN;
    for (int nb = 0; nb < NB; ++nb)
      for (int ks = 0; ks < 2; ++ks)
        for (int hi = 0; hi < 2; ++hi) {
          std::vector<int> src(64), addr(64);
          for (int lane = 0; lane < 64; ++lane) {
            src[lane] = l::gemm_w_rd(lane, wn, nb, BN) + ks * 16 * BN + hi * 4 * BN;
            addr[lane] = 2 * src[lane];
          }
          // W^T operand: lane l holds column wn + 32 nb + l % 32, k = 16 ks +
          // 8 (l / 32) + 4 hi + e: the contiguous k-slots of the X^T operand's
          // row reads (granule 2 ks + l / 32 of row m).
          for (int lane = 0; lane < 64; ++lane)
            for (int e = 0; e < 4; ++e) {
              const auto kc = elem(tr_element(src, lane, e));
              CHECK(kc.second == wn + 32 * nb + lane % 32 &&
                        kc.first == 16 * ks + 8 * (lane / 32) + 4 * hi + e,
                    "W operand BN %d wn %d nb %d ks %d hi %d lane %d e %d", BN, wn, nb, ks, hi,
                    lane, e);
            }
          for (int h = 0; h < 2; ++h)
            CHECK(covers_all_banks_once(std::vector<int>(addr.begin() + 32 * h, addr.begin() + 32 * h + 32), 8),
                  "W read banks BN %d nb %d ks %d hi %d half %d", BN, nb, ks, hi, h);
        }
  }
}

// The GEMM's X pair stage: BM rows x 8 granules (64 k).  The slot map is a
// bijection, DMA instruction i places (row, granule) where the layout wants
// them while reading whole 128-byte rows, and every X^T operand read gives
// lane l row wm + 32 mb + l % 32 and k = 32 sp + 16 ks + 8 (l / 32) .. + 7
// (the k-slots the W^T operand pairs with) and touches every bank once per
// 16 lanes.
static void check_gemm_x(int BM) {
  std::map<int, std::pair<int, int>> at;
  for (int m = 0; m < BM; ++m)
    for (int g = 0; g < 8; ++g) {
      const int s = l::gemm_x_slot(m, g);
      CHECK(s >= 0 && s < BM * 8, "X slot range BM %d m %d g %d", BM, m, g);
      CHECK(at.count(s) == 0, "X slot %d used twice", s);
      at[s] = {m, g};
    }
  for (int i = 0; i < BM / 8; ++i) {
    std::set<int> rows;
    for (int lane = 0; lane < 64; ++lane) {
      const int m = l::gemm_x_dma_row(lane, i), g = l::gemm_x_dma_gran(lane, i);
      CHECK(l::gemm_x_slot(m, g) == 64 * i + lane, "X dma BM %d i %d lane %d", BM, i, lane);
      rows.insert(m);
    }
    // whole rows: 8 rows, each with all 8 granules
    CHECK((int)rows.size() == 8, "X dma instruction %d covers %d rows", i, (int)rows.size());
  }
  for (int wm : {0, BM / 2})
    for (int mb = 0; mb < BM / 2 / 32; ++mb)
      for (int sp = 0; sp < 2; ++sp)
        for (int ks = 0; ks < 2; ++ks) {
          std::vector<int> addr(64);
          for (int lane = 0; lane < 64; ++lane) {
            const int e0 = l::gemm_x_rd(lane, wm) + 2048 * mb + 256 * sp + 128 * ks;
            CHECK(e0 % 8 == 0, "X read not slot aligned");
            const auto mg = at.at(e0 / 8);
            CHECK(mg.first == wm + 32 * mb + lane % 32 && 8 * mg.second == 32 * sp + 16 * ks + 8 * (lane / 32),
                  "X operand BM %d wm %d mb %d sp %d ks %d lane %d: row %d granule %d", BM, wm, mb, sp,
                  ks, lane, mg.first, mg.second);
            addr[lane] = 2 * e0;
          }
          for (int q = 0; q < 4; ++q)
            CHECK(covers_all_banks_once(std::vector<int>(addr.begin() + 16 * q, addr.begin() + 16 * q + 16), 16),
                  "X read banks BM %d wm %d mb %d sp %d ks %d quarter %d", BM, wm, mb, sp, ks, q);
        }
}

// The checker's own sensitivity: the unswizzled layout (slot (g / 4) * 256
// + (r / 16) * 64 + (g % 4) * 16 + r % 16, the forward's K layout) gives the
// same elements to every lane but a 4-way bank conflict on every column
// read, which the bank test must report.
static void check_detects_conflicts() {
  int conflicted = 0, reads = 0;
  for (int jb = 0; jb < 4; ++jb)
    for (int rb = 0; rb < 4; ++rb) {
      std::vector<int> addr(32);
      for (int lane = 0; lane < 32; ++lane) {
        const int g = lane >> 4, j = lane & 15;
        const int slot = (2 * (g & 1) + ((j >> 1) & 1)) * 16 + 4 * (g >> 1) + (j >> 2);
        addr[lane] = 2 * (slot * 8 + 4 * (j & 1) + l::bwd_col_off(jb, rb));
      }
      ++reads;
      conflicted += !covers_all_banks_once(addr, 8);
    }
  CHECK(conflicted == reads, "the unswizzled column reads should all conflict (%d of %d)",
        conflicted, reads);
}

int main() {
  check_detects_conflicts();
  for (int D : {64, 128}) check_bwd(D);
  for (int BN : {128, 256}) check_gemm_w(BN);
  for (int BM : {128, 256}) check_gemm_x(BM);
  std::printf("%ld checks: %ld failure(s)\n", g_checks, g_fail);
  return g_fail == 0 ? 0 : 1;
}
