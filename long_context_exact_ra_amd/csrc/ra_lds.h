// LDS layouts of the tiles that are read both as rows (ds_read_b128) and
// transposed (ds_read_b64_tr_b16): the backward's Q / dO / K / V tiles and
// the feedforward GEMM's W stage.  Plain constexpr functions of integers,
// compiled into the kernels and, by tests/lds_check.cpp, on the host, where
// every lane's operand is checked against the MFMA operand layout and every
// read against the 64 four-byte LDS banks.  Internal; not part of the C ABI.
//
// Units: 16-byte slots (8 bf16), element offsets in bf16.  LDS has 64 banks
// of 4 bytes, so 16 consecutive slots (256 bytes) cover every bank once; a
// ds_read_b128 serves 16 lanes per cycle, a ds_read_b64_tr_b16 32 lanes.
#pragma once

#include <stdint.h>

namespace ra {
namespace lds {

// ---------------------------------------------------------------------------
// Backward tiles: 64 rows x D columns (D / 8 granules of 16 bytes per row).
//   slot(r, g) = (g / 4) * 256 + (r / 16) * 64 + (g % 4) * 16 +
//                ((r % 16) ^ (4 * (g % 4)))
// A row read (16 lanes: 16 rows of one granule) and a column read (32
// lanes: 4 rows x 4 granules of a quad) each touch 16 slots that differ
// modulo 16.  Without the XOR the 4 rows of a column read would hit the same
// 4 of the 16 bank groups four times each.
// ---------------------------------------------------------------------------

constexpr int bwd_slot(int r, int g) {
  return (g / 4) * 256 + (r / 16) * 64 + (g % 4) * 16 + ((r % 16) ^ (4 * (g % 4)));
}

// A DMA instruction fills 64 consecutive slots (16 rows x one granule quad):
// lane l loads row dma_row(l) (within the 16) and granule dma_gran(l) (within
// the quad), the pair the layout puts in slot l of the block.
constexpr int bwd_dma_row(int lane) { return (lane & 15) ^ (4 * (lane >> 4)); }
constexpr int bwd_dma_gran(int lane) { return lane >> 4; }

// Row operand (the A operand of a 16-column k-step): lane l reads row
// 32 blk + l % 32, columns 16 c + 8 (l / 32) .. + 7.  row_rd is the lane's
// element offset for even c; odd c moves the granule by 2 within its quad,
// which flips bit 3 of the swizzled row: offset ^ 64.
constexpr int bwd_row_rd(int lane) {
  return 512 * ((lane & 31) >> 4) + 128 * (lane >> 5) + 8 * (((lane & 31) & 15) ^ (4 * (lane >> 5)));
}
constexpr int bwd_row_rd_c(int rd, int c) { return (c & 1) ? (rd ^ 64) : rd; }
constexpr int bwd_row_off(int c, int blk) { return 2048 * (c >> 1) + 256 * (c & 1) + 1024 * blk; }

// Column operand (the A operand of the transposed product) by two
// ds_read_b64_tr_b16: in each 16-lane group g, lane j reads 4 values of tile
// row 4 (g / 2) + j / 4 (+ 8 for the high read) at columns 32 jb + 16 (g % 2)
// + 4 (j % 4); rows + 8 flip bit 3 of the swizzled row: the high read is at
// offset ^ 64.  After the transpose, lane l holds for its column 32 jb +
// l % 32 the 8 tile rows 16 rb + 8 (l / 32) .. + 7.
constexpr int bwd_col_rd(int lane) {
  return ((2 * ((lane >> 4) & 1) + (((lane & 15) >> 1) & 1)) * 16 +
          ((4 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)) ^
           (4 * (2 * ((lane >> 4) & 1) + (((lane & 15) >> 1) & 1))))) * 8 +
         4 * (lane & 1);
}
constexpr int bwd_col_hi(int rd) { return rd ^ 64; }
constexpr int bwd_col_off(int jb, int rb) { return 2048 * jb + 512 * rb; }

// ---------------------------------------------------------------------------
// Feedforward GEMM, W stage: 32 rows k x BN / 8 granules, row-major with the
// granules of row k permuted: slot k * BN / 8 + j holds granule
// j ^ (4 (k % 4)).  Half a wave of one transposing read touches 4 rows x 4
// granules of a quad; a row is a multiple of 256 bytes, so the XOR puts the
// 4 rows in 4 different quads of bank groups.
// ---------------------------------------------------------------------------

constexpr int gemm_w_swz(int k) { return 4 * (k & 3); }
// The granule held by slot j of row k (and the slot of granule j): the
// permutation is its own inverse.
constexpr int gemm_w_gran(int k, int j) { return j ^ gemm_w_swz(k); }

// W^T operand of column block nb of a wave whose columns start at wn: lane
// (g16 = lane / 16, j16 = lane % 16) reads row kr = 8 (g16 / 2) + j16 / 4
// (+ 16 ks, + 4 for the second read; kr % 4 = j16 / 4 either way) at column
// wn + 32 nb + 16 (g16 % 2) + 4 (j16 % 4): element offset within the stage.
constexpr int gemm_w_rd(int lane, int wn, int nb, int bn) {
  return (8 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)) * bn +
         (((wn / 8 + 4 * nb + 2 * ((lane >> 4) & 1) + (((lane & 15) & 3) >> 1))) ^
          (4 * ((lane & 15) >> 2))) * 8 +
         4 * (lane & 1);
}

// ---------------------------------------------------------------------------
// Feedforward GEMM, X pair stage: BM rows m x 64 k (8 granules of 16 bytes:
// two 32-deep stages), so that a DMA instruction fetches whole 128-byte
// rows (8 rows x 8 granules): 16 rows x 64 bytes per instruction move at a
// fraction of the rate.  Blocks of 8 rows, granules permuted in odd blocks:
//   slot(m, g) = (m / 8) * 64 + (g ^ ((m / 8) % 2)) * 8 + m % 8
// A row read (ds_read_b128, 16 lanes: rows m0 .. m0 + 15 of one granule,
// m0 % 16 = 0) then touches 8 slots of an even block and 8 of an odd block
// that differ in bit 3: 16 slots distinct modulo 16, every bank once.
// ---------------------------------------------------------------------------

constexpr int gemm_x_slot(int m, int g) { return (m / 8) * 64 + (g ^ ((m / 8) & 1)) * 8 + m % 8; }
// DMA instruction i (rows 8 i .. 8 i + 7 of the pair tile), lane l writes
// slot 64 i + l: it loads row 8 i + l % 8 and granule (l / 8) ^ (i % 2).
constexpr int gemm_x_dma_row(int lane, int i) { return 8 * i + (lane & 7); }
constexpr int gemm_x_dma_gran(int lane, int i) { return (lane >> 3) ^ (i & 1); }
// X^T operand of row block mb (32 rows) of a wave whose rows start at wm
// (a multiple of 32), 16-k step ks of 32-deep stage sp within the pair:
// lane l reads row wm + 32 mb + l % 32, granule 4 sp + 2 ks + l / 32, as
// element offset gemm_x_rd(lane, wm) + 2048 mb + 256 sp + 128 ks.
constexpr int gemm_x_rd(int lane, int wm) {
  return 8 * gemm_x_slot(wm + (lane & 31), lane >> 5);
}

}  // namespace lds
}  // namespace ra
