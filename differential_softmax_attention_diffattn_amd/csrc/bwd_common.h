// Tile helpers shared by the backward kernels (V1 and V2): swizzled LDS
// layouts of 64-row bf16 tiles and their direct-to-LDS loader.
#pragma once

#include "device_common.h"

namespace diffattn {
namespace bwd {

constexpr int kWaves = 8;  // waves of the 512-thread backward workgroups

template <int D>
struct BTile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;  // 16-byte chunks per row
  static constexpr int kBytes = 64 * kRowBytes;
  static constexpr int kInstr = kBytes / 1024;
};

// Two LDS layouts of a 64-row bf16 tile (row-major, swizzled):
//  * rows: 16-byte chunk c of row r at position c ^ (r mod nchunks), for
//    16-byte row reads (an MFMA operand whose k index runs along a row);
//  * trans: 32-byte chunk c of row r at position c ^ trans_swz(r), for the
//    transposing read (an operand whose k index runs down the rows).
// trans_swz is a permutation of the D/16 chunk positions over rows r mod
// D/16.  For D = 128 (256-byte rows, one row per pass over the 64 banks) it
// is r mod 8 with its bits rotated, (r mod 4) * 2 + (r / 4 mod 2): then any 8
// consecutive rows fall on 8 different positions (the 16x16 transposing reads
// of 8 rows, the 16-byte row reads), and so do two adjacent chunks of any 4
// rows 4h .. 4h+3 (the 32x32 transposing reads, whose first 32 lanes take
// 4 rows x 64 bytes); with the plain r mod 8 those two chunks of 4 rows
// cover only 4 positions, a two-way bank conflict.  For D = 64 (two rows per
// pass) r mod 4 already keeps both patterns apart.
template <int D>
__device__ __forceinline__ int trans_swz(int row) {
  if constexpr (D / 16 == 8) return ((row & 3) << 1) | ((row >> 2) & 1);
  return row & (D / 16 - 1);
}
template <int D>
__device__ __forceinline__ int rows_offset(int row, int chunk) {
  return row * BTile<D>::kRowBytes + ((chunk ^ (row & (BTile<D>::kChunks - 1))) << 4);
}
template <int D>
__device__ __forceinline__ int trans_offset(int row, int byte_in_row) {
  const int c32 = byte_in_row >> 5;
  return row * BTile<D>::kRowBytes + ((c32 ^ trans_swz<D>(row)) << 5) + (byte_in_row & 31);
}

// The same offsets as one base per (row, byte) XORed with the chunk index:
// trans_offset<D>(row, 32 c + b) == trans_base<D>(row, b) ^ (c << 5) and
// rows_offset<D>(row, c) == rows_base<D>(row) ^ (c << 4) (the row's bits sit
// above the chunk bits), so a loop over chunks costs one XOR per read.
template <int D>
__device__ __forceinline__ int trans_base(int row, int byte_in_chunk) {
  return row * BTile<D>::kRowBytes | (trans_swz<D>(row) << 5) | byte_in_chunk;
}
template <int D>
__device__ __forceinline__ int rows_base(int row) {
  return row * BTile<D>::kRowBytes | ((row & (BTile<D>::kChunks - 1)) << 4);
}

// Direct-to-LDS load of a ROWS-row tile: rows r0 .. r0+ROWS-1 of a bf16 matrix
// whose consecutive rows are `stride` elements apart, rows >= n_valid clamped
// to the last valid row (their values are masked by the caller).  TRANS
// selects the layout.  The tile is ROWS * D * 2 / 1024 loads of 1 KiB, dealt
// round-robin to the NW waves.
template <int D, bool TRANS, int NW = kWaves, int ROWS = 64>
__device__ __forceinline__ void load_tile(const uint16_t* base, size_t stride, int n_valid,
                                          uint8_t* lds, int wave, int lane) {
  using TL = BTile<D>;
  constexpr int kInstr = ROWS * TL::kRowBytes / 1024;
#pragma unroll
  for (int j = 0; j < (kInstr + NW - 1) / NW; ++j) {
    const int blk = wave + j * NW;
    if (kInstr % NW != 0 && blk >= kInstr) break;
    const int off = blk * 1024 + lane * 16;  // LDS byte this lane fills
    const int r = off / TL::kRowBytes;
    const int pos = (off % TL::kRowBytes) >> 4;
    int lc;  // logical 16-byte chunk stored at that position
    if (TRANS) {
      lc = (((pos >> 1) ^ trans_swz<D>(r)) << 1) | (pos & 1);
    } else {
      lc = pos ^ (r & (TL::kChunks - 1));
    }
    const size_t row = (size_t)min(r, n_valid - 1);
    dma16(base, (uint32_t)((row * stride + lc * 8) * 2), lds + blk * 1024);
  }
}

// Loader of ROWS-row tiles of one layout and row stride that keeps, per lane,
// one 32-bit byte offset per load of a full tile (computed once), so a full
// tile costs no address arithmetic: the tile base moves in scalar registers.
// Only a ragged tile (fewer than ROWS valid rows, the last of a sequence)
// takes the clamping load_tile path, from a lane index made opaque there so
// that path's offsets are not hoisted and kept live across the caller's loop.
template <int D, bool TRANS, int NW = kWaves, int ROWS = 64>
struct TileLoader {
  static constexpr int kInstr = ROWS * BTile<D>::kRowBytes / 1024;
  static constexpr int kJ = (kInstr + NW - 1) / NW;
  uint32_t off[kJ];
  size_t stride;

  __device__ __forceinline__ TileLoader(size_t stride_, int wave, int lane) : stride(stride_) {
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int o = (wave + j * NW) * 1024 + lane * 16;  // LDS byte this lane fills
      const int r = o / BTile<D>::kRowBytes;
      const int pos = (o % BTile<D>::kRowBytes) >> 4;
      int lc;
      if (TRANS) {
        lc = (((pos >> 1) ^ trans_swz<D>(r)) << 1) | (pos & 1);
      } else {
        lc = pos ^ (r & (BTile<D>::kChunks - 1));
      }
      off[j] = (uint32_t)((r * stride + lc * 8) * 2);
    }
  }
  // rows 0 .. ROWS-1 of the tile at `base`, of which n_valid are valid
  __device__ __forceinline__ void load(const uint16_t* base, int n_valid, uint8_t* lds, int wave,
                                       int lane) const {
    if (n_valid >= ROWS) {
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const int blk = wave + j * NW;
        if (kInstr % NW != 0 && blk >= kInstr) break;
        dma16(base, off[j], lds + blk * 1024);
      }
    } else {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      load_tile<D, TRANS, NW, ROWS>(base, stride, n_valid, lds, wave, ln);
    }
  }
};

}  // namespace bwd
}  // namespace diffattn
