// Backward building blocks for eight-wavefront workgroups.
//
// Every staged tile is 64 rows x D, row-major, copied HBM -> LDS directly (no registers),
// with the 16-byte chunk c of row r stored at chunk position c ^ swz(r).  Two kinds of
// MFMA operand come out of such a tile:
//  * row fragments (lane = row, 8 consecutive columns): one 16-byte read;
//  * transposed fragments (lane = column, 8 rows in accumulator slot order): two
//    ds_read_b64_tr_b16 reads.  That instruction transposes 4x16 b16 blocks across each
//    group of 16 lanes: output lane i of a group receives, for j = 0..3, element i % 4 of
//    the 8 bytes addressed by source lane 4j + i / 4.  Source lane t therefore points at
//    row rb + t / 4, columns cb + 4 (t % 4) .. +3, and output lane i ends up holding
//    column cb + i of rows rb .. rb + 3.
// swz() keeps both kinds of read free of bank conflicts on gfx950 (checked with the LDS
// counters).  Row reads: 16 consecutive rows map to 16 distinct positions.  Transposed
// reads: the 32 lanes served together read 4 aligned rows (two 16-column halves); their
// positions must fall in different blocks of 4 chunks, i.e. swz >> 2 differs across the 4
// rows at d = 128, and between the two rows of each parity at d = 64 (where a 256-byte
// bank line holds two rows).  The previous map, ((r & 7) << 1) | ((r >> 3) & 1), cost every
// transposed read a second cycle.
#pragma once

#include "common.h"

namespace s2a {

typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1);
}

// Direct copy of a 64 x D tile (row stride `rstride` elements in HBM) into `lds`.
template <int D, int NW>
__device__ __forceinline__ void tile_direct(const bf16_t* base, long rstride, bf16_t* lds, int w, int lane) {
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;
  constexpr int INSTS = kTile / RPI;
  static_assert(INSTS % NW == 0, "tile copy must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < INSTS / NW; ++i) {
    const int inst = w * (INSTS / NW) + i;
    const int row = inst * RPI + lane / CPR;
    const int cpos = lane % CPR;
    load_lds16(base + row * rstride + (cpos ^ swz<D>(row)) * 8, lds + inst * 512);
  }
}

// Direct copy of 64 floats (one wave-instruction: 4 bytes per lane).
__device__ __forceinline__ void floats_direct(const float* src, float* lds, int lane) {
  __builtin_amdgcn_global_load_lds(src + lane, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// Row fragment: row `row`, logical chunk `chunk` (8 columns).
template <int D>
__device__ __forceinline__ bf16x8_t row_frag(const bf16_t* tile, int row, int chunk) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(tile + row * D + ((chunk ^ swz<D>(row)) << 3)));
}

// Transposed fragment for a K-step over rows 16 kb .. 16 kb + 15 and columns
// 32 nb + lq: slots 0..3 = rows 16kb + 4g + 0..3, slots 4..7 = rows 16kb + 8 + 4g + 0..3.
template <int D>
__device__ __forceinline__ bf16x8_t tr_frag(const bf16_t* tile, int nb, int kb, int lq, int g) {
  const int t = lq & 15;
  const int col = 32 * nb + 16 * (lq >> 4) + 4 * (t & 3);
  const int r1 = 16 * kb + 4 * g + (t >> 2);
  const int r2 = r1 + 8;
  const bf16_t* a1 = tile + r1 * D + (((col >> 3) ^ swz<D>(r1)) << 3) + (col & 7);
  const bf16_t* a2 = tile + r2 * D + (((col >> 3) ^ swz<D>(r2)) << 3) + (col & 7);
  const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t __attribute__((address_space(3)))*)a1);
  const s16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t __attribute__((address_space(3)))*)a2);
  const uint2 ux = __builtin_bit_cast(uint2, x), uy = __builtin_bit_cast(uint2, y);
  return as_bf16x8(uint4{ux.x, ux.y, uy.x, uy.y});
}

// Writes a transposed accumulator (lane = row lq, registers over columns) scaled by
// `mul` as bf16 into row `row` (D contiguous columns).
template <int D>
__device__ __forceinline__ void store_acc_row(const f32x16_t (&acc)[D / 32], float mul, bf16_t* row, int g) {
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint2 w;
      w.x = pack_bf16(acc[nb][4 * i + 0] * mul, acc[nb][4 * i + 1] * mul);
      w.y = pack_bf16(acc[nb][4 * i + 2] * mul, acc[nb][4 * i + 3] * mul);
      *reinterpret_cast<uint2*>(row + 32 * nb + 8 * i + 4 * g) = w;
    }
  }
}


}  // namespace s2a
