// Tile building blocks shared by the backward and the forward's P.V product.
//
// Every staged tile is rows x D, row-major, copied HBM -> LDS directly (no registers),
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
// transposed read a second cycle.  The kernels compute each lane's read and copy offsets
// once (attn_bwd.hip: KvfOffsets, CopyOffsets, HalfCopy).
#pragma once

#include "common.h"

namespace s2a {

typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1);
}

// Direct copy of 64 floats (one wave-instruction: 4 bytes per lane).
__device__ __forceinline__ void floats_direct(const float* src, float* lds, int lane) {
  __builtin_amdgcn_global_load_lds(src + lane, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// Per-lane source offsets (elements) of one wave's share of a 64-row tile copy:
// instruction i of wave w covers rows (w * PER + i) * RPI .. + RPI - 1, 16 bytes per lane
// into LDS at the swizzled chunk position; computed once, so a copy is one address add
// per instruction.
template <int D, int NW>
struct CopyOffsets {
  static constexpr int CPR = D / 8, RPI = 64 / CPR, PER = kTile / RPI / NW;
  int off[PER];
};

template <int D, int NW>
__device__ __forceinline__ CopyOffsets<D, NW> copy_offsets(int w, int lane, long rstride) {
  using C = CopyOffsets<D, NW>;
  C o;
#pragma unroll
  for (int i = 0; i < C::PER; ++i) {
    const int row = (w * C::PER + i) * C::RPI + lane / C::CPR;
    o.off[i] = (int)(row * rstride) + (((lane % C::CPR) ^ swz<D>(row)) << 3);
  }
  return o;
}

template <int D, int NW>
__device__ __forceinline__ void copy_tile(const bf16_t* src, const CopyOffsets<D, NW>& o, bf16_t* lds, int w) {
  using C = CopyOffsets<D, NW>;
#pragma unroll
  for (int i = 0; i < C::PER; ++i) load_lds16(src + o.off[i], lds + (w * C::PER + i) * 512);
}

// The same copy with the source offsets computed on the spot (no registers kept between
// tiles): wave w of NW copies its share of a 64-row tile whose rows are `rstride`
// elements apart.
template <int D, int NW>
__device__ __forceinline__ void copy_tile_direct(const bf16_t* src, long rstride, bf16_t* lds, int w, int lane) {
  using C = CopyOffsets<D, NW>;
#pragma unroll
  for (int i = 0; i < C::PER; ++i) {
    const int row = (w * C::PER + i) * C::RPI + lane / C::CPR;
    load_lds16(src + (long)((w * C::PER + i) * C::RPI) * rstride +
                   (unsigned)((lane / C::CPR) * rstride + (((lane % C::CPR) ^ swz<D>(row)) << 3)),
               lds + (w * C::PER + i) * 512);
  }
}

// Per-lane LDS element offsets of the transposed fragments of a swizzled tile: block nb
// covers columns 32 nb .. 32 nb + 31, and the two reads of K-step 0 cover rows
// 4g .. 4g + 3 and 8 + 4g .. 8 + 4g + 3 (K-step kb adds 16 kb rows, a constant).
template <int D>
struct TrOffsets {
  int tr[D / 32][2];
};

template <int D>
__device__ __forceinline__ TrOffsets<D> tr_offsets(int lane) {
  TrOffsets<D> o;
  const int lq = lane % 32, g = lane / 32, t = lq & 15;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
    const int col = 32 * nb + 16 * (lq >> 4) + 4 * (t & 3);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 4 * g + (t >> 2) + 8 * i;
      o.tr[nb][i] = r * D + (((col >> 3) ^ swz<D>(r)) << 3) + (col & 7);
    }
  }
  return o;
}

// The two offsets of one column block nb only (for a block chosen at run time).
template <int D>
__device__ __forceinline__ void tr_offsets_block(int lane, int nb, int (&tr)[2]) {
  const int lq = lane % 32, g = lane / 32, t = lq & 15;
  const int col = 32 * nb + 16 * (lq >> 4) + 4 * (t & 3);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 4 * g + (t >> 2) + 8 * i;
    tr[i] = r * D + (((col >> 3) ^ swz<D>(r)) << 3) + (col & 7);
  }
}

// Transposed fragment of K-step kb: lane (lq, g) gets column 32 nb + lq of rows
// 16 kb + 4g + 0..3 and 16 kb + 8 + 4g + 0..3, the row order of a 32x32 accumulator's
// registers, so it pairs with an operand packed from accumulator registers.
template <int D>
__device__ __forceinline__ bf16x8_t tr_frag(const bf16_t* tile, const int (&tr)[2], int kb) {
  const bf16_t* a1 = tile + 16 * kb * D + tr[0];
  const bf16_t* a2 = tile + 16 * kb * D + tr[1];
  const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t __attribute__((address_space(3)))*)a1);
  const s16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t __attribute__((address_space(3)))*)a2);
  const uint2 ux = __builtin_bit_cast(uint2, x), uy = __builtin_bit_cast(uint2, y);
  return as_bf16x8(uint4{ux.x, ux.y, uy.x, uy.y});
}

}  // namespace s2a
