// Device helpers shared by the attention kernels: bf16 packing, the gfx950 bf16 MFMA,
// and the K/V tile stagers that move 64-row tiles from HBM into LDS.
//
// Lane conventions of v_mfma_f32_32x32x16_bf16 (checked on gfx950): with l the lane,
// lq = l % 32 and g = l / 32,
//   A operand (32 x 16, M x K): lane holds A[lq][8g .. 8g+7]
//   B operand (16 x 32, K x N): lane holds B[8g .. 8g+7][lq]
//   C/D (32 x 32):              register r holds D[8(r/4) + 4g + (r%4)][lq]
// So a product whose N dimension is the query index leaves every value a lane holds in
// the same query row; all per-row softmax state is then a per-lane scalar.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s2a {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Keys per LDS tile and the LDS row padding (elements) that staggers rows across banks.
constexpr int kTile = 64;
constexpr int kPad = 8;

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Same lane layout with fp16 operands.  Used for products with the softmax
// probabilities P in [0, 1], which keep 11 significant bits in fp16 (8 in bf16).
__device__ __forceinline__ f32x16_t mfma32h(const f16x8_t& a, const f16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ f16x8_t as_f16x8(const uint4& u) { return __builtin_bit_cast(f16x8_t, u); }

__device__ __forceinline__ uint4 load16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Position of row `r` (0..63) of a tile once the quads of every 16-row block are
// reordered [0-3, 8-11, 4-7, 12-15].  In that order the 8 rows one lane half needs for
// one MFMA K-step (rows 4g..4g+3 and 8+4g..8+4g+3 of the block, matching the register
// order of a 32x32 accumulator) are contiguous, so they load with one 16-byte read.
__device__ __forceinline__ int quad_swizzle(int r) {
  const int q = (r >> 2) & 3;
  const int qs = (q == 1) ? 2 : (q == 2) ? 1 : q;
  return (r & ~15) | (qs << 2) | (r & 3);
}

// Stages a 64-row x D tile (row stride `rstride` elements in HBM) into LDS, either
// row-major ([64][D + kPad]) or transposed with swizzled rows ([D][64 + kPad]).
// load() issues the global reads into registers; store() writes them to LDS, so a caller
// can overlap the reads of the next tile with work on the current one.
template <int D, int NT>
struct RowTile {
  static constexpr int kChunks = kTile * D / 8;             // 16-byte pieces per tile
  static constexpr int kPer = (kChunks + NT - 1) / NT;
  uint4 r[kPer];
  __device__ __forceinline__ void load(const bf16_t* base, long rstride, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * NT;
      if (kChunks % NT == 0 || c < kChunks) {
        const int row = c / (D / 8), col = (c % (D / 8)) * 8;
        r[i] = load16(base + row * rstride + col);
      }
    }
  }
  __device__ __forceinline__ void store(bf16_t (*lds)[D + kPad], int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * NT;
      if (kChunks % NT == 0 || c < kChunks) {
        const int row = c / (D / 8), col = (c % (D / 8)) * 8;
        *reinterpret_cast<uint4*>(&lds[row][col]) = r[i];
      }
    }
  }
};

// ToF16: convert the bf16 values to fp16 on the way into LDS (exact for magnitudes in
// fp16's normal range; values beyond +-65504 become infinite).
template <int D, int NT, bool ToF16 = false>
struct TransTile {
  static constexpr int kBlocks = (kTile / 4) * (D / 8);     // 4-row x 8-column blocks
  static constexpr int kPer = (kBlocks + NT - 1) / NT;
  uint4 r[kPer][4];
  __device__ __forceinline__ void load(const bf16_t* base, long rstride, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int bidx = tid + i * NT;
      if (kBlocks % NT == 0 || bidx < kBlocks) {
        const int rq = bidx / (D / 8), col = (bidx % (D / 8)) * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[i][j] = load16(base + (4 * rq + j) * rstride + col);
      }
    }
  }
  __device__ __forceinline__ void store(bf16_t (*lds)[kTile + kPad], int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int bidx = tid + i * NT;
      if (kBlocks % NT == 0 || bidx < kBlocks) {
        const int rq = bidx / (D / 8), col = (bidx % (D / 8)) * 8;
        const int pos = quad_swizzle(4 * rq);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a0 = (&r[i][0].x)[w], a1 = (&r[i][1].x)[w];
          const uint32_t a2 = (&r[i][2].x)[w], a3 = (&r[i][3].x)[w];
          uint2 lo, hi;
          if constexpr (ToF16) {
            lo.x = pack_f16(bf16_lo(a0), bf16_lo(a1));
            lo.y = pack_f16(bf16_lo(a2), bf16_lo(a3));
            hi.x = pack_f16(bf16_hi(a0), bf16_hi(a1));
            hi.y = pack_f16(bf16_hi(a2), bf16_hi(a3));
          } else {
            lo.x = (a0 & 0xffffu) | (a1 << 16);
            lo.y = (a2 & 0xffffu) | (a3 << 16);
            hi.x = (a0 >> 16) | (a1 & 0xffff0000u);
            hi.y = (a2 >> 16) | (a3 & 0xffff0000u);
          }
          *reinterpret_cast<uint2*>(&lds[col + 2 * w][pos]) = lo;
          *reinterpret_cast<uint2*>(&lds[col + 2 * w + 1][pos]) = hi;
        }
      }
    }
  }
};

// Stages a 64-row x D tile into LDS in both layouts at once (row-major and transposed
// with swizzled rows) from one read of HBM: each thread moves 4-row x 8-column blocks.
template <int D, int NT>
struct DualTile {
  static constexpr int kBlocks = (kTile / 4) * (D / 8);
  static constexpr int kPer = (kBlocks + NT - 1) / NT;
  uint4 r[kPer][4];
  __device__ __forceinline__ void load(const bf16_t* base, long rstride, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int bidx = tid + i * NT;
      if (kBlocks % NT == 0 || bidx < kBlocks) {
        const int rq = bidx / (D / 8), col = (bidx % (D / 8)) * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[i][j] = load16(base + (4 * rq + j) * rstride + col);
      }
    }
  }
  __device__ __forceinline__ void store(bf16_t (*rows)[D + kPad], bf16_t (*trans)[kTile + kPad], int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int bidx = tid + i * NT;
      if (kBlocks % NT == 0 || bidx < kBlocks) {
        const int rq = bidx / (D / 8), col = (bidx % (D / 8)) * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(&rows[4 * rq + j][col]) = r[i][j];
        const int pos = quad_swizzle(4 * rq);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a0 = (&r[i][0].x)[w], a1 = (&r[i][1].x)[w];
          const uint32_t a2 = (&r[i][2].x)[w], a3 = (&r[i][3].x)[w];
          uint2 lo, hi;
          lo.x = (a0 & 0xffffu) | (a1 << 16);
          lo.y = (a2 & 0xffffu) | (a3 << 16);
          hi.x = (a0 >> 16) | (a1 & 0xffff0000u);
          hi.y = (a2 >> 16) | (a3 & 0xffff0000u);
          *reinterpret_cast<uint2*>(&trans[col + 2 * w][pos]) = lo;
          *reinterpret_cast<uint2*>(&trans[col + 2 * w + 1][pos]) = hi;
        }
      }
    }
  }
};

// Per-lane fragment of 32 rows x D loaded straight from HBM as MFMA operands: lane
// (lq, g) holds row lq, columns 16kk + 8g .. +7 for every K-step kk.
template <int D>
__device__ __forceinline__ void load_row_frag(bf16x8_t (&f)[D / 16], const bf16_t* row, int g) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) f[kk] = as_bf16x8(load16(row + 16 * kk + 8 * g));
}

// max / sum of a lane's value and its partner lane (l ^ 32), through a bpermute.
__device__ __forceinline__ float pair_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float pair_sum(float x) { return x + __shfl_xor(x, 32); }

// Direct HBM -> LDS copy of 16 bytes per lane: lane l's bytes land at lds_wave_base + 16 l.
__device__ __forceinline__ void load_lds16(const bf16_t* src, bf16_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

}  // namespace s2a
