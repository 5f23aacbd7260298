// Device helpers shared by the attention kernels: bf16 packing, the gfx950 bf16 MFMA,
// register fragments, direct HBM -> LDS copies and launch-order helpers.
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
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Groups at least this long (tokens) use eight-wave workgroups in the shifted-attention
// forward; shorter ones use four-wave workgroups, two per CU (measured on MI355X at
// d = 128: 6% faster at 2048, even at 512 and 1024, 1.5% slower at 256).
constexpr int kWideGroupFwd = 2048;
// Groups shorter than this run as persistent launches: exactly the resident workgroups,
// each looping over its XCD's units (measured on MI355X at N = 32768: 2.8% faster for
// G = 8192, forward and backward; 1.2% slower for the dense G = N forward).
constexpr int kPersistGroup = 16384;

// Keys (or queries) per LDS tile.
constexpr int kTile = 64;

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint4 load16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

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

// Work-item and workgroup indices read straight from the hardware registers.  HIP's
// threadIdx / blockIdx / gridDim go through device-library functions that are linked
// after optimisation and stay real calls, which puts a call frame into every kernel.
__device__ __forceinline__ int thread_x() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int group_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int group_y() { return (int)__builtin_amdgcn_workgroup_id_y(); }
__device__ __forceinline__ int group_z() { return (int)__builtin_amdgcn_workgroup_id_z(); }

// Stores a transposed accumulator tile (32 rows x D: lane = row lq, registers over
// columns) scaled by `mul` as bf16 to rows dst + r * rstride, through `lds` (32 x D
// elements owned by this wave).  Written straight from the registers every store
// instruction would put 16 bytes into each of 32 rows; through LDS each one writes four
// (D = 128) or eight (D = 64) whole rows, so no cache line is written back in pieces.
// The 16-byte chunk c of row r sits at chunk position c ^ (r % CPR), which keeps both
// the 8-byte writes and the 16-byte row reads free of bank conflicts.  A wave's LDS
// accesses complete in order, so no barrier is needed around it.
template <int D>
__device__ __forceinline__ void store_acc_tile(const f32x16_t (&acc)[D / 32], float mul, bf16_t* lds, bf16_t* dst,
                                               long rstride, int lane) {
  constexpr int CPR = D / 8, RPI = 64 / CPR;
  const int lq = lane % 32, g = lane / 32;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint2 w;
      w.x = pack_bf16(acc[nb][4 * i + 0] * mul, acc[nb][4 * i + 1] * mul);
      w.y = pack_bf16(acc[nb][4 * i + 2] * mul, acc[nb][4 * i + 3] * mul);
      const int chunk = 4 * nb + i;   // columns 32 nb + 8 i .. + 7
      *reinterpret_cast<uint2*>(lds + lq * D + ((chunk ^ (lq % CPR)) << 3) + 4 * g) = w;
    }
  }
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int row = k * RPI + lane / CPR, c = lane % CPR;
    const uint4 val = *reinterpret_cast<const uint4*>(lds + row * D + ((c ^ (row % CPR)) << 3));
    *reinterpret_cast<uint4*>(dst + row * rstride + c * 8) = val;
  }
}

}  // namespace s2a
