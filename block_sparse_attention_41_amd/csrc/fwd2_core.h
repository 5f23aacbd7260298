// Forward attention, eight-wavefront variant: one workgroup stages each 64-key K/V tile
// once for 8 x 32 query rows, double-buffered with a single barrier per tile.
//
//  * K tiles are copied HBM -> LDS directly (global_load_lds, no registers).  Rows are
//    unpadded; the 16-byte chunk c of row r is stored at chunk position c ^ (r % CPR)
//    (CPR = chunks per row), so the 16 lanes that read 16 consecutive rows at one logical
//    chunk hit 16 distinct positions.
//  * V tiles go through registers: each thread converts a 2-key x 8-column block to fp16
//    and writes it transposed (rows = head dim, keys quad-swizzled as in common.h).
//  * Per wave the math is the transposed product of fwd_core.h (query = MFMA column,
//    softmax state per lane).  The running max is only moved when some row's tile max
//    exceeds it by more than kRescale (base-2 units); until then O and l are not
//    rescaled and probabilities may reach 2^kRescale, well inside fp16 and fp32 range.
#pragma once

#include "common.h"

namespace s2a {

constexpr float kRescale = 8.f;

template <int D>
struct Fwd2Lds {
  static constexpr int CPR = D / 8;
  bf16_t k[2][kTile * D];             // swizzled rows
  bf16_t vt[2][D][kTile + kPad];      // fp16, transposed, quad-swizzled key order
};

// Direct K tile copy: wave w issues its share of the 1 KB wave-instructions.
template <int D, int NW>
__device__ __forceinline__ void k_tile_direct(const bf16_t* kbase, long rstride, bf16_t* lds, int w, int lane) {
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;                 // rows per wave-instruction
  constexpr int INSTS = kTile / RPI;            // wave-instructions per tile
  static_assert(INSTS % NW == 0, "tile copy must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < INSTS / NW; ++i) {
    const int inst = w * (INSTS / NW) + i;
    const int row = inst * RPI + lane / CPR;
    const int cpos = lane % CPR;
    const int c = cpos ^ (row % CPR);
    load_lds16(kbase + row * rstride + c * 8, lds + inst * 512);
  }
}

// 2-key x 8-column V blocks, converted to fp16 and stored transposed.
template <int D, int NT>
struct VStage {
  static constexpr int kBlocks = (kTile / 2) * (D / 8);
  static constexpr int kPer = (kBlocks + NT - 1) / NT;
  uint4 a[kPer], b[kPer];
  __device__ __forceinline__ void load(const bf16_t* base, long rstride, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int blk = tid + i * NT;
      if (kBlocks % NT == 0 || blk < kBlocks) {
        const int kp = blk / (D / 8), col = (blk % (D / 8)) * 8;
        a[i] = load16(base + (2 * kp) * rstride + col);
        b[i] = load16(base + (2 * kp + 1) * rstride + col);
      }
    }
  }
  __device__ __forceinline__ void store(bf16_t (*vt)[kTile + kPad], int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int blk = tid + i * NT;
      if (kBlocks % NT == 0 || blk < kBlocks) {
        const int kp = blk / (D / 8), col = (blk % (D / 8)) * 8;
        const int pos = quad_swizzle(2 * kp);
        const uint32_t aw[4] = {a[i].x, a[i].y, a[i].z, a[i].w};
        const uint32_t bw[4] = {b[i].x, b[i].y, b[i].z, b[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          *reinterpret_cast<uint32_t*>(&vt[col + 2 * e][pos]) = pack_f16(bf16_lo(aw[e]), bf16_lo(bw[e]));
          *reinterpret_cast<uint32_t*>(&vt[col + 2 * e + 1][pos]) = pack_f16(bf16_hi(aw[e]), bf16_hi(bw[e]));
        }
      }
    }
  }
};

template <int D>
__device__ __forceinline__ void fwd2_tile(const bf16_t* __restrict__ ks, const bf16_t (*vt)[kTile + kPad],
                                          const bf16x8_t (&qf)[D / 16], f32x16_t (&o)[D / 32], float& m, float& l,
                                          int lq, int g, bool diag, int kpos0, int qpos, float c) {
  constexpr int CPR = D / 8;
  f32x16_t sc[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    sc[mb] = f32x16_t{};
    const int row = 32 * mb + lq;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int pos = (2 * kk + g) ^ (row % CPR);
      const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(ks + row * D + pos * 8));
      sc[mb] = mfma32(a, qf[kk], sc[mb]);
    }
  }
  if (diag) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kp = kpos0 + 32 * mb + 8 * (r / 4) + 4 * g + (r % 4);
        if (kp > qpos) sc[mb][r] = kNegInf;
      }
    }
  }
  float mx = kNegInf;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(sc[mb][r], sc[mb][r + 1]));
  }
  const float mt = pair_max(mx) * c;
  if (__any(mt > m + kRescale)) {
    const float mn = fmaxf(m, mt);
    const float alpha = fast_exp2(m - mn);     // 0 on the first tile (m = -inf)
    m = mn;
    l *= alpha;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) o[nb] *= alpha;
  }
  const float nm = -m;
  float ls = 0.f;
  f16x8_t pb[4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = fast_exp2(__builtin_fmaf(sc[mb][8 * h + 2 * e], c, nm));
        const float p1 = fast_exp2(__builtin_fmaf(sc[mb][8 * h + 2 * e + 1], c, nm));
        ls += p0 + p1;
        wv[e] = pack_f16(p0, p1);
      }
      pb[2 * mb + h] = __builtin_bit_cast(f16x8_t, uint4{wv[0], wv[1], wv[2], wv[3]});
    }
  }
  l += ls;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const f16x8_t a = as_f16x8(*reinterpret_cast<const uint4*>(&vt[32 * nb + lq][16 * kb + 8 * g]));
      o[nb] = mfma32h(a, pb[kb], o[nb]);
    }
  }
}

}  // namespace s2a
