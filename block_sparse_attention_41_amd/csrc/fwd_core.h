// Forward attention over one staged K/V tile for one wavefront of 32 query rows.
//
// The wave computes S^T = K Q^T (keys as MFMA rows, its 32 queries as columns), so each
// lane owns one query row and the online-softmax state (running max m, partial sum l)
// is a per-lane scalar.  The output is accumulated transposed, O^T += V^T P^T, which
// keeps the per-row rescale a per-lane scalar too.  Scores are handled in the base-2
// domain: x = (q.k) * scale * log2(e), p = 2^(x - m).  P and V enter the P.V product
// as fp16 (P in [0, 1] keeps 11 significant bits there, against 8 in bf16).
#pragma once

#include "common.h"

namespace s2a {

template <int D>
struct FwdLds {
  bf16_t k[kTile][D + kPad];      // keys, row-major (bf16)
  bf16_t vt[D][kTile + kPad];     // values, transposed, rows quad-swizzled, stored as fp16
};

// diag: apply the causal test key_pos <= q_pos (positions in the caller's frame: the
// rolled order for shifted short attention, segment order for the local part of HGA).
template <int D>
__device__ __forceinline__ void fwd_tile(const FwdLds<D>& s, const bf16x8_t (&qf)[D / 16],
                                         f32x16_t (&o)[D / 32], float& m, float& l,
                                         int lq, int g, bool diag, int kpos0, int qpos, float c) {
  f32x16_t sc[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    sc[mb] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(&s.k[32 * mb + lq][16 * kk + 8 * g]));
      sc[mb] = mfma32(a, qf[kk], sc[mb]);
    }
  }
  float mt = kNegInf;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = sc[mb][r] * c;
      if (diag) {
        const int kp = kpos0 + 32 * mb + 8 * (r / 4) + 4 * g + (r % 4);
        x = (kp <= qpos) ? x : kNegInf;
      }
      sc[mb][r] = x;
      mt = fmaxf(mt, x);
    }
  }
  mt = pair_max(mt);
  const float mn = fmaxf(m, mt);
  const float base = (mn == kNegInf) ? 0.f : mn;
  const float alpha = fast_exp2(m - base);
  m = mn;
  float ls = 0.f;
  f16x8_t pb[4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = fast_exp2(sc[mb][8 * h + 2 * e] - base);
        const float p1 = fast_exp2(sc[mb][8 * h + 2 * e + 1] - base);
        ls += p0 + p1;
        w[e] = pack_f16(p0, p1);
      }
      pb[2 * mb + h] = __builtin_bit_cast(f16x8_t, uint4{w[0], w[1], w[2], w[3]});
    }
  }
  l = l * alpha + ls;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
    o[nb] *= alpha;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const f16x8_t a = as_f16x8(*reinterpret_cast<const uint4*>(&s.vt[32 * nb + lq][16 * kb + 8 * g]));
      o[nb] = mfma32h(a, pb[kb], o[nb]);
    }
  }
}

// Normalises and writes one wave's 32 output rows (token-order row pointer per lane) and
// the natural-log LSE.  orow points at O[token(lq)][h][0].
template <int D>
__device__ __forceinline__ void fwd_finish(const f32x16_t (&o)[D / 32], float m, float l, bf16_t* orow,
                                          float* lse_row, int g) {
  const float lt = pair_sum(l);
  const float inv = 1.f / lt;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint2 w;
      w.x = pack_bf16(o[nb][4 * i + 0] * inv, o[nb][4 * i + 1] * inv);
      w.y = pack_bf16(o[nb][4 * i + 2] * inv, o[nb][4 * i + 3] * inv);
      *reinterpret_cast<uint2*>(orow + 32 * nb + 8 * i + 4 * g) = w;
    }
  }
  if (g == 0) *lse_row = (m + __builtin_log2f(lt)) * kLn2;
}

}  // namespace s2a
