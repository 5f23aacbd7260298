// Backward attention tiles.  With P = exp(scale q.k - LSE) on the mask,
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q,
// where D = rowsum(dO * O).  Two wave-level tiles cover it without atomics:
//
//  * dq_tile   (query-major): the wave owns 32 queries and walks key tiles.  It forms
//    S^T and dP^T with keys as MFMA rows, so every value a lane holds belongs to its
//    query; dQ^T += K^T dS^T.
//  * dkdv_tile (key-major): the wave owns 32 keys and walks query tiles.  It forms S and
//    dP with queries as MFMA rows, so every value a lane holds belongs to its key;
//    dV^T += dO^T P and dK^T += Q^T dS.
//
// The recomputed probabilities use the forward's LSE, pre-multiplied by log2(e).
#pragma once

#include "common.h"

namespace s2a {

template <int D>
struct DqLds {
  bf16_t k[kTile][D + kPad];     // keys row-major: A operand of S^T
  bf16_t kt[D][kTile + kPad];    // keys transposed: A operand of dQ^T
  bf16_t v[kTile][D + kPad];     // values row-major: A operand of dP^T
};

template <int D>
__device__ __forceinline__ void dq_tile(const DqLds<D>& s, const bf16x8_t (&qf)[D / 16],
                                        const bf16x8_t (&dof)[D / 16], f32x16_t (&dq)[D / 32], float lse2,
                                        float dd, int lq, int g, bool diag, int kpos0, int qpos, float c) {
  f32x16_t sc[2], dp[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    sc[mb] = f32x16_t{};
    dp[mb] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(&s.k[32 * mb + lq][16 * kk + 8 * g]));
      sc[mb] = mfma32(a, qf[kk], sc[mb]);
      const bf16x8_t av = as_bf16x8(*reinterpret_cast<const uint4*>(&s.v[32 * mb + lq][16 * kk + 8 * g]));
      dp[mb] = mfma32(av, dof[kk], dp[mb]);
    }
  }
  bf16x8_t dsb[4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float ds2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int r = 8 * h + 2 * e + t;
          float p = fast_exp2(sc[mb][r] * c - lse2);
          if (diag) {
            const int kp = kpos0 + 32 * mb + 8 * (r / 4) + 4 * g + (r % 4);
            p = (kp <= qpos) ? p : 0.f;
          }
          ds2[t] = p * (dp[mb][r] - dd);
        }
        w[e] = pack_bf16(ds2[0], ds2[1]);
      }
      dsb[2 * mb + h] = __builtin_bit_cast(bf16x8_t, uint4{w[0], w[1], w[2], w[3]});
    }
  }
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(&s.kt[32 * nb + lq][16 * kb + 8 * g]));
      dq[nb] = mfma32(a, dsb[kb], dq[nb]);
    }
  }
}

template <int D>
struct KvLds {
  bf16_t q[kTile][D + kPad];      // queries row-major: A operand of S
  bf16_t qt[D][kTile + kPad];     // queries transposed: A operand of dK^T
  bf16_t dob[kTile][D + kPad];    // output grads row-major: A operand of dP
  bf16_t dot[D][kTile + kPad];    // output grads transposed: A operand of dV^T
  float lse2[kTile];              // LSE * log2(e) of the tile's queries
  float dd[kTile];                // D = rowsum(dO * O) of the tile's queries
};

// diag: the causal test key_pos <= q_pos applies (positions in the caller's frame).
template <int D>
__device__ __forceinline__ void dkdv_tile(const KvLds<D>& s, const bf16x8_t (&kf)[D / 16],
                                          const bf16x8_t (&vf)[D / 16], f32x16_t (&dk)[D / 32],
                                          f32x16_t (&dv)[D / 32], int lq, int g, bool diag, int qpos0, int kpos,
                                          float c) {
  f32x16_t sc[2], dp[2];
#pragma unroll
  for (int mq = 0; mq < 2; ++mq) {
    sc[mq] = f32x16_t{};
    dp[mq] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(&s.q[32 * mq + lq][16 * kk + 8 * g]));
      sc[mq] = mfma32(a, kf[kk], sc[mq]);
      const bf16x8_t ad = as_bf16x8(*reinterpret_cast<const uint4*>(&s.dob[32 * mq + lq][16 * kk + 8 * g]));
      dp[mq] = mfma32(ad, vf[kk], dp[mq]);
    }
  }
  bf16x8_t pb[4], dsb[4];
#pragma unroll
  for (int mq = 0; mq < 2; ++mq) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // rows 32mq + 16h + {4g..4g+3, 8+4g..8+4g+3} are this lane's 8 queries of the step
      const int q0 = 32 * mq + 16 * h + 4 * g;
      const float4 l0 = *reinterpret_cast<const float4*>(&s.lse2[q0]);
      const float4 l1 = *reinterpret_cast<const float4*>(&s.lse2[q0 + 8]);
      const float4 d0 = *reinterpret_cast<const float4*>(&s.dd[q0]);
      const float4 d1 = *reinterpret_cast<const float4*>(&s.dd[q0 + 8]);
      const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
      const float dv8[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
      uint32_t wp[4], wd[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p2[2], ds2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int sidx = 2 * e + t;               // slot within the 16-query step
          const int r = 8 * h + sidx;               // accumulator register
          float p = fast_exp2(sc[mq][r] * c - lv[sidx]);
          if (diag) {
            const int qp = qpos0 + 32 * mq + 8 * (r / 4) + 4 * g + (r % 4);
            p = (kpos <= qp) ? p : 0.f;
          }
          p2[t] = p;
          ds2[t] = p * (dp[mq][r] - dv8[sidx]);
        }
        wp[e] = pack_bf16(p2[0], p2[1]);
        wd[e] = pack_bf16(ds2[0], ds2[1]);
      }
      pb[2 * mq + h] = __builtin_bit_cast(bf16x8_t, uint4{wp[0], wp[1], wp[2], wp[3]});
      dsb[2 * mq + h] = __builtin_bit_cast(bf16x8_t, uint4{wd[0], wd[1], wd[2], wd[3]});
    }
  }
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(&s.dot[32 * nb + lq][16 * kb + 8 * g]));
      dv[nb] = mfma32(a, pb[kb], dv[nb]);
      const bf16x8_t aq = as_bf16x8(*reinterpret_cast<const uint4*>(&s.qt[32 * nb + lq][16 * kb + 8 * g]));
      dk[nb] = mfma32(aq, dsb[kb], dk[nb]);
    }
  }
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
