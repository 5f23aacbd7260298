// Forward attention tile step, shared by the shifted-attention, HGA and generation
// kernels: one wave, 32 query rows, one 64-key K/V tile staged in LDS.
//
//  * K and V tiles are copied HBM -> LDS directly (global_load_lds, no registers).  K
//    rows: the 16-byte chunk c of row r sits at chunk position c ^ (r % CPR) (CPR = chunks
//    per row), so the 16 lanes that read 16 consecutive rows at one logical chunk hit 16
//    distinct positions.  V rows: chunk c of row r at c ^ swz(r) (bwd2_core.h), the layout
//    whose transposed reads are free of bank conflicts.
//  * Each wave computes S^T = K Q^T (keys as MFMA rows, its 32 queries as columns), so a
//    lane owns one query row and the online-softmax state (running max m, partial sum l)
//    is a per-lane scalar; O is accumulated transposed, O^T += V^T P^T, with V^T read as
//    transposed fragments of the row-major V tile and P packed to bf16 straight from the
//    score registers (both in accumulator row order).  Scores live in the base-2 domain,
//    x = (q.k) * scale * log2(e), p = 2^(x - m).  P and V enter the product in bf16, the
//    input type: any finite V is exact there, and P keeps 8 significant bits.
//  * The running max is only moved when some row's tile max exceeds it by more than
//    kRescale (base-2 units); until then O and l are not rescaled and probabilities may
//    reach 2^kRescale, well inside bf16 and fp32 range.
#pragma once

#include "bwd2_core.h"

namespace s2a {

constexpr float kRescale = 8.f;

template <int D>
struct Fwd2Lds {
  bf16_t k[2][kTile * D];   // rows swizzled c ^ (r % CPR)
  bf16_t v[2][kTile * D];   // rows swizzled c ^ swz(r)
};

// Direct K tile copy: wave w issues its share of the 1 KB wave-instructions.
template <int D, int NW>
__device__ __forceinline__ void k_tile_direct(const bf16_t* kbase, long rstride, bf16_t* lds, int w, int lane) {
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;                 // rows per wave-instruction
  constexpr int INSTS = kTile / RPI;            // wave-instructions per tile
  static_assert(INSTS % NW == 0, "tile copy must split evenly over the waves");
  // a wave-uniform row base plus a 32-bit lane offset (no per-lane 64-bit arithmetic)
#pragma unroll
  for (int i = 0; i < INSTS / NW; ++i) {
    const int inst = w * (INSTS / NW) + i;
    const int row = inst * RPI + lane / CPR;
    const int cpos = lane % CPR;
    const int c = cpos ^ (row % CPR);
    load_lds16(kbase + (long)(inst * RPI) * rstride + (unsigned)((lane / CPR) * rstride + c * 8), lds + inst * 512);
  }
}

// The same copies (K tiles with KSW, V tiles swizzled by swz otherwise) from offsets kept
// in registers: wave w's instruction i covers rows (w PER + i) RPI .. + RPI - 1.  Both
// swizzles repeat every 16 rows, so a lane's offset within its instruction's rows takes
// NDIST = 16 / RPI values (PER is a multiple of NDIST, so instruction i uses off[i %
// NDIST]); the instruction's first row is a wave-uniform offset of the source, which
// leaves no per-lane 64-bit arithmetic in a tile loop.
template <int D, int NW, bool KSW>
struct TileCopy {
  static constexpr int CPR = D / 8, RPI = 64 / CPR, PER = kTile / RPI / NW, NDIST = 16 / RPI;
  static_assert(PER % NDIST == 0, "each wave's instructions start at a multiple of the swizzle period");
  unsigned off[NDIST];
};

template <int D, int NW, bool KSW>
__device__ __forceinline__ TileCopy<D, NW, KSW> tile_copy_offsets(int lane, long rstride) {
  using C = TileCopy<D, NW, KSW>;
  C o;
#pragma unroll
  for (int i = 0; i < C::NDIST; ++i) {
    const int row = i * C::RPI + lane / C::CPR;   // modulo 16, as the swizzles see it
    const int pos = lane % C::CPR;
    const int c = KSW ? pos ^ (row % C::CPR) : pos ^ swz<D>(row);
    o.off[i] = (unsigned)((lane / C::CPR) * rstride + c * 8);
  }
  return o;
}

template <int D, int NW, bool KSW>
__device__ __forceinline__ void copy_tile_swz(const TileCopy<D, NW, KSW>& o, const bf16_t* src, long rstride,
                                              bf16_t* lds, int w) {
  using C = TileCopy<D, NW, KSW>;
  const bf16_t* ws = src + (long)(w * C::PER * C::RPI) * rstride;
#pragma unroll
  for (int i = 0; i < C::PER; ++i)
    load_lds16(ws + (long)(i * C::RPI) * rstride + o.off[i % C::NDIST], lds + (w * C::PER + i) * 512);
}

// after_scores() runs once the tile's K fragments have been read and the S^T chain issued:
// a double-buffered caller issues the next tile's copies there, so its LDS reads above are
// not ordered behind copies still in flight.
template <int D, typename AfterScores>
__device__ __forceinline__ void fwd2_tile(const bf16_t* __restrict__ ks, const bf16_t* __restrict__ vs,
                                          const TrOffsets<D>& vo, const bf16x8_t (&qf)[D / 16],
                                          f32x16_t (&o)[D / 32], float& m, float& l, int lq, int g, bool diag,
                                          int kpos0, int qpos, float c, AfterScores&& after_scores) {
  constexpr int CPR = D / 8;
  // Fragment (mb, kk) of row 32 mb + lq sits at chunk (2 kk + g) ^ (row % CPR); the XOR
  // only touches bits below the row offset, so its element offset is
  // ((lq * D + z) ^ (kk << 4)) + 32 D mb with one per-lane base.
  const int kbase = lq * D + ((g ^ (lq % CPR)) << 3);
  // K fragments and the S^T chain, software-pipelined: half of the fragment reads go
  // first, the rest are issued two at a time behind the MFMAs, so the chain starts as
  // soon as its first operands arrive instead of after every read has returned
  constexpr int NR = 2 * (D / 16);   // fragment reads = MFMAs
  bf16x8_t ka[2][D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
      ka[mb][kk] = as_bf16x8(*reinterpret_cast<const uint4*>(ks + ((kbase ^ (kk << 4)) + 32 * D * mb)));
  }
  f32x16_t sc[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) sc[mb] = f32x16_t{};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) sc[mb] = mfma32(ka[mb][kk], qf[kk], sc[mb]);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, NR / 2, 0);   // DS reads
#pragma unroll
  for (int i = 0; i < NR / 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);      // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);      // DS reads
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NR / 2, 0);
  __builtin_amdgcn_sched_barrier(0);
  after_scores();

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
  // the first half of the V fragments is read now (after the cross-lane max, which
  // goes through the LDS queue); its latency hides behind the exponentials
  constexpr int NB = D / 32, NH = (NB + 1) / 2;
  bf16x8_t va[NB][4];
#pragma unroll
  for (int nb = 0; nb < NH; ++nb) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) va[nb][kb] = tr_frag<D>(vs, vo.tr[nb], kb);
  }
  __builtin_amdgcn_sched_barrier(0);
  const float nm = -m;
  float ls = 0.f;
  // P in the K order of the transposed V fragments: pb[2 mb + h] holds keys
  // 32 mb + 16 h + 4g + 0..3 and 32 mb + 16 h + 8 + 4g + 0..3, registers 8h .. 8h + 7
  bf16x8_t pb[4];
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
        wv[e] = pack_bf16(p0, p1);
      }
      pb[2 * mb + h] = __builtin_bit_cast(bf16x8_t, uint4{wv[0], wv[1], wv[2], wv[3]});
    }
  }
  l += ls;
#pragma unroll
  for (int nb = NH; nb < NB; ++nb) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) va[nb][kb] = tr_frag<D>(vs, vo.tr[nb], kb);
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb] = mfma32(va[nb][kb], pb[kb], o[nb]);
  }
}

}  // namespace s2a
