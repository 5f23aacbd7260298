// Forward attention, eight-wavefront variant: one workgroup stages each 64-key K/V tile
// once for 8 x 32 query rows, double-buffered with a single barrier per tile.
//
//  * K tiles are copied HBM -> LDS directly (global_load_lds, no registers).  Rows are
//    unpadded; the 16-byte chunk c of row r is stored at chunk position c ^ (r % CPR)
//    (CPR = chunks per row), so the 16 lanes that read 16 consecutive rows at one logical
//    chunk hit 16 distinct positions.
//  * V tiles go through registers: each thread converts a 2-key x 8-column block to fp16
//    and writes it transposed (rows = head dim, keys quad-swizzled as in common.h).
//  * Each wave computes S^T = K Q^T (keys as MFMA rows, its 32 queries as columns), so a
//    lane owns one query row and the online-softmax state (running max m, partial sum l)
//    is a per-lane scalar; O is accumulated transposed, O^T += V^T P^T.  Scores live in
//    the base-2 domain, x = (q.k) * scale * log2(e), p = 2^(x - m), and P and V enter the
//    P.V product as fp16 (P <= 2^kRescale keeps 11 significant bits, against 8 in bf16).
//  * The running max is only moved when some row's tile max exceeds it by more than
//    kRescale (base-2 units); until then O and l are not rescaled and probabilities may
//    reach 2^kRescale, well inside fp16 and fp32 range.
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

// Transposed fp16 V tile: row r (head-dim index) holds the 64 keys in quad-swizzled
// order, i.e. key pair P occupies dword P of the row.  The 16-byte chunk c of a row
// (dwords 4c..4c+3) is stored at chunk position c ^ vt_xor(r); with 160-byte rows this
// keeps the 16-byte fragment reads free of bank conflicts (measured on gfx950).
__device__ __forceinline__ int vt_xor(int row) { return (row >> 4) & 7; }

// V staging.  Work item i = (Q, j) = (i % 16, i / 16): key group Q (tile positions
// 4Q..4Q+3, four consecutive keys after the quad swizzle) and column block j (8 head-dim
// values).  Item i goes to lane i % 64 of wave-round i / 64, so one wave-instruction
// covers all 16 key groups of 4 column blocks.  A thread loads its 4 keys x 8 columns,
// converts them to fp16 and writes, for each of its 8 rows (columns), the two dwords of
// key pairs 2Q and 2Q + 1 with one 8-byte write (measured on gfx950: 4 cycles per write
// instruction, no conflicts, against 8 per 4-byte write of the two-key scheme).
template <int D, int NW>
struct VStage {
  static constexpr int CPR = D / 8;
  static constexpr int ITEMS = 16 * CPR;                  // (key group, column block) pairs
  static constexpr int ROUNDS = (ITEMS + 64 * NW - 1) / (64 * NW);
  uint4 r4[ROUNDS][4];
  __device__ __forceinline__ static bool has(int r, int w) { return ITEMS % (64 * NW) == 0 || (NW * r + w) * 64 < ITEMS; }
  __device__ __forceinline__ void load_round(const bf16_t* base, long rstride, int r, int w, int lane) {
    const int i = (NW * r + w) * 64 + lane, Q = i % 16, col = (i / 16) * 8;
    const int key = quad_swizzle(4 * Q);
#pragma unroll
    for (int t = 0; t < 4; ++t) r4[r][t] = load16(base + (key + t) * rstride + col);
  }
  __device__ __forceinline__ void store_round(bf16_t (*vt)[kTile + kPad], int r, int w, int lane) const {
    const int i = (NW * r + w) * 64 + lane, Q = i % 16, col = (i / 16) * 8;
    const uint32_t k0[4] = {r4[r][0].x, r4[r][0].y, r4[r][0].z, r4[r][0].w};
    const uint32_t k1[4] = {r4[r][1].x, r4[r][1].y, r4[r][1].z, r4[r][1].w};
    const uint32_t k2[4] = {r4[r][2].x, r4[r][2].y, r4[r][2].z, r4[r][2].w};
    const uint32_t k3[4] = {r4[r][3].x, r4[r][3].y, r4[r][3].z, r4[r][3].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int row = col + 2 * e + hi;
        const int dw = (((Q >> 1) ^ vt_xor(row)) << 2) | (2 * (Q & 1));
        const uint2 val = hi ? uint2{pack_f16(bf16_hi(k0[e]), bf16_hi(k1[e])), pack_f16(bf16_hi(k2[e]), bf16_hi(k3[e]))}
                             : uint2{pack_f16(bf16_lo(k0[e]), bf16_lo(k1[e])), pack_f16(bf16_lo(k2[e]), bf16_lo(k3[e]))};
        *reinterpret_cast<uint2*>(reinterpret_cast<uint32_t*>(&vt[row][0]) + dw) = val;
      }
    }
  }
  __device__ __forceinline__ void load(const bf16_t* base, long rstride, int w, int lane) {
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r)
      if (has(r, w)) load_round(base, rstride, r, w, lane);
  }
  __device__ __forceinline__ void store(bf16_t (*vt)[kTile + kPad], int w, int lane) const {
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r)
      if (has(r, w)) store_round(vt, r, w, lane);
  }
  // copy of a tile whose keys past `kmax` (relative to `base`) lie outside the buffer:
  // those positions get key kmax's values (callers mask them out of the softmax)
  __device__ __forceinline__ void copy_clamped(const bf16_t* base, long rstride, int kmax,
                                               bf16_t (*vt)[kTile + kPad], int w, int lane) {
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      if (has(r, w)) {
        const int i = (NW * r + w) * 64 + lane, Q = i % 16, col = (i / 16) * 8;
        const int key = quad_swizzle(4 * Q);
#pragma unroll
        for (int t = 0; t < 4; ++t) r4[r][t] = load16(base + (long)min(key + t, kmax) * rstride + col);
        store_round(vt, r, w, lane);
      }
    }
  }
  // load + store one round at a time: only one round's registers are ever live
  __device__ __forceinline__ void copy(const bf16_t* base, long rstride, bf16_t (*vt)[kTile + kPad], int w,
                                       int lane) {
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      if (has(r, w)) {
        load_round(base, rstride, r, w, lane);
        store_round(vt, r, w, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// after_scores() runs once the tile's K fragments have been read and the S^T chain issued:
// a double-buffered caller issues the next tile's copies there, so its LDS reads above are
// not ordered behind copies still in flight.
template <int D, typename AfterScores>
__device__ __forceinline__ void fwd2_tile(const bf16_t* __restrict__ ks, const bf16_t (*vt)[kTile + kPad],
                                          const bf16x8_t (&qf)[D / 16], f32x16_t (&o)[D / 32], float& m, float& l,
                                          int lq, int g, bool diag, int kpos0, int qpos, float c,
                                          AfterScores&& after_scores) {
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
  // V fragment (nb, kb): row 32 nb + lq, chunk (2 kb + g) ^ vt_xor(row) = 2 (kb ^ nb) + (g ^ (lq >> 4)),
  // i.e. a per-lane base plus a compile-time offset
  const bf16_t* vbase = &vt[lq][8 * (g ^ (lq >> 4))];
  f16x8_t va[NB][4];
#pragma unroll
  for (int nb = 0; nb < NH; ++nb) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      va[nb][kb] = as_f16x8(*reinterpret_cast<const uint4*>(vbase + 32 * nb * (kTile + kPad) + 16 * (kb ^ nb)));
  }
  __builtin_amdgcn_sched_barrier(0);
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
  for (int nb = NH; nb < NB; ++nb) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      va[nb][kb] = as_f16x8(*reinterpret_cast<const uint4*>(vbase + 32 * nb * (kTile + kPad) + 16 * (kb ^ nb)));
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb] = mfma32h(va[nb][kb], pb[kb], o[nb]);
  }
}

}  // namespace s2a
