// Backward kernels for shifted short attention and for HGA (active segment only).
//
//   1. bwd_rowdot_kernel: D = rowsum(dO * O) per (batch, head, token), float32 workspace.
//   2. dqw_kernel, hga_dqw_kernel: query-major; each wave owns two 32-query blocks and
//                     walks the same key tiles as the forward.  For HGA a two-wave
//                     workgroup per 64-query block deals the block's half tiles (local
//                     ones, then those of its selected history chunks) alternately to its
//                     waves and adds their float32 partials through LDS; blocks run
//                     heaviest first, so light blocks fill the early finishers' slots.
//                     Given room for them, the local half tiles use the dS tiles that the
//                     key-major kernel stored (then it runs first, after the statistics).
//   3. kvp_kernel: key-major; a workgroup of eight waves owns 128 keys as four wave pairs
//                     of 32 keys (two waves per SIMD).  Wave A of a pair holds the keys' K
//                     rows and the dV accumulator (S, P, dV); wave B holds the V rows and
//                     the dK accumulator (dP, dS, dK), one query tile behind A, and takes P
//                     from A through LDS.  Both walk the query tiles that can see the keys,
//                     over every q head of the kv head (grouped-query sum in registers).
//                     Short HGA segments run it split into parts whose float32 partial sums
//                     kv_reduce_kernel adds in order.  For HGA only active keys get
//                     gradients: the history is detached ("Long-Context Fine-Tuning with
//                     Limited VRAM", English abstract).
// No atomics anywhere, so results are bitwise reproducible.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "../../include/s2a.h"
#include "bwd2_core.h"
#include "dsq.h"
#include "launch.h"
#include "validate.h"

namespace s2a {

// D[b, h, t] = sum_e dO[b, t, h, e] * O[b, t, h, e]; 8 lanes per row.  When `lse` is
// given, also writes lse2 = LSE * log2(e) (the base-2 row statistic the recomputation of
// P uses) at the same index.  A workgroup takes T consecutive tokens of one batch and up
// to 32 heads: its rows are contiguous in O and dO (32 rows of 8 lanes per pass, four
// passes of loads in flight), and the statistics, token-contiguous per head, go out
// through LDS as whole 4T-byte runs (row-ordered writes would scatter 4-byte pieces of
// every line over the XCDs).  T = 16, or fewer when that leaves the chip short of
// workgroups (a 2048-token segment of 32 heads: 128 workgroups at T = 16).
template <int D, int T>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const bf16_t* __restrict__ o,
                                                          const bf16_t* __restrict__ dout, float* __restrict__ dd,
                                                          const float* __restrict__ lse, float* __restrict__ lse2,
                                                          int L, int H) {
  constexpr int PER = D / 8;  // elements per lane
  constexpr int UN = 4;       // passes in flight
  __shared__ float sd[32][T];
  const int nhc = (H + 31) / 32, ntb = (L + T - 1) / T;
  int x = group_x();
  const int hc = x % nhc;
  x /= nhc;
  const int tb = x % ntb;
  const int b = x / ntb;
  const int h0 = hc * 32, nh = min(32, H - h0), t0 = tb * T, nt = min(T, L - t0);
  const int sub = thread_x() % 8, rw = thread_x() / 8;   // row within a pass
  const int nrows = nt * nh, npass = (nrows + 31) / 32;
  for (int p0 = 0; p0 < npass; p0 += UN) {
    uint4 a[UN][PER / 8], c[UN][PER / 8];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int r = min((p0 + u) * 32 + rw, nrows - 1);   // clamped: a spare row reloads the last one
      const long row = ((long)b * L + t0 + r / nh) * H + h0 + r % nh;
#pragma unroll
      for (int i = 0; i < PER / 8; ++i) {
        a[u][i] = load16(o + row * D + sub * PER + 8 * i);
        c[u][i] = load16(dout + row * D + sub * PER + 8 * i);
      }
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < PER / 8; ++i) {
        const uint32_t aw[4] = {a[u][i].x, a[u][i].y, a[u][i].z, a[u][i].w};
        const uint32_t bw[4] = {c[u][i].x, c[u][i].y, c[u][i].z, c[u][i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += bf16_lo(aw[e]) * bf16_lo(bw[e]) + bf16_hi(aw[e]) * bf16_hi(bw[e]);
      }
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      acc += __shfl_xor(acc, 4);
      const int r = (p0 + u) * 32 + rw;
      if (sub == 0 && r < nrows) sd[r % nh][r / nh] = acc;
    }
  }
  __syncthreads();
  // D[(b H + h) L + t] and lse2 at the same index, T tokens of each head in a run
  for (int e = thread_x(); e < nh * T; e += 256) {
    const int hh = e / T, tt = e % T;
    if (tt >= nt) continue;
    const long idx = ((long)b * H + h0 + hh) * L + t0 + tt;
    dd[idx] = sd[hh][tt];
    if (lse) lse2[idx] = lse[idx] * kLog2e;
  }
}

// ---------------------------------------------------------------------------------------
// Shifted short attention (same rolled-group geometry and launch order as the forward):
// tiles copied HBM -> LDS directly, one barrier per tile.
// ---------------------------------------------------------------------------------------



// Work split of the key-major kernels.  Key block `tig` of a group (BN = 32 NW keys) loops
// over rep x (query tiles at or after it) iterations.  When a launch would have too few
// workgroups, these iterations are cut into parts of at most `m`, each part run by its
// own workgroup into a float32 partial sum; kv_reduce_kernel then adds the parts in part
// order, so the result stays deterministic.  upg = workgroups per (batch, kv head, group);
// upg == tpg (key blocks per group) means one part per key block.
__host__ __device__ inline int kv_iters(int rep, int G, int bn, int tig) { return rep * (G / kTile - tig * (bn / kTile)); }
__host__ __device__ inline int kv_parts(int rep, int G, int bn, int tig, int m) { return (kv_iters(rep, G, bn, tig) + m - 1) / m; }

// float32 row store of a transposed accumulator (lane = row lq, registers over columns)
template <int D>
__device__ __forceinline__ void store_acc_f32(const f32x16_t (&acc)[D / 32], float mul, float* row, int g) {
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<float4*>(row + 32 * nb + 8 * i + 4 * g) =
          float4{acc[nb][4 * i] * mul, acc[nb][4 * i + 1] * mul, acc[nb][4 * i + 2] * mul, acc[nb][4 * i + 3] * mul};
  }
}


// Per-lane LDS element offsets of the fragments the fused kernel reads from a staged
// tile: row fragments of K-step kk for rows 0..31, transposed fragments of block nb for
// the two row quads of K-step 0, and the first of a lane's four row statistics.  Rows
// 32 mq + r and K-steps kb of the transposed reads only add constants (the swizzle
// depends on the row modulo 16), so each read is one register plus an immediate.
template <int D>
struct KvfOffsets {
  int row[D / 16];
  int tr[D / 32][2];
  int stat;
};

template <int D>
__device__ __forceinline__ KvfOffsets<D> kvf_offsets(int lane) {
  KvfOffsets<D> o;
  const int lq = lane % 32, g = lane / 32, t = lq & 15;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) o.row[kk] = lq * D + (((2 * kk + g) ^ swz<D>(lq)) << 3);
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
    const int col = 32 * nb + 16 * (lq >> 4) + 4 * (t & 3);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 4 * g + (t >> 2) + 8 * i;
      o.tr[nb][i] = r * D + (((col >> 3) ^ swz<D>(r)) << 3) + (col & 7);
    }
  }
  o.stat = 4 * g;
  return o;
}

template <int D>
__device__ __forceinline__ bf16x8_t kvf_tr(const bf16_t* tile, const KvfOffsets<D>& o, int nb, int kb) {
  return tr_frag<D>(tile, o.tr[nb], kb);
}

// ---------------------------------------------------------------------------------------
// Key-major dK and dV with wave pairs (two waves per SIMD).  A workgroup of eight waves
// owns 128 keys as four pairs of 32.  In each pair:
//   wave A (waves 0-3) holds its keys' K rows and the dV^T accumulator; for query tile t
//     it computes S = Q K^T, P = exp2(S c - LSE log2 e) (masked on the diagonal),
//     dV^T += dO^T P, and writes P (bf16, register order) to the pair's LDS slot;
//   wave B (waves 4-7) holds the V rows and the dK^T accumulator; one phase behind, for
//     tile t - 1, it computes dP = dO V^T, reads A's P, dS = P (dP - D) and
//     dK^T += Q^T dS.
// Both do 32 MFMAs per 64-query tile on different tiles of their shared SIMD, each
// software-pipelined so that its own vector work runs between its MFMAs.  Three sets of
// Q/dO tiles are resident: B's tile, A's tile and the next tile, copied during the phase;
// one barrier per phase.  Both waves compute with lane = key and registers over queries,
// so P leaves A and reaches B in the same register order: the exchange is one 16-byte
// write and read per lane and register half.  (Per-phase timestamps at the 8K step: about
// 5400 shader cycles per phase against 2048 of MFMA work per SIMD; the two waves of a SIMD
// start each phase together at the barrier, so their matrix-only stages overlap each
// other rather than each other's vector work.)
// ---------------------------------------------------------------------------------------
template <int D>
struct KvpLds {
  bf16_t q[3][kTile * D];
  bf16_t o[3][kTile * D];
  float l2[3][kTile];
  float dd[3][kTile];
  uint4 px[3][4][2][2][64];   // [phase % 3][pair][query half][register half][lane]
};

// The vector work of one half runs between the matrix products of the other, in four
// stages per 64-query tile, so a wave's own exponentials (or dS arithmetic) execute under
// its MFMAs; the schedule is pinned with scheduling-group barriers (masks: 0x008 MFMA,
// 0x002 VALU, 0x100 LDS read, 0x200 LDS write).
//
// Wave A: S_0 | S_1 with P_0 = exp2(S_0 c - LSE log2 e) | dV^T += dO^T P_0 with P_1 |
// dV^T += dO^T P_1.  P goes to the pair's exchange slot in register order.  The causal
// mask (diagonal tiles only) is a wave-uniform branch around the vector work on P alone,
// so the matrix products stay on one straight path and the accumulator keeps its
// registers.
template <int D>
__device__ __forceinline__ void kvp_p(const f32x16_t& sc, const float* l2, const KvfOffsets<D>& o, int mq, float c,
                                      float (&x)[16]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // this lane's 8 queries: q0 + 4g + 0..3 and q0 + 8 + 4g + 0..3, q0 = 32 mq + 16 h
    const int q0 = 32 * mq + 16 * h;
    const float4 la = *reinterpret_cast<const float4*>(l2 + q0 + o.stat);
    const float4 lb = *reinterpret_cast<const float4*>(l2 + q0 + 8 + o.stat);
    const float lv[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[8 * h + i] = fast_exp2(__builtin_fmaf(sc[8 * h + i], c, -lv[i]));
  }
}

__device__ __forceinline__ void kvp_mask(float (&x)[16], int kpos, int qh, int g) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int qp = qh + 8 * (r / 4) + 4 * g + (r % 4);
    x[r] = (kpos <= qp) ? x[r] : 0.f;
  }
}

__device__ __forceinline__ void kvp_pack(const float (&x)[16], bf16x8_t (&pb)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) wv[e] = pack_bf16(x[8 * h + 2 * e], x[8 * h + 2 * e + 1]);
    pb[h] = __builtin_bit_cast(bf16x8_t, uint4{wv[0], wv[1], wv[2], wv[3]});
  }
}

template <int D, typename Copy>
__device__ __forceinline__ void kvp_tile_a(const bf16_t* qt, const bf16_t* dt, const float* l2, uint4* px,
                                           const bf16x8_t (&kf)[D / 16], f32x16_t (&av)[D / 32],
                                           const KvfOffsets<D>& o, int g, int qp, int kpos, float c, bool diag0,
                                           bool diag1, int lane, Copy&& docopy) {
  constexpr int KS = D / 16, NB = D / 32, NF = 2 * NB;
  __builtin_amdgcn_sched_barrier(0);
  // stage 1: S_0, each Q fragment two ahead of its MFMA
  f32x16_t sc0 = f32x16_t{}, sc1 = f32x16_t{};
  {
    bf16x8_t fq[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) fq[kk] = as_bf16x8(load16(qt + o.row[kk]));
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) sc0 = mfma32(fq[kk], kf[kk], sc0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < KS - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // stage 2: S_1 with P_0
  float x[16];
  {
    bf16x8_t fq[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) fq[kk] = as_bf16x8(load16(qt + 32 * D + o.row[kk]));
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) sc1 = mfma32(fq[kk], kf[kk], sc1);
    kvp_p<D>(sc0, l2, o, 0, c, x);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);   // two fragments, the LSE values
#pragma unroll
    for (int i = 0; i < KS - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the next tile's copies, issued here rather than at the phase start (where they
  // compete with the first fragment reads of all eight waves): measured 4% shorter phases
  docopy();
  if (diag0) kvp_mask(x, kpos, qp, g);
  bf16x8_t pb[2];
  kvp_pack(x, pb);
  px[lane] = __builtin_bit_cast(uint4, pb[0]);
  px[64 + lane] = __builtin_bit_cast(uint4, pb[1]);
  // stage 3: dV^T += dO^T P_0 with P_1
  {
    bf16x8_t td[NF];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) td[h * NB + nb] = kvf_tr<D>(dt, o, nb, h);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) av[nb] = mfma32(td[h * NB + nb], pb[h], av[nb]);
    kvp_p<D>(sc1, l2, o, 1, c, x);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // two fragments, the LSE values
#pragma unroll
    for (int i = 0; i < NF - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (diag1) kvp_mask(x, kpos, qp + 32, g);
  kvp_pack(x, pb);
  px[128 + lane] = __builtin_bit_cast(uint4, pb[0]);
  px[192 + lane] = __builtin_bit_cast(uint4, pb[1]);
  // stage 4: dV^T += dO^T P_1
  {
    bf16x8_t td[NF];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) td[h * NB + nb] = kvf_tr<D>(dt, o, nb, 2 + h);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) av[nb] = mfma32(td[h * NB + nb], pb[h], av[nb]);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NF - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Wave B: dP_0 | dP_1 with dS_0 = P_0 (dP_0 - D) | dK^T += Q^T dS_0 with dS_1 |
// dK^T += Q^T dS_1; P comes from the pair's exchange slot.
template <int D>
__device__ __forceinline__ void kvp_ds(const f32x16_t& dp, const float* ddl, const uint4* px,
                                       const KvfOffsets<D>& o, int mq, int lane, bf16x8_t (&sb)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q0 = 32 * mq + 16 * h;
    const float4 da = *reinterpret_cast<const float4*>(ddl + q0 + o.stat);
    const float4 db = *reinterpret_cast<const float4*>(ddl + q0 + 8 + o.stat);
    const float dv8[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
    const uint4 pw = px[128 * mq + 64 * h + lane];
    const uint32_t pu[4] = {pw.x, pw.y, pw.z, pw.w};
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r0 = 8 * h + 2 * e;
      wv[e] = pack_bf16(bf16_lo(pu[e]) * (dp[r0] - dv8[2 * e]), bf16_hi(pu[e]) * (dp[r0 + 1] - dv8[2 * e + 1]));
    }
    sb[h] = __builtin_bit_cast(bf16x8_t, uint4{wv[0], wv[1], wv[2], wv[3]});
  }
}

template <int D, typename Copy>
__device__ __forceinline__ void kvp_tile_b(const bf16_t* qt, const bf16_t* dt, const float* ddl, const uint4* px,
                                           const bf16x8_t (&vf)[D / 16], f32x16_t (&ak)[D / 32],
                                           const KvfOffsets<D>& o, int lane, Copy&& docopy, bf16_t* dsrow,
                                           bf16x8_t (&keep)[2]) {
  constexpr int KS = D / 16, NB = D / 32, NF = 2 * NB;
  __builtin_amdgcn_sched_barrier(0);
  f32x16_t dp0 = f32x16_t{}, dp1 = f32x16_t{};
  {
    bf16x8_t fd[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) fd[kk] = as_bf16x8(load16(dt + o.row[kk]));
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) dp0 = mfma32(fd[kk], vf[kk], dp0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < KS - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  bf16x8_t sb[2];
  {
    bf16x8_t fd[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) fd[kk] = as_bf16x8(load16(dt + 32 * D + o.row[kk]));
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) dp1 = mfma32(fd[kk], vf[kk], dp1);
    kvp_ds<D>(dp0, ddl, px, o, 0, lane, sb);
    if (dsrow) ds_store_pair(dsrow, sb, 0, lane);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // two fragments, D values, P
#pragma unroll
    for (int i = 0; i < KS - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  docopy();
  {
    bf16x8_t tq[NF];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) tq[h * NB + nb] = kvf_tr<D>(qt, o, nb, h);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) ak[nb] = mfma32(tq[h * NB + nb], sb[h], ak[nb]);
    kvp_ds<D>(dp1, ddl, px, o, 1, lane, sb);
    if (dsrow) {   // stored by the caller after the phase's barrier
      keep[0] = sb[0];
      keep[1] = sb[1];
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);   // two fragments, D values, P
#pragma unroll
    for (int i = 0; i < NF - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  {
    bf16x8_t tq[NF];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) tq[h * NB + nb] = kvf_tr<D>(qt, o, nb, 2 + h);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) ak[nb] = mfma32(tq[h * NB + nb], sb[h], ak[nb]);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NF - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The per-lane offsets pass through an empty asm in place: every read after it becomes
// offset register + immediate, and none of the address sums is kept across phases.
template <int D>
__device__ __forceinline__ void asm_fence_offsets(KvfOffsets<D>& o) {
#pragma unroll
  for (int i = 0; i < D / 16; ++i) asm volatile("" : "+v"(o.row[i]));
#pragma unroll
  for (int i = 0; i < D / 32; ++i) asm volatile("" : "+v"(o.tr[i][0]), "+v"(o.tr[i][1]));
  asm volatile("" : "+v"(o.stat));
}

// One phase of a wave: this wave's two halves of its own tile, with the copies of the next
// tile into the idle set issued in the middle (every wave issues its share, working or
// not).  All LDS buffers are
// restrict parameters of this one inlined function, so the compiler knows the tile's
// reads do not depend on the copies in flight and does not wait for them.
struct KvpCopy {
  const bf16_t* qsrc;
  const bf16_t* dsrc;
  const float* ssrc;
  bool on;
};

template <int D>
__device__ __forceinline__ void kvp_copy(const KvpCopy& cp, const CopyOffsets<D, 8>& co, bf16_t* __restrict__ nq,
                                         bf16_t* __restrict__ nd, float* __restrict__ ns, int wu, int lane) {
  if (cp.on) {
    copy_tile<D, 8>(cp.qsrc, co, nq, wu);
    copy_tile<D, 8>(cp.dsrc, co, nd, wu);
    floats_direct(cp.ssrc, ns, lane);
  }
}

template <int D>
__device__ __forceinline__ void kvp_phase_a(const bf16_t* __restrict__ qt, const bf16_t* __restrict__ dt,
                                            const float* __restrict__ l2, uint4* __restrict__ px,
                                            bf16_t* __restrict__ nq, bf16_t* __restrict__ nd,
                                            float* __restrict__ ns, const KvpCopy& cp, const CopyOffsets<D, 8>& co,
                                            bool work, const bf16x8_t (&kf)[D / 16], f32x16_t (&av)[D / 32],
                                            const KvfOffsets<D>& o, int kpw, int qp, float c, int wu, int lane) {
  auto docopy = [&]() { kvp_copy<D>(cp, co, nq, nd, ns, wu, lane); };
  if (!work) {
    docopy();
    return;
  }
  // diagonal halves need the causal mask; a half whose queries all come before the
  // pair's keys gets P = 0 from it (the whole tile is skipped when both do)
  kvp_tile_a<D>(qt, dt, l2, px, kf, av, o, lane >> 5, qp, kpw + (lane & 31), c, kpw + 31 > qp, kpw + 31 > qp + 32,
                lane, docopy);
}

template <int D>
__device__ __forceinline__ void kvp_phase_b(const bf16_t* __restrict__ qt, const bf16_t* __restrict__ dt,
                                            const float* __restrict__ ddl, const uint4* __restrict__ px,
                                            bf16_t* __restrict__ nq, bf16_t* __restrict__ nd,
                                            float* __restrict__ ns, const KvpCopy& cp, const CopyOffsets<D, 8>& co,
                                            bool work, const bf16x8_t (&vf)[D / 16], f32x16_t (&ak)[D / 32],
                                            const KvfOffsets<D>& o, int kpw, int qp, int wu, int lane,
                                            bf16_t* dsrow, bf16x8_t (&keep)[2]) {
  auto docopy = [&]() { kvp_copy<D>(cp, co, nq, nd, ns, wu, lane); };
  if (!work) {
    docopy();
    return;
  }
  kvp_tile_b<D>(qt, dt, ddl, px, vf, ak, o, lane, docopy, dsrow, keep);
}

template <int D, bool SPLIT, bool PERSIST, bool DSW = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void kvp_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, long kv_bstride,
    const float* __restrict__ lse2v, const float* __restrict__ ddv, const bf16_t* __restrict__ dout,
    bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, float* __restrict__ part_k, float* __restrict__ part_v, int N,
    int H, int Hkv, int G, int shift_on, float scale, int tpg, int upg, int m, int units, int slots,
    bf16_t* __restrict__ dsw) {
  constexpr int NP = 4, BN = 32 * NP, NW = 2 * NP;
  __shared__ __align__(16) KvpLds<D> lds;
  const float c = scale * kLog2e;
  const int tid = thread_x(), w = tid / 64, lane = tid % 64, lq = lane % 32, g = lane / 32;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const bool role_a = wu < NP;
  const int pr = wu % NP;   // pair
  const CopyOffsets<D, NW> coffs = copy_offsets<D, NW>(wu, lane, (long)H * D);
  KvfOffsets<D> offs = kvf_offsets<D>(lane);

  const int per = (units + 7) / 8;
  const int xcd = group_x() % 8, slot = group_x() / 8;
  const int nrounds = PERSIST ? (per + slots - 1) / slots : 1;
  for (int r = 0; r < nrounds; ++r) {
  const int vv = r * slots + ((r & 1) ? slots - 1 - slot : slot);
  const int u = xcd * per + vv;
  if (vv >= per || u >= units) continue;
  const int ngroups = N / G;
  const int rep = H / Hkv;
  int qq = u % upg;
  int rest = u / upg;
  const int grp = rest % ngroups;
  rest /= ngroups;
  const int kvh = rest % Hkv;
  const int b = rest / Hkv;
  int tig = qq, part = 0, nparts = 1;
  if (SPLIT) {
    tig = 0;
    for (;;) {
      nparts = kv_parts(rep, G, BN, tig, m);
      if (qq < nparts) break;
      qq -= nparts;
      ++tig;
    }
    part = qq;
  }
  const int s = (shift_on && ngroups >= 2 && kvh >= Hkv / 2) ? G / 2 : 0;
  const int gstart = grp * G;
  const int kp0 = gstart + tig * BN;
  const int kpw = kp0 + 32 * pr;   // first key of this wave's pair
  const bool active = kpw < gstart + G;
  const int qt0 = (kp0 - gstart) / kTile;
  const int nqt = G / kTile - qt0;

  const long qs = (long)H * D, ks = (long)Hkv * D;
  const int tokw = active ? (kpw + s) % N : 0;
  const long krow_in = b * kv_bstride + (long)(tokw + lq) * ks + (long)kvh * D;
  // wave A: K rows; wave B: V rows
  bf16x8_t kvf[D / 16];
  if (active) load_row_frag<D>(kvf, (role_a ? k : v) + krow_in, g);
  f32x16_t acc[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) acc[nb] = f32x16_t{};

  // the unit's share of the key block's iterations (parts of a split block differ by at
  // most one iteration); item i = (q head, query tile) in that order
  const int iters = rep * nqt;
  const int it0 = (int)((long)part * iters / nparts), it1 = (int)((long)(part + 1) * iters / nparts);
  const int n = it1 - it0;
  // item cursors, advanced one item at a time (no division in the loop): the item this
  // wave works on and the item whose tile is copied next
  struct Cur {
    int hh, qti;
  };
  auto advance = [&](Cur c_) {
    if (++c_.qti == qt0 + nqt) {
      c_.qti = qt0;
      ++c_.hh;
    }
    return c_;
  };
  const Cur first{it0 / nqt, qt0 + it0 % nqt};
  // source of the tile of an item; wave NW - 1 copies the LSE row, the others the D row
  // (identical writes)
  auto source = [&](Cur c_, bool on) {
    const int h = kvh * rep + c_.hh;
    int tok = gstart + kTile * c_.qti + s;
    if (tok >= N) tok -= N;
    const long off = ((long)b * N + tok) * qs + (long)h * D;
    const long soff = ((long)b * H + h) * N + tok;
    return KvpCopy{q + off, dout + off, (wu == NW - 1 ? lse2v : ddv) + soff, on};
  };
  {
    float* ns = wu == NW - 1 ? lds.l2[0] : lds.dd[0];
    kvp_copy<D>(source(first, true), coffs, lds.q[0], lds.o[0], ns, wu, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // phase ph: wave A works on item ph (set ph % 3), wave B on item ph - 1 (set (ph + 2) % 3),
  // and the tile of item ph + 1 is copied into set (ph + 1) % 3, whose item (ph - 2) wave B
  // finished in the previous phase.  Each role runs its own loop (one barrier per phase
  // in both), so each accumulator is written on one path only.  The offsets pass through
  // an empty asm at the top of each phase, so the compiler cannot keep one address per
  // read and buffer set across phases.
  Cur cw = first;               // this wave's next item (wave B: from phase 1 on)
  Cur cc = advance(first);      // next item to copy
  int ncopied = 1;
  if (role_a) {
    for (int ph = 0; ph <= n; ++ph) {
      const int sa = ph % 3, sn = (ph + 1) % 3;
      asm_fence_offsets(offs);
      const bool on = ncopied < n;
      kvp_phase_a<D>(lds.q[sa], lds.o[sa], lds.l2[sa], &lds.px[sa][pr][0][0][0], lds.q[sn], lds.o[sn],
                     wu == NW - 1 ? lds.l2[sn] : lds.dd[sn], source(cc, on), coffs,
                     active && ph < n && kpw <= gstart + kTile * cw.qti + 63, kvf, acc, offs, kpw,
                     gstart + kTile * cw.qti, c, wu, lane);
      if (on) {
        cc = advance(cc);
        ++ncopied;
      }
      cw = advance(cw);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  } else {
    // with DSW, wave B also writes dS (unscaled, bf16) for dQ = scale dS K: tile (query tile
    // qt, key tile kt) of a (batch, q head, group) at ((b H + h) ngroups + grp) tri +
    // qt (qt + 1) / 2 + kt (tri = its lower-triangle tile count), 4096 elements each, the
    // pair's keys in half (kpw - gstart) % 64 / 32 of it.  The second query half is stored
    // after the phase's barrier, so the wait for the next tile's copies does not also
    // wait for these stores.
    const int ntl = G / kTile;
    const long tri = (long)ntl * (ntl + 1) / 2;
    const int ktl = (kpw - gstart) / kTile;
    const int kpair = (kpw - gstart) % kTile / 32;
    bf16x8_t keep[2];
    for (int ph = 0; ph <= n; ++ph) {
      const int sb = (ph + 2) % 3, sn = (ph + 1) % 3;
      asm_fence_offsets(offs);
      const bool on = ncopied < n;
      const bool work = active && ph >= 1 && kpw <= gstart + kTile * cw.qti + 63;
      bf16_t* dsrow = nullptr;
      if (DSW) {
        const long h = (long)kvh * rep + cw.hh;
        const int qt = cw.qti;
        dsrow = dsw + ((((long)b * H + h) * ngroups + grp) * tri + (long)qt * (qt + 1) / 2 + ktl) * (kTile * kTile) +
                kpair * 2048;
      }
      kvp_phase_b<D>(lds.q[sb], lds.o[sb], lds.dd[sb], &lds.px[sb][pr][0][0][0], lds.q[sn], lds.o[sn],
                     wu == NW - 1 ? lds.l2[sn] : lds.dd[sn], source(cc, on), coffs, work, kvf, acc, offs, kpw,
                     gstart + kTile * cw.qti, wu, lane, dsrow, keep);
      if (on) {
        cc = advance(cc);
        ++ncopied;
      }
      if (ph >= 1) cw = advance(cw);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (DSW && work) ds_store_pair(dsrow, keep, 1, lane);
    }
  }
  if (active) {
    // wave A stores dV, wave B dK (scaled)
    const float mul = role_a ? 1.f : scale;
    if (!SPLIT || nparts == 1) {
      // through this wave's 32 x D share of the (now idle) tile sets
      bf16_t* st = (wu < 4 ? lds.q[wu / 2] : lds.o[(wu - 4) / 2]) + (wu % 2) * 32 * D;
      const long orow0 = ((long)b * N + tokw) * ks + (long)kvh * D;
      // an opaque copy of the lane index: the store addresses are computed here, not
      // hoisted out of the unit loop into registers (which spill)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      store_acc_tile<D>(acc, mul, st, (role_a ? dv : dk) + orow0, ks, ln);
    } else {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      store_acc_f32<D>(acc, mul, (role_a ? part_v : part_k) + ((long)u * BN + 32 * pr + (ln & 31)) * D, ln >> 5);
    }
  }
  __syncthreads();   // the next unit reuses the LDS tiles
  }
}

// Query-major dQ with two 32-query blocks per wave (one wave per SIMD, four per
// workgroup, 256 queries per unit).  Each K/V fragment read from LDS feeds both blocks,
// and the two blocks' MFMA chains are independent, so the matrix core always has work
// while a chain's result or a fragment is pending.  Per 32-key half, with lane = query
// and registers over keys: S^T = K Q^T and dP^T = V dO^T for both blocks, then
// dS = P (dP - D) packed to bf16; after both halves dQ^T += K^T dS^T from transposed
// fragments of the same K tile.  The exponentials of one half run between the MFMAs of
// the next.
template <int D, bool DIAG, typename Pre>
__device__ __forceinline__ void dqw_tile(const bf16_t* kt, const bf16_t* vt, const KvfOffsets<D>& o,
                                         const bf16x8_t (&qf)[2][D / 16], const bf16x8_t (&dof)[2][D / 16],
                                         f32x16_t (&acc)[2][D / 32], const float (&lse2)[2], const float (&dd)[2],
                                         int g, int kp0, const int (&qpos)[2], float c, Pre&& pre) {
  constexpr int KS = D / 16, NB = D / 32;
  bf16x8_t dsb[2][4];   // [block][32-key half * 2 + 16-key step]
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    bf16x8_t fk[KS], fv[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) fk[kk] = as_bf16x8(load16(kt + 32 * mb * D + o.row[kk]));
    if (mb == 0) pre();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) fv[kk] = as_bf16x8(load16(vt + 32 * mb * D + o.row[kk]));
    f32x16_t sc[2], dp[2];
    sc[0] = sc[1] = dp[0] = dp[1] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      sc[0] = mfma32(fk[kk], qf[0][kk], sc[0]);
      sc[1] = mfma32(fk[kk], qf[1][kk], sc[1]);
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      dp[0] = mfma32(fv[kk], dof[0][kk], dp[0]);
      dp[1] = mfma32(fv[kk], dof[1][kk], dp[1]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x2[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int r = 8 * h + 2 * e + t;
            float p = fast_exp2(__builtin_fmaf(sc[j][r], c, -lse2[j]));
            if constexpr (DIAG) {
              const int kp = kp0 + 32 * mb + 8 * (r / 4) + 4 * g + (r % 4);
              p = (kp <= qpos[j]) ? p : 0.f;
            }
            x2[t] = p * (dp[j][r] - dd[j]);
          }
          wv[e] = pack_bf16(x2[0], x2[1]);
        }
        dsb[j][2 * mb + h] = __builtin_bit_cast(bf16x8_t, uint4{wv[0], wv[1], wv[2], wv[3]});
      }
    }
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8_t t = kvf_tr<D>(kt, o, nb, kb);
      acc[0][nb] = mfma32(t, dsb[0][kb], acc[0][nb]);
      acc[1][nb] = mfma32(t, dsb[1][kb], acc[1][nb]);
    }
}

template <int D, bool PERSIST, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void dqw_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    float* __restrict__ lse2v, float* __restrict__ ddv, const bf16_t* __restrict__ dout, const bf16_t* __restrict__ o,
    const float* __restrict__ lse, bf16_t* __restrict__ dq, int N, int H, int Hkv, int G, int shift_on, float scale,
    int tpg, int units, int slots) {
  constexpr int NW = 4, BM = 64 * NW;
  // two K/V buffer sets as separate LDS objects, used alternately by a loop unrolled
  // twice (the compiler then does not make the reads of one set wait for the copies into
  // the other)
  __shared__ __align__(16) bf16_t ka[kTile * D], kb[kTile * D], va[kTile * D], vb[kTile * D];
  const float c = scale * kLog2e;
  const int tid = thread_x(), w = tid / 64, lane = tid % 64, lq = lane % 32, g = lane / 32;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const KvfOffsets<D> offs = kvf_offsets<D>(lane);
  const CopyOffsets<D, NW> coffs = copy_offsets<D, NW>(w, lane, (long)Hkv * D);

  const int per = (units + 7) / 8;
  const int xcd = group_x() % 8, slot = group_x() / 8;
  const int nrounds = PERSIST ? (per + slots - 1) / slots : 1;
  for (int r = 0; r < nrounds; ++r) {
  const int vv = r * slots + ((r & 1) ? slots - 1 - slot : slot);
  const int u = xcd * per + vv;
  if (vv >= per || u >= units) continue;
  const int ngroups = N / G;
  const int tig = tpg - 1 - u % tpg;
  int rest = u / tpg;
  const int grp = rest % ngroups;
  rest /= ngroups;
  const int h = rest % H;
  const int b = rest / H;
  const int s = (shift_on && ngroups >= 2 && h >= H / 2) ? G / 2 : 0;
  const int kvh = h / (H / Hkv);

  const int gstart = grp * G;
  const int qp0 = gstart + tig * BM;
  const int qlast = min(qp0 + BM, gstart + G) - 1;
  const int ntiles = (qlast - gstart) / kTile + 1;
  const long qs = (long)H * D, ks = (long)Hkv * D;

  bf16x8_t qf[2][D / 16], dof[2][D / 16];
  float lse2[2], dd[2];
  int qpos[2];
  long qbase[2];   // row 0 of each block (wave-uniform); lane lq owns row lq
  bool act[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qpw = qp0 + 64 * wu + 32 * j;
    act[j] = qpw < gstart + G;
    qpos[j] = qpw + lq;
    const int tok = act[j] ? (qpw + s) % N : 0;
    qbase[j] = ((long)b * N + tok) * qs + (long)h * D;
    if (act[j]) {
      load_row_frag<D>(qf[j], q + qbase[j] + lq * (int)qs, g);
      load_row_frag<D>(dof[j], dout + qbase[j] + lq * (int)qs, g);
      const long si = ((long)b * H + h) * N + tok + lq;
      if constexpr (FUSED) {
        // the row statistics of this block's rows, written for the key-major kernel that
        // follows: D = rowsum(dO * O) (lane halves g hold the two column halves) and
        // LSE * log2(e)
        bf16x8_t of[D / 16];
        load_row_frag<D>(of, o + qbase[j] + lq * (int)qs, g);
        float a = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
          for (int e = 0; e < 8; ++e) a = __builtin_fmaf((float)of[kk][e], (float)dof[j][kk][e], a);
        dd[j] = pair_sum(a);
        lse2[j] = lse[si] * kLog2e;
        if (g == 0) {
          ddv[si] = dd[j];
          lse2v[si] = lse2[j];
        }
      } else {
        lse2[j] = lse2v[si];
        dd[j] = ddv[si];
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) qf[j][kk] = dof[j][kk] = bf16x8_t{};
      lse2[j] = __builtin_huge_valf();   // P = 0 for rows outside the group
      dd[j] = 0.f;
    }
  }
  f32x16_t acc[2][D / 32];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) acc[j][nb] = f32x16_t{};

  const bf16_t* kb0 = k + (long)b * N * ks + (long)kvh * D;
  const bf16_t* vb0 = v + (long)b * N * ks + (long)kvh * D;
  auto tok_of = [&](int it) {
    int t = gstart + kTile * it + s;
    return t >= N ? t - N : t;
  };
  {
    const long off = (long)tok_of(0) * ks;
    copy_tile<D, NW>(kb0 + off, coffs, ka, wu);
    copy_tile<D, NW>(vb0 + off, coffs, va, wu);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // step it: tile it from one set, tile it + 1 (or it again, into the unused set, on the
  // last step) copied into the other
  auto step = [&](int it, const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, bf16_t* __restrict__ kn,
                  bf16_t* __restrict__ vn) {
    const long off = (long)tok_of(it + 1 < ntiles ? it + 1 : it) * ks;
    const bf16_t* __restrict__ ksrc = kb0 + off;
    const bf16_t* __restrict__ vsrc = vb0 + off;
    auto copy = [&]() {
      copy_tile<D, NW>(ksrc, coffs, kn, wu);
      copy_tile<D, NW>(vsrc, coffs, vn, wu);
    };
    const int kp0 = gstart + kTile * it;
    if (kp0 <= qp0 + 64 * w + 63 && (act[0] || act[1])) {
      KvfOffsets<D> o = offs;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) asm volatile("" : "+v"(o.row[i]));
#pragma unroll
      for (int i = 0; i < D / 32; ++i) asm volatile("" : "+v"(o.tr[i][0]), "+v"(o.tr[i][1]));
      if (kp0 + kTile - 1 <= qp0 + 64 * w)
        dqw_tile<D, false>(kc, vc, o, qf, dof, acc, lse2, dd, g, kp0, qpos, c, copy);
      else
        dqw_tile<D, true>(kc, vc, o, qf, dof, acc, lse2, dd, g, kp0, qpos, c, copy);
    } else {
      copy();
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(it, ka, va, kb, vb);
    if (it + 1 < ntiles) step(it + 1, kb, vb, ka, va);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (act[j])   // through this wave's share of the (now idle) tile buffers
      store_acc_tile<D>(acc[j], scale, wu == 0 ? ka : wu == 1 ? kb : wu == 2 ? va : vb, dq + qbase[j], qs, lane);
  __syncthreads();   // the next unit reuses the LDS tiles
  }
}

// Sum of the float32 partials of split key blocks, in part order, rounded once to bf16:
// dV (grid y = 0) and dK (y = 1) in one launch.  One workgroup per (batch, kv head, group,
// key block, 8-key slice), one thread per 4-column piece of a key row; key blocks that ran
// as a single part were written directly and are skipped.
template <int D>
__global__ __launch_bounds__(256) void kv_reduce_kernel(const float* __restrict__ part_v, const float* __restrict__ part_k,
                                                        bf16_t* __restrict__ dv, bf16_t* __restrict__ dk, int N, int H,
                                                        int Hkv, int G, int shift_on, int bn, int tpg, int upg, int m) {
  const float* __restrict__ part = group_y() ? part_k : part_v;
  bf16_t* __restrict__ out = group_y() ? dk : dv;
  constexpr int C4 = D / 4, RPW = 256 / C4;   // 4-column pieces per row, rows per workgroup
  const int slices = bn / RPW;
  int x = group_x();
  const int sl = x % slices;
  x /= slices;
  const int tig = x % tpg;
  x /= tpg;
  const int ngroups = N / G;
  const int grp = x % ngroups;
  x /= ngroups;
  const int kvh = x % Hkv;
  const int b = x / Hkv;
  const int rep = H / Hkv;
  const int np = kv_parts(rep, G, bn, tig, m);
  const int r = RPW * sl + thread_x() / C4;   // row within the key block
  const int key = tig * bn + r;                // group-relative
  if (np == 1 || key >= G) return;
  long u0 = ((long)(b * Hkv + kvh) * ngroups + grp) * upg;
  for (int t = 0; t < tig; ++t) u0 += kv_parts(rep, G, bn, t, m);
  const int col = 4 * (thread_x() % C4);
  const float* src = part + (u0 * bn + r) * D + col;
  const long pstride = (long)bn * D;
  float4 a = float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int p = 0; p < np; ++p) {
    const float4 t = *reinterpret_cast<const float4*>(src + p * pstride);
    a.x += t.x;
    a.y += t.y;
    a.z += t.z;
    a.w += t.w;
  }
  const int s = (shift_on && ngroups >= 2 && kvh >= Hkv / 2) ? G / 2 : 0;
  const int tok = (grp * G + key + s) % N;
  *reinterpret_cast<uint2*>(out + (((long)b * N + tok) * Hkv + kvh) * D + col) =
      uint2{pack_bf16(a.x, a.y), pack_bf16(a.z, a.w)};
}


// HGA dQ: each wave holds a query block of 64 (two 32-query sub-blocks) at one wave per
// SIMD and streams 32-key half tiles (causal local ones, then those of the selected
// history chunks) through two LDS buffer sets of its own, copying its next half tile
// while it computes the current one, with no barrier.  Per half tile: S^T and dP^T for
// both sub-blocks from the same K and V row fragments, dS, then dQ^T += K^T dS^T from
// transposed fragments of the same K half tile.

// Per-lane source offsets of a wave's copy of a 32-row tile (rows of `rstride` elements).
// Instruction i covers rows i * RPI .. + RPI - 1; the swizzle repeats every 16 rows, so
// only NDIST lane offsets differ and the rest is a wave-uniform row offset.
template <int D>
struct HalfCopy {
  static constexpr int CPR = D / 8, RPI = 64 / CPR, PER = 32 / RPI, NDIST = 16 / RPI;
  int off[NDIST];
  long rstride;
};

template <int D>
__device__ __forceinline__ HalfCopy<D> half_copy_offsets(int lane, long rstride) {
  using C = HalfCopy<D>;
  C o;
#pragma unroll
  for (int i = 0; i < C::NDIST; ++i) {
    const int row = i * C::RPI + lane / C::CPR;
    o.off[i] = (int)((lane / C::CPR) * rstride) + (((lane % C::CPR) ^ swz<D>(row)) << 3);
  }
  o.rstride = rstride;
  return o;
}

template <int D>
__device__ __forceinline__ void copy_half(const bf16_t* src, const HalfCopy<D>& o, bf16_t* lds) {
  using C = HalfCopy<D>;
#pragma unroll
  for (int i = 0; i < C::PER; ++i) load_lds16(src + i * C::RPI * o.rstride + o.off[i % C::NDIST], lds + i * 512);
}

template <int D, bool DIAG, typename Pre>
__device__ __forceinline__ void hga_dqw_half(const bf16_t* kt, const bf16_t* vt, const KvfOffsets<D>& o,
                                             const bf16x8_t (&qf)[2][D / 16], const bf16x8_t (&dof)[2][D / 16],
                                             f32x16_t (&acc)[2][D / 32], const float (&lse2)[2],
                                             const float (&dd)[2], int g, int kp0, const int (&qpos)[2], float c,
                                             Pre&& pre) {
  constexpr int KS = D / 16, NB = D / 32;
  bf16x8_t fk[KS], fv[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) fk[kk] = as_bf16x8(load16(kt + o.row[kk]));
  pre();
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) fv[kk] = as_bf16x8(load16(vt + o.row[kk]));
  f32x16_t sc[2], dp[2];
  sc[0] = sc[1] = dp[0] = dp[1] = f32x16_t{};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    sc[0] = mfma32(fk[kk], qf[0][kk], sc[0]);
    sc[1] = mfma32(fk[kk], qf[1][kk], sc[1]);
  }
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) dp[0] = mfma32(fv[kk], dof[0][kk], dp[0]);
  __builtin_amdgcn_sched_barrier(0);
  // The vector work of the two query sub-blocks runs under the products that follow
  // it: P of both (it needs S only) under dP of sub-block 1, dS of sub-block 0 under the
  // transposed K reads, dS of sub-block 1 under dQ of sub-block 0.
  float p[2][16];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) dp[1] = mfma32(fv[kk], dof[1][kk], dp[1]);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pr = fast_exp2(__builtin_fmaf(sc[j][r], c, -lse2[j]));
      if constexpr (DIAG) {
        const int kp = kp0 + 8 * (r / 4) + 4 * g + (r % 4);
        pr = (kp <= qpos[j]) ? pr : 0.f;
      }
      p[j][r] = pr;
    }
#pragma unroll
  for (int i = 0; i < KS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // dS = P (dP - D), packed to bf16 in the MFMA's K order
  auto ds_pack = [&](int j, bf16x8_t (&dsb)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * h + 2 * e;
        wv[e] = pack_bf16(p[j][r] * (dp[j][r] - dd[j]), p[j][r + 1] * (dp[j][r + 1] - dd[j]));
      }
      dsb[h] = __builtin_bit_cast(bf16x8_t, uint4{wv[0], wv[1], wv[2], wv[3]});
    }
  };
  bf16x8_t t[2][NB];
  bf16x8_t ds0[2], ds1[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) t[kb][nb] = kvf_tr<D>(kt, o, nb, kb);
  ds_pack(0, ds0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[0][nb] = mfma32(t[kb][nb], ds0[kb], acc[0][nb]);
  ds_pack(1, ds1);
#pragma unroll
  for (int i = 0; i < 2 * NB; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[1][nb] = mfma32(t[kb][nb], ds1[kb], acc[1][nb]);
}

// A local half tile from the stored dS instead (tile (j, t / 2) of the block's (batch,
// head), pair t % 2, masked on the diagonal by the key-major kernel that wrote it): only
// dQ^T += K^T dS^T.  The dS half tile (4 KB) is staged in the V buffer in the slot order
// of a full tile's first pair, so the transposed reads give the fragments directly.
__device__ __forceinline__ void copy_ds_half(const bf16_t* src, const int (&off)[4], bf16_t* lds) {
#pragma unroll
  for (int i = 0; i < 4; ++i) load_lds16_stream(src + off[i], lds + i * 512);
}

template <int D, typename Pre>
__device__ __forceinline__ void hga_dqw_half_ds(const bf16_t* kt, const bf16_t* dst, const KvfOffsets<D>& o,
                                                const int (&dso)[2], f32x16_t (&acc)[2][D / 32], Pre&& pre) {
  constexpr int NB = D / 32;
  bf16x8_t sb[2][2];   // [sub-block][16-key step]
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int j = 0; j < 2; ++j) sb[j][kb] = ds_frag(dst, dso[j], kb);
  pre();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8_t t = kvf_tr<D>(kt, o, nb, kb);
      acc[0][nb] = mfma32(t, sb[0][kb], acc[0][nb]);
      acc[1][nb] = mfma32(t, sb[1][kb], acc[1][nb]);
    }
}

// DSQ: the local half tiles come from the stored dS tiles at dsw (lower-triangle order per
// (batch, head), as the key-major kernel writes them for a single group of S keys), and the
// row statistics from the workspace; otherwise every half tile is recomputed and the kernel
// writes the statistics for the key-major kernel that follows.
template <int D, bool DSQ>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 1))) void hga_dqw_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_act, const bf16_t* __restrict__ v_act,
    long act_bstride, const bf16_t* __restrict__ k_hist, const bf16_t* __restrict__ v_hist, long hist_bstride,
    const int32_t* __restrict__ idx, const bf16_t* __restrict__ o, const float* __restrict__ lse,
    float* __restrict__ lse2v, float* __restrict__ ddv, const bf16_t* __restrict__ dout, bf16_t* __restrict__ dq,
    const bf16_t* __restrict__ dsw, int S, int H, int Hkv, int C, int chunk, int topk, float scale, int units,
    int hpl) {
  // per wave, two half-tile buffer sets (separate LDS objects, used alternately by a loop
  // unrolled twice, so the reads of one set do not wait for the copies into the other)
  __shared__ __align__(16) bf16_t ka_[2][32 * D], va_[2][32 * D], kb_[2][32 * D], vb_[2][32 * D];
  constexpr int NB = D / 32;
  const float c = scale * kLog2e;
  const int nqb = S / 64;
  const int nbh = units / nqb;   // (batch, head) pairs
  // heaviest query blocks first; within one block index, the heads of a kv head on one
  // XCD (workgroup i runs on XCD i mod 8) when the pairs divide evenly
  const int j = nqb - 1 - group_x() / nbh;
  const int i = group_x() % nbh;
  const int bh = (nbh % 8 == 0) ? (i % 8) * (nbh / 8) + i / 8 : i;
  const int h = bh % H;
  const int b = bh / H;
  const int kvh = h / (H / Hkv);
  const int tid = thread_x(), lane = tid % 64, lq = lane % 32, g = lane / 32;
  const int wu = __builtin_amdgcn_readfirstlane(tid / 64);
  const long qs = (long)H * D, ks = (long)Hkv * D;
  const KvfOffsets<D> offs = kvf_offsets<D>(lane);
  const HalfCopy<D> co = half_copy_offsets<D>(lane, ks);

  // chunk list of this block; entries outside [0, C) are skipped
  int cidx = -1;
  if (lane < topk) cidx = idx[(((long)b * (H / hpl) + h / hpl) * nqb + j) * topk + lane];
  unsigned long long rem = __ballot(lane < topk && cidx >= 0 && cidx < C);
  const int spc = chunk / 32;
  const int nloc = 2 * (j + 1);
  const int ntiles = nloc + __popcll(rem) * spc;

  bf16x8_t qf[2][D / 16], dof[2][D / 16];
  float lse2[2], dd[2];
  int qpos[2];
  // rows of this block: a wave-uniform base plus a 32-bit lane offset
  const long qbase = (long)b * S * qs + (long)h * D;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int qp = 64 * j + 32 * sb;
    qpos[sb] = qp + lq;
    const int roff = (qp + lq) * (int)qs;
    load_row_frag<D>(qf[sb], q + qbase + roff, g);
    load_row_frag<D>(dof[sb], dout + qbase + roff, g);
    const long si = ((long)b * H + h) * S + qp + lq;
    if constexpr (DSQ) {
      dd[sb] = ddv[si];
      lse2[sb] = lse2v[si];
    } else {
      // the row statistics, D = rowsum(dO * O) (lane halves g hold the two column halves)
      // and LSE * log2(e); wave 0 writes them for the key-major kernel that follows
      bf16x8_t of[D / 16];
      load_row_frag<D>(of, o + qbase + roff, g);
      float a = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) a = __builtin_fmaf((float)of[kk][e], (float)dof[sb][kk][e], a);
      dd[sb] = pair_sum(a);
      lse2[sb] = lse[si] * kLog2e;
      if (wu == 0 && g == 0) {
        ddv[si] = dd[sb];
        lse2v[si] = lse2[sb];
      }
    }
  }
  f32x16_t acc[2][NB];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[sb][nb] = f32x16_t{};

  const bf16_t* ka = k_act + b * act_bstride + (long)kvh * D;
  const bf16_t* va = v_act + b * act_bstride + (long)kvh * D;
  const bf16_t* kh = k_hist + b * hist_bstride + (long)kvh * D;
  const bf16_t* vh = v_hist + b * hist_bstride + (long)kvh * D;
  // DSQ: this (batch, head)'s dS tiles of query tile j, its copy offsets (LDS slot
  // 64 i + lane of a half tile holds chunk ds_chunk_of_slot(64 i + lane)) and the
  // transposed-read offsets of the two 32-query sub-blocks
  const bf16_t* dsj = nullptr;
  int dco[4], dso[2];
  if constexpr (DSQ) {
    const long tri = (long)nqb * (nqb + 1) / 2;
    dsj = dsw + (((long)b * H + h) * tri + (long)j * (j + 1) / 2) * (kTile * kTile);
#pragma unroll
    for (int i = 0; i < 4; ++i) dco[i] = 8 * ds_chunk_of_slot(64 * i + lane);
    dso[0] = ds_tr_offset(lane, 0);
    dso[1] = ds_tr_offset(lane, 1);
  }
  // copy cursor over the block's half tiles in order (local ones first, then each selected
  // chunk); past the end it stays on the last one.  A half tile's sources: K rows, and V
  // rows or (local, DSQ) its dS half tile.
  struct Src {
    const bf16_t* k;
    const bf16_t* v;
    bool ds;
  };
  int nxt = 0, cur = 0;
  auto next_src = [&]() {
    const int t = nxt < ntiles ? nxt : ntiles - 1;
    Src r;
    if (t < nloc) {
      r.k = ka + 32l * t * ks;
      r.ds = DSQ;
      r.v = DSQ ? dsj + (t >> 1) * (kTile * kTile) + (t & 1) * (32 * kTile) : va + 32l * t * ks;
    } else {
      const int sub = (t - nloc) % spc;
      if (sub == 0 && nxt < ntiles) {   // next selected chunk
        cur = __builtin_amdgcn_readlane(cidx, __builtin_ctzll(rem));
        rem &= rem - 1;
      }
      const long r0 = (long)cur * chunk + 32l * sub;
      r.k = kh + r0 * ks;
      r.v = vh + r0 * ks;
      r.ds = false;
    }
    ++nxt;
    return r;
  };
  auto issue = [&](const Src& sr, bf16_t* kn, bf16_t* vn) {
    copy_half<D>(sr.k, co, kn);
    if (DSQ && sr.ds)
      copy_ds_half(sr.v, dco, vn);
    else
      copy_half<D>(sr.v, co, vn);
  };
  // wave w takes half tiles w, w + 2, w + 4, ... (an equal share of the causal prefix,
  // one of the two diagonal half tiles, and half of each selected chunk)
  {
    if (wu == 1) next_src();
    issue(next_src(), ka_[wu], va_[wu]);
  }
  __builtin_amdgcn_s_waitcnt(0);
  auto step = [&](int it, const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, bf16_t* __restrict__ kn,
                  bf16_t* __restrict__ vn) {
    next_src();                    // the other wave's
    const Src sn = next_src();     // half tile it + 2 (past the end: the last one again, harmlessly)
    auto copy = [&]() { issue(sn, kn, vn); };
    KvfOffsets<D> o = offs;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) asm volatile("" : "+v"(o.row[i]));
#pragma unroll
    for (int i = 0; i < D / 32; ++i) asm volatile("" : "+v"(o.tr[i][0]), "+v"(o.tr[i][1]));
    const int kp0 = 32 * it;
    if constexpr (DSQ) {
      if (it < nloc) {
        int dz[2] = {dso[0], dso[1]};
        asm volatile("" : "+v"(dz[0]), "+v"(dz[1]));
        hga_dqw_half_ds<D>(kc, vc, o, dz, acc, copy);
      } else {
        hga_dqw_half<D, false>(kc, vc, o, qf, dof, acc, lse2, dd, g, kp0, qpos, c, copy);
      }
    } else {
      if (it >= nloc - 2 && it < nloc)   // the block's diagonal half tiles
        hga_dqw_half<D, true>(kc, vc, o, qf, dof, acc, lse2, dd, g, kp0, qpos, c, copy);
      else
        hga_dqw_half<D, false>(kc, vc, o, qf, dof, acc, lse2, dd, g, kp0, qpos, c, copy);
    }
    __builtin_amdgcn_s_waitcnt(0);
  };
  for (int it = wu; it < ntiles; it += 4) {
    step(it, ka_[wu], va_[wu], kb_[wu], vb_[wu]);
    if (it + 2 < ntiles) step(it + 2, kb_[wu], vb_[wu], ka_[wu], va_[wu]);
  }
  // wave 1's float32 partial goes to wave 0 through wave 1's (now idle) buffers: D / 64
  // accumulators of 64 lanes x 16 floats per buffer, float4 [register / 4][lane] order
  __syncthreads();
  constexpr int APB = D / 64;
  bf16_t* const xb[4] = {ka_[1], va_[1], kb_[1], vb_[1]};
  if (wu == 1) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int a = sb * NB + nb;
        float* x = reinterpret_cast<float*>(xb[a / APB]) + (a % APB) * 1024;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *reinterpret_cast<float4*>(x + (i4 * 64 + lane) * 4) =
              float4{acc[sb][nb][4 * i4], acc[sb][nb][4 * i4 + 1], acc[sb][nb][4 * i4 + 2], acc[sb][nb][4 * i4 + 3]};
      }
  }
  __syncthreads();
  if (wu == 0) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int a = sb * NB + nb;
        const float* x = reinterpret_cast<const float*>(xb[a / APB]) + (a % APB) * 1024;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const float4 t = *reinterpret_cast<const float4*>(x + (i4 * 64 + lane) * 4);
          acc[sb][nb][4 * i4] += t.x;
          acc[sb][nb][4 * i4 + 1] += t.y;
          acc[sb][nb][4 * i4 + 2] += t.z;
          acc[sb][nb][4 * i4 + 3] += t.w;
        }
      }
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)   // through wave 0's (idle) first buffer
      store_acc_tile<D>(acc[sb], scale, ka_[0], dq + qbase + (64 * j + 32 * sb) * qs, qs, lane);
  }
}

template <int D>
void launch_rowdot(const bf16_t* o, const bf16_t* dout, float* dd, const float* lse, float* lse2, int B, int L, int H,
                   hipStream_t st) {
  auto wgs = [&](int t) { return (long)B * ((L + t - 1) / t) * ((H + 31) / 32); };
  if (wgs(16) >= 512)
    hipLaunchKernelGGL((bwd_rowdot_kernel<D, 16>), dim3((unsigned)wgs(16)), dim3(256), 0, st, o, dout, dd, lse, lse2,
                       L, H);
  else
    hipLaunchKernelGGL((bwd_rowdot_kernel<D, 4>), dim3((unsigned)wgs(4)), dim3(256), 0, st, o, dout, dd, lse, lse2,
                       L, H);
}

// How the key-major kernels cover (B, N, H, Hkv, G): keys per workgroup (four waves of
// 32), key blocks per group, workgroups per group, iterations per part and workgroups in
// all; `partial_floats` is the float32 scratch a split needs (0 without split).
struct KvPlan {
  int bn, tpg, upg, m;
  long units;
  size_t partial_floats;
};

// Fewer workgroups than the chip's slots (256 CUs, one fused workgroup each) leave CUs
// idle, so the iterations are then split into at most that many parts of at least
// kKvMinPart iterations each (a part's partial writes and their reduction cost about one
// iteration), as even as the rounding allows.
constexpr int kKvMinPart = 8;

KvPlan kv_plan(int B, int N, int H, int Hkv, int G, bool allow_split) {
  const int rep = H / Hkv, ngroups = N / G;
  KvPlan p;
  p.bn = 128;
  p.tpg = (G + p.bn - 1) / p.bn;
  p.m = kv_iters(rep, G, p.bn, 0);
  p.upg = p.tpg;
  p.units = (long)B * Hkv * ngroups * p.tpg;
  p.partial_floats = 0;
  const long target = 256L;
  if (!allow_split || p.units >= target) return p;
  long itot = 0;
  for (int t = 0; t < p.tpg; ++t) itot += kv_iters(rep, G, p.bn, t);
  const long groups = (long)B * Hkv * ngroups;
  // each key block's part count rounds up, so grow the part length until the parts fit
  // in one round of the chip's slots (a second, mostly empty round would idle most CUs
  // for a whole part; one round of longer parts also halves the partial sums to add:
  // 0.296-0.300 -> 0.288-0.291 ms for the 16K HGA backward)
  int m = (int)std::max<long>(kKvMinPart, (itot * groups + target - 1) / target);
  int upg = 0;
  for (;; ++m) {
    if (m >= p.m) return p;
    upg = 0;
    for (int t = 0; t < p.tpg; ++t) upg += kv_parts(rep, G, p.bn, t, m);
    if (groups * upg <= target) break;
  }
  p.m = m;
  p.upg = upg;
  p.units = groups * upg;
  p.partial_floats = 2 * (size_t)p.units * p.bn * 128;  // dK and dV, sized for the largest head dim
  return p;
}

// Key-major gradients on one stream, with the fused dK/dV kernel (one resident workgroup
// per CU).  Without a split: persistent for groups shorter than kPersistGroup.  Split
// (HGA segments too short to fill the chip): float32 partials of dK and dV, then one
// ordered reduction for each.
template <int D>
void launch_kv(const KvPlan& pl, const bf16_t* q, const bf16_t* k, const bf16_t* v, long kv_bstride,
               const float* lse2, const float* dd, const bf16_t* dout, bf16_t* dk, bf16_t* dv, float* part, int B,
               int N, int H, int Hkv, int G, int shift, float scale, hipStream_t st, bf16_t* dsw = nullptr) {
  const int per = (int)((pl.units + 7) / 8);
  if (pl.upg == pl.tpg) {
    const int slots = G < kPersistGroup ? std::min(per, resident_per_xcd(1)) : per;
    if (dsw != nullptr) {   // also writes dS for the streaming dQ kernel
      if (G < kPersistGroup)
        hipLaunchKernelGGL((kvp_kernel<D, false, true, true>), dim3(8 * slots), dim3(512), 0, st, q, k, v, kv_bstride,
                           lse2, dd, dout, dk, dv, nullptr, nullptr, N, H, Hkv, G, shift, scale, pl.tpg, pl.upg, pl.m,
                           (int)pl.units, slots, dsw);
      else
        hipLaunchKernelGGL((kvp_kernel<D, false, false, true>), dim3(8 * slots), dim3(512), 0, st, q, k, v,
                           kv_bstride, lse2, dd, dout, dk, dv, nullptr, nullptr, N, H, Hkv, G, shift, scale, pl.tpg,
                           pl.upg, pl.m, (int)pl.units, slots, dsw);
      return;
    }
    if (G < kPersistGroup)
      hipLaunchKernelGGL((kvp_kernel<D, false, true>), dim3(8 * slots), dim3(512), 0, st, q, k, v, kv_bstride, lse2, dd,
                         dout, dk, dv, nullptr, nullptr, N, H, Hkv, G, shift, scale, pl.tpg, pl.upg, pl.m,
                         (int)pl.units, slots, nullptr);
    else
      hipLaunchKernelGGL((kvp_kernel<D, false, false>), dim3(8 * slots), dim3(512), 0, st, q, k, v, kv_bstride, lse2,
                         dd, dout, dk, dv, nullptr, nullptr, N, H, Hkv, G, shift, scale, pl.tpg, pl.upg, pl.m,
                         (int)pl.units, slots, nullptr);
    return;
  }
  constexpr int BN = 128;
  const int slots = std::min(per, resident_per_xcd(1));
  float* part_k = part;
  float* part_v = part + (size_t)pl.units * BN * D;
  const dim3 rgrid((unsigned)((long)B * Hkv * (N / G) * pl.tpg * (BN / (256 / (D / 4)))), 2), rblk(256);
  if (dsw != nullptr)
    hipLaunchKernelGGL((kvp_kernel<D, true, true, true>), dim3(8 * slots), dim3(512), 0, st, q, k, v, kv_bstride, lse2,
                       dd, dout, dk, dv, part_k, part_v, N, H, Hkv, G, shift, scale, pl.tpg, pl.upg, pl.m,
                       (int)pl.units, slots, dsw);
  else
    hipLaunchKernelGGL((kvp_kernel<D, true, true>), dim3(8 * slots), dim3(512), 0, st, q, k, v, kv_bstride, lse2, dd,
                       dout, dk, dv, part_k, part_v, N, H, Hkv, G, shift, scale, pl.tpg, pl.upg, pl.m, (int)pl.units,
                       slots, nullptr);
  hipLaunchKernelGGL((kv_reduce_kernel<D>), rgrid, rblk, 0, st, part_v, part_k, dv, dk, N, H, Hkv, G, shift, BN, pl.tpg,
                     pl.upg, pl.m);
}

// Query-major dQ: two 32-query blocks per wave, four waves per workgroup, one resident
// workgroup per CU, persistent for groups shorter than kPersistGroup.
// With o and lse given (fused), the kernel also computes the row statistics from them
// and writes lse2 and dd; otherwise it reads them from there.
template <int D>
void launch_dq(const bf16_t* q, const bf16_t* k, const bf16_t* v, float* lse2, float* dd, const bf16_t* dout,
               const bf16_t* o, const float* lse, bf16_t* dq, int B, int N, int H, int Hkv, int G, int shift,
               float scale, hipStream_t st) {
  const int tpg = (G + 255) / 256;
  const int units = tpg * (N / G) * H * B;
  const int per = (units + 7) / 8;
  const int slots = G < kPersistGroup ? std::min(per, resident_per_xcd(1)) : per;
  const dim3 grid(8 * slots), block(256);
  const bool fused = o != nullptr;
  if (G < kPersistGroup) {
    if (fused)
      hipLaunchKernelGGL((dqw_kernel<D, true, true>), grid, block, 0, st, q, k, v, lse2, dd, dout, o, lse, dq, N, H,
                         Hkv, G, shift, scale, tpg, units, slots);
    else
      hipLaunchKernelGGL((dqw_kernel<D, true, false>), grid, block, 0, st, q, k, v, lse2, dd, dout, o, lse, dq, N, H,
                         Hkv, G, shift, scale, tpg, units, slots);
  } else {
    if (fused)
      hipLaunchKernelGGL((dqw_kernel<D, false, true>), grid, block, 0, st, q, k, v, lse2, dd, dout, o, lse, dq, N, H,
                         Hkv, G, shift, scale, tpg, units, slots);
    else
      hipLaunchKernelGGL((dqw_kernel<D, false, false>), grid, block, 0, st, q, k, v, lse2, dd, dout, o, lse, dq, N,
                         H, Hkv, G, shift, scale, tpg, units, slots);
  }
}

}  // namespace s2a

using namespace s2a;

extern "C" size_t s2attn_bwd_workspace_bytes(int B, int N, int H, int Hkv, int d) {
  (void)Hkv;
  (void)d;
  if (B <= 0 || N <= 0 || H <= 0) return 0;
  return 2 * (size_t)B * H * N * sizeof(float);  // D = rowsum(dO * O), then LSE * log2(e)
}

// The backward runs in three stages on one stream: prep (D and LSE*log2e into the
// workspace), dQ (query-major) and dK/dV (key-major).  Run separately, dQ and dK/dV only
// read the workspace, so a caller may run them on two streams after prep; run together
// (s2attn_bwd, s2attn_bwd_dq_prep), prep happens inside the dQ kernel.  s2attn_bwd with a
// workspace of s2attn_bwd_workspace_bytes_dsq bytes runs prep, then dK/dV writing dS, then
// dQ from dS (dqs_kernel), which recomputes neither S nor dP.
namespace {
// The streaming dQ path keeps the dS tiles of every (batch, head, group) between the
// key-major kernel and dqs_kernel: 2 bytes per lower-triangle tile element (553 MB at 8K
// tokens in groups of 2048, 8.7 GB at 32K tokens in groups of 8192, 32 heads).
size_t ds_bytes(int B, int N, int H, int G) {
  if (G <= 0 || N % G || G % kTile) return 0;
  const long ntl = G / kTile;
  return (size_t)B * H * (N / G) * (size_t)(ntl * (ntl + 1) / 2) * kTile * kTile * sizeof(bf16_t);
}
size_t stats_bytes_aligned(int B, int N, int H) { return ((2 * (size_t)B * H * N * sizeof(float)) + 255) & ~(size_t)255; }

enum Stage { kPrep = 1, kDq = 2, kDkdv = 4 };

int s2attn_bwd_stages(int stages, const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B,
                      int N, int H, int Hkv, int d, int G, int shift, float scale, void* stream) {
  if ((stages & kPrep) && (!ptr_ok(o) || !ptr_ok(lse))) return S2A_ERR_INVALID_ARG;
  if (!ptr_ok(dout)) return S2A_ERR_INVALID_ARG;
  if ((stages & (kDq | kDkdv)) && (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v))) return S2A_ERR_INVALID_ARG;
  if ((stages & kDq) && !ptr_ok(dq)) return S2A_ERR_INVALID_ARG;
  if ((stages & kDkdv) && (!ptr_ok(dk) || !ptr_ok(dv))) return S2A_ERR_INVALID_ARG;
  int st = check_s2attn(B, N, H, Hkv, d, G, shift, scale);
  if (st) return st;
  if (!ptr_ok(workspace) || workspace_bytes < s2attn_bwd_workspace_bytes(B, N, H, Hkv, d)) return S2A_ERR_WORKSPACE;
  // unit counts must fit an int, and the kernels' per-lane tile offsets (64 rows of
  // H * d elements) 32 bits
  if ((long)((G + 127) / 128) * (N / G) * H * B >= (1l << 31) - 8) return S2A_ERR_UNSUPPORTED;
  if ((long)H * d * kTile >= (1l << 31)) return S2A_ERR_UNSUPPORTED;
  hipStream_t sm = reinterpret_cast<hipStream_t>(stream);
  auto qp = static_cast<const bf16_t*>(q);
  auto kp = static_cast<const bf16_t*>(k);
  auto vp = static_cast<const bf16_t*>(v);
  auto op = static_cast<const bf16_t*>(o);
  auto dop = static_cast<const bf16_t*>(dout);
  float* dd = static_cast<float*>(workspace);
  float* lse2 = dd + (size_t)B * H * N;
  auto dqp = static_cast<bf16_t*>(dq);
  auto dkp = static_cast<bf16_t*>(dk);
  auto dvp = static_cast<bf16_t*>(dv);
  const KvPlan pl = kv_plan(B, N, H, Hkv, G, false);
  const long kvb = (long)N * Hkv * d;
  // With a workspace of s2attn_bwd_workspace_bytes_dsq bytes the dK/dV stage also stores
  // dS, and dQ is formed from the stored tiles after it: in one call (prep, dK/dV, dQ) or
  // as a dq stage of its own after a dkdv stage.  dq_prep (prep and dQ in one call) always
  // recomputes: no tiles exist yet.
  const size_t dsb = ds_bytes(B, N, H, G);
  const bool dsq = dsb > 0 && pl.upg == pl.tpg && workspace_bytes >= stats_bytes_aligned(B, N, H) + dsb;
  bf16_t* dsw = dsq ? reinterpret_cast<bf16_t*>(static_cast<char*>(workspace) + stats_bytes_aligned(B, N, H)) : nullptr;
  const bool dq_from_ds = dsq && (stages & kDq) && ((stages & kDkdv) || !(stages & kPrep));
  // prep and dQ together otherwise: the dQ kernel computes the row statistics of the rows
  // it owns (every row is owned by exactly one of its units) and writes them for dK/dV
  const bool fuse = (stages & kPrep) && (stages & kDq) && !dq_from_ds;
  const bf16_t* of = fuse ? op : nullptr;
  const float* lf = fuse ? lse : nullptr;
  if (d == 128) {
    if ((stages & kPrep) && !fuse) launch_rowdot<128>(op, dop, dd, lse, lse2, B, N, H, sm);
    if ((stages & kDq) && !dq_from_ds)
      launch_dq<128>(qp, kp, vp, lse2, dd, dop, of, lf, dqp, B, N, H, Hkv, G, shift, scale, sm);
    if (stages & kDkdv)
      launch_kv<128>(pl, qp, kp, vp, kvb, lse2, dd, dop, dkp, dvp, nullptr, B, N, H, Hkv, G, shift, scale, sm, dsw);
  } else {
    if ((stages & kPrep) && !fuse) launch_rowdot<64>(op, dop, dd, lse, lse2, B, N, H, sm);
    if ((stages & kDq) && !dq_from_ds)
      launch_dq<64>(qp, kp, vp, lse2, dd, dop, of, lf, dqp, B, N, H, Hkv, G, shift, scale, sm);
    if (stages & kDkdv)
      launch_kv<64>(pl, qp, kp, vp, kvb, lse2, dd, dop, dkp, dvp, nullptr, B, N, H, Hkv, G, shift, scale, sm, dsw);
  }
  if (dq_from_ds) launch_dqs(d, kp, dsw, dqp, B, N, H, Hkv, G, shift, scale, sm);
  return hipGetLastError() == hipSuccess ? S2A_OK : S2A_ERR_HIP;
}
}  // namespace

extern "C" size_t s2attn_bwd_workspace_bytes_dsq(int B, int N, int H, int Hkv, int d, int G) {
  if (s2attn_bwd_workspace_bytes(B, N, H, Hkv, d) == 0) return 0;
  const size_t dsb = ds_bytes(B, N, H, G);   // 0 unless G > 0 splits N into groups of 64-multiples
  return dsb ? stats_bytes_aligned(B, N, H) + dsb : 0;
}

extern "C" int s2attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                          int B, int N, int H, int Hkv, int d, int G, int shift, float scale, void* stream) {
  return s2attn_bwd_stages(kPrep | kDq | kDkdv, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, N,
                           H, Hkv, d, G, shift, scale, stream);
}

extern "C" int s2attn_bwd_prep(const void* o, const float* lse, const void* dout, void* workspace,
                               size_t workspace_bytes, int B, int N, int H, int Hkv, int d, int G, int shift,
                               float scale, void* stream) {
  return s2attn_bwd_stages(kPrep, nullptr, nullptr, nullptr, o, lse, dout, nullptr, nullptr, nullptr, workspace,
                           workspace_bytes, B, N, H, Hkv, d, G, shift, scale, stream);
}

extern "C" int s2attn_bwd_dq_prep(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                  const void* dout, void* dq, void* workspace, size_t workspace_bytes, int B, int N,
                                  int H, int Hkv, int d, int G, int shift, float scale, void* stream) {
  return s2attn_bwd_stages(kPrep | kDq, q, k, v, o, lse, dout, dq, nullptr, nullptr, workspace, workspace_bytes, B, N,
                           H, Hkv, d, G, shift, scale, stream);
}

extern "C" int s2attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq,
                             const void* workspace, size_t workspace_bytes, int B, int N, int H, int Hkv, int d, int G,
                             int shift, float scale, void* stream) {
  return s2attn_bwd_stages(kDq, q, k, v, nullptr, nullptr, dout, dq, nullptr, nullptr, const_cast<void*>(workspace),
                           workspace_bytes, B, N, H, Hkv, d, G, shift, scale, stream);
}

extern "C" int s2attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                               const void* workspace, size_t workspace_bytes, int B, int N, int H, int Hkv, int d,
                               int G, int shift, float scale, void* stream) {
  return s2attn_bwd_stages(kDkdv, q, k, v, nullptr, nullptr, dout, nullptr, dk, dv, const_cast<void*>(workspace),
                           workspace_bytes, B, N, H, Hkv, d, G, shift, scale, stream);
}

// ---------------------------------------------------------------------------------------
// The backward without a workspace argument, for callers that cannot allocate: the row
// statistics live in `scratch`, a file-scope device array.  Each GPU holds its own copy
// for the life of the process; its device address is looked up once per device (the
// array's name is only a host-side stand-in and must never be passed to a kernel).
// ---------------------------------------------------------------------------------------
namespace {
__device__ __align__(256) unsigned char scratch[S2A_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

// Device address of `scratch` on the current device, or null if the runtime cannot
// report it.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  return p;
}
}  // namespace

extern "C" int s2attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                  const void* dout, void* dq, void* dk, void* dv, int B, int N, int H, int Hkv,
                                  int d, int G, int shift, float scale, void* stream) {
  // every host check that needs no runtime call first, so a rejected call touches nothing
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(o) || !ptr_ok(lse) || !ptr_ok(dout) || !ptr_ok(dq) ||
      !ptr_ok(dk) || !ptr_ok(dv))
    return S2A_ERR_INVALID_ARG;
  int st = check_s2attn(B, N, H, Hkv, d, G, shift, scale);
  if (st) return st;
  if (s2attn_bwd_workspace_bytes(B, N, H, Hkv, d) > (size_t)S2A_NOALLOC_SCRATCH_BYTES) return S2A_ERR_WORKSPACE;
  void* ws = scratch_address();
  if (ws == nullptr) return S2A_ERR_HIP;
  // every statistic the kernels read is written earlier in the same call (the dQ kernel
  // writes both values of each row before the dK/dV kernel reads them), so the array's
  // contents from an earlier call never matter.  The array is offered as a workspace of
  // the statistics' size only: the call runs the recompute path (no dS tiles), the bits
  // of s2attn_bwd with a workspace of s2attn_bwd_workspace_bytes bytes.
  return s2attn_bwd_stages(kPrep | kDq | kDkdv, q, k, v, o, lse, dout, dq, dk, dv, ws,
                           s2attn_bwd_workspace_bytes(B, N, H, Hkv, d), B, N, H, Hkv, d, G, shift, scale, stream);
}

// [D | LSE * log2(e)] row statistics (float32 [B, H, S] each), then the float32 partial
// sums of the split key-major kernels when the segment alone gives too few workgroups.
extern "C" size_t hga_bwd_workspace_bytes(int B, int S, int H, int Hkv, int d) {
  (void)d;
  if (B <= 0 || S <= 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || S % kTile != 0) return 0;
  const KvPlan pl = kv_plan(B, S, H, Hkv, S, true);
  return (2 * (size_t)B * H * S + pl.partial_floats) * sizeof(float);
}

// The same, then (256-byte aligned) the bf16 dS tiles of every (batch, head)'s lower
// triangle of 64 x 64 tiles over the segment: with this much workspace the key-major kernel
// stores dS and the dQ kernel reads the local part from it.
static size_t hga_ds_offset(int B, int S, int H, int Hkv, int d) {
  return (hga_bwd_workspace_bytes(B, S, H, Hkv, d) + 255) & ~(size_t)255;
}

extern "C" size_t hga_bwd_workspace_bytes_dsq(int B, int S, int H, int Hkv, int d) {
  if (hga_bwd_workspace_bytes(B, S, H, Hkv, d) == 0) return 0;
  const size_t nt = (size_t)(S / kTile);
  return hga_ds_offset(B, S, H, Hkv, d) + (size_t)B * H * (nt * (nt + 1) / 2) * (kTile * kTile) * sizeof(bf16_t);
}

static int hga_bwd_impl(const void* q, const void* k_act, const void* v_act, long long act_bstride,
                              const void* k_hist, const void* v_hist, long long hist_bstride, const int32_t* idx,
                              const void* o, const float* lse, const void* dout, void* dq, void* dk_act,
                              void* dv_act, void* workspace, size_t workspace_bytes, int B, int S, int H, int Hkv,
                              int d, int T, int chunk, int qblock, int topk, float scale, void* stream, bool shared) {
  if (!ptr_ok(q) || !ptr_ok(k_act) || !ptr_ok(v_act) || !ptr_ok(idx) || !ptr_ok(o) || !ptr_ok(lse) ||
      !ptr_ok(dout) || !ptr_ok(dq) || !ptr_ok(dk_act) || !ptr_ok(dv_act))
    return S2A_ERR_INVALID_ARG;
  int st = check_hga_shape(B, S, H, Hkv, d, T, chunk, qblock, topk);
  if (st) return st;
  if (check_scale(scale)) return S2A_ERR_INVALID_ARG;
  if (T > 0 && (!ptr_ok(k_hist) || !ptr_ok(v_hist))) return S2A_ERR_INVALID_ARG;
  if (!stride_ok(act_bstride, S, Hkv, d, B) || !stride_ok(hist_bstride, T, Hkv, d, B)) return S2A_ERR_INVALID_ARG;
  if ((long)B * H * (S / 64) >= (1l << 31) - 8) return S2A_ERR_UNSUPPORTED;
  if ((long)S * H * d >= (1l << 31)) return S2A_ERR_UNSUPPORTED;
  if (!ptr_ok(workspace) || workspace_bytes < hga_bwd_workspace_bytes(B, S, H, Hkv, d)) return S2A_ERR_WORKSPACE;
  hipStream_t sm = reinterpret_cast<hipStream_t>(stream);
  const int C = T / chunk;
  auto qp = static_cast<const bf16_t*>(q);
  auto ka = static_cast<const bf16_t*>(k_act);
  auto va = static_cast<const bf16_t*>(v_act);
  auto kh = static_cast<const bf16_t*>(T > 0 ? k_hist : k_act);
  auto vh = static_cast<const bf16_t*>(T > 0 ? v_hist : v_act);
  auto op = static_cast<const bf16_t*>(o);
  auto dop = static_cast<const bf16_t*>(dout);
  auto dqp = static_cast<bf16_t*>(dq);
  auto dkp = static_cast<bf16_t*>(dk_act);
  auto dvp = static_cast<bf16_t*>(dv_act);
  float* dd = static_cast<float*>(workspace);
  float* lse2 = dd + (size_t)B * H * S;
  float* part = lse2 + (size_t)B * H * S;
  const KvPlan pl = kv_plan(B, S, H, Hkv, S, true);
  const int hpl = shared ? H / Hkv : 1;   // q heads per chunk list
  const int uq = B * H * (S / 64);
  const dim3 gq(uq), bq(128);
  // with room for the dS tiles: row statistics, dK/dV storing dS, then dQ reading the local
  // part from it; otherwise dQ first (recomputing everything and writing the statistics)
  const size_t dsoff = hga_ds_offset(B, S, H, Hkv, d);
  const bool dsq = workspace_bytes >= hga_bwd_workspace_bytes_dsq(B, S, H, Hkv, d);
  bf16_t* dsw = dsq ? reinterpret_cast<bf16_t*>(static_cast<char*>(workspace) + dsoff) : nullptr;
  if (d == 128) {
    if (dsq) {
      launch_rowdot<128>(op, dop, dd, lse, lse2, B, S, H, sm);
      launch_kv<128>(pl, qp, ka, va, (long)act_bstride, lse2, dd, dop, dkp, dvp, part, B, S, H, Hkv, S, 0, scale, sm,
                     dsw);
      hipLaunchKernelGGL((hga_dqw_kernel<128, true>), gq, bq, 0, sm, qp, ka, va, (long)act_bstride, kh, vh,
                         (long)hist_bstride, idx, op, lse, lse2, dd, dop, dqp, dsw, S, H, Hkv, C, chunk, topk, scale,
                         uq, hpl);
    } else {
      hipLaunchKernelGGL((hga_dqw_kernel<128, false>), gq, bq, 0, sm, qp, ka, va, (long)act_bstride, kh, vh,
                         (long)hist_bstride, idx, op, lse, lse2, dd, dop, dqp, nullptr, S, H, Hkv, C, chunk, topk,
                         scale, uq, hpl);
      launch_kv<128>(pl, qp, ka, va, (long)act_bstride, lse2, dd, dop, dkp, dvp, part, B, S, H, Hkv, S, 0, scale, sm);
    }
  } else {
    if (dsq) {
      launch_rowdot<64>(op, dop, dd, lse, lse2, B, S, H, sm);
      launch_kv<64>(pl, qp, ka, va, (long)act_bstride, lse2, dd, dop, dkp, dvp, part, B, S, H, Hkv, S, 0, scale, sm,
                    dsw);
      hipLaunchKernelGGL((hga_dqw_kernel<64, true>), gq, bq, 0, sm, qp, ka, va, (long)act_bstride, kh, vh,
                         (long)hist_bstride, idx, op, lse, lse2, dd, dop, dqp, dsw, S, H, Hkv, C, chunk, topk, scale,
                         uq, hpl);
    } else {
      hipLaunchKernelGGL((hga_dqw_kernel<64, false>), gq, bq, 0, sm, qp, ka, va, (long)act_bstride, kh, vh,
                         (long)hist_bstride, idx, op, lse, lse2, dd, dop, dqp, nullptr, S, H, Hkv, C, chunk, topk,
                         scale, uq, hpl);
      launch_kv<64>(pl, qp, ka, va, (long)act_bstride, lse2, dd, dop, dkp, dvp, part, B, S, H, Hkv, S, 0, scale, sm);
    }
  }
  return hipGetLastError() == hipSuccess ? S2A_OK : S2A_ERR_HIP;
}

extern "C" int hga_bwd_active(const void* q, const void* k_act, const void* v_act, long long act_bstride,
                              const void* k_hist, const void* v_hist, long long hist_bstride, const int32_t* idx,
                              const void* o, const float* lse, const void* dout, void* dq, void* dk_act,
                              void* dv_act, void* workspace, size_t workspace_bytes, int B, int S, int H, int Hkv,
                              int d, int T, int chunk, int qblock, int topk, float scale, void* stream) {
  return hga_bwd_impl(q, k_act, v_act, act_bstride, k_hist, v_hist, hist_bstride, idx, o, lse, dout, dq, dk_act,
                      dv_act, workspace, workspace_bytes, B, S, H, Hkv, d, T, chunk, qblock, topk, scale, stream,
                      false);
}

extern "C" int hga_bwd_active_shared(const void* q, const void* k_act, const void* v_act, long long act_bstride,
                                     const void* k_hist, const void* v_hist, long long hist_bstride,
                                     const int32_t* idx, const void* o, const float* lse, const void* dout, void* dq,
                                     void* dk_act, void* dv_act, void* workspace, size_t workspace_bytes, int B,
                                     int S, int H, int Hkv, int d, int T, int chunk, int qblock, int topk,
                                     float scale, void* stream) {
  return hga_bwd_impl(q, k_act, v_act, act_bstride, k_hist, v_hist, hist_bstride, idx, o, lse, dout, dq, dk_act,
                      dv_act, workspace, workspace_bytes, B, S, H, Hkv, d, T, chunk, qblock, topk, scale, stream,
                      true);
}
