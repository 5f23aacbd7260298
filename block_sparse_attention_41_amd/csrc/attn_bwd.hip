// Backward kernels for shifted short attention and for HGA (active segment only).
//
//   1. bwd_rowdot_kernel: D = rowsum(dO * O) per (batch, head, token), float32 workspace.
//   2. dqw_kernel, hga_dqw_kernel: query-major; each wave owns two 32-query blocks and
//                     walks the same key tiles as the forward.  For HGA a two-wave
//                     workgroup per 64-query block deals the block's half tiles (local
//                     ones, then those of its selected history chunks) alternately to its
//                     waves and adds their float32 partials through LDS; blocks run
//                     heaviest first, so light blocks fill the early finishers' slots.
//   3. kvf_kernel: key-major; each wave owns 32 keys and walks the query tiles that can
//                     see them, over every q head of its kv head (grouped-query sum in
//                     registers), computing dK and dV together (one wave per SIMD, both
//                     accumulators resident).  Short HGA segments run it split into
//                     parts whose float32 partial sums kv_reduce_kernel adds in order.
//                     For HGA only active keys get gradients: the history is detached
//                     ("Long-Context Fine-Tuning with Limited VRAM", English abstract).
// No atomics anywhere, so results are bitwise reproducible.
#include <algorithm>

#include "../../include/s2a.h"
#include "bwd2_core.h"
#include "launch.h"
#include "validate.h"

namespace s2a {

// D[b, h, t] = sum_e dO[b, t, h, e] * O[b, t, h, e]; 8 lanes per row.  When `lse` is
// given, also writes lse2 = LSE * log2(e) (the base-2 row statistic the recomputation of
// P uses) at the same index.
template <int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const bf16_t* __restrict__ o,
                                                          const bf16_t* __restrict__ dout, float* __restrict__ dd,
                                                          const float* __restrict__ lse, float* __restrict__ lse2,
                                                          int L, int H, long rows) {
  constexpr int PER = D / 8;  // elements per lane
  const long row = (long)group_x() * 32 + thread_x() / 8;
  const int sub = thread_x() % 8;
  float acc = 0.f;
  if (row < rows) {
    const bf16_t* po = o + row * D + sub * PER;
    const bf16_t* pd = dout + row * D + sub * PER;
#pragma unroll
    for (int i = 0; i < PER; i += 8) {
      const uint4 a = load16(po + i), b = load16(pd + i);
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += bf16_lo(aw[e]) * bf16_lo(bw[e]) + bf16_hi(aw[e]) * bf16_hi(bw[e]);
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < rows && sub == 0) {
    // row = (b * L + t) * H + h  ->  D[(b * H + h) * L + t]
    const long bt = row / H;
    const int h = (int)(row % H);
    const long b = bt / L;
    const int t = (int)(bt % L);
    const long idx = (b * H + h) * L + t;
    dd[idx] = acc;
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
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const bf16_t* a1 = tile + 16 * kb * D + o.tr[nb][0];
  const bf16_t* a2 = tile + 16 * kb * D + o.tr[nb][1];
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)a1);
  const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)a2);
  const uint2 ux = __builtin_bit_cast(uint2, x), uy = __builtin_bit_cast(uint2, y);
  return as_bf16x8(uint4{ux.x, ux.y, uy.x, uy.y});
}

// Fused key-major dK and dV for one wave (32 keys) and one 32-query half of a staged
// tile.  With lane = key and registers over queries:
//   S^T = K Q^T and dP^T = V dO^T  (row fragments of the Q and dO tiles),
//   P = exp2(S c - LSE log2 e), dS = P (dP - D),
//   dV^T += dO^T P and dK^T += Q^T dS  (transposed fragments of the same tiles).
// The instruction order keeps the matrix core busy while the vector ALU works: the
// exponentials run between the dP MFMAs and dS between the dV MFMAs, and each phase's
// LDS reads are issued during the previous phase's MFMAs.
template <int D, bool DIAG, typename Pre>
__device__ __forceinline__ void kvf_half(const bf16_t* qt, const bf16_t* dt, const float* l2, const float* ddl,
                                         const bf16x8_t (&kf)[D / 16], const bf16x8_t (&vf)[D / 16],
                                         f32x16_t (&ak)[D / 32], f32x16_t (&av)[D / 32], const KvfOffsets<D>& o,
                                         int mq, int g, int qh, int kpos, float c, Pre&& pre) {
  constexpr int KS = D / 16;   // K-steps of the score chains
  constexpr int NB = D / 32;   // accumulator blocks over the head dim
  constexpr int NF = 2 * NB;   // transposed fragments (= MFMAs) per update
  bf16x8_t fq[KS], fd[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) fq[kk] = as_bf16x8(load16(qt + 32 * mq * D + o.row[kk]));
  // work the caller wants spread over the first MFMA chain (the next tile's copies)
  pre();
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) fd[kk] = as_bf16x8(load16(dt + 32 * mq * D + o.row[kk]));
  f32x16_t sc = f32x16_t{};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) sc = mfma32(fq[kk], kf[kk], sc);
  // phase A: S chain; the Q reads run four ahead of it, the dO reads follow
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < KS - 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  __builtin_amdgcn_sched_barrier(0);

  // phase B: dP chain, with P = exp2(...) and the dO^T fragment reads between its MFMAs
  f32x16_t dp = f32x16_t{};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) dp = mfma32(fd[kk], vf[kk], dp);
  float p[16];
  float dv8[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // this lane's 8 queries: q0..q0+3 and q0+8..q0+11, q0 = 32 mq + 16 h + 4 g
    const int q0 = 32 * mq + 16 * h;
    const float4 la = *reinterpret_cast<const float4*>(l2 + q0 + o.stat);
    const float4 lb = *reinterpret_cast<const float4*>(l2 + q0 + 8 + o.stat);
    const float lv[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
    const float4 da = *reinterpret_cast<const float4*>(ddl + q0 + o.stat);
    const float4 db = *reinterpret_cast<const float4*>(ddl + q0 + 8 + o.stat);
    dv8[h][0] = da.x; dv8[h][1] = da.y; dv8[h][2] = da.z; dv8[h][3] = da.w;
    dv8[h][4] = db.x; dv8[h][5] = db.y; dv8[h][6] = db.z; dv8[h][7] = db.w;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const int r = 8 * h + sl;
      float x = fast_exp2(__builtin_fmaf(sc[r], c, -lv[sl]));
      if constexpr (DIAG) {
        const int qp = qh + 8 * (r / 4) + 4 * g + (r % 4);
        x = (kpos <= qp) ? x : 0.f;
      }
      p[r] = x;
    }
  }
  bf16x8_t pb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) wv[e] = pack_bf16(p[8 * h + 2 * e], p[8 * h + 2 * e + 1]);
    pb[h] = __builtin_bit_cast(bf16x8_t, uint4{wv[0], wv[1], wv[2], wv[3]});
  }
  bf16x8_t td[NF];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) td[h * NB + nb] = kvf_tr<D>(dt, o, nb, 2 * mq + h);
#pragma unroll
  for (int i = 0; i < KS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
  }
  __builtin_amdgcn_sched_barrier(0);

  // phase C: dV^T += dO^T P, with dS = P (dP - D) and the Q^T fragment reads between
  bf16x8_t tq[NF];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) av[nb] = mfma32(td[h * NB + nb], pb[h], av[nb]);
  bf16x8_t sb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r0 = 8 * h + 2 * e;
      wv[e] = pack_bf16(p[r0] * (dp[r0] - dv8[h][2 * e]), p[r0 + 1] * (dp[r0 + 1] - dv8[h][2 * e + 1]));
    }
    sb[h] = __builtin_bit_cast(bf16x8_t, uint4{wv[0], wv[1], wv[2], wv[3]});
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) tq[h * NB + nb] = kvf_tr<D>(qt, o, nb, 2 * mq + h);
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_barrier(0);

  // phase D: dK^T += Q^T dS
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) ak[nb] = mfma32(tq[h * NB + nb], sb[h], ak[nb]);
  __builtin_amdgcn_sched_barrier(0);
}

// One step of the fused loop: the copies of the next tile into the other buffers, then
// this tile's two halves.  Both buffer sets are restrict parameters of this one inlined
// function, so the compiler knows the reads of this tile do not depend on the copies in
// flight and does not wait for them (the caller's wait and barrier order the tiles).
template <int D>
__device__ __forceinline__ void kvf_iter(const bf16_t* __restrict__ qt, const bf16_t* __restrict__ dt,
                                         const float* __restrict__ l2, const float* __restrict__ ddl,
                                         bf16_t* __restrict__ nqt, bf16_t* __restrict__ ndt,
                                         float* __restrict__ nl2, float* __restrict__ nddl,
                                         const bf16_t* __restrict__ qsrc, const bf16_t* __restrict__ dsrc,
                                         const float* __restrict__ l2src, const float* __restrict__ ddsrc, long qs,
                                         bool work, const bf16x8_t (&kf)[D / 16], const bf16x8_t (&vf)[D / 16],
                                         f32x16_t (&ak)[D / 32], f32x16_t (&av)[D / 32], KvfOffsets<D> o,
                                         const CopyOffsets<D, 4>& co, int w, int lane, int kpw, int qp, float c) {
  constexpr int NW = 4;
  // every wave issues the same copies without a branch (so they can be scheduled among
  // the first MFMAs): its share of both tiles and one row statistic, wave 3 the LSE row
  // and the others the D row (three identical writes)
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto copy = [&]() {
    copy_tile<D, NW>(qsrc, co, nqt, wu);
    copy_tile<D, NW>(dsrc, co, ndt, wu);
    floats_direct(wu == NW - 1 ? l2src : ddsrc, wu == NW - 1 ? nl2 : nddl, lane);
  };
  auto none = []() {};
  if (!work) {
    copy();
    return;
  }
  // the offsets pass through an empty asm in every step, so the compiler cannot hoist one
  // address per read and buffer out of the loop (which would take ~150 registers); each
  // read becomes offset register + immediate
#pragma unroll
  for (int i = 0; i < D / 16; ++i) asm volatile("" : "+v"(o.row[i]));
#pragma unroll
  for (int i = 0; i < D / 32; ++i) asm volatile("" : "+v"(o.tr[i][0]), "+v"(o.tr[i][1]));
  asm volatile("" : "+v"(o.stat));
  const int lq = lane % 32, g = lane / 32, kpos = kpw + lq;
  // a half whose queries all come after the wave's keys needs no mask; the first half
  // is skipped when every key of the wave is after its queries
  if (kpw + 31 <= qp) {
    kvf_half<D, false>(qt, dt, l2, ddl, kf, vf, ak, av, o, 0, g, qp, kpos, c, copy);
  } else {
    copy();
    if (kpw <= qp + 31) kvf_half<D, true>(qt, dt, l2, ddl, kf, vf, ak, av, o, 0, g, qp, kpos, c, none);
  }
  if (kpw + 31 <= qp + 32) kvf_half<D, false>(qt, dt, l2, ddl, kf, vf, ak, av, o, 1, g, qp + 32, kpos, c, none);
  else kvf_half<D, true>(qt, dt, l2, ddl, kf, vf, ak, av, o, 1, g, qp + 32, kpos, c, none);
}

// Fused key-major dK and dV for group-local causal attention, shared by shifted short
// attention (groups of G, half the kv heads rolled by G/2) and the active segment of HGA
// (one group, G = N = segment length, no roll; K/V rows of batch b start at
// b * kv_bstride).  One wave per SIMD (the two float32 accumulators and the K and V
// operands of a wave's 32 keys take ~200 registers), four waves per workgroup, one
// workgroup per CU, double-buffered Q/dO tiles.  Units are (batch, kv head, group, key
// block[, part]), low key blocks (most queries) first; XCD x owns units
// [x * per, (x + 1) * per) and, when PERSIST, its `slots` workgroups walk them in
// rounds, backwards in odd rounds, so heavy and light units alternate.  A split (see
// kv_iters) writes its dK partials to part_k and its dV partials to part_v.
template <int D, bool SPLIT, bool PERSIST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void kvf_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, long kv_bstride,
    const float* __restrict__ lse2v, const float* __restrict__ ddv, const bf16_t* __restrict__ dout,
    bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, float* __restrict__ part_k, float* __restrict__ part_v, int N,
    int H, int Hkv, int G, int shift_on, float scale, int tpg, int upg, int m, int units, int slots) {
  constexpr int NW = 4, BN = 32 * NW;
  // two buffer sets as separate LDS objects, used alternately by an unrolled loop: the
  // compiler then tells the reads of one set from the copies into the other and does not
  // make the reads wait for those copies
  __shared__ __align__(16) bf16_t qa[kTile * D], qb[kTile * D];
  __shared__ __align__(16) bf16_t da[kTile * D], db[kTile * D];
  __shared__ __align__(16) float la[kTile], lb[kTile], ea[kTile], eb[kTile];
  const float c = scale * kLog2e;
  const KvfOffsets<D> offs = kvf_offsets<D>(thread_x() % 64);
  const CopyOffsets<D, NW> coffs = copy_offsets<D, NW>(thread_x() / 64, thread_x() % 64, (long)H * D);

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
  const int tid = thread_x(), w = tid / 64, lane = tid % 64, lq = lane % 32, g = lane / 32;

  const int gstart = grp * G;
  const int kp0 = gstart + tig * BN;
  const int kpw = kp0 + 32 * w;
  const bool active = kpw < gstart + G;
  const int qt0 = (kp0 - gstart) / kTile;
  const int nqt = G / kTile - qt0;

  const long qs = (long)H * D, ks = (long)Hkv * D;
  const int tokw = active ? (kpw + s) % N : 0;
  const long krow_in = b * kv_bstride + (long)(tokw + lq) * ks + (long)kvh * D;
  bf16x8_t kf[D / 16], vf[D / 16];
  if (active) {
    load_row_frag<D>(kf, k + krow_in, g);
    load_row_frag<D>(vf, v + krow_in, g);
  }
  f32x16_t ak[D / 32], av[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) ak[nb] = av[nb] = f32x16_t{};

  // the unit's share of the key block's iterations (parts of a split block differ by at
  // most one iteration)
  const int iters = rep * nqt;
  const int it0 = (int)((long)part * iters / nparts), it1 = (int)((long)(part + 1) * iters / nparts);
  struct Pos {
    int hh, qti;
  };
  auto step = [&](Pos p) {
    if (++p.qti == qt0 + nqt) {
      p.qti = qt0;
      ++p.hh;
    }
    return p;
  };
  // source offsets of a tile: Q/dO rows and the row statistics
  auto src = [&](Pos p, long& off, long& soff) {
    const int h = kvh * rep + p.hh;
    int tok = gstart + kTile * p.qti + s;
    if (tok >= N) tok -= N;
    off = ((long)b * N + tok) * qs + (long)h * D;
    soff = ((long)b * H + h) * N + tok;
  };
  Pos cq{it0 / nqt, qt0 + it0 % nqt};
  {
    long off, soff;
    src(cq, off, soff);
    kvf_iter<D>(qb, db, lb, eb, qa, da, la, ea, q + off, dout + off, lse2v + soff, ddv + soff, qs, false, kf, vf, ak,
                av, offs, coffs, w, lane, 0, 0, c);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // iteration it computes tile cq from one set and copies the next tile into the other
  auto iter = [&](int it, bf16_t* qc, bf16_t* dc, float* lc, float* ec, bf16_t* qn, bf16_t* dn, float* ln_,
                  float* en) {
    const Pos nq = step(cq);
    long off, soff;
    // the last step copies its own tile again (into the unused set) instead of branching
    src(it + 1 < it1 ? nq : cq, off, soff);
    const int qp = gstart + kTile * cq.qti;
    cq = nq;
    kvf_iter<D>(qc, dc, lc, ec, qn, dn, ln_, en, q + off, dout + off, lse2v + soff, ddv + soff, qs,
                active && kpw <= qp + kTile - 1, kf, vf, ak, av, offs, coffs, w, lane, kpw, qp, c);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int it = it0; it < it1; it += 2) {
    iter(it, qa, da, la, ea, qb, db, lb, eb);
    if (it + 1 < it1) iter(it + 1, qb, db, lb, eb, qa, da, la, ea);
  }
  if (active) {
    if (!SPLIT || nparts == 1) {
      // through this wave's share of the (now idle) tile buffers, one output at a time
      bf16_t* st = w == 0 ? qa : w == 1 ? qb : w == 2 ? da : db;
      const long orow0 = ((long)b * N + tokw) * ks + (long)kvh * D;
      store_acc_tile<D>(ak, scale, st, dk + orow0, ks, lane);
      store_acc_tile<D>(av, 1.f, st, dv + orow0, ks, lane);
    } else {
      store_acc_f32<D>(ak, scale, part_k + ((long)u * BN + 32 * w + lq) * D, g);
      store_acc_f32<D>(av, 1.f, part_v + ((long)u * BN + 32 * w + lq) * D, g);
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
  for (int kk = 0; kk < KS; ++kk) {
    dp[0] = mfma32(fv[kk], dof[0][kk], dp[0]);
    dp[1] = mfma32(fv[kk], dof[1][kk], dp[1]);
  }
  bf16x8_t dsb[2][2];
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
            const int kp = kp0 + 8 * (r / 4) + 4 * g + (r % 4);
            p = (kp <= qpos[j]) ? p : 0.f;
          }
          x2[t] = p * (dp[j][r] - dd[j]);
        }
        wv[e] = pack_bf16(x2[0], x2[1]);
      }
      dsb[j][h] = __builtin_bit_cast(bf16x8_t, uint4{wv[0], wv[1], wv[2], wv[3]});
    }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8_t t = kvf_tr<D>(kt, o, nb, kb);
      acc[0][nb] = mfma32(t, dsb[0][kb], acc[0][nb]);
      acc[1][nb] = mfma32(t, dsb[1][kb], acc[1][nb]);
    }
}

template <int D>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 1))) void hga_dqw_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_act, const bf16_t* __restrict__ v_act,
    long act_bstride, const bf16_t* __restrict__ k_hist, const bf16_t* __restrict__ v_hist, long hist_bstride,
    const int32_t* __restrict__ idx, const bf16_t* __restrict__ o, const float* __restrict__ lse,
    float* __restrict__ lse2v, float* __restrict__ ddv, const bf16_t* __restrict__ dout, bf16_t* __restrict__ dq,
    int S, int H, int Hkv, int C, int chunk, int topk, float scale, int units, int hpl) {
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
    // the row statistics, D = rowsum(dO * O) (lane halves g hold the two column halves)
    // and LSE * log2(e); wave 0 writes them for the key-major kernel that follows
    bf16x8_t of[D / 16];
    load_row_frag<D>(of, o + qbase + roff, g);
    float a = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) a = __builtin_fmaf((float)of[kk][e], (float)dof[sb][kk][e], a);
    const long si = ((long)b * H + h) * S + qp + lq;
    dd[sb] = pair_sum(a);
    lse2[sb] = lse[si] * kLog2e;
    if (wu == 0 && g == 0) {
      ddv[si] = dd[sb];
      lse2v[si] = lse2[sb];
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
  // copy cursor over the block's half tiles in order (local ones first, then each selected
  // chunk); past the end it stays on the last one
  int nxt = 0, cur = 0;
  auto next_src = [&](const bf16_t*& ksrc, const bf16_t*& vsrc) {
    const int t = nxt < ntiles ? nxt : ntiles - 1;
    long r0;
    bool loc = t < nloc;
    if (loc) {
      r0 = 32l * t;
    } else {
      const int sub = (t - nloc) % spc;
      if (sub == 0 && nxt < ntiles) {   // next selected chunk
        cur = __builtin_amdgcn_readlane(cidx, __builtin_ctzll(rem));
        rem &= rem - 1;
      }
      r0 = (long)cur * chunk + 32l * sub;
    }
    ksrc = (loc ? ka : kh) + r0 * ks;
    vsrc = (loc ? va : vh) + r0 * ks;
    ++nxt;
  };
  // wave w takes half tiles w, w + 2, w + 4, ... (an equal share of the causal prefix,
  // one of the two diagonal half tiles, and half of each selected chunk)
  {
    const bf16_t *ks0, *vs0;
    if (wu == 1) next_src(ks0, vs0);
    next_src(ks0, vs0);
    copy_half<D>(ks0, co, ka_[wu]);
    copy_half<D>(vs0, co, va_[wu]);
  }
  __builtin_amdgcn_s_waitcnt(0);
  auto step = [&](int it, const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, bf16_t* __restrict__ kn,
                  bf16_t* __restrict__ vn) {
    const bf16_t *ksrc, *vsrc;
    next_src(ksrc, vsrc);   // the other wave's
    next_src(ksrc, vsrc);   // half tile it + 2 (past the end: the last one again, harmlessly)
    auto copy = [&]() {
      copy_half<D>(ksrc, co, kn);
      copy_half<D>(vsrc, co, vn);
    };
    KvfOffsets<D> o = offs;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) asm volatile("" : "+v"(o.row[i]));
#pragma unroll
    for (int i = 0; i < D / 32; ++i) asm volatile("" : "+v"(o.tr[i][0]), "+v"(o.tr[i][1]));
    const int kp0 = 32 * it;
    if (it >= nloc - 2 && it < nloc)   // the block's diagonal half tiles
      hga_dqw_half<D, true>(kc, vc, o, qf, dof, acc, lse2, dd, g, kp0, qpos, c, copy);
    else
      hga_dqw_half<D, false>(kc, vc, o, qf, dof, acc, lse2, dd, g, kp0, qpos, c, copy);
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
  const long rows = (long)B * L * H;
  dim3 grid((unsigned)((rows + 31) / 32)), block(256);
  hipLaunchKernelGGL((bwd_rowdot_kernel<D>), grid, block, 0, st, o, dout, dd, lse, lse2, L, H, rows);
}

// How the key-major kernels cover (B, N, H, Hkv, G): keys per workgroup (four waves of
// 32), key blocks per group, workgroups per group, iterations per part and workgroups in
// all; `partial_floats` is the float32 scratch a split needs (0 without split).
struct KvPlan {
  int bn, tpg, upg, m;
  long units;
  size_t partial_floats;
};

// Fewer workgroups than two rounds of the chip's slots (256 CUs, one fused workgroup
// each) leave CUs idle, so the iterations are then split into at most that many parts of
// at least kKvMinPart iterations each (a part's partial writes and their reduction cost
// about one iteration), as even as the rounding allows.
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
  const long target = 256L * 2;
  if (!allow_split || p.units >= target) return p;
  long itot = 0;
  for (int t = 0; t < p.tpg; ++t) itot += kv_iters(rep, G, p.bn, t);
  const long groups = (long)B * Hkv * ngroups;
  // each key block's part count rounds up, so grow the part length until the parts fit
  // in two rounds (a third, mostly empty round would idle most CUs for a whole part)
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
               int N, int H, int Hkv, int G, int shift, float scale, hipStream_t st) {
  const int per = (int)((pl.units + 7) / 8);
  if (pl.upg == pl.tpg) {
    const int slots = G < kPersistGroup ? std::min(per, resident_per_xcd(1)) : per;
    if (G < kPersistGroup)
      hipLaunchKernelGGL((kvf_kernel<D, false, true>), dim3(8 * slots), dim3(256), 0, st, q, k, v, kv_bstride, lse2, dd,
                         dout, dk, dv, nullptr, nullptr, N, H, Hkv, G, shift, scale, pl.tpg, pl.upg, pl.m,
                         (int)pl.units, slots);
    else
      hipLaunchKernelGGL((kvf_kernel<D, false, false>), dim3(8 * slots), dim3(256), 0, st, q, k, v, kv_bstride, lse2,
                         dd, dout, dk, dv, nullptr, nullptr, N, H, Hkv, G, shift, scale, pl.tpg, pl.upg, pl.m,
                         (int)pl.units, slots);
    return;
  }
  constexpr int BN = 128;
  const int slots = std::min(per, resident_per_xcd(1));
  float* part_k = part;
  float* part_v = part + (size_t)pl.units * BN * D;
  const dim3 rgrid((unsigned)((long)B * Hkv * (N / G) * pl.tpg * (BN / (256 / (D / 4)))), 2), rblk(256);
  hipLaunchKernelGGL((kvf_kernel<D, true, true>), dim3(8 * slots), dim3(256), 0, st, q, k, v, kv_bstride, lse2, dd,
                     dout, dk, dv, part_k, part_v, N, H, Hkv, G, shift, scale, pl.tpg, pl.upg, pl.m, (int)pl.units,
                     slots);
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
// (s2attn_bwd, s2attn_bwd_dq_prep), prep happens inside the dQ kernel.
namespace {
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
  // prep and dQ together: the dQ kernel computes the row statistics of the rows it owns
  // (every row is owned by exactly one of its units) and writes them for dK/dV
  const bool fuse = (stages & kPrep) && (stages & kDq);
  const bf16_t* of = fuse ? op : nullptr;
  const float* lf = fuse ? lse : nullptr;
  if (d == 128) {
    if ((stages & kPrep) && !fuse) launch_rowdot<128>(op, dop, dd, lse, lse2, B, N, H, sm);
    if (stages & kDq) launch_dq<128>(qp, kp, vp, lse2, dd, dop, of, lf, dqp, B, N, H, Hkv, G, shift, scale, sm);
    if (stages & kDkdv)
      launch_kv<128>(pl, qp, kp, vp, kvb, lse2, dd, dop, dkp, dvp, nullptr, B, N, H, Hkv, G, shift, scale, sm);
  } else {
    if ((stages & kPrep) && !fuse) launch_rowdot<64>(op, dop, dd, lse, lse2, B, N, H, sm);
    if (stages & kDq) launch_dq<64>(qp, kp, vp, lse2, dd, dop, of, lf, dqp, B, N, H, Hkv, G, shift, scale, sm);
    if (stages & kDkdv)
      launch_kv<64>(pl, qp, kp, vp, kvb, lse2, dd, dop, dkp, dvp, nullptr, B, N, H, Hkv, G, shift, scale, sm);
  }
  return hipGetLastError() == hipSuccess ? S2A_OK : S2A_ERR_HIP;
}
}  // namespace

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

// [D | LSE * log2(e)] row statistics (float32 [B, H, S] each), then the float32 partial
// sums of the split key-major kernels when the segment alone gives too few workgroups.
extern "C" size_t hga_bwd_workspace_bytes(int B, int S, int H, int Hkv, int d) {
  (void)d;
  if (B <= 0 || S <= 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || S % kTile != 0) return 0;
  const KvPlan pl = kv_plan(B, S, H, Hkv, S, true);
  return (2 * (size_t)B * H * S + pl.partial_floats) * sizeof(float);
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
  if (d == 128) {
    hipLaunchKernelGGL((hga_dqw_kernel<128>), gq, bq, 0, sm, qp, ka, va, (long)act_bstride, kh, vh,
                       (long)hist_bstride, idx, op, lse, lse2, dd, dop, dqp, S, H, Hkv, C, chunk, topk, scale, uq, hpl);
    launch_kv<128>(pl, qp, ka, va, (long)act_bstride, lse2, dd, dop, dkp, dvp, part, B, S, H, Hkv, S, 0, scale, sm);
  } else {
    hipLaunchKernelGGL((hga_dqw_kernel<64>), gq, bq, 0, sm, qp, ka, va, (long)act_bstride, kh, vh,
                       (long)hist_bstride, idx, op, lse, lse2, dd, dop, dqp, S, H, Hkv, C, chunk, topk, scale, uq, hpl);
    launch_kv<64>(pl, qp, ka, va, (long)act_bstride, lse2, dd, dop, dkp, dvp, part, B, S, H, Hkv, S, 0, scale, sm);
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
