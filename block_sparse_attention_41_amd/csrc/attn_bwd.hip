// Backward kernels for shifted short attention and for HGA (active segment only).
//
//   1. bwd_rowdot_kernel: D = rowsum(dO * O) per (batch, head, token), float32 workspace.
//   2. *_dq_kernel:   query-major; each wave owns 32 queries and walks the same key tiles
//                     as the forward (for HGA: local tiles, then the selected history).
//   3. *_dkdv_kernel: key-major; each wave owns 32 keys and walks the query tiles that
//                     can see them, over every q head of its kv head (grouped-query sum
//                     in registers).  For HGA only active keys get gradients: the
//                     history is detached ("Long-Context Fine-Tuning with Limited VRAM",
//                     English abstract).
// No atomics anywhere, so results are bitwise reproducible.
#include "../../include/s2a.h"
#include "bwd_core.h"
#include "bwd2_core.h"
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
  const long row = (long)blockIdx.x * 32 + threadIdx.x / 8;
  const int sub = threadIdx.x % 8;
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
// Shifted short attention (same rolled-group geometry as the forward), eight waves per
// workgroup, all tiles copied HBM -> LDS directly and double-buffered, one barrier per tile.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int xcd_order_b(int lin, int total) { return (lin % 8) * (total / 8) + lin / 8; }

// dQ for one wave: 32 queries against one 64-key tile (K and V row-major in LDS).
template <int D>
__device__ __forceinline__ void dq2_tile(const bf16_t* ks, const bf16_t* vs, const bf16x8_t (&qf)[D / 16],
                                         const bf16_t* dow, f32x16_t (&dq)[D / 32], float lse2, float dd, int lane,
                                         int lq, int g, bool diag, int kpos0, int qpos, float c) {
  // S^T and dP^T, one 32-key half at a time (8 fragment reads, then 8 MFMAs each)
  f32x16_t sc[2], dp[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    bf16x8_t fr[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) fr[kk] = row_frag<D>(ks, 32 * mb + lq, 2 * kk + g);
    __builtin_amdgcn_sched_barrier(0);
    sc[mb] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) sc[mb] = mfma32(fr[kk], qf[kk], sc[mb]);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) fr[kk] = row_frag<D>(vs, 32 * mb + lq, 2 * kk + g);
    bf16x8_t dof[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) dof[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(dow + (kk * 64 + lane) * 8));
    __builtin_amdgcn_sched_barrier(0);
    dp[mb] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) dp[mb] = mfma32(fr[kk], dof[kk], dp[mb]);
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
          float p = fast_exp2(__builtin_fmaf(sc[mb][r], c, -lse2));
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
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) dq[nb] = mfma32(tr_frag<D>(ks, nb, kb, lq, g), dsb[kb], dq[nb]);
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void s2attn_dq_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ lse2v, const float* __restrict__ ddv, const bf16_t* __restrict__ dout,
    bf16_t* __restrict__ dq, int N, int H, int Hkv, int G, int shift_on, float scale, int tpg, int units) {
  constexpr int BM = 32 * NW;
  __shared__ __align__(16) bf16_t kl[2][kTile * D];
  __shared__ __align__(16) bf16_t vl[2][kTile * D];
  const float c = scale * kLog2e;

  const int u = xcd_order_b(blockIdx.x, gridDim.x);
  if (u >= units) return;
  const int ngroups = N / G;
  const int tig = tpg - 1 - u % tpg;
  int rest = u / tpg;
  const int grp = rest % ngroups;
  rest /= ngroups;
  const int h = rest % H;
  const int b = rest / H;
  const int s = (shift_on && ngroups >= 2 && h >= H / 2) ? G / 2 : 0;
  const int kvh = h / (H / Hkv);
  const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, lq = lane % 32, g = lane / 32;

  const int gstart = grp * G;
  const int qp0 = gstart + tig * BM;
  const int qpw = qp0 + 32 * w;
  const bool active = qpw < gstart + G;
  const int qlast = min(qp0 + BM, gstart + G) - 1;
  const int ntiles = (qlast - gstart) / kTile + 1;

  const long qs = (long)H * D, ks = (long)Hkv * D;
  const int tokw = active ? (qpw + s) % N : 0;
  const long qrow_off = ((long)b * N + tokw + lq) * qs + (long)h * D;
  // the wave's dO fragments live in its own LDS region ([kk][lane] 16-byte pieces)
  __shared__ __align__(16) bf16_t dolds[NW][(D / 16) * 64 * 8];
  bf16_t* dow = dolds[w];
  bf16x8_t qf[D / 16];
  float lse2 = 0.f, dd = 0.f;
  if (active) {
    load_row_frag<D>(qf, q + qrow_off, g);
    bf16x8_t dof[D / 16];
    load_row_frag<D>(dof, dout + qrow_off, g);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) *reinterpret_cast<bf16x8_t*>(dow + (kk * 64 + lane) * 8) = dof[kk];
    lse2 = lse2v[((long)b * H + h) * N + tokw + lq];
    dd = ddv[((long)b * H + h) * N + tokw + lq];
  }
  f32x16_t acc[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) acc[nb] = f32x16_t{};

  const bf16_t* kb0 = k + (long)b * N * ks + (long)kvh * D;
  const bf16_t* vb0 = v + (long)b * N * ks + (long)kvh * D;
  {
    const int tok = (gstart + s) % N;
    tile_direct<D, NW>(kb0 + tok * ks, ks, kl[0], w, lane);
    tile_direct<D, NW>(vb0 + tok * ks, ks, vl[0], w, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    if (it + 1 < ntiles) {
      const int tok = (gstart + kTile * (it + 1) + s) % N;
      tile_direct<D, NW>(kb0 + tok * ks, ks, kl[cur ^ 1], w, lane);
      tile_direct<D, NW>(vb0 + tok * ks, ks, vl[cur ^ 1], w, lane);
    }
    const int kp0 = gstart + kTile * it;
    if (active && kp0 <= qpw + 31)
      dq2_tile<D>(kl[cur], vl[cur], qf, dow, acc, lse2, dd, lane, lq, g, kp0 + kTile - 1 > qpw, kp0, qpw + lq, c);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (active) store_acc_row<D>(acc, scale, dq + qrow_off, g);
}

// Key-major part.  WANT_DK = false: dV^T += dO^T P.  WANT_DK = true: dK^T += Q^T dS, with
// dS = P * (dP - D) and dP = dO V^T.  One wave owns 32 keys; a query tile of 64 rows is
// processed in two halves of 32.
template <int D, bool WANT_DK>
__device__ __forceinline__ void kv2_tile(const bf16_t* qt, const bf16_t* dt, const float* l2, const float* ddl,
                                         const bf16x8_t (&kf)[D / 16], const bf16x8_t (&vf)[D / 16],
                                         f32x16_t (&acc)[D / 32], int lq, int g, int qpos0, int kpos, float c) {
#pragma unroll
  for (int mq = 0; mq < 2; ++mq) {
    const int qh = qpos0 + 32 * mq;             // first query of this half
    if (kpos - lq > qh + 31) continue;          // every key of the wave is after every query
    const bool diag = kpos - lq + 31 > qh;
    bf16x8_t fr[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) fr[kk] = row_frag<D>(qt, 32 * mq + lq, 2 * kk + g);
    __builtin_amdgcn_sched_barrier(0);
    f32x16_t sc = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) sc = mfma32(fr[kk], kf[kk], sc);
    f32x16_t dp = f32x16_t{};
    if constexpr (WANT_DK) {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) fr[kk] = row_frag<D>(dt, 32 * mq + lq, 2 * kk + g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) dp = mfma32(fr[kk], vf[kk], dp);
    }
    bf16x8_t pb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q0 = 32 * mq + 16 * h + 4 * g;   // this lane's 8 queries: q0..q0+3, q0+8..q0+11
      const float4 la = *reinterpret_cast<const float4*>(l2 + q0);
      const float4 lb = *reinterpret_cast<const float4*>(l2 + q0 + 8);
      const float lv[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
      float dv8[8];
      if constexpr (WANT_DK) {
        const float4 da = *reinterpret_cast<const float4*>(ddl + q0);
        const float4 db = *reinterpret_cast<const float4*>(ddl + q0 + 8);
        dv8[0] = da.x; dv8[1] = da.y; dv8[2] = da.z; dv8[3] = da.w;
        dv8[4] = db.x; dv8[5] = db.y; dv8[6] = db.z; dv8[7] = db.w;
      }
      uint32_t wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int sl = 2 * e + t, r = 8 * h + sl;
          float p = fast_exp2(__builtin_fmaf(sc[r], c, -lv[sl]));
          if (diag) {
            const int qp = qh + 8 * (r / 4) + 4 * g + (r % 4);
            p = (kpos <= qp) ? p : 0.f;
          }
          if constexpr (WANT_DK) x2[t] = p * (dp[r] - dv8[sl]);
          else x2[t] = p;
        }
        wv[e] = pack_bf16(x2[0], x2[1]);
      }
      pb[h] = __builtin_bit_cast(bf16x8_t, uint4{wv[0], wv[1], wv[2], wv[3]});
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
        acc[nb] = mfma32(tr_frag<D>(WANT_DK ? qt : dt, nb, 2 * mq + h, lq, g), pb[h], acc[nb]);
  }
}

template <int D, int NW, bool WANT_DK>
__global__ __launch_bounds__(64 * NW) void s2attn_kv_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ lse2v, const float* __restrict__ ddv, const bf16_t* __restrict__ dout,
    bf16_t* __restrict__ out, int N, int H, int Hkv, int G, int shift_on, float scale, int tpg, int units) {
  constexpr int BN = 32 * NW;
  __shared__ __align__(16) bf16_t ql[2][kTile * D];
  __shared__ __align__(16) bf16_t dl[2][kTile * D];
  __shared__ __align__(16) float l2l[2][kTile];
  __shared__ __align__(16) float ddl[2][kTile];
  const float c = scale * kLog2e;

  const int u = xcd_order_b(blockIdx.x, gridDim.x);
  if (u >= units) return;
  const int ngroups = N / G;
  const int tig = u % tpg;               // low key tiles see the most queries: first
  int rest = u / tpg;
  const int grp = rest % ngroups;
  rest /= ngroups;
  const int kvh = rest % Hkv;
  const int b = rest / Hkv;
  const int rep = H / Hkv;
  // every q head of this kv head has the same shift (the H/2 boundary maps to Hkv/2)
  const int s = (shift_on && ngroups >= 2 && kvh >= Hkv / 2) ? G / 2 : 0;
  const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, lq = lane % 32, g = lane / 32;

  const int gstart = grp * G;
  const int kp0 = gstart + tig * BN;
  const int kpw = kp0 + 32 * w;
  const bool active = kpw < gstart + G;
  const int qt0 = (kp0 - gstart) / kTile;
  const int nqt = G / kTile - qt0;

  const long qs = (long)H * D, ks = (long)Hkv * D;
  const int tokw = active ? (kpw + s) % N : 0;
  const long krow_off = ((long)b * N + tokw + lq) * ks + (long)kvh * D;
  bf16x8_t kf[D / 16], vf[D / 16];
  if (active) {
    load_row_frag<D>(kf, k + krow_off, g);
    if constexpr (WANT_DK) load_row_frag<D>(vf, v + krow_off, g);
  }
  f32x16_t acc[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) acc[nb] = f32x16_t{};

  const int total = rep * nqt;
  auto issue = [&](int it, int buf) {
    const int hh = it / nqt, qti = qt0 + it % nqt;
    const int h = kvh * rep + hh;
    const int tok = (gstart + kTile * qti + s) % N;
    const long off = ((long)b * N + tok) * qs + (long)h * D;
    tile_direct<D, NW>(q + off, qs, ql[buf], w, lane);
    tile_direct<D, NW>(dout + off, qs, dl[buf], w, lane);
    if (w == NW - 1) floats_direct(lse2v + ((long)b * H + h) * N + tok, l2l[buf], lane);
    if (WANT_DK && w == NW - 2) floats_direct(ddv + ((long)b * H + h) * N + tok, ddl[buf], lane);
  };
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < total; ++it) {
    const int cur = it & 1;
    if (it + 1 < total) issue(it + 1, cur ^ 1);
    const int qp = gstart + kTile * (qt0 + it % nqt);
    if (active && kpw <= qp + kTile - 1)
      kv2_tile<D, WANT_DK>(ql[cur], dl[cur], l2l[cur], ddl[cur], kf, vf, acc, lq, g, qp, kpw + lq, c);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (active) store_acc_row<D>(acc, WANT_DK ? scale : 1.f, out + krow_off, g);
}

// ---------------------------------------------------------------------------------------
// HGA backward.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void hga_dq_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_act, const bf16_t* __restrict__ v_act,
    long act_bstride, const bf16_t* __restrict__ k_hist, const bf16_t* __restrict__ v_hist, long hist_bstride,
    const int32_t* __restrict__ idx, const float* __restrict__ lse, const float* __restrict__ ddv,
    const bf16_t* __restrict__ dout, bf16_t* __restrict__ dq, int S, int H, int Hkv, int C, int chunk, int topk,
    float scale) {
  constexpr int NT = 128;
  __shared__ __align__(16) DqLds<D> lds;
  __shared__ int sel[64];
  __shared__ int nsel;
  const float c = scale * kLog2e;

  const int b = blockIdx.z, h = blockIdx.y;
  const int nqb = S / 64;
  const int j = nqb - 1 - blockIdx.x;
  const int kvh = h / (H / Hkv);
  const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, lq = lane % 32, g = lane / 32;

  if (w == 0) {
    int cidx = -1;
    if (lane < topk) cidx = idx[(((long)b * H + h) * nqb + j) * topk + lane];
    const bool valid = lane < topk && cidx >= 0 && cidx < C;
    const unsigned long long bal = __ballot(valid);
    if (valid) sel[__popcll(bal & ((1ull << lane) - 1ull))] = cidx;
    if (lane == 0) nsel = __popcll(bal);
  }
  __syncthreads();
  const int spc = chunk / kTile;
  const int nloc = j + 1;
  const int ntiles = nloc + nsel * spc;

  const long qs = (long)H * D, ks = (long)Hkv * D;
  const int qpw = 64 * j + 32 * w;
  const long qrow_off = ((long)b * S + qpw + lq) * qs + (long)h * D;
  bf16x8_t qf[D / 16], dof[D / 16];
  load_row_frag<D>(qf, q + qrow_off, g);
  load_row_frag<D>(dof, dout + qrow_off, g);
  const float lse2 = lse[((long)b * H + h) * S + qpw + lq] * kLog2e;
  const float dd = ddv[((long)b * H + h) * S + qpw + lq];
  f32x16_t acc[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) acc[nb] = f32x16_t{};

  const bf16_t* ka = k_act + b * act_bstride + (long)kvh * D;
  const bf16_t* va = v_act + b * act_bstride + (long)kvh * D;
  const bf16_t* kh = k_hist + b * hist_bstride + (long)kvh * D;
  const bf16_t* vh = v_hist + b * hist_bstride + (long)kvh * D;
  auto issue = [&](int it, DualTile<D, NT>& kt, RowTile<D, NT>& vt) {
    const bool loc = it < nloc;
    long r0;
    if (loc) {
      r0 = (long)kTile * it;
    } else {
      const int u = it - nloc;
      r0 = (long)sel[u / spc] * chunk + (long)kTile * (u % spc);
    }
    kt.load((loc ? ka : kh) + r0 * ks, ks, tid);
    vt.load((loc ? va : vh) + r0 * ks, ks, tid);
  };
  DualTile<D, NT> kt;
  RowTile<D, NT> vt;
  issue(0, kt, vt);
  for (int it = 0; it < ntiles; ++it) {
    __syncthreads();
    kt.store(lds.k, lds.kt, tid);
    vt.store(lds.v, tid);
    __syncthreads();
    if (it + 1 < ntiles) issue(it + 1, kt, vt);
    const bool loc = it < nloc;
    const int kp0 = loc ? kTile * it : 0;
    if (!loc || kp0 <= qpw + 31)
      dq_tile<D>(lds, qf, dof, acc, lse2, dd, lq, g, loc && it == j, kp0, qpw + lq, c);
  }
  store_acc_row<D>(acc, scale, dq + qrow_off, g);
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void hga_dkdv_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_act, const bf16_t* __restrict__ v_act,
    long act_bstride, const float* __restrict__ lse, const float* __restrict__ ddv,
    const bf16_t* __restrict__ dout, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, int S, int H, int Hkv,
    float scale) {
  constexpr int NT = 64 * NW, BN = 32 * NW;
  __shared__ __align__(16) KvLds<D> lds;
  const float c = scale * kLog2e;

  const int b = blockIdx.z, kvh = blockIdx.y;
  const int tile = blockIdx.x;  // low key tiles see the most queries: first
  const int rep = H / Hkv;
  const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, lq = lane % 32, g = lane / 32;
  const int kp0 = tile * BN;
  const int kpw = kp0 + 32 * w;
  const bool active = kpw < S;
  const int qt0 = kp0 / kTile;
  const int nqt = S / kTile - qt0;

  const long qs = (long)H * D, ks = (long)Hkv * D;
  const long krow_in = b * act_bstride + (long)(active ? kpw + lq : 0) * ks + (long)kvh * D;
  const long krow_out = ((long)b * S + (active ? kpw + lq : 0)) * ks + (long)kvh * D;
  bf16x8_t kf[D / 16], vf[D / 16];
  if (active) {
    load_row_frag<D>(kf, k_act + krow_in, g);
    load_row_frag<D>(vf, v_act + krow_in, g);
  }
  f32x16_t dka[D / 32], dva[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) dka[nb] = dva[nb] = f32x16_t{};

  DualTile<D, NT> qt, dt;
  float pl = 0.f, pd = 0.f;
  const int total = rep * nqt;
  auto issue = [&](int it) {
    const int hh = it / nqt, qti = qt0 + it % nqt;
    const int h = kvh * rep + hh;
    const long off = ((long)b * S + kTile * qti) * qs + (long)h * D;
    qt.load(q + off, qs, tid);
    dt.load(dout + off, qs, tid);
    if (tid < kTile) {
      pl = lse[((long)b * H + h) * S + kTile * qti + tid] * kLog2e;
      pd = ddv[((long)b * H + h) * S + kTile * qti + tid];
    }
  };
  issue(0);
  for (int it = 0; it < total; ++it) {
    __syncthreads();
    qt.store(lds.q, lds.qt, tid);
    dt.store(lds.dob, lds.dot, tid);
    if (tid < kTile) {
      lds.lse2[tid] = pl;
      lds.dd[tid] = pd;
    }
    __syncthreads();
    if (it + 1 < total) issue(it + 1);
    const int qp = kTile * (qt0 + it % nqt);
    if (active && kpw <= qp + kTile - 1)
      dkdv_tile<D>(lds, kf, vf, dka, dva, lq, g, kpw + 31 > qp, qp, kpw + lq, c);
  }
  if (active) {
    store_acc_row<D>(dka, scale, dk + krow_out, g);
    store_acc_row<D>(dva, 1.f, dv + krow_out, g);
  }
}

template <int D>
void launch_rowdot(const bf16_t* o, const bf16_t* dout, float* dd, const float* lse, float* lse2, int B, int L, int H,
                   hipStream_t st) {
  const long rows = (long)B * L * H;
  dim3 grid((unsigned)((rows + 31) / 32)), block(256);
  hipLaunchKernelGGL((bwd_rowdot_kernel<D>), grid, block, 0, st, o, dout, dd, lse, lse2, L, H, rows);
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
// workspace), dQ (query-major) and dK/dV (key-major).  dQ and dK/dV only read the
// workspace, so a caller may also run them on two streams after prep.
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
  constexpr int NW = 8, BT = 32 * NW;
  const int tpg = (G + BT - 1) / BT;
  if ((long)tpg * (N / G) * H * B >= (1l << 31) - 8) return S2A_ERR_UNSUPPORTED;
  hipStream_t sm = reinterpret_cast<hipStream_t>(stream);
  auto qp = static_cast<const bf16_t*>(q);
  auto kp = static_cast<const bf16_t*>(k);
  auto vp = static_cast<const bf16_t*>(v);
  auto op = static_cast<const bf16_t*>(o);
  auto dop = static_cast<const bf16_t*>(dout);
  float* dd = static_cast<float*>(workspace);
  float* lse2 = dd + (size_t)B * H * N;
  const int uq = tpg * (N / G) * H * B, uk = tpg * (N / G) * Hkv * B;
  const dim3 blk(64 * NW), gq((uq + 7) / 8 * 8), gk((uk + 7) / 8 * 8);
  auto dqp = static_cast<bf16_t*>(dq);
  auto dkp = static_cast<bf16_t*>(dk);
  auto dvp = static_cast<bf16_t*>(dv);
  if (d == 128) {
    if (stages & kPrep) launch_rowdot<128>(op, dop, dd, lse, lse2, B, N, H, sm);
    if (stages & kDq)
      hipLaunchKernelGGL((s2attn_dq_kernel<128, NW>), gq, blk, 0, sm, qp, kp, vp, lse2, dd, dop, dqp, N, H, Hkv, G,
                         shift, scale, tpg, uq);
    if (stages & kDkdv) {
      hipLaunchKernelGGL((s2attn_kv_kernel<128, NW, false>), gk, blk, 0, sm, qp, kp, vp, lse2, dd, dop, dvp, N, H,
                         Hkv, G, shift, scale, tpg, uk);
      hipLaunchKernelGGL((s2attn_kv_kernel<128, NW, true>), gk, blk, 0, sm, qp, kp, vp, lse2, dd, dop, dkp, N, H, Hkv,
                         G, shift, scale, tpg, uk);
    }
  } else {
    if (stages & kPrep) launch_rowdot<64>(op, dop, dd, lse, lse2, B, N, H, sm);
    if (stages & kDq)
      hipLaunchKernelGGL((s2attn_dq_kernel<64, NW>), gq, blk, 0, sm, qp, kp, vp, lse2, dd, dop, dqp, N, H, Hkv, G,
                         shift, scale, tpg, uq);
    if (stages & kDkdv) {
      hipLaunchKernelGGL((s2attn_kv_kernel<64, NW, false>), gk, blk, 0, sm, qp, kp, vp, lse2, dd, dop, dvp, N, H, Hkv,
                         G, shift, scale, tpg, uk);
      hipLaunchKernelGGL((s2attn_kv_kernel<64, NW, true>), gk, blk, 0, sm, qp, kp, vp, lse2, dd, dop, dkp, N, H, Hkv,
                         G, shift, scale, tpg, uk);
    }
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

extern "C" size_t hga_bwd_workspace_bytes(int B, int S, int H, int Hkv, int d) {
  (void)Hkv;
  (void)d;
  if (B <= 0 || S <= 0 || H <= 0) return 0;
  return (size_t)B * H * S * sizeof(float);
}

extern "C" int hga_bwd_active(const void* q, const void* k_act, const void* v_act, long long act_bstride,
                              const void* k_hist, const void* v_hist, long long hist_bstride, const int32_t* idx,
                              const void* o, const float* lse, const void* dout, void* dq, void* dk_act,
                              void* dv_act, void* workspace, size_t workspace_bytes, int B, int S, int H, int Hkv,
                              int d, int T, int chunk, int qblock, int topk, float scale, void* stream) {
  if (!ptr_ok(q) || !ptr_ok(k_act) || !ptr_ok(v_act) || !ptr_ok(idx) || !ptr_ok(o) || !ptr_ok(lse) ||
      !ptr_ok(dout) || !ptr_ok(dq) || !ptr_ok(dk_act) || !ptr_ok(dv_act))
    return S2A_ERR_INVALID_ARG;
  int st = check_hga_shape(B, S, H, Hkv, d, T, chunk, qblock, topk);
  if (st) return st;
  if (check_scale(scale)) return S2A_ERR_INVALID_ARG;
  if (T > 0 && (!ptr_ok(k_hist) || !ptr_ok(v_hist))) return S2A_ERR_INVALID_ARG;
  if (!stride_ok(act_bstride, S, Hkv, d, B) || !stride_ok(hist_bstride, T, Hkv, d, B)) return S2A_ERR_INVALID_ARG;
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
  constexpr int NW = 4, BN = 32 * NW;
  dim3 gq(S / 64, H, B), bq(128), gk((S + BN - 1) / BN, Hkv, B), bk(64 * NW);
  if (d == 128) {
    launch_rowdot<128>(op, dop, dd, nullptr, nullptr, B, S, H, sm);
    hipLaunchKernelGGL((hga_dq_kernel<128>), gq, bq, 0, sm, qp, ka, va, (long)act_bstride, kh, vh,
                       (long)hist_bstride, idx, lse, dd, dop, dqp, S, H, Hkv, C, chunk, topk, scale);
    hipLaunchKernelGGL((hga_dkdv_kernel<128, NW>), gk, bk, 0, sm, qp, ka, va, (long)act_bstride, lse, dd, dop, dkp,
                       dvp, S, H, Hkv, scale);
  } else {
    launch_rowdot<64>(op, dop, dd, nullptr, nullptr, B, S, H, sm);
    hipLaunchKernelGGL((hga_dq_kernel<64>), gq, bq, 0, sm, qp, ka, va, (long)act_bstride, kh, vh,
                       (long)hist_bstride, idx, lse, dd, dop, dqp, S, H, Hkv, C, chunk, topk, scale);
    hipLaunchKernelGGL((hga_dkdv_kernel<64, NW>), gk, bk, 0, sm, qp, ka, va, (long)act_bstride, lse, dd, dop, dkp,
                       dvp, S, H, Hkv, scale);
  }
  return hipGetLastError() == hipSuccess ? S2A_OK : S2A_ERR_HIP;
}
