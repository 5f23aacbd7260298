// HGA generation step ("Long-Context Fine-Tuning with Limited VRAM", English abstract: the
// method also serves retrieval and generation): the last nq (<= 32) tokens of an active
// segment of Sa tokens attend, under one softmax, to their causal prefix in the segment
// and to every token of the history chunks listed for their query block.
//
// With one to a few queries per head there is too little work per head for one
// workgroup, so the key set is split: each single-wave workgroup takes a few consecutive
// 64-key tiles of one (batch, head) (the segment's tiles first, then the 64-key pieces of
// the listed chunks in list order), stages them in its own LDS and runs the forward tile
// step on its 32 query rows (rows past nq repeat the last query and are not stored).  It
// writes its unnormalised float32 partial output with its running max and sum; a second
// launch combines the splits of each head and normalises.
#include "../../include/s2a.h"
#include <algorithm>

#include "fwd2_core.h"
#include "validate.h"

namespace s2a {

constexpr float kDecEmptyMax = -1e30f;  // running max of a row that has seen no key yet

// 64-key tiles per split: the (batch, head) key sets cut into about 2048 single-wave
// workgroups (two rounds of the four per CU that fit, one per SIMD: each holds about 400
// registers per lane), at least one tile each
struct DecPlan {
  int per, nsplit;
};
inline DecPlan decode_plan(int B, int Sa, int H, int chunk, int topk) {
  const long tiles = (Sa + kTile - 1) / kTile + (long)topk * (chunk / kTile);
  const long total = tiles * B * H;
  const int per = (int)std::max(1l, (total + 2047) / 2048);
  return {per, (int)((tiles + per - 1) / per)};
}

// One wave copies a K or V tile through registers into the swizzled LDS layout of the
// forward tile step (chunk c of row r at chunk position c ^ (r % CPR) for K, c ^ swz(r)
// for V); rows past rmax read row rmax.
template <int D, bool V>
__device__ __forceinline__ void tile_clamped(const bf16_t* base, long rstride, long r0, long rmax, bf16_t* lds,
                                             int lane) {
  constexpr int CPR = D / 8, RPI = 64 / CPR, INSTS = kTile / RPI;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint4 v[INSTS / 2];
#pragma unroll
    for (int i = 0; i < INSTS / 2; ++i) {
      const int row = (h * INSTS / 2 + i) * RPI + lane / CPR;
      const int c = (lane % CPR) ^ (V ? swz<D>(row) : row % CPR);
      v[i] = load16(base + std::min(r0 + row, rmax) * rstride + c * 8);
    }
#pragma unroll
    for (int i = 0; i < INSTS / 2; ++i) *reinterpret_cast<uint4*>(lds + (h * INSTS / 2 + i) * 512 + lane * 8) = v[i];
  }
}

// Partial record of a split, per query row (D + 4 floats, so records stay 16-byte
// aligned): D unnormalised output values, then the running max (base-2 units) and the sum.
template <int D>
__global__ __launch_bounds__(64) void hga_decode_part_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_act, const bf16_t* __restrict__ v_act,
    long act_bstride, const bf16_t* __restrict__ k_hist, const bf16_t* __restrict__ v_hist, long hist_bstride,
    const int32_t* __restrict__ idx, float* __restrict__ part, int nq, int Sa, int H, int Hkv, int C, int chunk,
    int topk, float c, int per, int nsplit) {
  __shared__ __align__(16) bf16_t lk[kTile * D];
  __shared__ __align__(16) bf16_t lv[kTile * D];
  const int sp = group_x(), h = group_y(), b = group_z();
  const int kvh = h / (H / Hkv);
  const int lane = thread_x(), lq = lane % 32, g = lane / 32;

  int cidx = -1;
  if (lane < topk) cidx = idx[((long)b * H + h) * topk + lane];
  unsigned long long rem = __ballot(lane < topk && cidx >= 0 && cidx < C);
  const int spc = chunk / kTile;
  const int nloc = (Sa + kTile - 1) / kTile;
  const int ntiles = nloc + __popcll(rem) * spc;
  const int t0 = sp * per, t1 = std::min(ntiles, t0 + per);
  const int p0 = Sa - nq;   // segment position of query 0
  const int qr = std::min(lq, nq - 1);

  const long qs = (long)H * D, ks = (long)Hkv * D;
  bf16x8_t qf[D / 16];
  load_row_frag<D>(qf, q + ((long)b * nq + qr) * qs + (long)h * D, g);
  f32x16_t acc[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) acc[nb] = f32x16_t{};
  // a finite start: a row whose first tiles are all masked keeps p = 0 instead of NaN
  float m = kDecEmptyMax, l = 0.f;

  const bf16_t* ka = k_act + b * act_bstride + (long)kvh * D;
  const bf16_t* va = v_act + b * act_bstride + (long)kvh * D;
  const bf16_t* kh = k_hist + b * hist_bstride + (long)kvh * D;
  const bf16_t* vh = v_hist + b * hist_bstride + (long)kvh * D;
  // chunks wholly before this split's first tile are passed over
  for (int k = (std::max(t0, nloc) - nloc) / spc; k > 0; --k) rem &= rem - 1;
  bool have = false;
  int cur = 0;
  const TrOffsets<D> vo = tr_offsets<D>(lane);
  const TileCopy<D, 1, true> kco = tile_copy_offsets<D, 1, true>(lane, ks);
  const TileCopy<D, 1, false> vco = tile_copy_offsets<D, 1, false>(lane, ks);
  for (int t = t0; t < t1; ++t) {
    const bool loc = t < nloc;
    long r0, rmax;
    if (loc) {
      r0 = (long)kTile * t;
      rmax = Sa - 1;
    } else {
      const int sub = (t - nloc) % spc;
      if (!have || sub == 0) {
        cur = __builtin_amdgcn_readlane(cidx, __builtin_ctzll(rem));
        rem &= rem - 1;
        have = true;
      }
      r0 = (long)cur * chunk + (long)kTile * sub;
      rmax = r0 + kTile - 1;
    }
    if (rmax - r0 == kTile - 1) {   // a whole tile: straight from HBM into LDS
      copy_tile_swz(kco, (loc ? ka : kh) + r0 * ks, ks, lk, 0);
      copy_tile_swz(vco, (loc ? va : vh) + r0 * ks, ks, lv, 0);
    } else {
      tile_clamped<D, false>(loc ? ka : kh, ks, r0, rmax, lk, lane);
      tile_clamped<D, true>(loc ? va : vh, ks, r0, rmax, lv, lane);
    }
    __builtin_amdgcn_s_waitcnt(0);   // the copies have landed
    const int kp0 = loc ? kTile * t : 0;
    // keys past a row's position (and past the segment's end) are masked
    fwd2_tile<D>(lk, lv, vo, qf, acc, m, l, lq, g, loc && kp0 + kTile - 1 > p0, kp0, p0 + qr, c, [] {});
  }
  const float lt = pair_sum(l);
  if (lq >= nq) return;   // rows past nq repeat the last query
  float* rec = part + ((((long)b * H + h) * nsplit + sp) * 32 + lq) * (D + 4);
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<float4*>(rec + 32 * nb + 8 * i + 4 * g) =
          float4{acc[nb][4 * i], acc[nb][4 * i + 1], acc[nb][4 * i + 2], acc[nb][4 * i + 3]};
  if (g == 0) {
    rec[D] = m;
    rec[D + 1] = lt;
  }
}

// The split kernel for kv heads whose rep = H / Hkv q heads fit one 32-row tile with their
// nq queries each (rep * nq <= 32): tile row r holds query r % nq of q head kvh * rep +
// r / nq.  A workgroup takes `per` consecutive tiles of the kv head's key set: its
// segment's tiles, then the 64-key pieces of the chunks its q heads list, in the order of
// the concatenated lists; a chunk listed by several of the heads is taken at its first
// entry only, with the rows of heads that do not list it masked (they see no key of it),
// and a chunk a list names twice is taken twice for that list, as the per-head kernel does.
// So each segment tile and each listed chunk is staged once per kv head instead of once
// per q head.  Records are per (batch, kv head, split) and row, as in the per-head kernel.
template <int D>
__global__ __launch_bounds__(64) void hga_decode_grp_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_act, const bf16_t* __restrict__ v_act,
    long act_bstride, const bf16_t* __restrict__ k_hist, const bf16_t* __restrict__ v_hist, long hist_bstride,
    const int32_t* __restrict__ idx, float* __restrict__ part, int nq, int Sa, int H, int Hkv, int C, int chunk,
    int topk, float c, int per, int nsplit) {
  __shared__ __align__(16) bf16_t lk[kTile * D];
  __shared__ __align__(16) bf16_t lv[kTile * D];
  const int sp = group_x(), kvh = group_y(), b = group_z();
  const int rep = H / Hkv, rows = rep * nq;
  const int lane = thread_x(), lq = lane % 32, g = lane / 32;

  // lane e < rep * topk holds entry e % topk of head e / topk's list
  int cidx = -1;
  if (lane < rep * topk) cidx = idx[((long)b * H + (long)kvh * rep + lane / topk) * topk + lane % topk];
  const bool valid = lane < rep * topk && cidx >= 0 && cidx < C;
  const int spc = chunk / kTile;
  const int nloc = (Sa + kTile - 1) / kTile;
  const int ntiles = nloc + rep * topk * spc;
  const int t0 = sp * per, t1 = std::min(ntiles, t0 + per);
  const int p0 = Sa - nq;
  const int r = std::min(lq, rows - 1);   // rows past rep * nq repeat the last one
  const int hh = r / nq, qi = r % nq;

  const long qs = (long)H * D, ks = (long)Hkv * D;
  bf16x8_t qf[D / 16];
  load_row_frag<D>(qf, q + ((long)b * nq + qi) * qs + ((long)kvh * rep + hh) * D, g);
  f32x16_t acc[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) acc[nb] = f32x16_t{};
  float m = kDecEmptyMax, l = 0.f;

  const bf16_t* ka = k_act + b * act_bstride + (long)kvh * D;
  const bf16_t* va = v_act + b * act_bstride + (long)kvh * D;
  const bf16_t* kh = k_hist + b * hist_bstride + (long)kvh * D;
  const bf16_t* vh = v_hist + b * hist_bstride + (long)kvh * D;
  const TrOffsets<D> vo = tr_offsets<D>(lane);
  const TileCopy<D, 1, true> kco = tile_copy_offsets<D, 1, true>(lane, ks);
  const TileCopy<D, 1, false> vco = tile_copy_offsets<D, 1, false>(lane, ks);
  for (int t = t0; t < t1; ++t) {
    const bool loc = t < nloc;
    long r0, rmax;
    bool diag;
    int kp0, qpos;
    if (loc) {
      r0 = (long)kTile * t;
      rmax = Sa - 1;
      kp0 = kTile * t;
      qpos = p0 + qi;
      diag = kp0 + kTile - 1 > p0;
    } else {
      const int e = (t - nloc) / spc, sub = (t - nloc) % spc;
      const int ch = __builtin_amdgcn_readlane(cidx, e);
      if (__builtin_amdgcn_readlane((int)valid, e) == 0) continue;
      // entries naming this chunk; a list that names it n times attends to it n times, so
      // entry e, the k-th occurrence in its own list, stands for the k-th occurrence in
      // every list, unless an earlier head's list has one (then that entry takes it)
      const unsigned long long same = __ballot(valid && cidx == ch);
      const unsigned long long hmask = (topk == 64) ? ~0ull : ((1ull << topk) - 1ull);
      const int he = e / topk;
      const int k = __popcll(same & (hmask << (he * topk)) & ((1ull << e) - 1ull));
      bool taken = false;
      for (int x = 0; x < he; ++x) taken = taken || __popcll((same >> (x * topk)) & hmask) > k;
      if (taken) continue;
      // heads whose list names the chunk more than k times see its keys; the others none
      const bool listed = __popcll((same >> (hh * topk)) & hmask) > k;
      r0 = (long)ch * chunk + (long)kTile * sub;
      rmax = r0 + kTile - 1;
      kp0 = 0;
      qpos = listed ? 0x7fffffff : -1;
      diag = __ballot(lq < rows && !listed) != 0ull;
    }
    if (rmax - r0 == kTile - 1) {
      copy_tile_swz(kco, (loc ? ka : kh) + r0 * ks, ks, lk, 0);
      copy_tile_swz(vco, (loc ? va : vh) + r0 * ks, ks, lv, 0);
    } else {
      tile_clamped<D, false>(loc ? ka : kh, ks, r0, rmax, lk, lane);
      tile_clamped<D, true>(loc ? va : vh, ks, r0, rmax, lv, lane);
    }
    __builtin_amdgcn_s_waitcnt(0);
    fwd2_tile<D>(lk, lv, vo, qf, acc, m, l, lq, g, diag, kp0, qpos, c, [] {});
    __builtin_amdgcn_s_waitcnt(0);   // this tile's LDS reads are done before the next copy
  }
  const float lt = pair_sum(l);
  if (lq >= rows) return;
  float* rec = part + ((((long)b * Hkv + kvh) * nsplit + sp) * 32 + lq) * (D + 4);
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<float4*>(rec + 32 * nb + 8 * i + 4 * g) =
          float4{acc[nb][4 * i], acc[nb][4 * i + 1], acc[nb][4 * i + 2], acc[nb][4 * i + 3]};
  if (g == 0) {
    rec[D] = m;
    rec[D + 1] = lt;
  }
}

// One workgroup per (batch, head, query row).  Thread (g, q) sums column quad q of the
// splits g, g + NG, ... scaled to the row's largest running max; the NG group sums are
// then added in group order (a fixed order: the result does not depend on timing).  The
// records of a split come from other XCDs' caches, so each thread issues the loads of
// its first MAXS splits together before using any.  `grp` q heads share one record set
// (the grouped split kernel: head h's rows sit at (h % grp) * nq + row of kv head h / grp).
template <int D>
__global__ __launch_bounds__(256) void hga_decode_merge_kernel(const float* __restrict__ part,
                                                               bf16_t* __restrict__ o, float* __restrict__ lse,
                                                               int nq, int H, int nsplit, int grp) {
  constexpr int NQ = D / 4, NG = 256 / NQ, MAXS = 12;
  __shared__ __align__(16) float4 sa[NG][NQ];
  __shared__ float sm[NG], ss[NG];
  const int h = group_x(), b = group_y(), row = group_z();
  const int tid = thread_x(), cq = tid % NQ, gi = tid / NQ;
  const long rs = 32l * (D + 4);   // split stride
  const float* base =
      part + ((((long)b * (H / grp) + h / grp) * nsplit) * 32 + (h % grp) * nq + row) * (D + 4);
  float xm[MAXS], xl[MAXS];
  float4 xa[MAXS];
  // unconditional loads (split index clamped, the extra ones ignored below): a guarded
  // load became a branch of its own with a wait after it
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    const float* rec = base + min(gi + NG * i, nsplit - 1) * rs;
    xm[i] = rec[D];
    xl[i] = rec[D + 1];
    xa[i] = *reinterpret_cast<const float4*>(rec + 4 * cq);
  }
  float mx = kDecEmptyMax;
#pragma unroll
  for (int i = 0; i < MAXS; ++i)
    if (gi + NG * i < nsplit) mx = fmaxf(mx, xm[i]);
  for (int s = gi + NG * MAXS; s < nsplit; s += NG) mx = fmaxf(mx, base[s * rs + D]);
  if (cq == 0) sm[gi] = mx;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NG; ++k) mx = fmaxf(mx, sm[k]);
  float sum = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    if (gi + NG * i < nsplit) {
      const float wgt = fast_exp2(xm[i] - mx);
      sum += xl[i] * wgt;
      a.x += xa[i].x * wgt;
      a.y += xa[i].y * wgt;
      a.z += xa[i].z * wgt;
      a.w += xa[i].w * wgt;
    }
  }
  for (int s = gi + NG * MAXS; s < nsplit; s += NG) {
    const float* rec = base + s * rs;
    const float wgt = fast_exp2(rec[D] - mx);
    sum += rec[D + 1] * wgt;
    const float4 x = *reinterpret_cast<const float4*>(rec + 4 * cq);
    a.x += x.x * wgt;
    a.y += x.y * wgt;
    a.z += x.z * wgt;
    a.w += x.w * wgt;
  }
  sa[gi][cq] = a;
  if (cq == 0) ss[gi] = sum;
  __syncthreads();
  if (gi != 0) return;
  float tot = 0.f;
  float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    tot += ss[k];
    t.x += sa[k][cq].x;
    t.y += sa[k][cq].y;
    t.z += sa[k][cq].z;
    t.w += sa[k][cq].w;
  }
  const float inv = 1.f / tot;
  *reinterpret_cast<uint2*>(o + (((long)b * nq + row) * H + h) * D + 4 * cq) =
      uint2{pack_bf16(t.x * inv, t.y * inv), pack_bf16(t.z * inv, t.w * inv)};
  if (cq == 0) lse[((long)b * H + h) * nq + row] = (mx + __builtin_log2f(tot)) * kLn2;
}

}  // namespace s2a

using namespace s2a;

extern "C" size_t hga_decode_workspace_bytes(int B, int nq, int Sa, int H, int d, int chunk, int topk) {
  if (B <= 0 || nq <= 0 || nq > 32 || Sa < nq || H <= 0 || (d != 64 && d != 128) || chunk <= 0 || chunk % 64 ||
      topk <= 0 || topk > 64)
    return 0;
  return (size_t)B * H * decode_plan(B, Sa, H, chunk, topk).nsplit * 32 * (d + 4) * sizeof(float);
}

extern "C" int hga_decode(const void* q, const void* k_act, const void* v_act, long long act_bstride,
                          const void* k_hist, const void* v_hist, long long hist_bstride, const int32_t* idx,
                          void* o, float* lse, void* workspace, size_t workspace_bytes, int B, int nq, int Sa,
                          int H, int Hkv, int d, int T, int chunk, int topk, float scale, void* stream) {
  if (!ptr_ok(q) || !ptr_ok(k_act) || !ptr_ok(v_act) || !ptr_ok(idx) || !ptr_ok(o) || !ptr_ok(lse))
    return S2A_ERR_INVALID_ARG;
  int st = check_common_heads(B, Sa, H, Hkv, d);
  if (st) return st;
  if (nq <= 0 || nq > Sa || T < 0 || chunk <= 0 || topk <= 0 || T % chunk) return S2A_ERR_INVALID_ARG;
  if (nq > 32 || chunk % 64 || topk > 64) return S2A_ERR_UNSUPPORTED;
  if (check_scale(scale)) return S2A_ERR_INVALID_ARG;
  if (T > 0 && (!ptr_ok(k_hist) || !ptr_ok(v_hist))) return S2A_ERR_INVALID_ARG;
  if (!stride_ok(act_bstride, Sa, Hkv, d, B) || !stride_ok(hist_bstride, T, Hkv, d, B)) return S2A_ERR_INVALID_ARG;
  if ((long long)B * nq * H * d >= (1ll << 31)) return S2A_ERR_UNSUPPORTED;
  if (!ptr_ok(workspace) || workspace_bytes < hga_decode_workspace_bytes(B, nq, Sa, H, d, chunk, topk))
    return S2A_ERR_WORKSPACE;
  const int C = T / chunk;
  const int rep = H / Hkv;
  // the grouped split kernel when a kv head's q heads fit one tile and its lists one wave,
  // and its records fit the workspace sized for the per-head kernel
  const DecPlan pg = decode_plan(B, Sa, Hkv, chunk, rep * topk);
  const bool grouped = rep > 1 && rep * nq <= 32 && rep * topk <= 64 &&
                       (size_t)B * Hkv * pg.nsplit * 32 * (d + 4) * sizeof(float) <= workspace_bytes;
  const DecPlan pl = grouped ? pg : decode_plan(B, Sa, H, chunk, topk);
  const int nsplit = pl.nsplit;
  const float c = scale * kLog2e;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto qp = static_cast<const bf16_t*>(q);
  auto ka = static_cast<const bf16_t*>(k_act);
  auto va = static_cast<const bf16_t*>(v_act);
  auto kh = static_cast<const bf16_t*>(T > 0 ? k_hist : k_act);
  auto vh = static_cast<const bf16_t*>(T > 0 ? v_hist : v_act);
  auto op = static_cast<bf16_t*>(o);
  float* part = static_cast<float*>(workspace);
  const dim3 gp(nsplit, grouped ? Hkv : H, B), gm(H, B, nq);
  const int grp = grouped ? rep : 1;
  if (d == 128) {
    if (grouped)
      hipLaunchKernelGGL((hga_decode_grp_kernel<128>), gp, dim3(64), 0, s, qp, ka, va, (long)act_bstride, kh, vh,
                         (long)hist_bstride, idx, part, nq, Sa, H, Hkv, C, chunk, topk, c, pl.per, nsplit);
    else
      hipLaunchKernelGGL((hga_decode_part_kernel<128>), gp, dim3(64), 0, s, qp, ka, va, (long)act_bstride, kh, vh,
                         (long)hist_bstride, idx, part, nq, Sa, H, Hkv, C, chunk, topk, c, pl.per, nsplit);
    hipLaunchKernelGGL((hga_decode_merge_kernel<128>), gm, dim3(256), 0, s, part, op, lse, nq, H, nsplit, grp);
  } else {
    if (grouped)
      hipLaunchKernelGGL((hga_decode_grp_kernel<64>), gp, dim3(64), 0, s, qp, ka, va, (long)act_bstride, kh, vh,
                         (long)hist_bstride, idx, part, nq, Sa, H, Hkv, C, chunk, topk, c, pl.per, nsplit);
    else
      hipLaunchKernelGGL((hga_decode_part_kernel<64>), gp, dim3(64), 0, s, qp, ka, va, (long)act_bstride, kh, vh,
                         (long)hist_bstride, idx, part, nq, Sa, H, Hkv, C, chunk, topk, c, pl.per, nsplit);
    hipLaunchKernelGGL((hga_decode_merge_kernel<64>), gm, dim3(256), 0, s, part, op, lse, nq, H, nsplit, grp);
  }
  return hipGetLastError() == hipSuccess ? S2A_OK : S2A_ERR_HIP;
}
