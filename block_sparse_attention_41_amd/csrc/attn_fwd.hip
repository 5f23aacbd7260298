// Forward kernels: shifted short attention (group-local causal, half the heads rolled by
// G/2) and HGA (local causal segment plus gathered history chunks, one softmax).
//
// One workgroup owns NW wavefronts x 32 query rows of one (batch, head).  K/V tiles of 64
// keys are copied HBM -> LDS directly, both row-major (fwd2_core.h).  The shifted kernel
// double-buffers them, issuing tile i+1's copies once tile i's scores are under way; the
// per-head HGA kernel single-buffers them and relies on two workgroups per CU instead.
#include "../../include/s2a.h"
#include <algorithm>

#include "fwd2_core.h"
#include "launch.h"
#include "select_core.h"
#include "validate.h"

namespace s2a {

// ---------------------------------------------------------------------------------------
// Shifted short attention.
//
// LongLoRA's shift short attention (LongLoRA abstract; LongQLoRA post, section 03): a
// shifted head sees token t at rolled position p = (t - s) mod N with s = G/2, and
// attends causally (in rolled order) inside its rolled group floor(p / G).  Every tile of
// 64 rolled positions maps to 64 consecutive tokens because s and N are multiples of 64,
// so the roll costs one base-offset per tile.
// ---------------------------------------------------------------------------------------
// Workgroup ids are dealt round-robin to the 8 XCDs.  Logical work units are ordered
// (batch, head, group, tile-in-group heaviest first) and every XCD gets a contiguous run
// of them, so the q tiles that share one group's K/V run on the same XCD and its L2.
// ---------------------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void s2attn_fwd_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    bf16_t* __restrict__ o, float* __restrict__ lse, int B, int N, int H, int Hkv, int G, int shift_on, float c,
    int tiles_per_group, int units, int slots) {
  constexpr int BM = 32 * NW;
  __shared__ __align__(16) Fwd2Lds<D> lds;
  // per-lane V copy offsets and transposed-read offsets, fixed for the whole launch
  const CopyOffsets<D, NW> vco = copy_offsets<D, NW>(thread_x() / 64, thread_x() % 64, (long)Hkv * D);
  const TrOffsets<D> vo = tr_offsets<D>(thread_x() % 64);

  // XCD x (workgroup index mod 8) owns units [x * per, (x + 1) * per), ordered by (batch,
  // head, group) and heaviest tile first within a group.  Each of its `slots` workgroups
  // walks that range in rounds, forwards in even rounds and backwards in odd ones, so a
  // workgroup that drew a heavy unit draws a light one next.  With one workgroup per unit
  // (slots = per) this is a plain launch; with slots = the chip's resident workgroups
  // per XCD it is persistent: no workgroup waits to be dispatched after the first.
  const int per = (units + 7) / 8;
  const int xcd = group_x() % 8, slot = group_x() / 8;
  for (int r = 0; r * slots < per; ++r) {
  const int vv = r * slots + ((r & 1) ? slots - 1 - slot : slot);
  const int u = xcd * per + vv;
  if (vv >= per || u >= units) continue;
  const int ngroups = N / G;
  const int tig = tiles_per_group - 1 - u % tiles_per_group;  // heaviest tiles first
  int rest = u / tiles_per_group;
  const int grp = rest % ngroups;
  rest /= ngroups;
  const int h = rest % H;
  const int b = rest / H;
  const int s = (shift_on && ngroups >= 2 && h >= H / 2) ? G / 2 : 0;
  const int kvh = h / (H / Hkv);
  const int tid = thread_x(), w = tid / 64, lane = tid % 64, lq = lane % 32, g = lane / 32;

  const int gstart = grp * G;
  const int qp0 = gstart + tig * BM;
  const int qpw = qp0 + 32 * w;
  const bool active = qpw < gstart + G;
  const int qlast = min(qp0 + BM, gstart + G) - 1;
  const int ntiles = (qlast - gstart) / kTile + 1;

  const long qs = (long)H * D, ks = (long)Hkv * D;
  const int tokw = active ? (qpw + s) % N : 0;
  bf16x8_t qf[D / 16];
  if (active) load_row_frag<D>(qf, q + ((long)b * N + tokw + lq) * qs + (long)h * D, g);

  f32x16_t acc[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) acc[nb] = f32x16_t{};
  float m = kNegInf, l = 0.f;

  const bf16_t* kb0 = k + (long)b * N * ks + (long)kvh * D;
  const bf16_t* vb0 = v + (long)b * N * ks + (long)kvh * D;
  {
    const int tok = (gstart + s) % N;
    k_tile_direct<D, NW>(kb0 + tok * ks, ks, lds.k[0], w, lane);
    copy_tile<D, NW>(vb0 + tok * ks, vco, lds.v[0], w);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < ntiles;
    // copies of tile it + 1 into the other buffers, issued once this tile's K fragments
    // have been read (by every wave, also one that skips the tile)
    auto issue_next = [&]() {
      if (more) {
        const int tok = (gstart + kTile * (it + 1) + s) % N;
        k_tile_direct<D, NW>(kb0 + tok * ks, ks, lds.k[cur ^ 1], w, lane);
        copy_tile<D, NW>(vb0 + tok * ks, vco, lds.v[cur ^ 1], w);
      }
    };
    const int kp0 = gstart + kTile * it;
    if (active && kp0 <= qpw + 31)
      fwd2_tile<D>(lds.k[cur], lds.v[cur], vo, qf, acc, m, l, lq, g, kp0 + kTile - 1 > qpw, kp0, qpw + lq, c,
                   issue_next);
    else
      issue_next();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (active) {
    const float lt = pair_sum(l);
    // whole rows of O through this wave's 32 x D share of the (now idle) tile buffers
    bf16_t* st = w < 4 ? lds.k[w / 2] + (w % 2) * 32 * D : lds.v[(w - 4) / 2] + (w % 2) * 32 * D;
    int ln = lane;
    asm volatile("" : "+v"(ln));   // its LDS addresses are not kept in registers across units
    store_acc_tile<D>(acc, 1.f / lt, st, o + ((long)b * N + tokw) * qs + (long)h * D, qs, ln);
    if (g == 0) lse[((long)b * H + h) * N + tokw + lq] = (m + __builtin_log2f(lt)) * kLn2;
  }
  __syncthreads();   // the next unit reuses the LDS tiles
  }
}

// ---------------------------------------------------------------------------------------
// HGA forward ("Long-Context Fine-Tuning with Limited VRAM", English abstract): each query
// block attends, under one softmax, to its causal segment prefix and to every token of
// the history chunks selected for it.  One workgroup = one query block of 64 = 4 waves.
// ---------------------------------------------------------------------------------------
// Four waves per workgroup: two key streams of two waves each (one wave per 32-query
// half of the block).  The block's 64-key tiles (its causal prefix, then the 64-key halves
// of each selected chunk) are dealt alternately to the streams, each with its own
// single-buffered K and V tiles (32 KB at d = 128), so the two streams get equal shares; at the
// end stream 1 hands its softmax state (running max, partial sum, unnormalised O) to
// stream 0 through LDS and stream 0 merges and normalises.  Workgroups run heaviest block
// first; two share a CU (eight waves), and the light blocks of the second half take the
// places of the first half's early finishers.  The chunk list stays in lane registers
// (lane e holds entry e) and is walked with a ballot mask.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void hga_fwd_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_act, const bf16_t* __restrict__ v_act,
    long act_bstride, const bf16_t* __restrict__ k_hist, const bf16_t* __restrict__ v_hist,
    long hist_bstride, const int32_t* __restrict__ idx, bf16_t* __restrict__ o, float* __restrict__ lse,
    int S, int H, int Hkv, int C, int chunk, int topk, float c, int units, int hpl) {
  constexpr int NW = 2;   // waves per key stream
  __shared__ __align__(16) bf16_t lk[2][kTile * D];
  __shared__ __align__(16) bf16_t lv[2][kTile * D];

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
  const int w = __builtin_amdgcn_readfirstlane((tid / 64) % NW);   // query half
  const int ps = __builtin_amdgcn_readfirstlane(tid / (64 * NW));  // key stream

  // chunk list of this block; entries outside [0, C) are skipped
  int cidx = -1;
  if (lane < topk) cidx = idx[(((long)b * (H / hpl) + h / hpl) * nqb + j) * topk + lane];
  unsigned long long rem = __ballot(lane < topk && cidx >= 0 && cidx < C);
  const int spc = chunk / kTile;
  const int nloc = j + 1;
  const int ntiles = nloc + __popcll(rem) * spc;

  const long qs = (long)H * D, ks = (long)Hkv * D;
  const int qpw = 64 * j + 32 * w;
  bf16x8_t qf[D / 16];
  load_row_frag<D>(qf, q + ((long)b * S + qpw + lq) * qs + (long)h * D, g);
  const TileCopy<D, NW, true> kco = tile_copy_offsets<D, NW, true>(lane, ks);
  const TileCopy<D, NW, false> vco = tile_copy_offsets<D, NW, false>(lane, ks);

  f32x16_t acc[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) acc[nb] = f32x16_t{};
  float m = kNegInf, l = 0.f;

  const bf16_t* ka = k_act + b * act_bstride + (long)kvh * D;
  const bf16_t* va = v_act + b * act_bstride + (long)kvh * D;
  const bf16_t* kh = k_hist + b * hist_bstride + (long)kvh * D;
  const bf16_t* vh = v_hist + b * hist_bstride + (long)kvh * D;
  // tile t: local tiles 0..j first (token-causal on tile j), then the selected history
  // chunks in 64-key sub-tiles; every wave walks all tiles in order and stream ps works on
  // t = 2 i + ps
  int cur = 0;
  auto row_of = [&](int t) {   // first key row of tile t (advances the chunk cursor)
    if (t < nloc) return (long)kTile * t;
    const int sub = (t - nloc) % spc;
    if (sub == 0) {   // next selected chunk
      cur = __builtin_amdgcn_readlane(cidx, __builtin_ctzll(rem));
      rem &= rem - 1;
    }
    return (long)cur * chunk + (long)kTile * sub;
  };
  for (int t0 = 0; t0 < ntiles; t0 += 2) {
    const long ra = row_of(t0);
    const long rb = t0 + 1 < ntiles ? row_of(t0 + 1) : 0;
    const int it = t0 + ps;
    const bool has = it < ntiles;
    const bool loc = it < nloc;
    const long r0 = ps ? rb : ra;
    // an opaque copy of the lane index: the LDS read offsets derived from it are
    // recomputed each iteration instead of being hoisted into registers (which spill)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lqi = ln & 31, gi = ln >> 5;
    if (has) {
      copy_tile_swz(kco, (loc ? ka : kh) + r0 * ks, ks, lk[ps], w);
      copy_tile_swz(vco, (loc ? va : vh) + r0 * ks, ks, lv[ps], w);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int kp0 = loc ? kTile * it : 0;
    if (has && (!loc || kp0 <= qpw + 31))
      fwd2_tile<D>(lk[ps], lv[ps], tr_offsets<D>(ln), qf, acc, m, l, lqi, gi, loc && it == j, kp0, qpw + lqi, c,
                   [] {});
    __syncthreads();
  }
  // stream 1's state to stream 0 through the (idle) tile buffers: the accumulators of the
  // wave of query half 0 in lk[1], those of half 1 in lv[1], running max and partial sum
  // of both in lv[0]
  constexpr int NA = D / 32 * 16;   // accumulator floats per lane
  static_assert(NA * 64 * 4 == kTile * D * 2, "one tile buffer holds one wave's accumulators");
  float* xa = reinterpret_cast<float*>(w == 0 ? lk[1] : lv[1]);
  float* xs = reinterpret_cast<float*>(lv[0]) + 128 * w;
  if (ps == 1) {
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<float4*>(xa + ((nb * 4 + i4) * 64 + lane) * 4) =
            float4{acc[nb][4 * i4], acc[nb][4 * i4 + 1], acc[nb][4 * i4 + 2], acc[nb][4 * i4 + 3]};
    xs[lane] = m;
    xs[64 + lane] = l;
  }
  __syncthreads();
  if (ps == 1) return;
  {
    const float m1 = xs[lane], l1 = xs[64 + lane];
    const float mf = fmaxf(m, m1);
    const float a0 = fast_exp2(m - mf), a1 = fast_exp2(m1 - mf);   // a1 = 0 if stream 1 saw no key
    m = mf;
    l = l * a0 + l1 * a1;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 t = *reinterpret_cast<const float4*>(xa + ((nb * 4 + i4) * 64 + lane) * 4);
        acc[nb][4 * i4] = acc[nb][4 * i4] * a0 + t.x * a1;
        acc[nb][4 * i4 + 1] = acc[nb][4 * i4 + 1] * a0 + t.y * a1;
        acc[nb][4 * i4 + 2] = acc[nb][4 * i4 + 2] * a0 + t.z * a1;
        acc[nb][4 * i4 + 3] = acc[nb][4 * i4 + 3] * a0 + t.w * a1;
      }
  }
  const float lt = pair_sum(l);
  // whole rows of O through this wave's half of stream 0's (idle) K tile
  store_acc_tile<D>(acc, 1.f / lt, lk[0] + w * 32 * D, o + ((long)b * S + qpw) * qs + (long)h * D, qs, lane);
  if (g == 0) lse[((long)b * H + h) * S + qpw + lq] = (m + __builtin_log2f(lt)) * kLn2;
}


// HGA forward with one chunk list per kv head, for kv heads with four q heads: one
// workgroup = the 32 rows of one half query block for all four q heads (eight waves: two
// key streams x four heads).  The block's tiles are dealt to the streams as in
// hga_fwd_kernel, so every (head, row) sees the same tiles in the same order and gets the
// same bits; each staged tile now feeds four heads, and each wave copies a quarter of it.
// With eight waves of up to 256 registers a CU holds one workgroup, so each stream
// double-buffers its tiles (128 KB of LDS at d = 128) and issues the copies of its next
// tile once the current tile's scores are under way.
//
// With SEL the workgroup also chooses its block's chunk list ("Long-Context Fine-Tuning
// with Limited VRAM", English abstract: a capped set of history chunks per query block):
// waves 0-3 form the block means of the kv head's four q heads (all 64 rows of the block),
// wave 0 sums them, each of the eight waves scores every eighth 64-chunk tile of the
// summaries (lane = chunk, rows read from L2) and keeps its running top 64, and wave 0
// merges the eight lists.  The arithmetic is the selection kernel's (select_core.h), so
// the list is the one hga_select_topk_shared writes.  Both half-block workgroups of a
// block compute the same list; the one of half 0 writes it to idx for the backward.
template <int D, bool SEL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void hga_fwd_grp_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_act, const bf16_t* __restrict__ v_act,
    long act_bstride, const bf16_t* __restrict__ k_hist, const bf16_t* __restrict__ v_hist,
    long hist_bstride, int32_t* __restrict__ idx, const float* __restrict__ summ, long sbs,
    bf16_t* __restrict__ o, float* __restrict__ lse, int S, int H, int Hkv, int C, int chunk, int topk, float c,
    int units) {
  constexpr int R = 4;   // q heads per kv head = waves per key stream
  struct Bufs {
    bf16_t k[2][2][kTile * D];   // [stream][buffer]
    bf16_t v[2][2][kTile * D];
  };
  __shared__ __align__(16) Bufs lds;
  auto& lk = lds.k;
  auto& lv = lds.v;

  const int nqb = S / 64;
  const int npj = units / nqb;   // (batch, kv head, half block) per block index
  // heaviest query blocks first; within one block index the two halves of a kv head's
  // block on one XCD (workgroup i runs on XCD i mod 8) when the pairs divide evenly
  const int j = nqb - 1 - group_x() / npj;
  const int i = group_x() % npj;
  const int u = (npj % 16 == 0) ? (i % 8) * (npj / 8) + i / 8 : i;
  const int half = u % 2;
  const int kvh = (u / 2) % Hkv;
  const int b = u / 2 / Hkv;
  const int tid = thread_x(), lane = tid % 64, lq = lane % 32, g = lane / 32;
  const int w = (tid / 64) % R;    // q head within the kv head's group
  // transposed-read offsets taken from the lane index itself (not from the opaque copy
  // below): with addresses the compiler can trace to the V buffers, it sees that this
  // tile's V reads do not depend on the next tile's copies in flight and does not wait
  const TrOffsets<D> vo = tr_offsets<D>(lane);
  const int ps = tid / (64 * R);   // key stream
  const int h = kvh * R + w;

  int cidx = -1;
  const long list_off = (((long)b * Hkv + kvh) * nqb + j) * topk;
  if constexpr (SEL) {
    float(*qbar)[D] = reinterpret_cast<float(*)[D]>(&lds.v[0][0][0]);
    float* qsum = reinterpret_cast<float*>(&lds.v[0][1][0]);
    int* list = reinterpret_cast<int*>(&lds.v[1][0][0]);
    unsigned long long(*bests)[64] = reinterpret_cast<unsigned long long(*)[64]>(&lds.k[0][0][0]);
    constexpr int NWV = 2 * R;   // waves of the workgroup
    const int wv = tid / 64;
    if (C > 0 && tid < 64 * R) {
      // the selection kernel's grouped slots with one head each: 0 + mean
      float m[8];
      block_mean_rows<D>(q + (((long)b * S + 64 * j) * H + kvh * R + w) * D, (long)H * D, lane, m);
      if (lane < D / 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qbar[w][8 * lane + e] = 0.f + m[e];
      }
    }
    __syncthreads();
    if (C > 0 && tid < 64) {
#pragma unroll
      for (int e = lane; e < D; e += 64) qsum[e] = ((qbar[0][e] + qbar[1][e]) + qbar[2][e]) + qbar[3][e];
    }
    __syncthreads();
    unsigned long long best = 0ull;
    const float* sb = summ + b * sbs + (long)kvh * D;
    for (int c0 = kTile * wv; c0 < C; c0 += kTile * NWV)
      best = score_merge_rows<D>(qsum, sb, (long)Hkv * D, c0, C, best, lane);
    bests[wv][63 - lane] = best;   // reversed, ready for merge_best
    __syncthreads();
    if (tid < 64) {
      for (int x = 1; x < NWV && kTile * x < C; ++x) best = merge_best(best, bests[x][lane], lane);
      const int e = final_entry(best, C, topk, lane);
      list[lane] = e;
      if (half == 0 && lane < topk) idx[list_off + lane] = e;
    }
    __syncthreads();
    if (lane < topk) cidx = list[lane];
    __syncthreads();   // the staging space holds K/V tiles from here on
  } else {
    if (lane < topk) cidx = idx[list_off + lane];
  }
  unsigned long long rem = __ballot(lane < topk && cidx >= 0 && cidx < C);
  const int spc = chunk / kTile;
  const int nloc = j + 1;
  const int ntiles = nloc + __popcll(rem) * spc;

  const long qs = (long)H * D, ks = (long)Hkv * D;
  const int qpw = 64 * j + 32 * half;
  bf16x8_t qf[D / 16];
  load_row_frag<D>(qf, q + ((long)b * S + qpw + lq) * qs + (long)h * D, g);

  f32x16_t acc[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) acc[nb] = f32x16_t{};
  float m = kNegInf, l = 0.f;

  const bf16_t* ka = k_act + b * act_bstride + (long)kvh * D;
  const bf16_t* va = v_act + b * act_bstride + (long)kvh * D;
  const bf16_t* kh = k_hist + b * hist_bstride + (long)kvh * D;
  const bf16_t* vh = v_hist + b * hist_bstride + (long)kvh * D;
  int cur = 0;
  auto row_of = [&](int t) {   // first key row of tile t < ntiles (advances the chunk cursor)
    if (t < nloc) return (long)kTile * t;
    const int sub = (t - nloc) % spc;
    if (sub == 0) {
      cur = __builtin_amdgcn_readlane(cidx, __builtin_ctzll(rem));
      rem &= rem - 1;
    }
    return (long)cur * chunk + (long)kTile * sub;
  };
  {
    const long r0 = row_of(0);
    const long r1 = ntiles > 1 ? row_of(1) : 0;
    if (ps < ntiles) {
      const long r = ps ? r1 : r0;
      const bool loc = ps < nloc;
      k_tile_direct<D, R>((loc ? ka : kh) + r * ks, ks, lk[ps][0], w, lane);
      copy_tile_direct<D, R>((loc ? va : vh) + r * ks, ks, lv[ps][0], w, lane);
    }
  }
  long na = ntiles > 2 ? row_of(2) : 0;
  long nb2 = ntiles > 3 ? row_of(3) : 0;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int niter = (ntiles + 1) / 2;
  for (int it2 = 0; it2 < niter; ++it2) {
    const int cb = it2 & 1;
    const int it = 2 * it2 + ps;
    const bool has = it < ntiles;
    const bool loc = it < nloc;
    const int nt = it + 2;
    const bool more = nt < ntiles;
    const bool nloc2 = nt < nloc;
    const long rn = ps ? nb2 : na;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lqi = ln & 31, gi = ln >> 5;
    auto issue_next = [&]() {
      if (more) {
        k_tile_direct<D, R>((nloc2 ? ka : kh) + rn * ks, ks, lk[ps][cb ^ 1], w, ln);
        copy_tile_direct<D, R>((nloc2 ? va : vh) + rn * ks, ks, lv[ps][cb ^ 1], w, ln);
      }
    };
    const int kp0 = loc ? kTile * it : 0;
    if (has && (!loc || kp0 <= qpw + 31))
      fwd2_tile<D>(lk[ps][cb], lv[ps][cb], vo, qf, acc, m, l, lqi, gi, loc && it == j, kp0, qpw + lqi, c,
                   issue_next);
    else
      issue_next();
    na = 2 * it2 + 4 < ntiles ? row_of(2 * it2 + 4) : 0;
    nb2 = 2 * it2 + 5 < ntiles ? row_of(2 * it2 + 5) : 0;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // stream 1's softmax state to stream 0: accumulators of head w in the w-th K buffer,
  // running max and partial sum in the first V buffer; stream 0 then stages its O rows
  // in stream 1's V buffers, which nothing else touches now
  constexpr int NA = D / 32 * 16;
  float* xa = reinterpret_cast<float*>(lk[w / 2][w % 2]);
  float* xs = reinterpret_cast<float*>(lv[0][0]) + 128 * w;
  if (ps == 1) {
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<float4*>(xa + ((nb * 4 + i4) * 64 + lane) * 4) =
            float4{acc[nb][4 * i4], acc[nb][4 * i4 + 1], acc[nb][4 * i4 + 2], acc[nb][4 * i4 + 3]};
    xs[lane] = m;
    xs[64 + lane] = l;
  }
  __syncthreads();
  if (ps == 1) return;
  {
    const float m1 = xs[lane], l1 = xs[64 + lane];
    const float mf = fmaxf(m, m1);
    const float a0 = fast_exp2(m - mf), a1 = fast_exp2(m1 - mf);
    m = mf;
    l = l * a0 + l1 * a1;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 t = *reinterpret_cast<const float4*>(xa + ((nb * 4 + i4) * 64 + lane) * 4);
        acc[nb][4 * i4] = acc[nb][4 * i4] * a0 + t.x * a1;
        acc[nb][4 * i4 + 1] = acc[nb][4 * i4 + 1] * a0 + t.y * a1;
        acc[nb][4 * i4 + 2] = acc[nb][4 * i4 + 2] * a0 + t.z * a1;
        acc[nb][4 * i4 + 3] = acc[nb][4 * i4 + 3] * a0 + t.w * a1;
      }
  }
  static_assert(NA * 64 * 4 == kTile * D * 2, "one K buffer holds one wave's accumulators");
  const float lt = pair_sum(l);
  store_acc_tile<D>(acc, 1.f / lt, lv[1][w / 2] + (w % 2) * 32 * D,
                    o + ((long)b * S + qpw) * qs + (long)h * D, qs, lane);
  if (g == 0) lse[((long)b * H + h) * S + qpw + lq] = (m + __builtin_log2f(lt)) * kLn2;
}

}  // namespace s2a

using namespace s2a;

extern "C" int s2attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int N,
                          int H, int Hkv, int d, int G, int shift, float scale, void* stream) {
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(o) || !ptr_ok(lse)) return S2A_ERR_INVALID_ARG;
  int st = check_s2attn(B, N, H, Hkv, d, G, shift, scale);
  if (st) return st;
  // Short groups: four-wave workgroups, two per CU, cover each other's prologues and
  // causal tails.  Longer groups: eight-wave workgroups stage each K/V tile for twice as
  // many query rows, which halves the L2 -> LDS traffic, and keep a CU's waves in step:
  // of two four-wave workgroups sharing a CU the older one's waves win the issue slots,
  // it ends its (equal) share well before the other, and the CU then runs one wave per
  // SIMD (at the 8K step 149 against 192 us).
  const bool wide = G >= kWideGroupFwd;
  const int bm = 32 * (wide ? 8 : 4);
  const int tpg = (G + bm - 1) / bm;
  const long units = (long)tpg * (N / G) * H * B;
  if (units >= (1l << 31) - 8) return S2A_ERR_UNSUPPORTED;
  // groups shorter than kPersistGroup: persistent launch, as many workgroups as stay
  // resident (one eight-wave or two four-wave workgroups per CU), each looping over its
  // XCD's units, so none waits to be dispatched; longer groups: one workgroup per unit,
  // where the hardware's dynamic dispatch balances the long units better
  const int per = (int)((units + 7) / 8);
  const int slots = G < kPersistGroup ? std::min(per, resident_per_xcd(wide ? 1 : 2)) : per;
  const int grid = 8 * slots;
  const float c = scale * kLog2e;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto qp = static_cast<const bf16_t*>(q);
  auto kp = static_cast<const bf16_t*>(k);
  auto vp = static_cast<const bf16_t*>(v);
  auto op = static_cast<bf16_t*>(o);
  if (d == 128) {
    if (wide)
      hipLaunchKernelGGL((s2attn_fwd_kernel<128, 8>), dim3(grid), dim3(512), 0, s, qp, kp, vp, op, lse, B, N, H, Hkv,
                         G, shift, c, tpg, (int)units, slots);
    else
      hipLaunchKernelGGL((s2attn_fwd_kernel<128, 4>), dim3(grid), dim3(256), 0, s, qp, kp, vp, op, lse, B, N, H, Hkv,
                         G, shift, c, tpg, (int)units, slots);
  } else {
    if (wide)
      hipLaunchKernelGGL((s2attn_fwd_kernel<64, 8>), dim3(grid), dim3(512), 0, s, qp, kp, vp, op, lse, B, N, H, Hkv,
                         G, shift, c, tpg, (int)units, slots);
    else
      hipLaunchKernelGGL((s2attn_fwd_kernel<64, 4>), dim3(grid), dim3(256), 0, s, qp, kp, vp, op, lse, B, N, H, Hkv,
                         G, shift, c, tpg, (int)units, slots);
  }
  return hipGetLastError() == hipSuccess ? S2A_OK : S2A_ERR_HIP;
}

static int hga_fwd_impl(const void* q, const void* k_act, const void* v_act, long long act_bstride,
                       const void* k_hist, const void* v_hist, long long hist_bstride, const int32_t* idx,
                       void* o, float* lse, int B, int S, int H, int Hkv, int d, int T, int chunk, int qblock,
                       int topk, float scale, void* stream, bool shared) {
  if (!ptr_ok(q) || !ptr_ok(k_act) || !ptr_ok(v_act) || !ptr_ok(o) || !ptr_ok(lse) || !ptr_ok(idx))
    return S2A_ERR_INVALID_ARG;
  int st = check_hga_shape(B, S, H, Hkv, d, T, chunk, qblock, topk);
  if (st) return st;
  if (check_scale(scale)) return S2A_ERR_INVALID_ARG;
  if (T > 0 && (!ptr_ok(k_hist) || !ptr_ok(v_hist))) return S2A_ERR_INVALID_ARG;
  if (!stride_ok(act_bstride, S, Hkv, d, B) || !stride_ok(hist_bstride, T, Hkv, d, B)) return S2A_ERR_INVALID_ARG;
  if ((long)B * H * (S / 64) >= (1l << 31) - 8) return S2A_ERR_UNSUPPORTED;
  const int C = T / chunk;
  const int units = B * H * (S / 64);
  const int hpl = shared ? H / Hkv : 1;   // q heads per chunk list
  dim3 grid(units), block(256);
  const float c = scale * kLog2e;
  if (hpl == 4) {   // one workgroup per half block of a kv head, its four q heads together
    const int ug = 2 * units / 4;
    hipStream_t sg = reinterpret_cast<hipStream_t>(stream);
    auto kh = static_cast<const bf16_t*>(T > 0 ? k_hist : k_act);
    auto vh = static_cast<const bf16_t*>(T > 0 ? v_hist : v_act);
    auto qp = static_cast<const bf16_t*>(q);
    auto ka = static_cast<const bf16_t*>(k_act);
    auto va = static_cast<const bf16_t*>(v_act);
    auto op = static_cast<bf16_t*>(o);
    auto ip = const_cast<int32_t*>(idx);   // read only (SEL = false)
    if (d == 128)
      hipLaunchKernelGGL((hga_fwd_grp_kernel<128, false>), dim3(ug), dim3(512), 0, sg, qp, ka, va, (long)act_bstride,
                         kh, vh, (long)hist_bstride, ip, nullptr, 0l, op, lse, S, H, Hkv, C, chunk, topk, c, ug);
    else
      hipLaunchKernelGGL((hga_fwd_grp_kernel<64, false>), dim3(ug), dim3(512), 0, sg, qp, ka, va, (long)act_bstride,
                         kh, vh, (long)hist_bstride, ip, nullptr, 0l, op, lse, S, H, Hkv, C, chunk, topk, c, ug);
    return hipGetLastError() == hipSuccess ? S2A_OK : S2A_ERR_HIP;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto qp = static_cast<const bf16_t*>(q);
  auto ka = static_cast<const bf16_t*>(k_act);
  auto va = static_cast<const bf16_t*>(v_act);
  auto kh = static_cast<const bf16_t*>(T > 0 ? k_hist : k_act);
  auto vh = static_cast<const bf16_t*>(T > 0 ? v_hist : v_act);
  auto op = static_cast<bf16_t*>(o);
  if (d == 128)
    hipLaunchKernelGGL((hga_fwd_kernel<128>), grid, block, 0, s, qp, ka, va, (long)act_bstride, kh, vh,
                       (long)hist_bstride, idx, op, lse, S, H, Hkv, C, chunk, topk, c, units, hpl);
  else
    hipLaunchKernelGGL((hga_fwd_kernel<64>), grid, block, 0, s, qp, ka, va, (long)act_bstride, kh, vh,
                       (long)hist_bstride, idx, op, lse, S, H, Hkv, C, chunk, topk, c, units, hpl);
  return hipGetLastError() == hipSuccess ? S2A_OK : S2A_ERR_HIP;
}

extern "C" int hga_fwd(const void* q, const void* k_act, const void* v_act, long long act_bstride,
                       const void* k_hist, const void* v_hist, long long hist_bstride, const int32_t* idx,
                       void* o, float* lse, int B, int S, int H, int Hkv, int d, int T, int chunk, int qblock,
                       int topk, float scale, void* stream) {
  return hga_fwd_impl(q, k_act, v_act, act_bstride, k_hist, v_hist, hist_bstride, idx, o, lse, B, S, H, Hkv, d, T,
                      chunk, qblock, topk, scale, stream, false);
}

extern "C" int hga_fwd_shared(const void* q, const void* k_act, const void* v_act, long long act_bstride,
                              const void* k_hist, const void* v_hist, long long hist_bstride, const int32_t* idx,
                              void* o, float* lse, int B, int S, int H, int Hkv, int d, int T, int chunk,
                              int qblock, int topk, float scale, void* stream) {
  return hga_fwd_impl(q, k_act, v_act, act_bstride, k_hist, v_hist, hist_bstride, idx, o, lse, B, S, H, Hkv, d, T,
                      chunk, qblock, topk, scale, stream, true);
}

extern "C" int hga_fwd_select_shared(const void* q, const void* k_act, const void* v_act, long long act_bstride,
                                     const void* k_hist, const void* v_hist, long long hist_bstride,
                                     const float* summ, long long summ_bstride, int32_t* idx, void* o, float* lse,
                                     int B, int S, int H, int Hkv, int d, int T, int chunk, int qblock, int topk,
                                     float scale, void* stream) {
  if (!ptr_ok(q) || !ptr_ok(k_act) || !ptr_ok(v_act) || !ptr_ok(o) || !ptr_ok(lse) || !ptr_ok(idx))
    return S2A_ERR_INVALID_ARG;
  int st = check_hga_shape(B, S, H, Hkv, d, T, chunk, qblock, topk);
  if (st) return st;
  if (check_scale(scale)) return S2A_ERR_INVALID_ARG;
  const int C = T / chunk;
  if (T > 0 && (!ptr_ok(k_hist) || !ptr_ok(v_hist) || !ptr_ok(summ))) return S2A_ERR_INVALID_ARG;
  if (!stride_ok(act_bstride, S, Hkv, d, B) || !stride_ok(hist_bstride, T, Hkv, d, B) ||
      !stride_ok(summ_bstride, C, Hkv, d, B))
    return S2A_ERR_INVALID_ARG;
  if ((long)B * H * (S / 64) >= (1l << 31) - 8) return S2A_ERR_UNSUPPORTED;
  if (H / Hkv != 4) {
    // the selecting forward is built for kv heads with four q heads (the grouped kernel);
    // other group sizes run the two launches it fuses, which give the same lists and bits
    st = hga_select_topk_shared(q, summ, summ_bstride, idx, B, S, H, Hkv, d, C, qblock, topk, stream);
    if (st) return st;
    return hga_fwd_shared(q, k_act, v_act, act_bstride, k_hist, v_hist, hist_bstride, idx, o, lse, B, S, H, Hkv, d,
                          T, chunk, qblock, topk, scale, stream);
  }
  const int units = B * H * (S / 64);
  const int ug = 2 * units / 4;
  hipStream_t sg = reinterpret_cast<hipStream_t>(stream);
  auto qp = static_cast<const bf16_t*>(q);
  auto ka = static_cast<const bf16_t*>(k_act);
  auto va = static_cast<const bf16_t*>(v_act);
  auto kh = static_cast<const bf16_t*>(T > 0 ? k_hist : k_act);
  auto vh = static_cast<const bf16_t*>(T > 0 ? v_hist : v_act);
  auto op = static_cast<bf16_t*>(o);
  const float c = scale * kLog2e;
  if (d == 128)
    hipLaunchKernelGGL((hga_fwd_grp_kernel<128, true>), dim3(ug), dim3(512), 0, sg, qp, ka, va, (long)act_bstride,
                       kh, vh, (long)hist_bstride, idx, summ, (long)summ_bstride, op, lse, S, H, Hkv, C, chunk, topk,
                       c, ug);
  else
    hipLaunchKernelGGL((hga_fwd_grp_kernel<64, true>), dim3(ug), dim3(512), 0, sg, qp, ka, va, (long)act_bstride,
                       kh, vh, (long)hist_bstride, idx, summ, (long)summ_bstride, op, lse, S, H, Hkv, C, chunk, topk,
                       c, ug);
  return hipGetLastError() == hipSuccess ? S2A_OK : S2A_ERR_HIP;
}
