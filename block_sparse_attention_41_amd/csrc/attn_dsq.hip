// Query-major dQ from stored dS tiles (LongLoRA S2-Attn backward; the dS tile layout and
// the kernel that writes it are described in dsq.h).  Built with matrix products that
// accumulate in VGPRs: with one wave per SIMD the compiler otherwise keeps the accumulators
// in AGPRs and copies them around every step.
#include <algorithm>

#include "bwd2_core.h"
#include "dsq.h"
#include "launch.h"

namespace s2a {

// Query-major dQ from the dS tiles the key-major kernel wrote (dQ = scale dS K, no
// recomputation of S or dP).  A unit is a run of QT consecutive 64-query tiles
// (qa .. qa + QT - 1) of one (batch, head, group), walking key tiles t = 0 .. qa + QT - 1:
// each step stages the K tile and the dS tiles (qa + j, t) present (t <= qa + j) and forms
// dQ^T += K^T dS^T for those query tiles, so each K tile read serves 64 QT queries.  One
// persistent workgroup per CU (eight waves, two per SIMD); the steps of all of a
// workgroup's units form one stream, copied S - 1 steps ahead into a ring of S buffer sets,
// so the copies of the next unit are in flight while one finishes.  Units pair a long and a
// short run of one (batch, head, group) (p and np - 1 - p), so the workgroups get (nearly)
// equal numbers of steps, and each XCD takes a contiguous run of such pairs (K of a few
// heads stays in its L2).  The kernel streams dS, about 2 bytes per (query, key) pair.
//
// wave w's 16-byte pieces of a dS tile copy (slots (DPW w + i) 64 + lane, DPW = 8 / NW)
template <int NW>
__device__ __forceinline__ void ds_copy(const bf16_t* src, const int (&co)[8 / NW], bf16_t* lds, int w) {
#pragma unroll
  for (int i = 0; i < 8 / NW; ++i) load_lds16_stream(src + co[i], lds + ((8 / NW) * w + i) * 512);
}

// Query tiles per unit: each staged K tile serves 64 QT queries.
#ifndef S2A_DQS_QT
#define S2A_DQS_QT 4
#endif
constexpr int kDqsQT = S2A_DQS_QT;

// One unit's place in a workgroup's step stream.
struct DqsCur {
  int k, t, n;          // unit index within the workgroup, step, steps of the unit
  int qa, nt;           // first query tile of the unit, query tiles in it
  bool done;            // stream ended
  const bf16_t* kb;     // K of the (batch, kv head), token 0
  const bf16_t* dsb;    // the (batch, head, group)'s dS tiles
  bf16_t* qo;           // dQ of the (batch, head), token 0
  int gs, sh;           // group start, shift
};

struct DqsPlan {
  const bf16_t* k;
  const bf16_t* dsw;
  bf16_t* dq;
  int N, H, Hkv, G, shift_on;
  int ntl, np, nsu, tsu, per, slots;   // np: units (runs of QT query tiles) per (b, h, group)
};

template <int D, int QT>
__device__ __forceinline__ DqsCur dqs_unit(const DqsPlan& P, int k, int xcd, int slot) {
  DqsCur c{};
  // rounds in reverse: the key-major kernel walks each XCD's run of (batch, head, group)s
  // in the same order, so the last round here reads the dS it wrote first and the first
  // round the dS it wrote last, the tiles most likely still in the Infinity Cache
  const int nr = (P.per + P.slots - 1) / P.slots;
  for (;; ++k) {
    if ((k >> 1) >= nr) {
      c.done = true;
      return c;
    }
    const int r = (nr - 1 - (k >> 1)) * P.slots + slot;
    const int su = xcd * P.per + r;
    if (r >= P.per || su >= P.tsu) {   // no unit for this slot in this round
      k |= 1;
      continue;
    }
    const int si = su % P.nsu, bhg = su / P.nsu;
    const int pair = (k & 1) ? si : P.np - 1 - si;
    if ((k & 1) && si >= P.np - 1 - si) continue;   // the middle unit runs alone
    const int ngroups = P.N / P.G;
    const int grp = bhg % ngroups, h = (bhg / ngroups) % P.H, b = bhg / (ngroups * P.H);
    c.k = k;
    c.t = 0;
    c.qa = QT * pair;
    c.nt = min(QT, P.ntl - c.qa);
    c.n = c.qa + c.nt;
    c.done = false;
    const long ks = (long)P.Hkv * D;
    c.kb = P.k + (long)b * P.N * ks + (long)(h / (P.H / P.Hkv)) * D;
    const long tri = (long)P.ntl * (P.ntl + 1) / 2;
    c.dsb = P.dsw + (long)bhg * tri * (kTile * kTile);
    c.qo = P.dq + (long)b * P.N * P.H * D + (long)h * D;
    c.gs = grp * P.G;
    c.sh = (P.shift_on && ngroups >= 2 && h >= P.H / 2) ? P.G / 2 : 0;
    return c;
  }
}

template <int D, int QT>
__device__ __forceinline__ DqsCur dqs_next(const DqsPlan& P, DqsCur c, int xcd, int slot) {
  if (++c.t < c.n) return c;
  return dqs_unit<D, QT>(P, c.k + 1, xcd, slot);
}

__device__ __forceinline__ int dqs_tok(const DqsCur& c, int N, int tile) {
  const int x = c.gs + kTile * tile + c.sh;
  return x >= N ? x - N : x;
}

// Issue step c's copies (K tile, the dS tiles present: tile qa + j needs t <= qa + j) into
// one buffer set.
template <int D, int QT, int NW>
__device__ __forceinline__ void dqs_issue(const DqsPlan& P, const DqsCur& c, const CopyOffsets<D, NW>& kco,
                                          const int (&dco)[8 / NW], bf16_t* __restrict__ kn,
                                          bf16_t* __restrict__ nd, int wu) {
  const long ks = (long)P.Hkv * D;
  copy_tile<D, NW>(c.kb + (long)dqs_tok(c, P.N, c.t) * ks, kco, kn, wu);
#pragma unroll
  for (int j = 0; j < QT; ++j) {
    const int qt = c.qa + j;
    if (j < c.nt && c.t <= qt)
      ds_copy<NW>(c.dsb + ((long)qt * (qt + 1) / 2 + c.t) * (kTile * kTile), dco, nd + j * (kTile * kTile), wu);
  }
}

// Copies one wave issues for step c: the K tile's, and each present dS tile's.
template <int D, int QT, int NW>
__device__ __forceinline__ int dqs_ops(const DqsCur& c) {
  int n = CopyOffsets<D, NW>::PER;
#pragma unroll
  for (int j = 0; j < QT; ++j) n += (j < c.nt && c.t <= c.qa + j) ? 8 / NW : 0;
  return n;
}

// This wave's products of one step: its QTW query tiles (from jt0) x its NBW head-dim blocks.
template <int D, int NBW, int QTW>
__device__ __forceinline__ void dqs_compute(const bf16_t* __restrict__ kc, const bf16_t* __restrict__ dc,
                                            const DqsCur& c, int jt0, const int (&ko)[NBW][2], int dso,
                                            f32x16_t (&acc)[QTW][NBW]) {
  // an absent tile's buffer is read anyway (in bounds, stale) and masked to zeros: one
  // branch-free path for every step, so all reads can be issued ahead of the products
  constexpr int QT = QTW;
  unsigned m[QT];
#pragma unroll
  for (int j = 0; j < QT; ++j) m[j] = (jt0 + j < c.nt && c.t <= c.qa + jt0 + j) ? ~0u : 0u;
  dc += jt0 * (kTile * kTile);
  auto masked = [](bf16x8_t x, unsigned mk) {
    uint4 u = __builtin_bit_cast(uint4, x);
    u.x &= mk;
    u.y &= mk;
    u.z &= mk;
    u.w &= mk;
    return __builtin_bit_cast(bf16x8_t, u);
  };
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    bf16x8_t a[NBW];
#pragma unroll
    for (int jn = 0; jn < NBW; ++jn) a[jn] = tr_frag<D>(kc, ko[jn], kb);
#pragma unroll
    for (int j = 0; j < QT; ++j) {
      const bf16x8_t b = masked(ds_frag(dc + j * (kTile * kTile), dso, kb), m[j]);
#pragma unroll
      for (int jn = 0; jn < NBW; ++jn) acc[j][jn] = mfma32(a[jn], b, acc[j][jn]);
    }
  }
}

// One step: issue the copies of step `cp` (if any) into buffer set n, then (when `comp`)
// compute step `cc` from buffer set c.  Every LDS buffer is a restrict parameter of this
// inlined function, and it is the only place copies are issued, so the compiler can tell
// the reads of set c from the copies in flight and does not wait for them.
template <int D, int NBW, int QT, int NW, int QTW>
__device__ __forceinline__ void dqs_step(const DqsPlan& P, const DqsCur& cc, const DqsCur& cp, bool comp,
                                         const bf16_t* __restrict__ kc, const bf16_t* __restrict__ dc,
                                         bf16_t* __restrict__ kn, bf16_t* __restrict__ nd,
                                         const CopyOffsets<D, NW>& kco, const int (&dco)[8 / NW], int jt0,
                                         const int (&ko)[NBW][2], int dso, f32x16_t (&acc)[QTW][NBW], int wu) {
  if (!cp.done) dqs_issue<D, QT, NW>(P, cp, kco, dco, kn, nd, wu);
  if (!comp) return;
  dqs_compute<D, NBW, QTW>(kc, dc, cc, jt0, ko, dso, acc);
}

// Wait until at most N vector memory operations of this wave are outstanding and all its
// LDS reads have returned (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// The same for a wave-uniform n in [LO, HI] (the immediate is chosen by a binary search),
// then a barrier with the other waves.  No memory fence: the LDS buffers are written only
// by direct copies, which the vmcnt wait covers, and a fence would wait for every copy in
// flight.
template <int LO, int HI>
__device__ __forceinline__ void wait_vm_range(int n) {
  if constexpr (LO == HI) {
    wait_vm_lgkm<LO>();
  } else {
    constexpr int MID = (LO + HI + 1) / 2;
    if (n >= MID) wait_vm_range<MID, HI>(n);
    else wait_vm_range<LO, MID - 1>(n);
  }
}

__device__ __forceinline__ void wait_vm_barrier(int n) {
  wait_vm_range<0, 31>(n < 0 ? 0 : (n > 31 ? 31 : n));   // waiting for more is always correct
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, int NBW>
__device__ __forceinline__ void dqs_store(const DqsCur& c, int N, int H, int tile, f32x16_t (&acc)[NBW], int nb0,
                                          int mq, int lane, float scale) {
  const int lq = lane % 32, g = lane / 32;
  bf16_t* row = c.qo + (long)(dqs_tok(c, N, tile) + 32 * mq + lq) * H * D;
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint2 wv;
      wv.x = pack_bf16(acc[j][4 * i + 0] * scale, acc[j][4 * i + 1] * scale);
      wv.y = pack_bf16(acc[j][4 * i + 2] * scale, acc[j][4 * i + 3] * scale);
      *reinterpret_cast<uint2*>(row + 32 * (nb0 + j) + 8 * i + 4 * g) = wv;
    }
    acc[j] = f32x16_t{};
  }
}

// Buffer sets in the copy ring: as many as fit 160 KB of LDS, at most four.
template <int D, int QT>
constexpr int dqs_stages() {
  constexpr int set = (kTile * D + QT * kTile * kTile) * 2;
  return (160 * 1024) / set >= 4 ? 4 : (160 * 1024) / set;
}

#ifndef S2A_DQS_NW
#define S2A_DQS_NW 8
#endif
constexpr int kDqsNW = S2A_DQS_NW;

// NW waves: wave w owns queries 32 (w % 2) .. + 31 and head-dim blocks NB/2 (w / 2 % 2) ..
// of the unit's query tiles QTW (w / 4) .. + QTW - 1, QTW = 4 QT / NW (with eight waves,
// two per SIMD, one wave's fragment reads run under the other's products).
template <int D>
__global__ __launch_bounds__(64 * kDqsNW) void dqs_kernel(DqsPlan P, float scale) {
  constexpr int NW = kDqsNW, NB = D / 32, NBW = NB / 2, QT = kDqsQT, QTW = 4 * QT / NW, S = dqs_stages<D, QT>();
  static_assert(QTW >= 1 && QTW * NW == 4 * QT, "waves per unit");
  static_assert(S >= 2 && S <= 5, "buffer sets");
  __shared__ __align__(16) bf16_t ks[S][kTile * D];
  __shared__ __align__(16) bf16_t ds[S][QT * kTile * kTile];
  const int tid = thread_x(), w = tid / 64, lane = tid % 64;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int mq = wu % 2, nb0 = NBW * ((wu / 2) % 2), jt0 = QTW * (wu / 4);
  const int xcd = group_x() % 8, slot = group_x() / 8;
  const CopyOffsets<D, NW> kco = copy_offsets<D, NW>(wu, lane, (long)P.Hkv * D);
  int dco[8 / NW];
#pragma unroll
  for (int i = 0; i < 8 / NW; ++i) dco[i] = 8 * ds_chunk_of_slot(((8 / NW) * wu + i) * 64 + lane);
  int ko[NBW][2];
#pragma unroll
  for (int j = 0; j < NBW; ++j) tr_offsets_block<D>(lane, nb0 + j, ko[j]);
  const int dso = ds_tr_offset(lane, mq);
  f32x16_t acc[QTW][NBW];
#pragma unroll
  for (int j = 0; j < QTW; ++j)
#pragma unroll
    for (int jn = 0; jn < NBW; ++jn) acc[j][jn] = f32x16_t{};

  DqsCur cc = dqs_unit<D, QT>(P, 0, xcd, slot);
  DqsCur cp = cc;
  // copies this wave has issued, and the count right after each of the steps s .. s + S - 2
  int ops = 0;
  int mark[S - 1];
#pragma unroll
  for (int i = 0; i < S - 1; ++i) mark[i] = 0;
  // iterations s < 0 only issue copies (the first S - 1 steps)
  for (int s = 1 - S; !cc.done; ++s) {
    if (s >= 0) {
      // this wave's copies of step s have landed once only those issued after them are
      // outstanding (loads complete in order); the barrier then makes every wave's copies
      // visible and frees the set step s - 1 used
      wait_vm_barrier(ops - mark[0]);
    }
    const int c = (s + S) % S, n = (s + S - 1) % S;
    const int nops = cp.done ? 0 : dqs_ops<D, QT, NW>(cp);
    dqs_step<D, NBW, QT, NW, QTW>(P, cc, cp, s >= 0, ks[c], ds[c], ks[n], ds[n], kco, dco, jt0, ko, dso, acc, wu);
#pragma unroll
    for (int i = 0; i < S - 2; ++i) mark[i] = mark[i + 1];
    ops += nops;
    mark[S - 2] = ops;
    if (!cp.done) cp = dqs_next<D, QT>(P, cp, xcd, slot);
    if (s < 0) continue;
    if (cc.t == cc.n - 1) {
#pragma unroll
      for (int j = 0; j < QTW; ++j)
        if (jt0 + j < cc.nt) dqs_store<D, NBW>(cc, P.N, P.H, cc.qa + jt0 + j, acc[j], nb0, mq, lane, scale);
    }
    cc = dqs_next<D, QT>(P, cc, xcd, slot);
  }
}

// at most one workgroup per CU (the kernel's LDS ring allows no second); the units split
// evenly over the eight XCDs
void launch_dqs(int d, const bf16_t* k, const bf16_t* dsw, bf16_t* dq, int B, int N, int H, int Hkv, int G,
                int shift, float scale, hipStream_t st) {
  DqsPlan p;
  p.k = k;
  p.dsw = dsw;
  p.dq = dq;
  p.N = N;
  p.H = H;
  p.Hkv = Hkv;
  p.G = G;
  p.shift_on = shift;
  p.ntl = G / kTile;
  p.np = (p.ntl + kDqsQT - 1) / kDqsQT;
  p.nsu = (p.np + 1) / 2;
  p.tsu = B * H * (N / G) * p.nsu;
  p.per = (p.tsu + 7) / 8;
  p.slots = std::min(p.per, resident_per_xcd(1));
  if (d == 128) hipLaunchKernelGGL((dqs_kernel<128>), dim3(8 * p.slots), dim3(64 * kDqsNW), 0, st, p, scale);
  else hipLaunchKernelGGL((dqs_kernel<64>), dim3(8 * p.slots), dim3(64 * kDqsNW), 0, st, p, scale);
}

}  // namespace s2a
