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
// recomputation of S or dP).  A unit is a pair of 64-query tiles (qa = 2p, qa + 1) of one
// (batch, head, group), walking key tiles t = 0 .. qa + 1: each step stages the K tile and
// the two dS tiles (t, qa) and (t, qa + 1) (the first absent at t = qa + 1) and forms
// dQ^T += K^T dS^T for both query tiles, so each K tile read serves 128 queries.  One
// persistent workgroup of four waves per CU; wave w owns queries 32 (w % 2) .. + 31 of both
// tiles and head-dim blocks NB/2 (w / 2) ...  The steps of all of a workgroup's units form
// one stream, copied S - 1 steps ahead into a ring of S buffer sets, so the copies of the
// next unit are in flight while one finishes.  Units pair a long and a short query-tile
// pair of one (batch, head, group) (p and np - 1 - p: qa + 2 steps each, sum ntl + 2), and
// each XCD takes a contiguous run of such pairs (K of a few heads stays in its L2).
// The kernel streams dS, about 2 bytes per (query, key) pair: it is bound by HBM.
//
// In LDS, chunk c of a dS tile (fields p, mq, h, g, l as in dsq.h) sits at slot s with
// s bits 0-1 = l bits 0-1, bit 2 = g, bit 3 = h,
// bits 4-6 = l bits 2-4, bit 7 = mq, bit 8 = p: the 32 lanes that one transposed read
// serves together then touch 16 distinct 16-byte slots of one 256-byte bank line.
__device__ __forceinline__ int ds_chunk_of_slot(int s) {
  return (s & 0x180) | (((s >> 3) & 1) << 6) | (((s >> 2) & 1) << 5) | (((s >> 4) & 7) << 2) | (s & 3);
}

// LDS element offset of this lane's first transposed read of a dS tile (K-step 0, keys
// 4g .. 4g + 3, query half mq): source lane t of its 16-lane group points at keys
// 4g + t / 4 and queries 32 mq + 16 (lq / 16) + 4 (t % 4) .. + 3.  The second read (keys
// 8 + 4g ..) adds 256 elements, K-step kb adds 512 (kb % 2) + 2048 (kb / 2).
__device__ __forceinline__ int ds_tr_offset(int lane, int mq) {
  const int lq = lane % 32, g = lane / 32, t = lq & 15;
  const int slot = (t >> 2) | ((t & 1) << 2) | ((lq >> 4) << 3) | (g << 4) | (mq << 7);
  return 8 * slot + 4 * ((t >> 1) & 1);
}

__device__ __forceinline__ bf16x8_t ds_frag(const bf16_t* tile, int off, int kb) {
  const bf16_t* a1 = tile + off + 512 * (kb & 1) + 2048 * (kb >> 1);
  const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t __attribute__((address_space(3)))*)a1);
  const s16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t __attribute__((address_space(3)))*)(a1 + 256));
  const uint2 ux = __builtin_bit_cast(uint2, x), uy = __builtin_bit_cast(uint2, y);
  return as_bf16x8(uint4{ux.x, ux.y, uy.x, uy.y});
}

// wave w's two 16-byte pieces of a dS tile copy (slots 128 w + 64 i + lane)
__device__ __forceinline__ void ds_copy(const bf16_t* src, const int (&co)[2], bf16_t* lds, int w) {
#pragma unroll
  for (int i = 0; i < 2; ++i) load_lds16(src + co[i], lds + (2 * w + i) * 512);
}

// One unit's place in a workgroup's step stream.
struct DqsCur {
  int k, t, n;          // unit index within the workgroup, step, steps of the unit
  int qa;               // first query tile of the pair
  bool two, done;       // second query tile present; stream ended
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
  int ntl, np, nsu, tsu, per, slots;
};

template <int D>
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
    if ((k & 1) && si >= P.np - 1 - si) continue;   // the middle pair runs alone
    const int ngroups = P.N / P.G;
    const int grp = bhg % ngroups, h = (bhg / ngroups) % P.H, b = bhg / (ngroups * P.H);
    c.k = k;
    c.t = 0;
    c.qa = 2 * pair;
    c.two = c.qa + 1 < P.ntl;
    c.n = c.two ? c.qa + 2 : c.qa + 1;
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

template <int D>
__device__ __forceinline__ DqsCur dqs_next(const DqsPlan& P, DqsCur c, int xcd, int slot) {
  if (++c.t < c.n) return c;
  return dqs_unit<D>(P, c.k + 1, xcd, slot);
}

__device__ __forceinline__ int dqs_tok(const DqsCur& c, int N, int tile) {
  const int x = c.gs + kTile * tile + c.sh;
  return x >= N ? x - N : x;
}

// Issue step c's copies (K tile, the dS tiles present) into one buffer set.
template <int D>
__device__ __forceinline__ void dqs_issue(const DqsPlan& P, const DqsCur& c, const CopyOffsets<D, 4>& kco,
                                          const int (&dco)[2], bf16_t* __restrict__ kn, bf16_t* __restrict__ na,
                                          bf16_t* __restrict__ nb, int wu) {
  const long ks = (long)P.Hkv * D;
  copy_tile<D, 4>(c.kb + (long)dqs_tok(c, P.N, c.t) * ks, kco, kn, wu);
  const long ta = (long)c.qa * (c.qa + 1) / 2 + c.t;
  if (c.t <= c.qa) ds_copy(c.dsb + ta * (kTile * kTile), dco, na, wu);
  if (c.two) ds_copy(c.dsb + (ta + c.qa + 1) * (kTile * kTile), dco, nb, wu);
}

template <int D, int NBW>
__device__ __forceinline__ void dqs_compute(const bf16_t* __restrict__ kc, const bf16_t* __restrict__ ca,
                                            const bf16_t* __restrict__ cb, bool da, bool db,
                                            const int (&ko)[NBW][2], int dso, f32x16_t (&aa)[NBW],
                                            f32x16_t (&ab)[NBW]) {
  // an absent tile's buffer is read anyway (in bounds, stale) and masked to zeros: one
  // branch-free path for every step, so all reads can be issued ahead of the products
  const unsigned ma = da ? ~0u : 0u, mb = db ? ~0u : 0u;
  auto masked = [](bf16x8_t x, unsigned m) {
    uint4 u = __builtin_bit_cast(uint4, x);
    u.x &= m;
    u.y &= m;
    u.z &= m;
    u.w &= m;
    return __builtin_bit_cast(bf16x8_t, u);
  };
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    bf16x8_t a[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) a[j] = tr_frag<D>(kc, ko[j], kb);
    const bf16x8_t ba = masked(ds_frag(ca, dso, kb), ma);
    const bf16x8_t bb = masked(ds_frag(cb, dso, kb), mb);
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      aa[j] = mfma32(a[j], ba, aa[j]);
      ab[j] = mfma32(a[j], bb, ab[j]);
    }
  }
}

// One step: issue the copies of step `cp` (if any) into buffer set n, then (when `comp`)
// compute step `cc` from buffer set c.  Every LDS buffer is a restrict parameter of this
// inlined function, and it is the only place copies are issued, so the compiler can tell
// the reads of set c from the copies in flight and does not wait for them.
template <int D, int NBW>
__device__ __forceinline__ void dqs_step(const DqsPlan& P, const DqsCur& cc, const DqsCur& cp, bool comp,
                                         const bf16_t* __restrict__ kc, const bf16_t* __restrict__ ca,
                                         const bf16_t* __restrict__ cb, bf16_t* __restrict__ kn,
                                         bf16_t* __restrict__ na, bf16_t* __restrict__ nb,
                                         const CopyOffsets<D, 4>& kco, const int (&dco)[2], const int (&ko)[NBW][2],
                                         int dso, f32x16_t (&aa)[NBW], f32x16_t (&ab)[NBW], int wu) {
  if (!cp.done) dqs_issue<D>(P, cp, kco, dco, kn, na, nb, wu);
  if (!comp) return;
  dqs_compute<D, NBW>(kc, ca, cb, cc.t <= cc.qa, cc.two, ko, dso, aa, ab);
}

// Wait until at most N vector memory operations of this wave are outstanding and all its
// LDS reads have returned (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14, lgkmcnt 11:8),
// then meet the other waves at a barrier.  No memory fence: the LDS buffers are written
// only by direct copies, which the vmcnt wait covers, and a fence would wait for every
// copy in flight.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
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

#ifndef S2A_DQS_STAGES
#define S2A_DQS_STAGES 4
#endif
constexpr int kDqsStages = S2A_DQS_STAGES;

template <int D>
__global__ __launch_bounds__(256) void dqs_kernel(DqsPlan P, float scale) {
  constexpr int NW = 4, NB = D / 32, NBW = NB / 2, S = kDqsStages;
  // copies per wave per step: the K tile's, plus at least one dS tile's two
  constexpr int LMIN = CopyOffsets<D, NW>::PER + 2;
  static_assert(S >= 2 && S <= 5 && (S - 2) * LMIN < 64, "the waits below cover up to three steps ahead");
  __shared__ __align__(16) bf16_t ks[S][kTile * D];
  __shared__ __align__(16) bf16_t ds[S][2][kTile * kTile];
  const int tid = thread_x(), w = tid / 64, lane = tid % 64;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int mq = wu % 2, nb0 = NBW * (wu / 2);
  const int xcd = group_x() % 8, slot = group_x() / 8;
  const CopyOffsets<D, NW> kco = copy_offsets<D, NW>(wu, lane, (long)P.Hkv * D);
  int dco[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) dco[i] = 8 * ds_chunk_of_slot((2 * wu + i) * 64 + lane);
  int ko[NBW][2];
#pragma unroll
  for (int j = 0; j < NBW; ++j) tr_offsets_block<D>(lane, nb0 + j, ko[j]);
  const int dso = ds_tr_offset(lane, mq);
  f32x16_t aa[NBW], ab[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) aa[j] = ab[j] = f32x16_t{};

  DqsCur cc = dqs_unit<D>(P, 0, xcd, slot);
  DqsCur cp = cc;
  int issued = 0;
  // iterations s < 0 only issue copies (the first S - 1 steps)
  for (int s = 1 - S; !cc.done; ++s) {
    if (s >= 0) {
      // this wave's copies of step s have landed once at most those of the steps issued
      // after it (at least LMIN each) are outstanding; the barrier then makes every
      // wave's copies visible and frees the set step s - 1 used
      const int ahead = issued - s - 1;   // at most S - 2
      if (ahead >= 3) wait_vm_barrier<3 * LMIN>();
      else if (ahead == 2) wait_vm_barrier<2 * LMIN>();
      else if (ahead == 1) wait_vm_barrier<LMIN>();
      else wait_vm_barrier<0>();
    }
    const int c = (s + S) % S, n = (s + S - 1) % S;
    dqs_step<D, NBW>(P, cc, cp, s >= 0, ks[c], ds[c][0], ds[c][1], ks[n], ds[n][0], ds[n][1], kco, dco, ko, dso, aa,
                     ab, wu);
    if (!cp.done) {
      ++issued;
      cp = dqs_next<D>(P, cp, xcd, slot);
    }
    if (s < 0) continue;
    if (cc.t == cc.n - 1) {
      dqs_store<D, NBW>(cc, P.N, P.H, cc.qa, aa, nb0, mq, lane, scale);
      if (cc.two) dqs_store<D, NBW>(cc, P.N, P.H, cc.qa + 1, ab, nb0, mq, lane, scale);
    }
    cc = dqs_next<D>(P, cc, xcd, slot);
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
  p.np = (p.ntl + 1) / 2;
  p.nsu = (p.np + 1) / 2;
  p.tsu = B * H * (N / G) * p.nsu;
  p.per = (p.tsu + 7) / 8;
  p.slots = std::min(p.per, resident_per_xcd(1));
  if (d == 128) hipLaunchKernelGGL((dqs_kernel<128>), dim3(8 * p.slots), dim3(256), 0, st, p, scale);
  else hipLaunchKernelGGL((dqs_kernel<64>), dim3(8 * p.slots), dim3(256), 0, st, p, scale);
}

}  // namespace s2a
