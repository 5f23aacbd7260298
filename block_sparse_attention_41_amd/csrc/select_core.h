// Chunk selection building blocks ("Long-Context Fine-Tuning with Limited VRAM", BMW
// Group, English abstract: each query block attends to a capped number of whole history
// chunks, chosen with the help of per-chunk summaries), shared by the selection kernel and
// the forward that selects its own chunks, so both choose with the same arithmetic in the
// same order and get the same bits.
//
// Score of chunk c for a list: (mean of the list's queries) . summary[c]; a list is one q
// head's query block, or one kv head's query block with the block means of its q heads
// summed.  Top-k runs as a wavefront bitonic network on 64-bit keys (orderable score bits
// above the complemented chunk index, so a larger key is a higher score, then a lower
// index): each tile of 64 candidates is sorted, merged with the running best 64
// (elementwise max against the reversed list keeps the top 64 of the union as a bitonic
// sequence), and the merge is re-sorted.
#pragma once

#include "common.h"

namespace s2a {

__device__ __forceinline__ uint32_t orderable(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The key of lane l ^ J.  Within a row of 16 lanes this is a DPP move on the vector ALU
// (quad permutations for J = 1, 2; for J = 4, 8 a row shift down for lanes whose bit J is
// clear and up for the others); across rows a bpermute through the LDS unit.
template <int J>
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t x, int lane) {
  if constexpr (J == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  } else if constexpr (J == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  } else if constexpr (J == 4 || J == 8) {
    const uint32_t up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x100 + J, 0xF, 0xF, false);   // lane + J
    const uint32_t dn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x110 + J, 0xF, 0xF, false);   // lane - J
    return (lane & J) ? dn : up;
  } else {
    return (uint32_t)__shfl_xor((int)x, J);
  }
}

template <int J>
__device__ __forceinline__ unsigned long long xor_lane(unsigned long long key, int lane) {
  const uint32_t lo = xor_lane_u32<J>((uint32_t)key, lane), hi = xor_lane_u32<J>((uint32_t)(key >> 32), lane);
  return ((unsigned long long)hi << 32) | lo;
}

template <int J>
__device__ __forceinline__ unsigned long long bitonic_stage(unsigned long long key, int lane, int k) {
  const unsigned long long o = xor_lane<J>(key, lane);
  const bool up = (lane & k) != 0;        // the final k = 64 stage sorts descending
  const bool lower = (lane & J) == 0;
  const bool take_min = (lower == up);
  return take_min ? (o < key ? o : key) : (o > key ? o : key);
}

__device__ __forceinline__ unsigned long long bitonic_sort_desc(unsigned long long key, int lane) {
  key = bitonic_stage<1>(key, lane, 2);
  key = bitonic_stage<2>(key, lane, 4);
  key = bitonic_stage<1>(key, lane, 4);
  key = bitonic_stage<4>(key, lane, 8);
  key = bitonic_stage<2>(key, lane, 8);
  key = bitonic_stage<1>(key, lane, 8);
  key = bitonic_stage<8>(key, lane, 16);
  key = bitonic_stage<4>(key, lane, 16);
  key = bitonic_stage<2>(key, lane, 16);
  key = bitonic_stage<1>(key, lane, 16);
  key = bitonic_stage<16>(key, lane, 32);
  key = bitonic_stage<8>(key, lane, 32);
  key = bitonic_stage<4>(key, lane, 32);
  key = bitonic_stage<2>(key, lane, 32);
  key = bitonic_stage<1>(key, lane, 32);
  key = bitonic_stage<32>(key, lane, 64);
  key = bitonic_stage<16>(key, lane, 64);
  key = bitonic_stage<8>(key, lane, 64);
  key = bitonic_stage<4>(key, lane, 64);
  key = bitonic_stage<2>(key, lane, 64);
  key = bitonic_stage<1>(key, lane, 64);
  return key;
}

template <int J>
__device__ __forceinline__ unsigned long long merge_stage(unsigned long long key, int lane) {
  const unsigned long long o = xor_lane<J>(key, lane);
  const bool lower = (lane & J) == 0;
  return lower ? (o > key ? o : key) : (o < key ? o : key);
}

__device__ __forceinline__ unsigned long long bitonic_merge_desc(unsigned long long key, int lane) {
  key = merge_stage<32>(key, lane);
  key = merge_stage<16>(key, lane);
  key = merge_stage<8>(key, lane);
  key = merge_stage<4>(key, lane);
  key = merge_stage<2>(key, lane);
  key = merge_stage<1>(key, lane);
  return key;
}

// Mean of one q head's 64-query block (`base` = its first row, rows `step` elements
// apart), float32, with whole rows in flight: lane (p, piece) = (lane / PPR, lane % PPR)
// reads the 16-byte piece `piece` (elements 8 piece .. 8 piece + 7) of rows p, p + NPH,
// ... (PPR = D / 8 pieces per row, NPH = 64 / PPR row phases), all loads issued before
// any is used; the phase sums (each in row order) are then added across the phases by
// xor-shuffles, first partners PPR apart, then 2 PPR, ... (float addition commutes, so
// both partners get the same bits).  Every lane returns the mean of its piece's eight
// columns.
template <int D>
__device__ __forceinline__ void block_mean_rows(const bf16_t* base, long step, int lane, float (&m)[8]) {
  constexpr int PPR = D / 8, NPH = 64 / PPR, RPP = 64 / NPH;
  const int p = lane / PPR, piece = lane % PPR;
  uint4 u[RPP];
#pragma unroll
  for (int i = 0; i < RPP; ++i) u[i] = *reinterpret_cast<const uint4*>(base + (long)(p + NPH * i) * step + 8 * piece);
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = 0.f;
#pragma unroll
  for (int i = 0; i < RPP; ++i) {
    const uint32_t wv[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m[2 * e] += bf16_lo(wv[e]);
      m[2 * e + 1] += bf16_hi(wv[e]);
    }
  }
#pragma unroll
  for (int x = PPR; x < 64; x *= 2)
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = m[e] + __shfl_xor(m[e], x);
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] *= (1.f / 64.f);
}

// One tile of 64 summaries (chunks c0 .. c0 + 63, rows `rstride` floats apart), staged
// through registers into LDS rows of D + 4 floats (16-byte aligned rows whose float4
// reads by 64 lanes, one row each, fall on distinct bank groups) by the NT threads of the
// workgroup.  Chunks at or past C read as zeros.
template <int D, int NT>
struct SummaryTile {
  static constexpr int PT = kTile * (D / 4) / NT;
  float4 pf[PT];
  __device__ __forceinline__ void load(const float* sb, long rstride, int c0, int C, int tid) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int x = tid + NT * i, r = x / (D / 4), col = (x % (D / 4)) * 4;
      pf[i] = (c0 + r < C) ? *reinterpret_cast<const float4*>(sb + (long)(c0 + r) * rstride + col)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ void store(float (*st)[D + 4], int tid) const {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int x = tid + NT * i, r = x / (D / 4), col = (x % (D / 4)) * 4;
      *reinterpret_cast<float4*>(&st[r][col]) = pf[i];
    }
  }
};

// Scores the staged tile for one list (lane = chunk c0 + lane) and merges them into the
// running best 64.  The list's query is qbar[0], or with `ngroup` > 1 the sum of qbar[0..
// ngroup-1] (added in that order, element by element).
template <int D>
__device__ __forceinline__ unsigned long long score_merge(const float (*qbar)[D], int ngroup,
                                                          const float (*st)[D + 4], int c0, int C,
                                                          unsigned long long best, int lane) {
  float sc = 0.f;
#pragma unroll 8
  for (int e = 0; e < D; e += 4) {
    float4 a = *reinterpret_cast<const float4*>(&qbar[0][e]);
    for (int p = 1; p < ngroup; ++p) {
      const float4 x = *reinterpret_cast<const float4*>(&qbar[p][e]);
      a.x += x.x;
      a.y += x.y;
      a.z += x.z;
      a.w += x.w;
    }
    const float4 t = *reinterpret_cast<const float4*>(&st[lane][e]);
    sc = __builtin_fmaf(a.x, t.x, sc);
    sc = __builtin_fmaf(a.y, t.y, sc);
    sc = __builtin_fmaf(a.z, t.z, sc);
    sc = __builtin_fmaf(a.w, t.w, sc);
  }
  const int cidx = c0 + lane;
  unsigned long long key = 0ull;
  if (cidx < C) key = ((unsigned long long)orderable(sc) << 32) | (unsigned long long)(~(uint32_t)cidx);
  key = bitonic_sort_desc(key, lane);
  const unsigned long long rev = __shfl(key, 63 - lane);
  best = best > rev ? best : rev;
  return bitonic_merge_desc(best, lane);
}

// The same scoring and merge for chunks c0 .. c0 + 63 with each lane reading its own
// chunk's summary row (row c at sb + c * rstride) from memory instead of a staged tile,
// so that several waves can score different tiles at once; `qs` is the list's query in
// LDS (for several q heads, their block means already summed in order 0, 1, ...).  Every
// score is the same chain of fused multiply-adds as score_merge's, so the same bits.
template <int D>
__device__ __forceinline__ unsigned long long score_merge_rows(const float* qs, const float* sb, long rstride,
                                                               int c0, int C, unsigned long long best, int lane) {
  const int cidx = c0 + lane;
  unsigned long long key = 0ull;
  if (cidx < C) {
    const float* row = sb + (long)cidx * rstride;
    float sc = 0.f;
#pragma unroll 8
    for (int e = 0; e < D; e += 4) {
      const float4 a = *reinterpret_cast<const float4*>(qs + e);
      const float4 t = *reinterpret_cast<const float4*>(row + e);
      sc = __builtin_fmaf(a.x, t.x, sc);
      sc = __builtin_fmaf(a.y, t.y, sc);
      sc = __builtin_fmaf(a.z, t.z, sc);
      sc = __builtin_fmaf(a.w, t.w, sc);
    }
    key = ((unsigned long long)orderable(sc) << 32) | (unsigned long long)(~(uint32_t)cidx);
  }
  key = bitonic_sort_desc(key, lane);
  const unsigned long long rev = __shfl(key, 63 - lane);
  best = best > rev ? best : rev;
  return bitonic_merge_desc(best, lane);
}

// Merges another wave's running best 64 (sorted descending, `other` = its entry `lane`)
// into `best`: the top 64 of a set of distinct keys does not depend on the order in
// which its parts were merged, so tiles can be scored by different waves.
__device__ __forceinline__ unsigned long long merge_best(unsigned long long best, unsigned long long other_rev,
                                                         int lane) {
  best = best > other_rev ? best : other_rev;
  return bitonic_merge_desc(best, lane);
}

// Entry `lane` of the final list: the chosen chunk indices in ascending order (unused
// lanes sort to the end), -1 past k_eff = min(topk, C).
__device__ __forceinline__ int final_entry(unsigned long long best, int C, int topk, int lane) {
  const int keff = min(topk, C);
  const uint32_t cidx = ~(uint32_t)(best & 0xffffffffull);
  unsigned long long key2 = (lane < keff && best != 0ull) ? (unsigned long long)cidx : ~0ull;
  // ascending sort == descending sort of the complement
  key2 = ~bitonic_sort_desc(~key2, lane);
  return (lane < keff) ? (int)key2 : -1;
}

}  // namespace s2a
