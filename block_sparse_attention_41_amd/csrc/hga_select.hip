// HGA chunk summaries and per-query-block chunk selection.
//
// "Long-Context Fine-Tuning with Limited VRAM" (BMW Group, English abstract) keeps
// resident chunk summaries and, for each query block, loads a bounded set of exact
// historical tokens.  Here the summary is the mean key of a chunk per kv head, and a
// block picks the top-k chunks by the dot product of its mean query with the summaries
// (ties to the lower chunk index), reported ascending with -1 padding.
#include "../../include/s2a.h"
#include "common.h"
#include "validate.h"

namespace s2a {

// ---------------------------------------------------------------------------------------
// Summaries: grid (C, column blocks, B), 256 threads = 64 column groups of 8 elements x 4
// token phases.  A wave reads 64 consecutive 16-byte pieces of one token row (coalesced);
// the four phases are combined through LDS.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void hga_summarize_kernel(const bf16_t* __restrict__ kh, long hbs,
                                                             float* __restrict__ summ, long sbs, int W, int chunk) {
  __shared__ float part[3][64][9];
  const int c = group_x(), b = group_z();
  const int tid = thread_x(), cgl = tid % 64, phase = tid / 64;
  const int cg = group_y() * 64 + cgl;
  const bool valid = cg * 8 < W;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (valid) {
    const bf16_t* base = kh + b * hbs + ((long)c * chunk) * W + cg * 8;
    int t = phase;
    for (; t + 12 < chunk; t += 16) {
      uint4 u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) u[i] = load16(base + (long)(t + 4 * i) * W);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t wv[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += bf16_lo(wv[e]);
          acc[2 * e + 1] += bf16_hi(wv[e]);
        }
      }
    }
    for (; t < chunk; t += 4) {
      const uint4 u = load16(base + (long)t * W);
      const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_lo(wv[e]);
        acc[2 * e + 1] += bf16_hi(wv[e]);
      }
    }
  }
  if (phase > 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) part[phase - 1][cgl][e] = acc[e];
  }
  __syncthreads();
  if (phase == 0 && valid) {
    const float inv = 1.f / (float)chunk;
    float out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (((acc[e] + part[0][cgl][e]) + part[1][cgl][e]) + part[2][cgl][e]) * inv;
    float4* dst = reinterpret_cast<float4*>(summ + b * sbs + (long)c * W + cg * 8);
    dst[0] = make_float4(out[0], out[1], out[2], out[3]);
    dst[1] = make_float4(out[4], out[5], out[6], out[7]);
  }
}

// ---------------------------------------------------------------------------------------
// History append: a finished segment's keys and values are copied (detached) into the
// history buffer behind its first T tokens, and the summaries of the segment's chunks are
// written in the same pass over the keys.  Same grid and thread layout as the summaries:
// (S/chunk, column blocks, B); each thread copies its 16-byte pieces of K and V and sums
// the K pieces.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void hga_append_kernel(const bf16_t* __restrict__ ks, const bf16_t* __restrict__ vs,
                                                          long sbs, bf16_t* __restrict__ kh, bf16_t* __restrict__ vh,
                                                          long hbs, float* __restrict__ summ, long smbs, int W,
                                                          int chunk, int T) {
  __shared__ float part[3][64][9];
  const int c = group_x(), b = group_z();
  const int tid = thread_x(), cgl = tid % 64, phase = tid / 64;
  const int cg = group_y() * 64 + cgl;
  const bool valid = cg * 8 < W;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (valid) {
    const long src = b * sbs + ((long)c * chunk) * W + cg * 8;
    const long dst = b * hbs + ((long)T + (long)c * chunk) * W + cg * 8;
    for (int t = phase; t < chunk; t += 4) {
      const uint4 uk = load16(ks + src + (long)t * W);
      const uint4 uv = load16(vs + src + (long)t * W);
      *reinterpret_cast<uint4*>(kh + dst + (long)t * W) = uk;
      *reinterpret_cast<uint4*>(vh + dst + (long)t * W) = uv;
      const uint32_t wv[4] = {uk.x, uk.y, uk.z, uk.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_lo(wv[e]);
        acc[2 * e + 1] += bf16_hi(wv[e]);
      }
    }
  }
  if (phase > 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) part[phase - 1][cgl][e] = acc[e];
  }
  __syncthreads();
  if (phase == 0 && valid) {
    const float inv = 1.f / (float)chunk;
    float out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (((acc[e] + part[0][cgl][e]) + part[1][cgl][e]) + part[2][cgl][e]) * inv;
    float4* d4 = reinterpret_cast<float4*>(summ + b * smbs + ((long)T / chunk + c) * W + cg * 8);
    d4[0] = make_float4(out[0], out[1], out[2], out[3]);
    d4[1] = make_float4(out[4], out[5], out[6], out[7]);
  }
}

// ---------------------------------------------------------------------------------------
// Selection: one wave per (q head, query block) row; the 4 waves of a workgroup share a
// kv head, so each tile of 64 summaries is staged in LDS once for all of them.
// Top-k runs as a wavefront bitonic network on 64-bit keys (orderable score bits above
// the complemented chunk index, so larger key = higher score, then lower index): each
// tile of 64 candidates is sorted, merged with the running best 64 (elementwise max
// against the reversed list keeps the top 64 of the union as a bitonic sequence), and the
// merge is re-sorted.
// ---------------------------------------------------------------------------------------
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

template <int D>
__global__ __launch_bounds__(256) void hga_select_kernel(const bf16_t* __restrict__ q, const float* __restrict__ summ,
                                                          long sbs, int32_t* __restrict__ idx, int S, int H, int Hkv,
                                                          int C, int topk, int grouped) {
  // row stride D + 4 floats: 16-byte aligned rows whose float4 reads by 64 lanes (one row
  // each) fall on distinct bank groups
  __shared__ __align__(16) float st[kTile][D + 4];
  __shared__ __align__(16) float qbar[4][D];
  const int b = group_z(), kvh = group_y();
  const int rep = H / Hkv, nqb = S / 64;
  const int tid = thread_x(), w = tid / 64, lane = tid % 64;
  // a row is one (q head, query block), four per workgroup (one per wave); with `grouped`
  // one (kv head, query block) per workgroup, scored with the sum of the block means of
  // the kv head's q heads: wave w forms the means of heads w, w + 4, ... and wave 0 adds
  // the four partial sums and scores
  const int row = grouped ? group_x() : group_x() * 4 + w;
  const bool in = row < (grouped ? 1 : rep) * nqb;
  const bool active = in && (!grouped || w == 0);
  const int j = grouped ? row : row / rep;
  const int h = kvh * rep + (grouped ? 0 : row % rep);

  // mean query of the block, one or two elements per lane
  constexpr int EPL = D / 64;
  if (in && C > 0) {
    float a[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) a[e] = 0.f;
    const long step = (long)H * D;
    for (int e2 = grouped ? w : 0; e2 < (grouped ? rep : 1); e2 += 4) {
      const bf16_t* base = q + (((long)b * S + 64 * j) * H + h + e2) * D + lane * EPL;
#pragma unroll 8
      for (int t = 0; t < 64; ++t) {
        if constexpr (EPL == 2) {
          const uint32_t u = *reinterpret_cast<const uint32_t*>(base + t * step);
          a[0] += bf16_lo(u);
          a[1] += bf16_hi(u);
        } else {
          a[0] += __builtin_bit_cast(float, (uint32_t)base[t * step] << 16);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) qbar[w][lane * EPL + e] = a[e] * (1.f / 64.f);
  }

  unsigned long long best = 0ull;
  const float* sb = summ + b * sbs + (long)kvh * D;
  // summaries of chunks c0 .. c0+63, float4 pieces: the next tile's loads are in flight
  // while this tile is scored and merged
  constexpr int PT = kTile * (D / 4) / 256;
  float4 pf[PT];
  auto load_tile = [&](int c0) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int x = tid + 256 * i, r = x / (D / 4), col = (x % (D / 4)) * 4;
      pf[i] = (c0 + r < C) ? *reinterpret_cast<const float4*>(sb + (long)(c0 + r) * Hkv * D + col)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  if (C > 0) load_tile(0);
  for (int c0 = 0; c0 < C; c0 += kTile) {
    __syncthreads();   // the previous tile's reads are done
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int x = tid + 256 * i, r = x / (D / 4), col = (x % (D / 4)) * 4;
      *reinterpret_cast<float4*>(&st[r][col]) = pf[i];
    }
    __syncthreads();
    if (c0 + kTile < C) load_tile(c0 + kTile);
    if (active) {
      float sc = 0.f;
#pragma unroll 8
      for (int e = 0; e < D; e += 4) {
        float4 a = *reinterpret_cast<const float4*>(&qbar[w][e]);
        if (grouped) {
#pragma unroll
          for (int p = 1; p < 4; ++p) {
            const float4 x = *reinterpret_cast<const float4*>(&qbar[p][e]);
            a.x += x.x;
            a.y += x.y;
            a.z += x.z;
            a.w += x.w;
          }
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
      best = bitonic_merge_desc(best, lane);
    }
  }
  if (active) {
    const int keff = min(topk, C);
    // the chosen chunk indices, sorted ascending (unused lanes sort to the end)
    const uint32_t cidx = ~(uint32_t)(best & 0xffffffffull);
    unsigned long long key2 = (lane < keff && best != 0ull) ? (unsigned long long)cidx : ~0ull;
    // ascending sort == descending sort of the complement
    key2 = ~bitonic_sort_desc(~key2, lane);
    if (lane < topk) {
      const int out = (lane < keff) ? (int)key2 : -1;
      const long ih = grouped ? (long)b * Hkv + kvh : (long)b * H + h;
      idx[(ih * nqb + j) * topk + lane] = out;
    }
  }
}

}  // namespace s2a

using namespace s2a;

extern "C" int hga_summarize(const void* k_hist, long long hist_bstride, float* summ, long long summ_bstride, int B,
                             int T, int Hkv, int d, int chunk, void* stream) {
  if (B <= 0 || T < 0 || Hkv <= 0 || d <= 0 || chunk <= 0) return S2A_ERR_INVALID_ARG;
  if (T % chunk) return S2A_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return S2A_ERR_UNSUPPORTED;
  if (chunk % 64) return S2A_ERR_UNSUPPORTED;
  if (T == 0) return S2A_OK;
  if (!ptr_ok(k_hist) || !ptr_ok(summ)) return S2A_ERR_INVALID_ARG;
  const int C = T / chunk;
  if (!stride_ok(hist_bstride, T, Hkv, d, B) || !stride_ok(summ_bstride, C, Hkv, d, B)) return S2A_ERR_INVALID_ARG;
  if (B > 1 && (hist_bstride % 8 || summ_bstride % 4)) return S2A_ERR_INVALID_ARG;
  const int W = Hkv * d;
  dim3 grid(C, (W / 8 + 63) / 64, B), block(256);
  hipLaunchKernelGGL(hga_summarize_kernel, grid, block, 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const bf16_t*>(k_hist), (long)hist_bstride, summ, (long)summ_bstride, W, chunk);
  return hipGetLastError() == hipSuccess ? S2A_OK : S2A_ERR_HIP;
}

extern "C" int hga_append_history(const void* k_seg, const void* v_seg, long long seg_bstride, void* k_hist,
                                  void* v_hist, long long hist_bstride, float* summ, long long summ_bstride, int B,
                                  int S, int Hkv, int d, int T, int chunk, void* stream) {
  if (B <= 0 || S < 0 || T < 0 || Hkv <= 0 || d <= 0 || chunk <= 0) return S2A_ERR_INVALID_ARG;
  if (S % chunk || T % chunk) return S2A_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return S2A_ERR_UNSUPPORTED;
  if (chunk % 64) return S2A_ERR_UNSUPPORTED;
  if (S == 0) return S2A_OK;
  if (!ptr_ok(k_seg) || !ptr_ok(v_seg) || !ptr_ok(k_hist) || !ptr_ok(v_hist) || !ptr_ok(summ))
    return S2A_ERR_INVALID_ARG;
  const long long C = (long long)(T + S) / chunk;
  if (!stride_ok(seg_bstride, S, Hkv, d, B) || !stride_ok(hist_bstride, (long long)T + S, Hkv, d, B) ||
      !stride_ok(summ_bstride, C, Hkv, d, B))
    return S2A_ERR_INVALID_ARG;
  if (B > 1 && (seg_bstride % 8 || hist_bstride % 8 || summ_bstride % 4)) return S2A_ERR_INVALID_ARG;
  if (((long long)T + S) * Hkv * d >= (1ll << 31)) return S2A_ERR_UNSUPPORTED;
  const int W = Hkv * d;
  dim3 grid(S / chunk, (W / 8 + 63) / 64, B), block(256);
  hipLaunchKernelGGL(hga_append_kernel, grid, block, 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const bf16_t*>(k_seg), static_cast<const bf16_t*>(v_seg), (long)seg_bstride,
                     static_cast<bf16_t*>(k_hist), static_cast<bf16_t*>(v_hist), (long)hist_bstride, summ,
                     (long)summ_bstride, W, chunk, T);
  return hipGetLastError() == hipSuccess ? S2A_OK : S2A_ERR_HIP;
}

static int hga_select_impl(const void* q, const float* summ, long long summ_bstride, int32_t* idx, int B, int S,
                               int H, int Hkv, int d, int C, int qblock, int topk, void* stream, bool grouped) {
  int st = check_common_heads(B, S, H, Hkv, d);
  if (st) return st;
  if (C < 0 || qblock <= 0 || topk <= 0 || S % qblock) return S2A_ERR_INVALID_ARG;
  if (qblock != 64 || topk > 64) return S2A_ERR_UNSUPPORTED;
  if (!ptr_ok(q) || !ptr_ok(idx) || (C > 0 && !ptr_ok(summ))) return S2A_ERR_INVALID_ARG;
  if (C > 0 && !stride_ok(summ_bstride, C, Hkv, d, B)) return S2A_ERR_INVALID_ARG;
  if (B > 1 && summ_bstride % 4) return S2A_ERR_INVALID_ARG;
  const int rows = (grouped ? 1 : H / Hkv) * (S / 64);
  dim3 grid(grouped ? rows : (rows + 3) / 4, Hkv, B), block(256);
  hipStream_t sm = reinterpret_cast<hipStream_t>(stream);
  auto qp = static_cast<const bf16_t*>(q);
  if (d == 128)
    hipLaunchKernelGGL((hga_select_kernel<128>), grid, block, 0, sm, qp, summ, (long)summ_bstride, idx, S, H, Hkv, C,
                       topk, (int)grouped);
  else
    hipLaunchKernelGGL((hga_select_kernel<64>), grid, block, 0, sm, qp, summ, (long)summ_bstride, idx, S, H, Hkv, C,
                       topk, (int)grouped);
  return hipGetLastError() == hipSuccess ? S2A_OK : S2A_ERR_HIP;
}

extern "C" int hga_select_topk(const void* q, const float* summ, long long summ_bstride, int32_t* idx, int B, int S,
                               int H, int Hkv, int d, int C, int qblock, int topk, void* stream) {
  return hga_select_impl(q, summ, summ_bstride, idx, B, S, H, Hkv, d, C, qblock, topk, stream, false);
}

extern "C" int hga_select_topk_shared(const void* q, const float* summ, long long summ_bstride, int32_t* idx, int B,
                                      int S, int H, int Hkv, int d, int C, int qblock, int topk, void* stream) {
  return hga_select_impl(q, summ, summ_bstride, idx, B, S, H, Hkv, d, C, qblock, topk, stream, true);
}
