// HGA chunk summaries and per-query-block chunk selection.
//
// "Long-Context Fine-Tuning with Limited VRAM" (BMW Group, English abstract) keeps one
// summary per history chunk in memory and lets every query block attend to a capped
// number of whole history chunks.  Here the summary is the mean key of a chunk per kv head, and a
// block picks the top-k chunks by the dot product of its mean query with the summaries
// (ties to the lower chunk index), reported ascending with -1 padding.
#include "../../include/s2a.h"
#include "common.h"
#include "select_core.h"
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
// kv head, so each tile of 64 summaries is staged in LDS once for all of them.  With
// `grouped`, one (kv head, query block) row per workgroup, scored with the sum of the
// block means of the kv head's q heads: wave w forms the means of heads w, w + 4, ...,
// wave 0 adds the four partial sums once, wave w scores tiles w, w + 4, ... reading the
// summary rows itself, and wave 0 merges the four running lists (select_core.h).
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void hga_select_kernel(const bf16_t* __restrict__ q, const float* __restrict__ summ,
                                                          long sbs, int32_t* __restrict__ idx, int S, int H, int Hkv,
                                                          int C, int topk, int grouped) {
  __shared__ __align__(16) float st[kTile][D + 4];
  __shared__ __align__(16) float qbar[4][D];
  const int b = group_z(), kvh = group_y();
  const int rep = H / Hkv, nqb = S / 64;
  const int tid = thread_x(), w = tid / 64, lane = tid % 64;
  const int row = grouped ? group_x() : group_x() * 4 + w;
  const bool in = row < (grouped ? 1 : rep) * nqb;
  const bool active = in && (!grouped || w == 0);
  const int j = grouped ? row : row / rep;
  const int h = kvh * rep + (grouped ? 0 : row % rep);

  // per-head rows: the first summary tile's loads go out before the query rows', so the
  // two reads from HBM overlap
  const float* sb = summ + b * sbs + (long)kvh * D;
  SummaryTile<D, 256> tile;
  if (!grouped && C > 0) tile.load(sb, (long)Hkv * D, 0, C, tid);
  if (in && C > 0) {
    const long step = (long)H * D;
    // rep q heads summed in four wave slots: slot w holds heads w, w + 4, ... (one head
    // per wave without `grouped`)
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int e2 = grouped ? w : 0; e2 < (grouped ? rep : 1); e2 += 4) {
      float m[8];
      block_mean_rows<D>(q + (((long)b * S + 64 * j) * H + h + e2) * D, step, lane, m);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += m[e];
    }
    if (lane < D / 8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qbar[w][8 * lane + e] = acc[e];
    }
  }

  if (grouped) {
    float* qs = &st[0][0];
    unsigned long long(*bests)[64] = reinterpret_cast<unsigned long long(*)[64]>(&st[8][0]);
    __syncthreads();
    if (in && C > 0 && w == 0) {
      const int ng = min(rep, 4);
      for (int e = lane; e < D; e += 64) {
        float a = qbar[0][e];
        for (int p = 1; p < ng; ++p) a += qbar[p][e];
        qs[e] = a;
      }
    }
    __syncthreads();
    unsigned long long gbest = 0ull;
    if (in)
      for (int c0 = kTile * w; c0 < C; c0 += 4 * kTile)
        gbest = score_merge_rows<D>(qs, sb, (long)Hkv * D, c0, C, gbest, lane);
    bests[w][63 - lane] = gbest;   // reversed, ready for merge_best
    __syncthreads();
    if (in && w == 0) {
      for (int x = 1; x < 4 && kTile * x < C; ++x) gbest = merge_best(gbest, bests[x][lane], lane);
      const int out = final_entry(gbest, C, topk, lane);
      if (lane < topk) idx[(((long)b * Hkv + kvh) * nqb + j) * topk + lane] = out;
    }
    return;
  }

  unsigned long long best = 0ull;
  // the next tile's loads are in flight while this tile is scored and merged
  for (int c0 = 0; c0 < C; c0 += kTile) {
    __syncthreads();   // the previous tile's reads are done
    tile.store(st, tid);
    __syncthreads();
    if (c0 + kTile < C) tile.load(sb, (long)Hkv * D, c0 + kTile, C, tid);
    if (active) best = score_merge<D>(qbar + w, 1, st, c0, C, best, lane);
  }
  if (active) {
    const int out = final_entry(best, C, topk, lane);
    if (lane < topk) idx[(((long)b * H + h) * nqb + j) * topk + lane] = out;
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
