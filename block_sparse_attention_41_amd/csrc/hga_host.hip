// Host-tier history for HGA.
//
// "Long-Context Fine-Tuning with Limited VRAM" (BMW Group, English abstract) moves the
// older key/value rows out of GPU memory into host RAM (or NVMe); each query block then
// needs only the few whole history chunks selected for it.  Here the older rows live in
// pinned host memory that the GPU reads and writes directly over the host link, while the
// per-chunk mean keys stay in HBM so that selection never touches host memory.  One
// segment goes through:
//   1. hga_detach_segment: the finished segment's K/V rows are written into the host
//      history and its chunk summaries into the HBM table (one kernel);
//   2. hga_select_topk(_shared): chunk lists from the HBM summaries;
//   3. hga_stage_selected: per (batch, kv head), the union of the chunks its lists name is
//      gathered from host memory into an HBM staging history, and the lists are rewritten
//      to staging slots (a plan kernel, then a gather kernel); or hga_stage_update, which
//      keeps the staging history as a cache and gathers only the chunks it does not hold;
//   4. the attention kernels run on the staging history as on a resident one.
// Every rewritten list keeps its entry order and every slot holds its chunk's exact rows,
// so the attention sees the same tiles in the same order as on the resident history and
// gives the same bits, whichever slot a chunk sits in.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "../../include/s2a.h"
#include "common.h"
#include "validate.h"

namespace s2a {

constexpr int kStageWords = S2A_STAGE_MAX_CHUNKS / 32;

// ---------------------------------------------------------------------------------------
// Plan: one workgroup per (kv head, batch).  The chunks named by the kv head's lists are
// marked in an LDS bitmap; a prefix count over the bitmap gives each marked chunk its slot
// (ascending chunk order), which is written to chunk_of and used to rewrite the lists.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void stage_plan_kernel(const int32_t* __restrict__ idx, int lists, int nqb,
                                                         int topk, int Hkv, int C, int max_slots,
                                                         int32_t* __restrict__ chunk_of, int32_t* __restrict__ count,
                                                         int32_t* __restrict__ idx_staged) {
  __shared__ uint32_t bits[kStageWords];
  __shared__ int pre[kStageWords];
  __shared__ int part[256];
  const int h = group_x(), b = group_y(), tid = thread_x();
  const int W = (C + 31) / 32;
  const int rep = lists / Hkv;   // lists per kv head: its q heads, or 1 for shared lists
  const long n = (long)rep * nqb * topk;
  const long base = ((long)b * lists + (long)h * rep) * nqb * topk;
  for (int w = tid; w < W; w += 256) bits[w] = 0u;
  __syncthreads();
  for (long i = tid; i < n; i += 256) {
    const int c = idx[base + i];
    if (c >= 0 && c < C) atomicOr(&bits[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  // thread t counts the marked chunks of words [t * per, (t + 1) * per); an inclusive scan
  // over the 256 counts gives every word the number of marked chunks before it
  const int per = (W + 255) / 256;
  const int w0 = min(tid * per, W), w1 = min(w0 + per, W);
  int own = 0;
  for (int w = w0; w < w1; ++w) own += __popc(bits[w]);
  part[tid] = own;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int run = part[tid] - own;
  for (int w = w0; w < w1; ++w) {
    pre[w] = run;
    run += __popc(bits[w]);
  }
  const int total = part[255];
  __syncthreads();
  const long bh = (long)b * Hkv + h;
  int32_t* co = chunk_of + bh * max_slots;
  if (tid == 0) count[bh] = total;
  for (int w = tid; w < W; w += 256) {
    uint32_t m = bits[w];
    int sl = pre[w];
    while (m) {
      co[sl++] = 32 * w + (__ffs(m) - 1);
      m &= m - 1u;
    }
  }
  for (int sl = total + tid; sl < max_slots; sl += 256) co[sl] = -1;
  for (long i = tid; i < n; i += 256) {
    const int c = idx[base + i];
    int s = -1;
    if (c >= 0 && c < C) s = pre[c >> 5] + __popc(bits[c >> 5] & ((1u << (c & 31)) - 1u));
    idx_staged[base + i] = s;
  }
}

// One chunk of one kv head: rows c*chunk .. of the host history to rows slot*chunk .. of
// the staging history, K then V.
__device__ __forceinline__ void gather_item(const bf16_t* __restrict__ kh, const bf16_t* __restrict__ vh, long hbs,
                                            int c, bf16_t* __restrict__ ks, bf16_t* __restrict__ vs, long sbs, int h,
                                            long b, int slot, int Hkv, int d, int chunk, int tid) {
  const int ppr = d / 8;               // 16-byte pieces per row
  const int P = chunk * ppr;           // pieces per tensor
  const long W = (long)Hkv * d;
  const long src0 = b * hbs + (long)c * chunk * W + (long)h * d;
  const long dst0 = b * sbs + (long)slot * chunk * W + (long)h * d;
  // pieces past the end repeat the last one (the same 16 bytes loaded and stored again),
  // so the loop has no branches and its eight loads stay in registers
  for (int p0 = 0; p0 < 2 * P; p0 += 8 * 256) {
    uint4 r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = min(p0 + u * 256 + tid, 2 * P - 1);
      const int t = p < P ? p : p - P;
      r[u] = *reinterpret_cast<const uint4*>((p < P ? kh : vh) + src0 + (long)(t / ppr) * W + (t % ppr) * 8);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = min(p0 + u * 256 + tid, 2 * P - 1);
      const int t = p < P ? p : p - P;
      *reinterpret_cast<uint4*>((p < P ? ks : vs) + dst0 + (long)(t / ppr) * W + (t % ppr) * 8) = r[u];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Gather: a few persistent workgroups of 256 threads loop over the (slot, kv head, batch)
// items; an item whose slot is in use copies that chunk's K and V rows of its kv head
// (chunk x d each) from host memory to the staging history, eight 16-byte pieces per
// thread in flight at a time.  The host link is saturated by about a hundred kilobytes in
// flight, i.e. a handful of workgroups; keeping the gather on few compute units leaves the
// others to attention kernels running beside it on another stream, whose memory traffic
// would otherwise queue behind the slow host reads.
// ---------------------------------------------------------------------------------------
#ifndef S2A_STAGE_GROUPS
#define S2A_STAGE_GROUPS 64
#endif

__global__ __launch_bounds__(256) void stage_gather_kernel(const bf16_t* __restrict__ kh, const bf16_t* __restrict__ vh,
                                                           long hbs, const int32_t* __restrict__ chunk_of,
                                                           const int32_t* __restrict__ count,
                                                           bf16_t* __restrict__ ks, bf16_t* __restrict__ vs, long sbs,
                                                           int Hkv, int d, int chunk, int max_slots, int used,
                                                           long items) {
  const int tid = thread_x();
  for (long it = group_x(); it < items; it += (long)gridDim.x) {
    const int slot = (int)(it % used);
    const long bh = it / used;
    if (slot >= count[bh]) continue;
    gather_item(kh, vh, hbs, chunk_of[bh * max_slots + slot], ks, vs, sbs, (int)(bh % Hkv), bh / Hkv, slot, Hkv, d,
                chunk, tid);
  }
}

// ---------------------------------------------------------------------------------------
// Cached staging: the staging history keeps the chunks it holds.  One workgroup per (kv
// head, batch): chunks still named by the lists keep their slots; the slots of the others
// are freed; the named chunks not yet staged (ascending) take the free slots (ascending)
// and are listed for the gather.  Each slot is written by the thread that owns it.
// ---------------------------------------------------------------------------------------
constexpr int kUpdSlots = S2A_STAGE_MAX_SLOTS;

__device__ __forceinline__ int scan_256(int* part, int own, int tid) {
  part[tid] = own;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  return part[tid] - own;   // exclusive prefix; part[255] is the total
}

__global__ __launch_bounds__(256) void stage_update_kernel(const int32_t* __restrict__ idx, int lists, int nqb,
                                                           int topk, int Hkv, int C, int max_slots,
                                                           int32_t* __restrict__ chunk_of, int32_t* __restrict__ count,
                                                           int32_t* __restrict__ copied,
                                                           int32_t* __restrict__ copy_list,
                                                           int32_t* __restrict__ idx_staged) {
  __shared__ uint32_t need[kStageWords];
  __shared__ uint32_t present[kStageWords];
  __shared__ int pre[kStageWords];
  __shared__ uint16_t slot_of[S2A_STAGE_MAX_CHUNKS];
  __shared__ uint16_t missing[kUpdSlots];
  __shared__ int part[256];
  const int h = group_x(), b = group_y(), tid = thread_x();
  const int W = (C + 31) / 32;
  const int rep = lists / Hkv;
  const long n = (long)rep * nqb * topk;
  const long base = ((long)b * lists + (long)h * rep) * nqb * topk;
  const long bh = (long)b * Hkv + h;
  int32_t* co = chunk_of + bh * max_slots;
  for (int w = tid; w < W; w += 256) need[w] = present[w] = 0u;
  __syncthreads();
  for (long i = tid; i < n; i += 256) {
    const int c = idx[base + i];
    if (c >= 0 && c < C) atomicOr(&need[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  // slots: thread t owns [s0, s1); a slot whose chunk is still named keeps it
  const int sp = (max_slots + 255) / 256;
  const int s0 = min(tid * sp, max_slots), s1 = min(s0 + sp, max_slots);
  int nfree = 0;
  for (int s = s0; s < s1; ++s) {
    const int c = co[s];
    if (c >= 0 && c < C && (need[c >> 5] >> (c & 31) & 1u)) {
      atomicOr(&present[c >> 5], 1u << (c & 31));
      slot_of[c] = (uint16_t)s;
    } else {
      ++nfree;
    }
  }
  const int free0 = scan_256(part, nfree, tid);   // rank of this thread's first free slot
  __syncthreads();
  // named chunks not staged: thread t owns words [w0, w1)
  const int per = (W + 255) / 256;
  const int w0 = min(tid * per, W), w1 = min(w0 + per, W);
  int own = 0;
  for (int w = w0; w < w1; ++w) own += __popc(need[w] & ~present[w]);
  int run = scan_256(part, own, tid);
  const int nmiss = part[255];
  for (int w = w0; w < w1; ++w) {
    pre[w] = run;
    run += __popc(need[w] & ~present[w]);
  }
  __syncthreads();
  for (int w = tid; w < W; w += 256) {
    uint32_t m = need[w] & ~present[w];
    int r = pre[w];
    while (m) {
      missing[r++] = (uint16_t)(32 * w + (__ffs(m) - 1));
      m &= m - 1u;
    }
  }
  __syncthreads();
  // free slots in ascending order take the missing chunks in ascending order
  int fr = free0;
  for (int s = s0; s < s1; ++s) {
    const int c = co[s];
    if (c >= 0 && c < C && (need[c >> 5] >> (c & 31) & 1u)) continue;   // kept
    if (fr < nmiss) {
      const int nc = missing[fr];
      co[s] = nc;
      slot_of[nc] = (uint16_t)s;
      copy_list[bh * max_slots + fr] = (s << 16) | nc;
    } else {
      co[s] = -1;
    }
    ++fr;
  }
  __syncthreads();
  if (tid == 0) {
    int used = 0;
    for (int w = 0; w < W; ++w) used += __popc(need[w]);
    count[bh] = used;
    copied[bh] = nmiss;
  }
  for (long i = tid; i < n; i += 256) {
    const int c = idx[base + i];
    idx_staged[base + i] = (c >= 0 && c < C) ? (int)slot_of[c] : -1;
  }
}

// Gather of the cached staging's new chunks: item (r, kv head, batch) copies the r-th
// listed chunk into its slot, for r below the pair's count.
__global__ __launch_bounds__(256) void stage_gather_list_kernel(const bf16_t* __restrict__ kh,
                                                                const bf16_t* __restrict__ vh, long hbs,
                                                                const int32_t* __restrict__ copy_list,
                                                                const int32_t* __restrict__ copied,
                                                                bf16_t* __restrict__ ks, bf16_t* __restrict__ vs,
                                                                long sbs, int Hkv, int d, int chunk, int max_slots,
                                                                long items) {
  const int tid = thread_x();
  for (long it = group_x(); it < items; it += (long)gridDim.x) {
    const int r = (int)(it % max_slots);
    const long bh = it / max_slots;
    if (r >= copied[bh]) continue;
    const int e = copy_list[bh * max_slots + r];
    gather_item(kh, vh, hbs, e & 0xffff, ks, vs, sbs, (int)(bh % Hkv), bh / Hkv, e >> 16, Hkv, d, chunk, tid);
  }
}

// Device address of pinned host memory (hipHostMalloc and allocators built on it), or
// nullptr when `p` is not such memory (pageable host memory, device memory).
static void* host_device_address(const void* p) {
  hipPointerAttribute_t a;
  void* dp = nullptr;
  if (hipPointerGetAttributes(&a, p) != hipSuccess || a.type != hipMemoryTypeHost ||
      hipHostGetDevicePointer(&dp, const_cast<void*>(p), 0) != hipSuccess) {
    (void)hipGetLastError();   // a rejected pointer leaves no error pending for later calls
    return nullptr;
  }
  return dp;
}

}  // namespace s2a

using namespace s2a;

extern "C" int hga_append_history(const void* k_seg, const void* v_seg, long long seg_bstride, void* k_hist,
                                  void* v_hist, long long hist_bstride, float* summ, long long summ_bstride, int B,
                                  int S, int Hkv, int d, int T, int chunk, void* stream);

extern "C" int hga_detach_segment(const void* k_seg, const void* v_seg, long long seg_bstride, void* k_host,
                                  void* v_host, long long host_bstride, float* summ, long long summ_bstride, int B,
                                  int S, int Hkv, int d, int T, int chunk, void* stream) {
  if (B <= 0 || S < 0 || T < 0 || Hkv <= 0 || d <= 0 || chunk <= 0) return S2A_ERR_INVALID_ARG;
  if (S % chunk || T % chunk) return S2A_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return S2A_ERR_UNSUPPORTED;
  if (chunk % 64) return S2A_ERR_UNSUPPORTED;
  if (S == 0) return S2A_OK;
  if (!ptr_ok(k_seg) || !ptr_ok(v_seg) || !ptr_ok(k_host) || !ptr_ok(v_host) || !ptr_ok(summ))
    return S2A_ERR_INVALID_ARG;
  void* kd = host_device_address(k_host);
  void* vd = host_device_address(v_host);
  if (kd == nullptr || vd == nullptr) return S2A_ERR_INVALID_ARG;
  // the same kernel as the resident append: it writes the rows through the device address
  return hga_append_history(k_seg, v_seg, seg_bstride, kd, vd, host_bstride, summ, summ_bstride, B, S, Hkv, d, T,
                            chunk, stream);
}

extern "C" int hga_stage_selected(const int32_t* idx, int lists, int nqb, int topk, const void* k_host,
                                  const void* v_host, long long host_bstride, int T, int32_t* chunk_of,
                                  int32_t* count, int32_t* idx_staged, void* k_stage, void* v_stage,
                                  long long stage_bstride, int max_slots, int B, int Hkv, int d, int chunk,
                                  void* stream) {
  if (B <= 0 || lists <= 0 || nqb <= 0 || topk <= 0 || Hkv <= 0 || d <= 0 || chunk <= 0 || T < 0 || max_slots <= 0)
    return S2A_ERR_INVALID_ARG;
  if (lists % Hkv || T % chunk) return S2A_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return S2A_ERR_UNSUPPORTED;
  if (chunk % 64 || topk > 64) return S2A_ERR_UNSUPPORTED;
  const long long C = T / chunk;
  if (C > S2A_STAGE_MAX_CHUNKS) return S2A_ERR_UNSUPPORTED;
  // every slot the union of one kv head's lists can need
  const long long picks = (long long)(lists / Hkv) * nqb * topk;
  if (max_slots < std::min(C, picks)) return S2A_ERR_INVALID_ARG;
  if (!ptr_ok(idx) || !ptr_ok(chunk_of) || !ptr_ok(count) || !ptr_ok(idx_staged) || !ptr_ok(k_stage) ||
      !ptr_ok(v_stage))
    return S2A_ERR_INVALID_ARG;
  if (C > 0 && (!ptr_ok(k_host) || !ptr_ok(v_host))) return S2A_ERR_INVALID_ARG;
  if (!stride_ok(host_bstride, T, Hkv, d, B) || !stride_ok(stage_bstride, (long long)max_slots * chunk, Hkv, d, B))
    return S2A_ERR_INVALID_ARG;
  if (B > 1 && (host_bstride % 8 || stage_bstride % 8)) return S2A_ERR_INVALID_ARG;
  if ((long long)B * lists * nqb * topk >= (1ll << 31) || (long long)max_slots * chunk * Hkv * d >= (1ll << 31) ||
      (long long)B * Hkv * max_slots >= (1ll << 31))
    return S2A_ERR_UNSUPPORTED;
  const void* kd = C > 0 ? host_device_address(k_host) : nullptr;
  const void* vd = C > 0 ? host_device_address(v_host) : nullptr;
  if (C > 0 && (kd == nullptr || vd == nullptr)) return S2A_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(stage_plan_kernel, dim3(Hkv, B), dim3(256), 0, s, idx, lists, nqb, topk, Hkv, (int)C, max_slots,
                     chunk_of, count, idx_staged);
  if (hipGetLastError() != hipSuccess) return S2A_ERR_HIP;
  if (C == 0) return S2A_OK;
  const int used = (int)std::min<long long>(C, max_slots);
  const long items = (long)B * Hkv * used;
  hipLaunchKernelGGL(stage_gather_kernel, dim3((unsigned)std::min<long>(items, S2A_STAGE_GROUPS)), dim3(256), 0, s,
                     static_cast<const bf16_t*>(kd), static_cast<const bf16_t*>(vd), (long)host_bstride, chunk_of,
                     count, static_cast<bf16_t*>(k_stage), static_cast<bf16_t*>(v_stage), (long)stage_bstride, Hkv, d,
                     chunk, max_slots, used, items);
  return hipGetLastError() == hipSuccess ? S2A_OK : S2A_ERR_HIP;
}

extern "C" int hga_stage_update(const int32_t* idx, int lists, int nqb, int topk, const void* k_host,
                                const void* v_host, long long host_bstride, int T, int32_t* chunk_of, int32_t* count,
                                int32_t* copied, int32_t* copy_list, int32_t* idx_staged, void* k_stage,
                                void* v_stage, long long stage_bstride, int max_slots, int B, int Hkv, int d,
                                int chunk, void* stream) {
  if (B <= 0 || lists <= 0 || nqb <= 0 || topk <= 0 || Hkv <= 0 || d <= 0 || chunk <= 0 || T < 0 || max_slots <= 0)
    return S2A_ERR_INVALID_ARG;
  if (lists % Hkv || T % chunk) return S2A_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return S2A_ERR_UNSUPPORTED;
  if (chunk % 64 || topk > 64) return S2A_ERR_UNSUPPORTED;
  const long long C = T / chunk;
  if (C > S2A_STAGE_MAX_CHUNKS || max_slots > S2A_STAGE_MAX_SLOTS) return S2A_ERR_UNSUPPORTED;
  const long long picks = (long long)(lists / Hkv) * nqb * topk;
  if (max_slots < std::min(C, picks)) return S2A_ERR_INVALID_ARG;
  if (!ptr_ok(idx) || !ptr_ok(chunk_of) || !ptr_ok(count) || !ptr_ok(copied) || !ptr_ok(copy_list) ||
      !ptr_ok(idx_staged) || !ptr_ok(k_stage) || !ptr_ok(v_stage))
    return S2A_ERR_INVALID_ARG;
  if (C > 0 && (!ptr_ok(k_host) || !ptr_ok(v_host))) return S2A_ERR_INVALID_ARG;
  if (!stride_ok(host_bstride, T, Hkv, d, B) || !stride_ok(stage_bstride, (long long)max_slots * chunk, Hkv, d, B))
    return S2A_ERR_INVALID_ARG;
  if (B > 1 && (host_bstride % 8 || stage_bstride % 8)) return S2A_ERR_INVALID_ARG;
  if ((long long)B * lists * nqb * topk >= (1ll << 31) || (long long)max_slots * chunk * Hkv * d >= (1ll << 31) ||
      (long long)B * Hkv * max_slots >= (1ll << 31))
    return S2A_ERR_UNSUPPORTED;
  const void* kd = C > 0 ? host_device_address(k_host) : nullptr;
  const void* vd = C > 0 ? host_device_address(v_host) : nullptr;
  if (C > 0 && (kd == nullptr || vd == nullptr)) return S2A_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(stage_update_kernel, dim3(Hkv, B), dim3(256), 0, s, idx, lists, nqb, topk, Hkv, (int)C,
                     max_slots, chunk_of, count, copied, copy_list, idx_staged);
  if (hipGetLastError() != hipSuccess) return S2A_ERR_HIP;
  if (C == 0) return S2A_OK;
  const long items = (long)B * Hkv * max_slots;
  hipLaunchKernelGGL(stage_gather_list_kernel, dim3((unsigned)std::min<long>(items, S2A_STAGE_GROUPS)), dim3(256), 0,
                     s, static_cast<const bf16_t*>(kd), static_cast<const bf16_t*>(vd), (long)host_bstride,
                     copy_list, copied, static_cast<bf16_t*>(k_stage), static_cast<bf16_t*>(v_stage),
                     (long)stage_bstride, Hkv, d, chunk, max_slots, items);
  return hipGetLastError() == hipSuccess ? S2A_OK : S2A_ERR_HIP;
}
