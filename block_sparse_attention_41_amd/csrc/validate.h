// Host-side argument checks for the C ABI (plain C++; nothing here touches the GPU).
// Every entry point runs its check before launching anything and returns the status.
#pragma once

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "../../include/s2a.h"

namespace s2a {

inline bool ptr_ok(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int check_common_heads(int B, int L, int H, int Hkv, int d) {
  if (B <= 0 || L <= 0 || H <= 0 || Hkv <= 0 || d <= 0) return S2A_ERR_INVALID_ARG;
  if (H % Hkv) return S2A_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return S2A_ERR_UNSUPPORTED;
  return S2A_OK;
}

inline int check_scale(float scale) {
  return (std::isfinite(scale) && scale > 0.f) ? S2A_OK : S2A_ERR_INVALID_ARG;
}

// Shifted short attention shape rules (shared by forward and backward).
inline int check_s2attn(int B, int N, int H, int Hkv, int d, int G, int shift, float scale) {
  int st = check_common_heads(B, N, H, Hkv, d);
  if (st) return st;
  if (G <= 0 || N % G) return S2A_ERR_INVALID_ARG;
  if (check_scale(scale)) return S2A_ERR_INVALID_ARG;
  const bool shifting = shift && (N / G) >= 2;
  if (shifting && (G % 2 || Hkv % 2 || H % 2)) return S2A_ERR_INVALID_ARG;
  if (G % 64) return S2A_ERR_UNSUPPORTED;
  if (shifting && (G / 2) % 64) return S2A_ERR_UNSUPPORTED;
  // the kernels index tokens with 32-bit integers per (batch, head) plane
  if ((long long)N * H * d >= (1ll << 31) || (long long)N * Hkv * d >= (1ll << 31)) return S2A_ERR_UNSUPPORTED;
  return S2A_OK;
}

inline int check_hga_shape(int B, int S, int H, int Hkv, int d, int T, int chunk, int qblock, int topk) {
  int st = check_common_heads(B, S, H, Hkv, d);
  if (st) return st;
  if (T < 0 || chunk <= 0 || qblock <= 0 || topk <= 0) return S2A_ERR_INVALID_ARG;
  if (S % qblock || T % chunk) return S2A_ERR_INVALID_ARG;
  if (qblock != 64 || chunk % 64 || topk > 64) return S2A_ERR_UNSUPPORTED;
  return S2A_OK;
}

// A batch stride must at least cover one batch's rows; for B == 1 it is never used.
inline bool stride_ok(long long bstride, long long rows, int heads, int d, int B) {
  return B == 1 || bstride >= rows * heads * (long long)d;
}

}  // namespace s2a
