// Host-side launch helpers shared by the attention entry points.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace s2a {

// Workgroups that stay resident per XCD when each CU holds `per_cu` of them: the current
// device's CU count / 8 XCDs x per_cu.  The CU count is read once per device.
inline int resident_per_xcd(int per_cu) {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  const int per_xcd = n / 8 > 0 ? n / 8 : 1;
  return per_xcd * per_cu;
}

}  // namespace s2a
