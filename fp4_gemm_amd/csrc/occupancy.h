// Host-side sizing of persistent grids: how many workgroups of a kernel can
// be resident on the current device at once.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace epilora {

// Compute units of the current device (queried once per device).
inline int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  std::atomic<int>& slot = cache[dev & 63];
  int n = slot.load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    slot.store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workgroups of `kernel` (block threads, dyn_lds bytes of dynamic LDS) that
// fit on the device at once; at least one per compute unit.
template <typename Kernel>
inline int resident_groups(Kernel kernel, int block, size_t dyn_lds) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, dyn_lds) != hipSuccess || per_cu < 1)
    per_cu = 1;
  return per_cu * device_cus();
}

}  // namespace epilora
