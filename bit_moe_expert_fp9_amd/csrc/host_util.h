// host_util.h - small host-side helpers shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

namespace duckmoe {

inline bool aligned(const void *p, size_t n) { return ((uintptr_t)p % n) == 0; }

// Compute units of the current device, cached per device id.
inline int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return -1;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Grid of a persistent kernel: resident workgroups per CU from the occupancy
// API (at most waves_per_cu waves per CU), times the CUs, capped at `cap`.
template <typename K>
hipError_t persistent_grid(K kern, int threads, int waves_per_cu, int cap, int &grid) {
  int per_cu = 0;
  hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0);
  if (err != hipSuccess) return err;
  const int cus = device_cus();
  if (cus <= 0 || per_cu <= 0) return hipErrorInvalidConfiguration;
  per_cu = std::max(1, std::min(per_cu, waves_per_cu / (threads / 64)));
  grid = std::max(1, std::min(cus * per_cu, cap));
  return hipSuccess;
}

}  // namespace duckmoe
