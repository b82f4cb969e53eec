// host_util.h - small host-side helpers shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

namespace duckmoe {

inline bool aligned(const void *p, size_t n) { return ((uintptr_t)p % n) == 0; }

constexpr int kMaxDevices = 64;  // device ids the per-device caches cover

// Compute units of the current device, cached per device id.
inline int device_cus() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return -1;
  if (dev < kMaxDevices) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Resident workgroups per CU of one kernel at one dynamic-LDS size, from the
// occupancy API, cached per launch site (each site holds its own OccCache)
// and device, so a layer call makes no runtime queries after the first.  The
// entry packs (lds bytes << 32 | workgroups); another LDS size is recomputed.
// attr_lds > 0 sets the kernel's dynamic-LDS limit once per device, to the
// largest size the site ever launches (a fixed value, so concurrent callers
// never lower it under each other).
struct OccCache {
  std::atomic<uint64_t> entry[kMaxDevices];
  std::atomic<int> attr_set[kMaxDevices];
};

template <typename K>
hipError_t occupancy(OccCache &c, K kern, int threads, size_t lds, size_t attr_lds,
                     int &per_cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return hipErrorInvalidDevice;
  const bool cached = dev < kMaxDevices;
  if (cached) {
    const uint64_t e = c.entry[dev].load(std::memory_order_relaxed);
    if (e != 0 && (e >> 32) == (uint64_t)lds) {
      per_cu = (int)(e & 0xffffffffu);
      return hipSuccess;
    }
  }
  if (attr_lds > 0 && !(cached && c.attr_set[dev].load(std::memory_order_relaxed))) {
    const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)attr_lds);
    if (err != hipSuccess) return err;
    if (cached) c.attr_set[dev].store(1, std::memory_order_relaxed);
  }
  int v = 0;
  const hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kern, threads, lds);
  if (err != hipSuccess) return err;
  if (v <= 0) return hipErrorInvalidConfiguration;
  if (cached) c.entry[dev].store(((uint64_t)lds << 32) | (uint32_t)v, std::memory_order_relaxed);
  per_cu = v;
  return hipSuccess;
}

// CUs a launch may use: the device's, or fewer when the caller runs on a
// stream limited to a CU subset (budget > 0: that many CUs).
inline int cu_budget(int budget) {
  const int cus = device_cus();
  return (budget > 0 && cus > 0) ? std::min(budget, cus) : cus;
}

// Grid of a persistent kernel: resident workgroups per CU from the occupancy
// API (at most waves_per_cu waves per CU), times the CUs it may use (budget,
// see cu_budget), capped at `cap`.
template <typename K>
hipError_t persistent_grid(OccCache &c, K kern, int threads, int waves_per_cu, int cap,
                           int budget, int &grid) {
  int per_cu = 0;
  hipError_t err = occupancy(c, kern, threads, 0, 0, per_cu);
  if (err != hipSuccess) return err;
  const int cus = cu_budget(budget);
  if (cus <= 0) return hipErrorInvalidConfiguration;
  per_cu = std::max(1, std::min(per_cu, waves_per_cu / (threads / 64)));
  grid = std::max(1, std::min(cus * per_cu, cap));
  return hipSuccess;
}

}  // namespace duckmoe
