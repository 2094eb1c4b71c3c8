// fa_host.hpp — host-side helpers shared by the entry points of include/fa.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

namespace fa_host {

// hipError_t behind the last FA_ERR_HIP on this thread (one variable for the library).
inline thread_local int g_last_hip_error = 0;

// CU count of the current device, read once per device (immutable afterwards).
inline int cu_count() {
  static std::once_flag once[64];
  static int count[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::call_once(once[dev], [dev]() {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    count[dev] = n;
  });
  return count[dev];
}

// LDS bytes per CU of the current device, read once per device (0 if unknown).
inline size_t lds_per_cu() {
  static std::once_flag once[64];
  static size_t bytes[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::call_once(once[dev], [dev]() {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
        hipSuccess)
      n = 0;
    bytes[dev] = n > 0 ? static_cast<size_t>(n) : 0;
  });
  return bytes[dev];
}

inline bool ranges_overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a);
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace fa_host
