// Per-device facts the launchers need: the CU count and the one-time
// dynamic-LDS limit of a kernel.  Both are cached per device (up to 64
// devices) in atomics, so concurrent callers on several threads or devices
// see consistent values; nothing here is ever freed or reset.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

namespace convrot {

constexpr int kMaxDevices = 64;

// Compute units of the current device (256 if the runtime cannot say).
inline int device_cus() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Raise the dynamic LDS limit of `kern` to `bytes` on the current device,
// once per device; `done` is the caller's per-kernel record of the devices
// already set (setting it twice is harmless, so a race costs one extra call).
inline hipError_t set_lds_limit(const void* kern, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < kMaxDevices) ? (uint64_t{1} << dev) : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
  return e;
}

}  // namespace convrot
