// Host-side helpers of the launchers: the current device, device attributes
// cached per device, and the dynamic-LDS attribute of a kernel raised once
// per (kernel, device).  Every cache is an array of atomics indexed by the
// device, so concurrent calls from several host threads, on one device or on
// several, share no unsynchronized state.
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>

namespace lora {

constexpr int kMaxDevices = 64;

// The calling thread's current device, checked against the caches' size.
inline hipError_t current_device(int* dev) {
  hipError_t e = hipGetDevice(dev);
  if (e == hipSuccess && (*dev < 0 || *dev >= kMaxDevices)) return hipErrorInvalidDevice;
  return e;
}

// An attribute of the current device, queried once per device.  A value of 0
// marks "not yet queried"; every attribute read here is positive.
template <hipDeviceAttribute_t kAttr>
inline hipError_t device_attribute(int* out) {
  static std::atomic<int> cache[kMaxDevices];  // static storage: zero-initialized
  int dev = 0;
  hipError_t e = current_device(&dev);
  if (e != hipSuccess) return e;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    e = hipDeviceGetAttribute(&v, kAttr, dev);
    if (e != hipSuccess) return e;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  *out = v;
  return hipSuccess;
}

// Compute units of the current device (256 on an MI355X); 256 if the query
// fails, which only sizes grids.
inline int cu_count() {
  int v = 0;
  return device_attribute<hipDeviceAttributeMultiprocessorCount>(&v) == hipSuccess && v > 0 ? v : 256;
}

// The largest dynamic LDS a kernel has been allowed on each device.  One
// object per kernel (a function-local static of its launcher).
struct DynLdsLimit {
  std::atomic<size_t> raised[kMaxDevices];
};

// Allow `fn` `lds` bytes of dynamic LDS on the current device (above 48 KiB
// the attribute must be set).  Two threads racing here both set the
// attribute, which is idempotent, and the recorded limit only grows.
inline hipError_t ensure_dynamic_lds(DynLdsLimit& lim, const void* fn, size_t lds) {
  if (lds <= 48 * 1024) return hipSuccess;
  int dev = 0;
  hipError_t e = current_device(&dev);
  if (e != hipSuccess) return e;
  size_t cur = lim.raised[dev].load(std::memory_order_acquire);
  if (lds <= cur) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  while (cur < lds && !lim.raised[dev].compare_exchange_weak(cur, lds, std::memory_order_acq_rel)) {
  }
  return hipSuccess;
}

}  // namespace lora
