// Host-side helpers shared by the launchers: per-device facts queried once per device.
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

constexpr int kFgMaxDevices = 64;

// Compute units of the current device (the workgroup count that fills one round), cached per device;
// 256 if the runtime cannot say.
inline int fg_device_cus() {
    static std::atomic<int> cached[kFgMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kFgMaxDevices) return 256;
    int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    cached[dev].store(c, std::memory_order_relaxed);
    return c;
}

// Raises a kernel's dynamic LDS limit to `bytes` once per device (`done` is the caller's per-kernel bit
// set of devices already done). Setting it twice is harmless, so racing callers need no lock.
inline hipError_t fg_set_lds_limit_once(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    const uint64_t bit = dev >= 0 && dev < kFgMaxDevices ? (1ull << dev) : 0;
    if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_relaxed);
    return e;
}
