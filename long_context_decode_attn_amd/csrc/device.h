// device.h - host-side facts about the current device that size launches.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace lcda {

// Compute units of the current device (cached per device, safe to call from
// several host threads; 0 if the query fails).
inline int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

}  // namespace lcda
