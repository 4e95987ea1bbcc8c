// device.h - host-side facts about the current device that size launches.
#pragma once

#include <hip/hip_runtime.h>

namespace lcda {

// Compute units of the current device (cached per device; 0 if the query fails).
inline int device_cus() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cache[dev] == 0) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev] = c;
    }
    return cache[dev];
}

}  // namespace lcda
