// Internal host helpers shared by the kernel launchers of this library.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace mx {

// Compute units of the current device (cached per device; 256 if the query fails).
inline int num_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace mx
