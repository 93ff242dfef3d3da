// Host-side launch helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace canon {

// Workgroups of kernel KERN (with `threads` threads each) that fit on the
// current device at once, cached per device.  Grid-stride and ticket-driven
// kernels are launched with about this many workgroups: one workgroup per
// tile or row would be bounded by the workgroup launch rate, not by memory.
template <auto KERN>
uint64_t resident_grid(int threads)
{
    static uint64_t cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cache[dev] == 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, KERN, threads, 0) != hipSuccess)
            per = 0;
        cache[dev] = (uint64_t)(cus > 0 ? cus : 256) * (uint64_t)(per > 0 ? per : 1);
    }
    return cache[dev];
}

}  // namespace canon
