// Host-side launch helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

namespace canon {

// Schedule override (canon_set_schedule; 0 = none), process-wide and meant
// for tests: a cap on the workgroups of the persistent (ticket-driven) and
// grid-stride kernels, and the workgroups the streaming reduce aims for.
// Both change how the work is spread over workgroups, never the results.
inline std::atomic<uint64_t> g_sched_grid_cap{0};
inline std::atomic<uint64_t> g_sched_reduce_wg{0};
inline std::atomic<uint64_t> g_sched_spin_limit{0};  // polls of a bounded wait (0: default)

// Compute units of the current device (cached per device; 256 if unknown).
inline uint64_t device_cus()
{
    static uint64_t cache[64] = {};
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cache[dev] = (uint64_t)cus;
    }
    return cache[dev];
}

// `grid` workgroups, or fewer under the schedule override.
inline uint64_t capped_grid(uint64_t grid)
{
    const uint64_t cap = g_sched_grid_cap.load(std::memory_order_relaxed);
    return (cap != 0 && grid > cap) ? cap : grid;
}

// Workgroups of kernel KERN (with `threads` threads and `shmem` bytes of
// dynamic shared memory each) that fit on the current device at once, cached
// per device and shared-memory size.  Grid-stride and ticket-driven kernels
// are launched with about this many workgroups: one workgroup per tile or row
// would be bounded by the workgroup launch rate, not by memory.
template <auto KERN>
uint64_t resident_grid(int threads, size_t shmem = 0)
{
    struct Entry {
        int dev;
        size_t shmem;
        uint64_t grid;
    };
    static Entry cache[32] = {};
    static int used = 0;
    static std::mutex mu;  // host threads may launch concurrently
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].dev == dev && cache[i].shmem == shmem) return cache[i].grid;
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, KERN, threads, shmem) != hipSuccess)
        per = 0;
    const uint64_t grid = (uint64_t)(cus > 0 ? cus : 256) * (uint64_t)(per > 0 ? per : 1);
    if (used < 32) cache[used++] = Entry{dev, shmem, grid};
    return grid;
}

}  // namespace canon
