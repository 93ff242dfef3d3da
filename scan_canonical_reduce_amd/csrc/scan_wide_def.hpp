// Definitions of launch_wide and launch_lane_block (declared in
// scan_kernels.hpp), for the translation units that instantiate the WideTile
// and LaneBlockTile kernels.
#pragma once

#include "scan_kernels.hpp"

namespace canon {

template <typename T, bool OUTX>
hipError_t launch_wide(const T* x, T* y, uint64_t n, int b_log, bool aligned, uint64_t* ws,
                       const ScanLayout& lay, const ScanOut<T>& out, hipStream_t s)
{
    return launch_wide_impl<T, OUTX>(x, y, n, b_log, aligned, ws, lay, out, s);
}

template <typename T, bool OUTX>
hipError_t launch_lane_block(const T* x, T* y, uint64_t n, int b_log, bool aligned, uint64_t* ws,
                             const ScanLayout& lay, const ScanOut<T>& out, hipStream_t s)
{
    return launch_lane_block_impl<T, OUTX>(x, y, n, b_log, aligned, ws, lay, out, s);
}

}  // namespace canon
