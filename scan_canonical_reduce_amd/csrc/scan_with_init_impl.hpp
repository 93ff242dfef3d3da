// Canonical scan with an initial value, single pass (pairwise,
// block_dyadic<B>): the kernels of scan_kernels.hpp with the output stage
// that adds init and, for the exclusive and include_initial kinds, shifts
// every value one position up.
#pragma once
#include "scan_kernels.hpp"

namespace canon {

template <typename T>
__global__ __launch_bounds__(256) void k_put_column(T* y, uint64_t ldy, uint64_t rows, T v)
{
    for (uint64_t r = (uint64_t)blockIdx.x * 256 + threadIdx.x; r < rows;
         r += (uint64_t)gridDim.x * 256)
        y[r * ldy] = v;
}

template <typename T>
hipError_t launch_put_column(T* y, uint64_t ldy, uint64_t rows, T v, hipStream_t s)
{
    if (rows == 0) return hipSuccess;
    uint64_t grid = (rows + 255) / 256;
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL((k_put_column<T>), dim3((unsigned)grid), dim3(256), 0, s, y, ldy, rows, v);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_scan_with_init(const T* x, T* y, uint64_t n, bool pairwise, int b_log,
                                 bool aligned, uint64_t* ws, const ScanLayout& lay,
                                 const ScanOut<T>& out, hipStream_t s)
{
    if (n == 0)
        return out.kind == kScanIncludeInitial ? launch_put_column(y, 1, 1, out.init, s)
                                               : hipSuccess;
    return launch_scan_impl<T, true>(x, y, n, pairwise, b_log, aligned, ws, lay, out, s);
}

// For operators whose every parenthesisation gives the same value (minimum,
// maximum), so that every policy's scan equals every other's: the
// block_dyadic tiles with blocks of one wave-wide vector, which apply the
// operator fewer times per element than the pairwise tiles.
template <typename T>
hipError_t launch_scan_order_free(const T* x, T* y, uint64_t n, bool aligned, uint64_t* ws,
                                  const ScanLayout& lay, const ScanOut<T>& out, hipStream_t s)
{
    if (n == 0)
        return out.kind == kScanIncludeInitial ? launch_put_column(y, 1, 1, out.init, s)
                                               : hipSuccess;
    launch_scan_init<T>(ws, lay, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int LOGV = scan_log_v<T>();
    constexpr int b_log = Elem<T>::LOGE + 6;
    if (aligned)
        return launch_k<WideTile<T, true, LOGV, 0, true>>(x, y, n, b_log, ws, lay, 0, out, s);
    return launch_k<WideTile<T, false, LOGV, 0, true>>(x, y, n, b_log, ws, lay, 0, out, s);
}

}  // namespace canon
