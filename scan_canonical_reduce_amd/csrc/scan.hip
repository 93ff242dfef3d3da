// Canonical inclusive scan, single pass (pairwise, block_dyadic<B>): the
// kernels of scan_kernels.hpp with the plain inclusive output.
#include "scan_kernels.hpp"

namespace canon {

template <typename T>
hipError_t launch_scan(const T* x, T* y, uint64_t n, bool pairwise, int b_log, bool aligned,
                       uint64_t* ws, const ScanLayout& lay, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    return launch_scan_impl<T, false>(x, y, n, pairwise, b_log, aligned, ws, lay, ScanOut<T>{},
                                      s);
}

template hipError_t launch_scan<double>(const double*, double*, uint64_t, bool, int, bool,
                                        uint64_t*, const ScanLayout&, hipStream_t);
template hipError_t launch_scan<float>(const float*, float*, uint64_t, bool, int, bool, uint64_t*,
                                       const ScanLayout&, hipStream_t);

}  // namespace canon
