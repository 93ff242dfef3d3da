// The block_dyadic kernels for blocks of whole vectors inside one wave
// (WideTile in scan_kernels.hpp), plain inclusive output.
#include "scan_kernels.hpp"

namespace canon {

template <typename T, bool OUTX>
hipError_t launch_wide(const T* x, T* y, uint64_t n, int b_log, bool aligned, uint64_t* ws,
                       const ScanLayout& lay, const ScanOut<T>& out, hipStream_t s)
{
    return launch_wide_impl<T, OUTX>(x, y, n, b_log, aligned, ws, lay, out, s);
}

template hipError_t launch_wide<double, false>(const double*, double*, uint64_t, int, bool,
                                               uint64_t*, const ScanLayout&,
                                               const ScanOut<double>&, hipStream_t);
template hipError_t launch_wide<float, false>(const float*, float*, uint64_t, int, bool,
                                              uint64_t*, const ScanLayout&, const ScanOut<float>&,
                                              hipStream_t);

}  // namespace canon
