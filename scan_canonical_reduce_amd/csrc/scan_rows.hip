// Row-batched scan kernels (scan_rows_impl.hpp), instantiated for double
// and float with IEEE addition.
#include "scan_rows_impl.hpp"

namespace canon {

template hipError_t launch_scan_rows<double, true, false>(const double*, uint64_t, double*, uint64_t, uint64_t,
                                             uint64_t, bool, int, bool, const ScanOut<double>*,
                                             hipStream_t);
template hipError_t launch_scan_rows<float, true, false>(const float*, uint64_t, float*, uint64_t, uint64_t,
                                            uint64_t, bool, int, bool, const ScanOut<float>*,
                                            hipStream_t);

}  // namespace canon
