// Scan with an initial value (scan_with_init_impl.hpp), instantiated for
// double and float with IEEE addition.
#include "scan_with_init_impl.hpp"

namespace canon {

template hipError_t launch_put_column<double>(double*, uint64_t, uint64_t, double, hipStream_t);
template hipError_t launch_put_column<float>(float*, uint64_t, uint64_t, float, hipStream_t);
template hipError_t launch_scan_with_init<double>(const double*, double*, uint64_t, bool, int,
                                                  bool, uint64_t*, const ScanLayout&,
                                                  const ScanOut<double>&, hipStream_t);
template hipError_t launch_scan_with_init<float>(const float*, float*, uint64_t, bool, int, bool,
                                                 uint64_t*, const ScanLayout&,
                                                 const ScanOut<float>&, hipStream_t);

}  // namespace canon
