// Single-pass iterated_pairwise scan (scan_ip1_impl.hpp), instantiated for
// double and float with IEEE addition.
#include "scan_ip1_impl.hpp"

namespace canon {

template hipError_t launch_scan_ip_single<double, true>(const double*, uint64_t, double*, uint64_t,
                                                        uint64_t, uint64_t*, const IpSingleLayout&,
                                                        const ScanOut<double>*, bool, hipStream_t);
template hipError_t launch_scan_ip_single<float, true>(const float*, uint64_t, float*, uint64_t,
                                                       uint64_t, uint64_t*, const IpSingleLayout&,
                                                       const ScanOut<float>*, bool, hipStream_t);

}  // namespace canon
