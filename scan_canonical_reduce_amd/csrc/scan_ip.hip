// Three-kernel iterated_pairwise scan (scan_ip_impl.hpp), instantiated for
// double and float with IEEE addition.
#include "scan_ip_impl.hpp"

namespace canon {

template hipError_t launch_scan_ip<double, true>(const double*, uint64_t, double*, uint64_t, uint64_t,
                                           uint64_t, uint32_t*, double*, const IpLayout&,
                                           const ScanOut<double>*, hipStream_t);
template hipError_t launch_scan_ip<float, true>(const float*, uint64_t, float*, uint64_t, uint64_t,
                                          uint64_t, uint32_t*, float*, const IpLayout&,
                                          const ScanOut<float>*, hipStream_t);

}  // namespace canon
