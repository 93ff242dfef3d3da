// Single-pass iterated_pairwise scan over narrow rows (L < 64 E lanes,
// scan_ip1_impl.hpp), instantiated for double with IEEE addition.
#include "scan_ip1_impl.hpp"

namespace canon {

template hipError_t launch_ip1_narrow<double, true>(const double*, uint64_t, double*, uint64_t, uint64_t,
                                                 uint64_t*, const IpSingleLayout&,
                                                 const ScanOut<double>&, bool, hipStream_t);
template hipError_t launch_ip1_narrow<double, false>(const double*, uint64_t, double*, uint64_t, uint64_t,
                                                  uint64_t*, const IpSingleLayout&,
                                                  const ScanOut<double>&, bool, hipStream_t);

}  // namespace canon
