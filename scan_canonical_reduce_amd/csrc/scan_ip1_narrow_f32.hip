// Single-pass iterated_pairwise scan over narrow rows (L < 64 E lanes,
// scan_ip1_impl.hpp), instantiated for float with IEEE addition.
#include "scan_ip1_impl.hpp"

namespace canon {

template hipError_t launch_ip1_narrow<float, true>(const float*, uint64_t, float*, uint64_t, uint64_t,
                                                 uint64_t*, const IpSingleLayout&,
                                                 const ScanOut<float>&, bool, hipStream_t);
template hipError_t launch_ip1_narrow<float, false>(const float*, uint64_t, float*, uint64_t, uint64_t,
                                                  uint64_t*, const IpSingleLayout&,
                                                  const ScanOut<float>&, bool, hipStream_t);

}  // namespace canon
