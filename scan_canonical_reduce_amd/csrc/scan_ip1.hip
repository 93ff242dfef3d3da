// Single-pass iterated_pairwise scan (scan_ip1_impl.hpp), instantiated for
// double and float with IEEE addition.
#include "scan_ip1_impl.hpp"

namespace canon {

// narrow rows: scan_ip1_narrow_f64.hip, scan_ip1_narrow_f32.hip
#define CANON_IP1_NARROW(V, OUTX)                                                               \
    extern template hipError_t launch_ip1_narrow<V, OUTX>(const V*, uint64_t, V*, uint64_t,   \
                                                          uint64_t, uint64_t*,                \
                                                          const IpSingleLayout&,              \
                                                          const ScanOut<V>&, bool, hipStream_t);
CANON_IP1_NARROW(double, true)
CANON_IP1_NARROW(double, false)
CANON_IP1_NARROW(float, true)
CANON_IP1_NARROW(float, false)
#undef CANON_IP1_NARROW

template hipError_t launch_scan_ip_single<double, true>(const double*, uint64_t, double*, uint64_t,
                                                        uint64_t, uint64_t*, const IpSingleLayout&,
                                                        const ScanOut<double>*, bool, hipStream_t);
template hipError_t launch_scan_ip_single<float, true>(const float*, uint64_t, float*, uint64_t,
                                                       uint64_t, uint64_t*, const IpSingleLayout&,
                                                       const ScanOut<float>*, bool, hipStream_t);

}  // namespace canon
