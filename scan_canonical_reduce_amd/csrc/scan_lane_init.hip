// The block_dyadic kernels for blocks inside one vector row (LaneBlockTile
// in scan_kernels.hpp), output stage of a scan with an initial
// value.
#include "scan_wide_def.hpp"

namespace canon {

template hipError_t launch_lane_block<double, true>(const double*, double*, uint64_t, int, bool,
                                                     uint64_t*, const ScanLayout&,
                                                     const ScanOut<double>&, hipStream_t);
template hipError_t launch_lane_block<float, true>(const float*, float*, uint64_t, int, bool,
                                                    uint64_t*, const ScanLayout&,
                                                    const ScanOut<float>&, hipStream_t);

}  // namespace canon
