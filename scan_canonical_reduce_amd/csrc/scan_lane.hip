// The block_dyadic kernels for blocks inside one vector row (LaneBlockTile
// in scan_kernels.hpp), plain inclusive output.
#include "scan_wide_def.hpp"

namespace canon {

template hipError_t launch_lane_block<double, false>(const double*, double*, uint64_t, int, bool,
                                                     uint64_t*, const ScanLayout&,
                                                     const ScanOut<double>&, hipStream_t);
template hipError_t launch_lane_block<float, false>(const float*, float*, uint64_t, int, bool,
                                                    uint64_t*, const ScanLayout&,
                                                    const ScanOut<float>&, hipStream_t);

}  // namespace canon
