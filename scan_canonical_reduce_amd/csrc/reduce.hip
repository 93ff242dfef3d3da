// Canonical reduction kernels (reduce_impl.hpp), instantiated for double
// and float with IEEE addition.
#include "reduce_impl.hpp"

namespace canon {

template hipError_t launch_reduce<double, true>(const double*, uint64_t, uint32_t, double,
                                                double*, void*, const ReducePlan&, uint64_t,
                                                hipStream_t);
template hipError_t launch_reduce<float, true>(const float*, uint64_t, uint32_t, float, float*,
                                               void*, const ReducePlan&, uint64_t, hipStream_t);
template hipError_t launch_reduce_rows<double>(const double*, uint64_t, uint64_t, uint64_t,
                                               uint32_t, double, double*, hipStream_t);
template hipError_t launch_reduce_rows<float>(const float*, uint64_t, uint64_t, uint64_t, uint32_t,
                                              float, float*, hipStream_t);

}  // namespace canon
