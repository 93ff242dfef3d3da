// The kernels reached by the operator entry points, for double with the
// operator OpMin (device.hpp) in place of addition.
#include "ops_instantiate.hpp"

namespace canon {

using OpValue = OpVal<double, OpMin>;
CANON_INSTANTIATE_ORDER_FREE_OP(OpValue)

}  // namespace canon
