// The kernels reached by the operator entry points, for float with the
// operator OpMax (device.hpp) in place of addition.
#include "ops_instantiate.hpp"

namespace canon {

using OpValue = OpVal<float, OpMax>;
CANON_INSTANTIATE_ORDER_FREE_OP(OpValue)

}  // namespace canon
