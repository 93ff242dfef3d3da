// Every kernel reached by the operator entry points, for double with the
// operator OpMul (device.hpp) in place of addition.
#include "ops_instantiate.hpp"

namespace canon {

using OpValue = OpVal<double, OpMul>;
CANON_INSTANTIATE_OP(OpValue)

}  // namespace canon
