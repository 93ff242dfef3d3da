// Every kernel reached by the operator entry points, for float with the
// operator OpMul (device.hpp) in place of addition.
#include "ops_instantiate.hpp"

namespace canon {

using OpValue = OpVal<float, OpMul>;
CANON_INSTANTIATE_OP(OpValue)

}  // namespace canon
