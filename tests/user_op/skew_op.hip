// A caller-defined operator built through canon_user_op.hpp, for the GPU
// tests: a (+) b = (a + b) + ((a / 4) * b) * b, neither commutative nor
// associative, so any change of operand order or of parenthesisation in a
// kernel changes its results.  -0.0 is an exact two-sided identity for
// finite operands: a (+) -0.0 = (a + -0.0) + (a / 4 * -0.0) * -0.0 = a, and
// -0.0 (+) b = (-0.0 + b) + (-0.0 * b) * b = b, signed zeros included.
#include "canon_user_op.hpp"

struct OpSkew {
    template <typename B>
    static __host__ __device__ __forceinline__ B f(B a, B b)
    {
        const B s = a + b;
        const B q = (a * B(0.25)) * b;
        return s + q * b;
    }
    template <typename B>
    static __host__ __device__ __forceinline__ B identity()
    {
        return B(-0.0);
    }
};

CANON_USER_OP(canon_skew, OpSkew)
