/* canon_user_op.hpp -- a caller-defined binary operator (C++ / HIP extension
 * point of libcanon).
 *
 * The canonical expression (canonical-reduce README, P4016R0 "Summary" and
 * "Key Design Points") is defined for any binary operator; the C ABI of
 * canon.h carries four built in (canon_op_t).  Any other operator is
 * compiled into the caller's own shared library from this header: one HIP
 * translation unit defines the operator as
 *
 *     struct MyOp {
 *         template <typename B>
 *         static __host__ __device__ B f(B a, B b);   // a (+) b, a on the left
 *         template <typename B>
 *         static __host__ __device__ B identity();    // the absent value e
 *     };
 *
 * (B is double or float) and expands, at file scope,
 *
 *     CANON_USER_OP(prefix, MyOp)
 *
 * The operator need be neither commutative nor associative: every kernel
 * applies it in the expression's order, left operand on the left.  It must
 * be deterministic, and e must satisfy f(e, x) == x and f(x, e) == x bit for
 * bit for every value the data can produce, because ragged tiles and absent
 * lanes are padded with e.  Values passed between workgroups are
 * canonicalised, so NaN payloads are not preserved.
 *
 * CANON_USER_OP defines, with C linkage, for T in {f64, f32} (double, float):
 *
 *   canon_status_t prefix_reduce_T(const T* x, size_t n, uint32_t L, T init,
 *                                  T* out, void* ws, size_t ws_bytes,
 *                                  void* stream);
 *   canon_status_t prefix_reduce_rows_T(const T* x, size_t rows, size_t cols,
 *                                       size_t ldx, uint32_t L, T init,
 *                                       T* out, void* ws, size_t ws_bytes,
 *                                       void* stream);
 *   canon_status_t prefix_scan_T(const T* x, T* y, size_t n, int policy,
 *                                uint32_t param, int kind, T init, void* ws,
 *                                size_t ws_bytes, void* stream);
 *   canon_status_t prefix_scan_rows_T(const T* x, size_t ldx, T* y,
 *                                     size_t ldy, size_t rows, size_t cols,
 *                                     int policy, uint32_t param, int kind,
 *                                     T init, void* ws, size_t ws_bytes,
 *                                     void* stream);
 *   int prefix_last_hip_error(void);
 *
 * Arguments, layouts, ownership, argument checks and status codes are those
 * of canon_reduce_op_T, canon_reduce_rows_op_T, canon_scan_op_T and
 * canon_scan_rows_op_T in canon.h without the `op` argument; workspace sizes
 * are canon.h's *_workspace_bytes (they do not depend on the operator).
 * prefix_last_hip_error reports the HIP error of the last failed launch made
 * through these entry points.
 *
 * Build (one translation unit, a few minutes: every kernel is instantiated
 * for the operator):
 *   hipcc --offload-arch=gfx950 -std=c++17 -O3 -ffp-contract=off -fPIC
 *         -shared -I <repo>/include -I <repo>/scan_canonical_reduce_amd/csrc
 *         my_op.hip -o libmy_op.so
 */
#pragma once

#include "canon.h"
#include "api_impl.hpp"
#include "ops_instantiate.hpp"

#define CANON_USER_OP_TYPE(PREFIX, T, B, OPV)                                                  \
    extern "C" canon_status_t PREFIX##_reduce_##T(const B* x, size_t n, uint32_t L, B init,    \
                                                  B* out, void* ws, size_t ws_bytes,           \
                                                  void* stream)                                \
    {                                                                                          \
        return canon::abi::reduce_as<OPV>(x, n, L, init, out, ws, ws_bytes, stream);           \
    }                                                                                          \
    extern "C" canon_status_t PREFIX##_reduce_rows_##T(const B* x, size_t rows, size_t cols,   \
                                                       size_t ldx, uint32_t L, B init, B* out, \
                                                       void* ws, size_t ws_bytes,              \
                                                       void* stream)                           \
    {                                                                                          \
        return canon::abi::reduce_rows_as<OPV>(x, rows, cols, ldx, L, init, out, ws, ws_bytes, \
                                               stream);                                        \
    }                                                                                          \
    extern "C" canon_status_t PREFIX##_scan_##T(const B* x, B* y, size_t n, int policy,        \
                                                uint32_t param, int kind, B init, void* ws,    \
                                                size_t ws_bytes, void* stream)                 \
    {                                                                                          \
        return canon::abi::scan_as<OPV>(x, y, n, policy, param, kind, init, ws, ws_bytes,      \
                                        stream);                                               \
    }                                                                                          \
    extern "C" canon_status_t PREFIX##_scan_rows_##T(                                          \
        const B* x, size_t ldx, B* y, size_t ldy, size_t rows, size_t cols, int policy,        \
        uint32_t param, int kind, B init, void* ws, size_t ws_bytes, void* stream)             \
    {                                                                                          \
        return canon::abi::scan_rows_as<OPV>(x, ldx, y, ldy, rows, cols, policy, param, kind,  \
                                             init, ws, ws_bytes, stream);                      \
    }

#define CANON_USER_OP(PREFIX, OP)                                                              \
    namespace canon {                                                                          \
    using PREFIX##_value_f64 = OpVal<double, OP>;                                              \
    using PREFIX##_value_f32 = OpVal<float, OP>;                                               \
    CANON_INSTANTIATE_OP(PREFIX##_value_f64)                                                   \
    CANON_INSTANTIATE_OP(PREFIX##_value_f32)                                                   \
    }                                                                                          \
    CANON_USER_OP_TYPE(PREFIX, f64, double, canon::PREFIX##_value_f64)                         \
    CANON_USER_OP_TYPE(PREFIX, f32, float, canon::PREFIX##_value_f32)                          \
    extern "C" int PREFIX##_last_hip_error(void) { return canon::abi::g_last_hip_error; }
