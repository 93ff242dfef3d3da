// Explicit instantiations of the launchers for one value type V (an
// OpVal<B, Op>: the kernels with the operator Op in place of addition).
// Only the kernels that the operator entry points reach are built: the
// reduce kernels, and the scans with an output stage (for an order-free
// operator, minimum or maximum, one scan kernel for every policy).
#pragma once

#include "reduce_impl.hpp"
#include "scan_ip1_impl.hpp"
#include "scan_ip_impl.hpp"
#include "scan_rows_impl.hpp"
#include "scan_wide_def.hpp"
#include "scan_with_init_impl.hpp"

#define CANON_INSTANTIATE_OP(V)                                                                  \
    template hipError_t launch_reduce<V, true>(const V*, uint64_t, uint32_t, V, V*, void*,        \
                                               const ReducePlan&, uint64_t, hipStream_t);          \
    template hipError_t launch_reduce_rows<V>(const V*, uint64_t, uint64_t, uint64_t, uint32_t, V, \
                                              V*, hipStream_t);                                    \
    template hipError_t launch_put_column<V>(V*, uint64_t, uint64_t, V, hipStream_t);             \
    template hipError_t launch_scan_with_init<V>(const V*, V*, uint64_t, bool, int, bool,         \
                                                 uint64_t*, const ScanLayout&, const ScanOut<V>&, \
                                                 hipStream_t);                                     \
    template hipError_t launch_wide<V, true>(const V*, V*, uint64_t, int, bool, uint64_t*,        \
                                             const ScanLayout&, const ScanOut<V>&, hipStream_t);   \
    template hipError_t launch_lane_block<V, true>(const V*, V*, uint64_t, int, bool, uint64_t*,  \
                                                   const ScanLayout&, const ScanOut<V>&,           \
                                                   hipStream_t);                                   \
    template hipError_t launch_scan_rows<V, false, false>(const V*, uint64_t, V*, uint64_t,       \
                                                          uint64_t, uint64_t, bool, int, bool,     \
                                                          const ScanOut<V>*, hipStream_t);         \
    template hipError_t launch_scan_ip<V, false>(const V*, uint64_t, V*, uint64_t, uint64_t,      \
                                                 uint64_t, uint32_t*, V*, const IpLayout&,        \
                                                 const ScanOut<V>*, hipStream_t);                  \
    template hipError_t launch_scan_ip_single<V, false>(const V*, uint64_t, V*, uint64_t,         \
                                                        uint64_t, uint64_t*,                       \
                                                        const IpSingleLayout&,                     \
                                                        const ScanOut<V>*, bool, hipStream_t);

// Minimum and maximum: every parenthesisation gives the same value, so one
// scan kernel (block_dyadic with one-vector blocks) serves every policy.
#define CANON_INSTANTIATE_ORDER_FREE_OP(V)                                                       \
    template hipError_t launch_reduce<V, true>(const V*, uint64_t, uint32_t, V, V*, void*,        \
                                               const ReducePlan&, uint64_t, hipStream_t);          \
    template hipError_t launch_reduce_rows<V>(const V*, uint64_t, uint64_t, uint64_t, uint32_t, V, \
                                              V*, hipStream_t);                                    \
    template hipError_t launch_put_column<V>(V*, uint64_t, uint64_t, V, hipStream_t);             \
    template hipError_t launch_scan_order_free<V>(const V*, V*, uint64_t, bool, uint64_t*,        \
                                                  const ScanLayout&, const ScanOut<V>&,           \
                                                  hipStream_t);                                    \
    template hipError_t launch_scan_rows<V, false, true>(const V*, uint64_t, V*, uint64_t,        \
                                                         uint64_t, uint64_t, bool, int, bool,      \
                                                         const ScanOut<V>*, hipStream_t);
