// Argument checking, workspace sizing and launch planning of the C ABI,
// as templates over the kernels' value type (double / float for IEEE
// addition, OpVal<B, Op> for another operator).  api.cpp instantiates them
// for the built-in operators; a translation unit that adds its own
// operator (canon_user_op.hpp) instantiates the same code for it.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "../../include/canon.h"
#include "device.hpp"
#include "launch.hpp"
#include "reduce.hpp"
#include "scan.hpp"
#include "scan_ip.hpp"

namespace canon {
namespace abi {

// V is the kernels' value type: double / float for +, or OpVal<B, Op> for
// another operator (whose calls reach the reduce kernels and the scan
// kernels with an output stage).
template <typename V>
inline constexpr bool is_op_v = !std::is_same<V, typename Elem<V>::base_t>::value;

// Minimum and maximum are associative and commutative with the semantics of
// device.hpp (NaN payloads aside), so every policy's expression has the same
// value: their scans run one kernel (launch_scan_order_free) whatever the
// policy.
template <typename V>
inline constexpr bool is_order_free_v =
    std::is_same<V, OpVal<typename Elem<V>::base_t, OpMin>>::value ||
    std::is_same<V, OpVal<typename Elem<V>::base_t, OpMax>>::value;

inline thread_local int g_last_hip_error = 0;

inline constexpr uint64_t kReduceTargetWG = 256;  // one streaming workgroup per MI355X CU
inline constexpr size_t kWsAlign = 256;

// Workgroups the streaming reduce aims for (the schedule override's value
// when set): one per CU, fewer for small inputs, where the call's time is
// latency: as few as keep the finishing workgroup's partial values (one per
// workgroup and lane) at 8192 or below, but no fewer than give each
// workgroup at most 128 KiB of input (measured on MI355X at 2^20 doubles:
// L = 128 with 64 workgroups 10.0 us a call back to back, with 256 12.4 us).
inline uint64_t reduce_target_wg(uint64_t n, uint32_t L, size_t es)
{
    const uint64_t v = g_sched_reduce_wg.load(std::memory_order_relaxed);
    if (v) return v;
    uint64_t lp = 1;
    while (lp < L) lp *= 2;
    const uint64_t by_partials = lp < 8192 ? 8192 / lp : 1;
    const uint64_t by_bytes = (n * es + (128u << 10) - 1) >> 17;
    const uint64_t t = by_partials > by_bytes ? by_partials : by_bytes;
    return t < kReduceTargetWG ? t : kReduceTargetWG;
}

inline bool is_pow2(uint64_t v) { return v && !(v & (v - 1)); }

inline int log2_exact(uint64_t v)
{
    int l = 0;
    while ((1ull << l) < v) ++l;
    return l;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline canon_status_t hip_status(hipError_t e)
{
    if (e == hipSuccess) return CANON_OK;
    g_last_hip_error = (int)e;
    return CANON_EHIP;
}

inline canon_status_t check_ws(const void* ws, size_t ws_bytes, size_t need)
{
    if (need == 0) return CANON_OK;
    if (ws == nullptr || ws_bytes < need) return CANON_EWORKSPACE;
    if (((uintptr_t)ws & (kWsAlign - 1)) != 0) return CANON_EWORKSPACE;
    return CANON_OK;
}

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ------------------------------------------------------------------ reduce
inline size_t reduce_ws(uint64_t n, uint32_t L, size_t es)
{
    if (L == 0 || L > CANON_MAX_L || (es != 4 && es != 8)) return 0;
    // the larger of the two possible plans (16-byte aligned input or not)
    const ReducePlan a = plan_reduce(n, L, es, true, reduce_target_wg(n, L, es));
    const ReducePlan b = plan_reduce(n, L, es, false, reduce_target_wg(n, L, es));
    uint64_t need = reduce_ws_layout(a, L, es).bytes;
    const uint64_t nb = reduce_ws_layout(b, L, es).bytes;
    if (nb > need) need = nb;
    return need ? round_up(need, kWsAlign) : 0;
}

// A 64-bit id unique to one reduction call: a per-instance start (the clock
// and the address of the counter, which differs between library instances
// in one process, mixed by the splitmix64 finaliser) plus a counter, never
// 0, so that no earlier call of this or any other library instance, and no
// other data left in a workspace, holds it (a collision needs two 64-bit
// starts within the number of calls made).
inline uint64_t splitmix64(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

inline uint64_t next_reduce_call_id()
{
    static std::atomic<uint64_t> next{0};
    static std::atomic<bool> seeded{false};
    if (!seeded.load(std::memory_order_acquire)) {
        static std::mutex mu;
        std::lock_guard<std::mutex> lock(mu);
        if (!seeded.load(std::memory_order_relaxed)) {
            const uint64_t t =
                (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
            next.store(splitmix64(t ^ splitmix64((uint64_t)(uintptr_t)&next)),
                       std::memory_order_relaxed);
            seeded.store(true, std::memory_order_release);
        }
    }
    uint64_t v;
    do {
        v = next.fetch_add(1, std::memory_order_relaxed);
    } while (v == 0);
    return v;
}

template <typename T>
canon_status_t reduce_impl(const T* x, size_t n, uint32_t L, T init, T* out, void* ws,
                           size_t ws_bytes, void* stream)
{
    if (out == nullptr || L == 0 || (n > 0 && x == nullptr)) return CANON_EINVAL;
    if (L > CANON_MAX_L) return CANON_EUNSUPPORTED;
    const ReducePlan pl =
        plan_reduce(n, L, sizeof(T), aligned16(x), reduce_target_wg(n, L, sizeof(T)));
    // the documented size (covers either plan), so that a caller who sizes by
    // canon_reduce_workspace_bytes is never rejected and never overrun
    if (canon_status_t s = check_ws(ws, ws_bytes, reduce_ws(n, L, sizeof(T)))) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (n == 0) return hip_status(launch_put_column<T>(out, 1, 1, init, st));
    return hip_status(launch_reduce<T>(x, n, L, init, out, ws, pl, next_reduce_call_id(), st));
}

template <typename T>
canon_status_t reduce_rows_impl(const T* x, size_t rows, size_t cols, size_t ldx, uint32_t L,
                                T init, T* out, void* ws, size_t ws_bytes, void* stream)
{
    (void)ws;
    (void)ws_bytes;
    if (L == 0 || ldx < cols || (rows > 0 && out == nullptr) ||
        (rows > 0 && cols > 0 && x == nullptr))
        return CANON_EINVAL;
    if (L > CANON_MAX_L || !reduce_rows_supported(cols, L)) return CANON_EUNSUPPORTED;
    if (rows == 0) return CANON_OK;
    return hip_status(launch_reduce_rows<T>(x, rows, cols, ldx, L, init, out,
                                            static_cast<hipStream_t>(stream)));
}

// -------------------------------------------------------------------- scan
inline canon_status_t check_policy(int policy, uint32_t param)
{
    switch (policy) {
        case CANON_PAIRWISE:
            return (param <= 1) ? CANON_OK : CANON_EINVAL;
        case CANON_ITERATED_PAIRWISE:
            if (param == 0) return CANON_EINVAL;
            return param <= CANON_MAX_IP_L ? CANON_OK : CANON_EUNSUPPORTED;
        case CANON_BLOCK_DYADIC:
            if (param == 0 || !is_pow2(param)) return CANON_EINVAL;
            return param <= CANON_MAX_B ? CANON_OK : CANON_EUNSUPPORTED;
        default:
            return CANON_EINVAL;
    }
}

template <typename T>
ScanLayout scan_layout(uint64_t n, int policy, uint32_t param)
{
    (void)policy;
    (void)param;
    const uint64_t S = 1ull << scan_tile_log<T>();
    return make_scan_layout((n + S - 1) / S, 1);
}

// Node storage of an iterated_pairwise scan, after the 256-byte header whose
// first word is the error word every scan workspace carries.
template <typename T>
T* ip_nodes(void* ws)
{
    return reinterpret_cast<T*>(static_cast<unsigned char*>(ws) + kWsAlign);
}

// iterated_pairwise with L = 1 is the pairwise expression: CR_1 = PW.
inline bool is_ip(int policy, uint32_t param) { return policy == CANON_ITERATED_PAIRWISE && param > 1; }

// The register geometry of the iterated_pairwise scan runs in one pass (its
// items must fit one launch); any other geometry in three kernels.
inline bool ip_single(const IpLayout& ip) { return ip.fast_logrv != kIpNoFast; }
inline bool ip_fits(const IpLayout& ip) { return ip.nseg * ip.tps < (1ull << 31); }

// Workspace of an iterated_pairwise scan: the one-pass plan of the register
// geometry when it applies (it runs at any alignment), else the largest of
// the three-kernel plans (16-byte aligned or not).
inline size_t ip_ws(uint64_t nseg, uint64_t cols, uint32_t L, size_t es)
{
    const IpLayout reg = make_ip_layout(nseg, cols, L, es, true);
    if (ip_single(reg) && ip_fits(reg))
        return round_up(make_ip_single_layout(reg).total_words * 8, kWsAlign);
    size_t need = 0;
    for (int al = 0; al < 2; ++al) {
        const IpLayout ip = make_ip_layout(nseg, cols, L, es, al != 0);
        size_t b = kWsAlign + round_up(ip.total * es, kWsAlign);
        if (ip_single(ip)) {
            const size_t b1 = round_up(make_ip_single_layout(ip).total_words * 8, kWsAlign);
            if (b1 > b) b = b1;
        }
        if (b > need) need = b;
    }
    return need;
}

inline size_t scan_ws(uint64_t n, int policy, uint32_t param, size_t es)
{
    if (check_policy(policy, param) != CANON_OK || (es != 4 && es != 8) || n == 0) return 0;
    if (is_ip(policy, param)) {
        // also enough for the tile layout (the order-free operators run one
        // single-pass scan whatever the policy)
        const size_t a = ip_ws(1, n, param, es);
        const ScanLayout p = es == 8 ? scan_layout<double>(n, CANON_PAIRWISE, 0)
                                     : scan_layout<float>(n, CANON_PAIRWISE, 0);
        const size_t b = round_up(p.total_words * 8, kWsAlign);
        return a > b ? a : b;
    }
    const ScanLayout lay = es == 8 ? scan_layout<double>(n, policy, param)
                                   : scan_layout<float>(n, policy, param);
    return round_up(lay.total_words * 8, kWsAlign);
}

inline size_t scan_rows_ws(uint64_t rows, uint64_t cols, int policy, uint32_t param, size_t es)
{
    if (check_policy(policy, param) != CANON_OK || (es != 4 && es != 8)) return 0;
    if (rows == 0 || cols == 0 || !is_ip(policy, param)) return 0;
    return ip_ws(rows, cols, param, es);
}

// out == null: the plain inclusive scan; else the scan with an initial value.
template <typename T>
canon_status_t scan_impl(const T* x, T* y, size_t n, int policy, uint32_t param,
                         const ScanOut<T>* out, void* ws, size_t ws_bytes, void* stream)
{
    if (canon_status_t s = check_policy(policy, param)) return s;
    if (out && (out->kind < CANON_SCAN_INCLUSIVE || out->kind > CANON_SCAN_INCLUDE_INITIAL))
        return CANON_EINVAL;
    if (n > 0 && (x == nullptr || y == nullptr)) return CANON_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (n == 0) {
        if (!out || out->kind != CANON_SCAN_INCLUDE_INITIAL) return CANON_OK;
        if (y == nullptr) return CANON_EINVAL;
        return hip_status(launch_put_column<T>(y, 1, 1, out->init, st));
    }
    if constexpr (is_order_free_v<T>) {
        const ScanLayout lay = scan_layout<T>(n, CANON_PAIRWISE, 0);
        if (lay.ntiles > 0xFFFFFFFFull) return CANON_EUNSUPPORTED;
        if (canon_status_t s = check_ws(ws, ws_bytes, scan_ws(n, policy, param, sizeof(T))))
            return s;
        return hip_status(launch_scan_order_free<T>(x, y, n, aligned16(x) && aligned16(y),
                                                    static_cast<uint64_t*>(ws), lay, *out, st));
    } else if (is_ip(policy, param)) {
        const bool al = aligned16(x) && aligned16(y);
        if (canon_status_t s = check_ws(ws, ws_bytes, scan_ws(n, policy, param, sizeof(T))))
            return s;
        // the register geometry runs in one pass at any alignment
        const IpLayout reg = make_ip_layout(1, n, param, sizeof(T), true);
        if (ip_single(reg) && ip_fits(reg))
            return hip_status(launch_scan_ip_single<T, !is_op_v<T>>(
                x, n, y, n, n, static_cast<uint64_t*>(ws), make_ip_single_layout(reg), out, al,
                st));
        const IpLayout ip = make_ip_layout(1, n, param, sizeof(T), al);
        if (ip_single(ip)) return CANON_EUNSUPPORTED;  // too many tiles for one launch
        return hip_status(launch_scan_ip<T, !is_op_v<T>>(x, n, y, n, 1, n,
                                                         static_cast<uint32_t*>(ws),
                                                         ip_nodes<T>(ws), ip, out, st));
    }
    const ScanLayout lay = scan_layout<T>(n, policy, param);
    if (lay.ntiles > 0xFFFFFFFFull) return CANON_EUNSUPPORTED;
    if (canon_status_t s = check_ws(ws, ws_bytes, round_up(lay.total_words * 8, kWsAlign)))
        return s;
    const bool pairwise = policy != CANON_BLOCK_DYADIC;  // pairwise, or iterated_pairwise<1>
    const int b_log = pairwise ? 0 : log2_exact(param);
    const bool al = aligned16(x) && aligned16(y);
    if (out)
        return hip_status(launch_scan_with_init<T>(x, y, n, pairwise, b_log, al,
                                                   static_cast<uint64_t*>(ws), lay, *out, st));
    if constexpr (!is_op_v<T>)
        return hip_status(
            launch_scan<T>(x, y, n, pairwise, b_log, al, static_cast<uint64_t*>(ws), lay, st));
    return CANON_EINVAL;
}

template <typename T>
canon_status_t scan_rows_impl(const T* x, size_t ldx, T* y, size_t ldy, size_t rows, size_t cols,
                              int policy, uint32_t param, const ScanOut<T>* out, void* ws,
                              size_t ws_bytes, void* stream)
{
    if (canon_status_t s = check_policy(policy, param)) return s;
    if (out && (out->kind < CANON_SCAN_INCLUSIVE || out->kind > CANON_SCAN_INCLUDE_INITIAL))
        return CANON_EINVAL;
    const size_t ycols = out && out->kind == CANON_SCAN_INCLUDE_INITIAL ? cols + 1 : cols;
    if (ldx < cols || ldy < ycols) return CANON_EINVAL;
    if (rows > 0 && cols > 0 && x == nullptr) return CANON_EINVAL;
    if (rows > 0 && ycols > 0 && y == nullptr) return CANON_EINVAL;
    if (rows == 0 || ycols == 0) return CANON_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (cols == 0) return hip_status(launch_put_column<T>(y, ldy, rows, out->init, st));
    if constexpr (is_order_free_v<T>) {
        const bool al = aligned16(x) && aligned16(y) && (ldx * sizeof(T)) % 16 == 0 &&
                        (ldy * sizeof(T)) % 16 == 0;
        // this row kernel waits for nothing; a workspace it was given still
        // gets a cleared error word (its first bytes), as every scan's does
        if (ws != nullptr && ws_bytes >= sizeof(T)) {
            using bits_t = typename Elem<T>::bits_t;
            const hipError_t e = launch_put_column<T>(static_cast<T*>(ws), 1, 1,
                                                      __builtin_bit_cast(T, bits_t(0)), st);
            if (e != hipSuccess) return hip_status(e);
        }
        return hip_status(launch_scan_rows<T, false, true>(x, ldx, y, ldy, rows, cols, true, 0, al,
                                                           out, st));
    } else if (is_ip(policy, param)) {
        const bool al = aligned16(x) && aligned16(y) && (ldx * sizeof(T)) % 16 == 0 &&
                        (ldy * sizeof(T)) % 16 == 0;
        if (canon_status_t s =
                check_ws(ws, ws_bytes, scan_rows_ws(rows, cols, policy, param, sizeof(T))))
            return s;
        // the register geometry runs in one pass at any alignment
        const IpLayout reg = make_ip_layout(rows, cols, param, sizeof(T), true);
        if (ip_single(reg) && ip_fits(reg))
            return hip_status(launch_scan_ip_single<T, !is_op_v<T>>(
                x, ldx, y, ldy, cols, static_cast<uint64_t*>(ws), make_ip_single_layout(reg), out,
                al, st));
        const IpLayout ip = make_ip_layout(rows, cols, param, sizeof(T), al);
        if (ip_single(ip)) return CANON_EUNSUPPORTED;  // too many tiles for one launch
        return hip_status(launch_scan_ip<T, !is_op_v<T>>(x, ldx, y, ldy, rows, cols,
                                            static_cast<uint32_t*>(ws), ip_nodes<T>(ws), ip, out,
                                            st));
    }
    const bool pairwise = policy != CANON_BLOCK_DYADIC;
    const int b_log = pairwise ? 0 : log2_exact(param);
    const bool al = aligned16(x) && aligned16(y) && (ldx * sizeof(T)) % 16 == 0 &&
                    (ldy * sizeof(T)) % 16 == 0;
    return hip_status(launch_scan_rows<T, !is_op_v<T>>(x, ldx, y, ldy, rows, cols, pairwise, b_log,
                                                       al, out, st));
}

// The entry points for one value type V whose base type is B (the caller's
// element type): argument bits passed through unchanged.
template <typename V, typename B>
canon_status_t reduce_as(const B* x, size_t n, uint32_t L, B init, B* out, void* ws,
                         size_t ws_bytes, void* stream)
{
    return reduce_impl<V>(reinterpret_cast<const V*>(x), n, L, __builtin_bit_cast(V, init),
                          reinterpret_cast<V*>(out), ws, ws_bytes, stream);
}

template <typename V, typename B>
canon_status_t reduce_rows_as(const B* x, size_t rows, size_t cols, size_t ldx, uint32_t L,
                              B init, B* out, void* ws, size_t ws_bytes, void* stream)
{
    return reduce_rows_impl<V>(reinterpret_cast<const V*>(x), rows, cols, ldx, L,
                               __builtin_bit_cast(V, init), reinterpret_cast<V*>(out), ws,
                               ws_bytes, stream);
}

template <typename V, typename B>
canon_status_t scan_as(const B* x, B* y, size_t n, int policy, uint32_t param, int kind, B init,
                       void* ws, size_t ws_bytes, void* stream)
{
    const ScanOut<V> out{__builtin_bit_cast(V, init), kind};
    return scan_impl<V>(reinterpret_cast<const V*>(x), reinterpret_cast<V*>(y), n, policy, param,
                        &out, ws, ws_bytes, stream);
}

template <typename V, typename B>
canon_status_t scan_rows_as(const B* x, size_t ldx, B* y, size_t ldy, size_t rows, size_t cols,
                            int policy, uint32_t param, int kind, B init, void* ws,
                            size_t ws_bytes, void* stream)
{
    const ScanOut<V> out{__builtin_bit_cast(V, init), kind};
    return scan_rows_impl<V>(reinterpret_cast<const V*>(x), ldx, reinterpret_cast<V*>(y), ldy,
                             rows, cols, policy, param, &out, ws, ws_bytes, stream);
}

}  // namespace abi
}  // namespace canon
