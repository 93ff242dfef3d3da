// libcanon C ABI: argument checking, workspace sizing, launch planning.
//
// Every entry point validates its arguments before anything is enqueued,
// then enqueues its kernels on the caller's stream and returns.  The library
// keeps no device memory and no state between calls, apart from the
// thread-local HIP error code of the last failed launch.
#include "api_impl.hpp"

using namespace canon;
using namespace canon::abi;

namespace {

// Calls f with a value of type Tag<V>, V the kernels' value type for the
// operator `op` over base type B (CANON_EINVAL for an unknown operator).
template <typename V>
struct Tag {
    using type = V;
};

template <typename B, class F>
canon_status_t with_op(int op, F&& f)
{
    switch (op) {
        case CANON_OP_ADD: return f(Tag<B>{});
        case CANON_OP_MUL: return f(Tag<OpVal<B, OpMul>>{});
        case CANON_OP_MIN: return f(Tag<OpVal<B, OpMin>>{});
        case CANON_OP_MAX: return f(Tag<OpVal<B, OpMax>>{});
        default: return CANON_EINVAL;
    }
}

template <typename B>
canon_status_t reduce_op(const B* x, size_t n, uint32_t L, int op, B init, B* out, void* ws,
                         size_t ws_bytes, void* stream)
{
    return with_op<B>(op, [&](auto tag) {
        return reduce_as<typename decltype(tag)::type>(x, n, L, init, out, ws, ws_bytes, stream);
    });
}

template <typename B>
canon_status_t reduce_rows_op(const B* x, size_t rows, size_t cols, size_t ldx, uint32_t L,
                              int op, B init, B* out, void* ws, size_t ws_bytes, void* stream)
{
    return with_op<B>(op, [&](auto tag) {
        return reduce_rows_as<typename decltype(tag)::type>(x, rows, cols, ldx, L, init, out, ws,
                                                            ws_bytes, stream);
    });
}

template <typename B>
canon_status_t scan_op(const B* x, B* y, size_t n, int policy, uint32_t param, int op, int kind,
                       B init, void* ws, size_t ws_bytes, void* stream)
{
    return with_op<B>(op, [&](auto tag) {
        return scan_as<typename decltype(tag)::type>(x, y, n, policy, param, kind, init, ws,
                                                     ws_bytes, stream);
    });
}

template <typename B>
canon_status_t scan_rows_op(const B* x, size_t ldx, B* y, size_t ldy, size_t rows, size_t cols,
                            int policy, uint32_t param, int op, int kind, B init, void* ws,
                            size_t ws_bytes, void* stream)
{
    return with_op<B>(op, [&](auto tag) {
        return scan_rows_as<typename decltype(tag)::type>(x, ldx, y, ldy, rows, cols, policy,
                                                          param, kind, init, ws, ws_bytes,
                                                          stream);
    });
}

}  // namespace

extern "C" {

int canon_abi_version(void) { return CANON_ABI_VERSION; }

const char* canon_status_str(int s)
{
    switch (s) {
        case CANON_OK: return "CANON_OK";
        case CANON_EINVAL: return "CANON_EINVAL: invalid argument";
        case CANON_EUNSUPPORTED: return "CANON_EUNSUPPORTED: parameter outside the supported range";
        case CANON_EWORKSPACE: return "CANON_EWORKSPACE: workspace too small or misaligned";
        case CANON_EHIP: return "CANON_EHIP: HIP launch failed";
        default: return "unknown canon status";
    }
}

int canon_last_hip_error(void) { return g_last_hip_error; }

size_t canon_reduce_workspace_bytes(size_t n, uint32_t L, size_t elem_size)
{
    return reduce_ws(n, L, elem_size);
}

canon_status_t canon_reduce_f64(const double* x, size_t n, uint32_t L, double init, double* out,
                                void* ws, size_t ws_bytes, void* stream)
{
    return reduce_impl<double>(x, n, L, init, out, ws, ws_bytes, stream);
}

canon_status_t canon_reduce_f32(const float* x, size_t n, uint32_t L, float init, float* out,
                                void* ws, size_t ws_bytes, void* stream)
{
    return reduce_impl<float>(x, n, L, init, out, ws, ws_bytes, stream);
}

size_t canon_reduce_rows_workspace_bytes(size_t rows, size_t cols, uint32_t L, size_t elem_size)
{
    (void)rows;
    (void)cols;
    (void)L;
    (void)elem_size;
    return 0;
}

canon_status_t canon_reduce_rows_f64(const double* x, size_t rows, size_t cols, size_t ldx,
                                     uint32_t L, double init, double* out, void* ws,
                                     size_t ws_bytes, void* stream)
{
    return reduce_rows_impl<double>(x, rows, cols, ldx, L, init, out, ws, ws_bytes, stream);
}

canon_status_t canon_reduce_rows_f32(const float* x, size_t rows, size_t cols, size_t ldx,
                                     uint32_t L, float init, float* out, void* ws,
                                     size_t ws_bytes, void* stream)
{
    return reduce_rows_impl<float>(x, rows, cols, ldx, L, init, out, ws, ws_bytes, stream);
}

size_t canon_scan_workspace_bytes(size_t n, int policy, uint32_t param, size_t elem_size)
{
    return scan_ws(n, policy, param, elem_size);
}

canon_status_t canon_scan_f64(const double* x, double* y, size_t n, int policy, uint32_t param,
                              void* ws, size_t ws_bytes, void* stream)
{
    return scan_impl<double>(x, y, n, policy, param, nullptr, ws, ws_bytes, stream);
}

canon_status_t canon_scan_f32(const float* x, float* y, size_t n, int policy, uint32_t param,
                              void* ws, size_t ws_bytes, void* stream)
{
    return scan_impl<float>(x, y, n, policy, param, nullptr, ws, ws_bytes, stream);
}

size_t canon_scan_rows_workspace_bytes(size_t rows, size_t cols, int policy, uint32_t param,
                                       size_t elem_size)
{
    return scan_rows_ws(rows, cols, policy, param, elem_size);
}

canon_status_t canon_scan_rows_f64(const double* x, size_t ldx, double* y, size_t ldy,
                                   size_t rows, size_t cols, int policy, uint32_t param,
                                   void* ws, size_t ws_bytes, void* stream)
{
    return scan_rows_impl<double>(x, ldx, y, ldy, rows, cols, policy, param, nullptr, ws, ws_bytes,
                                  stream);
}

canon_status_t canon_scan_rows_f32(const float* x, size_t ldx, float* y, size_t ldy, size_t rows,
                                   size_t cols, int policy, uint32_t param, void* ws,
                                   size_t ws_bytes, void* stream)
{
    return scan_rows_impl<float>(x, ldx, y, ldy, rows, cols, policy, param, nullptr, ws, ws_bytes,
                                 stream);
}

canon_status_t canon_scan_with_init_f64(const double* x, double* y, size_t n, int policy,
                                       uint32_t param, int kind, double init, void* ws,
                                       size_t ws_bytes, void* stream)
{
    const ScanOut<double> out{init, kind};
    return scan_impl<double>(x, y, n, policy, param, &out, ws, ws_bytes, stream);
}

canon_status_t canon_scan_with_init_f32(const float* x, float* y, size_t n, int policy,
                                       uint32_t param, int kind, float init, void* ws,
                                       size_t ws_bytes, void* stream)
{
    const ScanOut<float> out{init, kind};
    return scan_impl<float>(x, y, n, policy, param, &out, ws, ws_bytes, stream);
}

canon_status_t canon_scan_rows_with_init_f64(const double* x, size_t ldx, double* y, size_t ldy,
                                            size_t rows, size_t cols, int policy, uint32_t param,
                                            int kind, double init, void* ws, size_t ws_bytes,
                                            void* stream)
{
    const ScanOut<double> out{init, kind};
    return scan_rows_impl<double>(x, ldx, y, ldy, rows, cols, policy, param, &out, ws, ws_bytes,
                                  stream);
}

canon_status_t canon_scan_rows_with_init_f32(const float* x, size_t ldx, float* y, size_t ldy,
                                            size_t rows, size_t cols, int policy, uint32_t param,
                                            int kind, float init, void* ws, size_t ws_bytes,
                                            void* stream)
{
    const ScanOut<float> out{init, kind};
    return scan_rows_impl<float>(x, ldx, y, ldy, rows, cols, policy, param, &out, ws, ws_bytes,
                                 stream);
}

canon_status_t canon_reduce_op_f64(const double* x, size_t n, uint32_t L, int op, double init,
                                   double* out, void* ws, size_t ws_bytes, void* stream)
{
    return reduce_op<double>(x, n, L, op, init, out, ws, ws_bytes, stream);
}

canon_status_t canon_reduce_op_f32(const float* x, size_t n, uint32_t L, int op, float init,
                                   float* out, void* ws, size_t ws_bytes, void* stream)
{
    return reduce_op<float>(x, n, L, op, init, out, ws, ws_bytes, stream);
}

canon_status_t canon_reduce_rows_op_f64(const double* x, size_t rows, size_t cols, size_t ldx,
                                        uint32_t L, int op, double init, double* out, void* ws,
                                        size_t ws_bytes, void* stream)
{
    return reduce_rows_op<double>(x, rows, cols, ldx, L, op, init, out, ws, ws_bytes, stream);
}

canon_status_t canon_reduce_rows_op_f32(const float* x, size_t rows, size_t cols, size_t ldx,
                                        uint32_t L, int op, float init, float* out, void* ws,
                                        size_t ws_bytes, void* stream)
{
    return reduce_rows_op<float>(x, rows, cols, ldx, L, op, init, out, ws, ws_bytes, stream);
}

canon_status_t canon_scan_op_f64(const double* x, double* y, size_t n, int policy, uint32_t param,
                                 int op, int kind, double init, void* ws, size_t ws_bytes,
                                 void* stream)
{
    return scan_op<double>(x, y, n, policy, param, op, kind, init, ws, ws_bytes, stream);
}

canon_status_t canon_scan_op_f32(const float* x, float* y, size_t n, int policy, uint32_t param,
                                 int op, int kind, float init, void* ws, size_t ws_bytes,
                                 void* stream)
{
    return scan_op<float>(x, y, n, policy, param, op, kind, init, ws, ws_bytes, stream);
}

canon_status_t canon_scan_rows_op_f64(const double* x, size_t ldx, double* y, size_t ldy,
                                      size_t rows, size_t cols, int policy, uint32_t param,
                                      int op, int kind, double init, void* ws, size_t ws_bytes,
                                      void* stream)
{
    return scan_rows_op<double>(x, ldx, y, ldy, rows, cols, policy, param, op, kind, init, ws,
                                ws_bytes, stream);
}

canon_status_t canon_scan_rows_op_f32(const float* x, size_t ldx, float* y, size_t ldy,
                                      size_t rows, size_t cols, int policy, uint32_t param,
                                      int op, int kind, float init, void* ws, size_t ws_bytes,
                                      void* stream)
{
    return scan_rows_op<float>(x, ldx, y, ldy, rows, cols, policy, param, op, kind, init, ws,
                               ws_bytes, stream);
}

canon_status_t canon_workspace_error(const void* ws, uint32_t* err_out, void* stream)
{
    if (ws == nullptr || err_out == nullptr) return CANON_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(err_out, ws, sizeof(uint32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return hip_status(e);
}

size_t canon_scan_tile_elems(int policy, uint32_t param, size_t elem_size)
{
    if (check_policy(policy, param) != CANON_OK || (elem_size != 4 && elem_size != 8)) return 0;
    if (is_ip(policy, param)) {
        const IpLayout ip = make_ip_layout(1, 1, param, elem_size, true);
        return (size_t)(1ull << ip.r_log) * param;
    }
    return (size_t)1 << (elem_size == 8 ? scan_tile_log<double>() : scan_tile_log<float>());
}

size_t canon_scan_rows_tile_elems(int policy, uint32_t param, size_t elem_size)
{
    if (check_policy(policy, param) != CANON_OK || (elem_size != 4 && elem_size != 8)) return 0;
    if (is_ip(policy, param)) return canon_scan_tile_elems(policy, param, elem_size);
    // E elements per vector, 64 lanes, 2^scan_rows_log_v vectors, 4 waves
    return elem_size == 8 ? (size_t)2 << (6 + scan_rows_log_v<double>() + 2)
                          : (size_t)4 << (6 + scan_rows_log_v<float>() + 2);
}

canon_status_t canon_set_schedule(int knob, uint64_t value)
{
    switch (knob) {
        case CANON_SCHED_GRID: g_sched_grid_cap.store(value, std::memory_order_relaxed); break;
        case CANON_SCHED_REDUCE_PARTIALS:
            g_sched_reduce_wg.store(value, std::memory_order_relaxed);
            break;
        case CANON_SCHED_SPIN_LIMIT: g_sched_spin_limit.store(value, std::memory_order_relaxed); break;
        default: return CANON_EINVAL;
    }
    return CANON_OK;
}

uint64_t canon_get_schedule(int knob)
{
    switch (knob) {
        case CANON_SCHED_GRID: return g_sched_grid_cap.load(std::memory_order_relaxed);
        case CANON_SCHED_REDUCE_PARTIALS: return g_sched_reduce_wg.load(std::memory_order_relaxed);
        case CANON_SCHED_SPIN_LIMIT: return g_sched_spin_limit.load(std::memory_order_relaxed);
        default: return 0;
    }
}

}  // extern "C"
