// canon_scan_noalloc_f64: canon_scan_f64 with the workspace in a static
// device array of the library, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// `scratch` below is that array.  Each device the library runs on holds its
// own copy until the process ends; its device address differs per device and
// is resolved once per device with hipGetSymbolAddress (in host code the
// array's name is only a host-side stand-in, never a device address).  The
// scan kernels set every word they read before reading it (the status and
// node words are re-marked by the scan's own init kernel on every call, the
// error word and ticket cleared), so the contents a previous call left behind
// do not matter.  Every call on one device shares the array: calls that may
// overlap on one device (other streams, other host threads) race and must
// not be issued.
#include <mutex>

#include "api_impl.hpp"

using namespace canon;
using namespace canon::abi;

namespace {

constexpr size_t kScratchBytes = CANON_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte units");

static __device__ __align__(256) uint64_t scratch[kScratchBytes / sizeof(uint64_t)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// The device address of `scratch` on the current device, resolved on the
// first call made with that device current.
canon_status_t scratch_on_current_device(void** out)
{
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return CANON_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (g != hipSuccess) return hip_status(g);
        if (p == nullptr) return hip_status(hipErrorInvalidSymbol);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CANON_OK;
}

}  // namespace

extern "C" canon_status_t canon_scan_noalloc_f64(const double* x, double* y, size_t n, int policy,
                                                 uint32_t param, void* stream)
{
    if (canon_status_t s = check_policy(policy, param)) return s;
    if (n > 0 && (x == nullptr || y == nullptr)) return CANON_EINVAL;
    if (n == 0) return CANON_OK;
    if (scan_ws(n, policy, param, sizeof(double)) > kScratchBytes) return CANON_EUNSUPPORTED;
    void* ws = nullptr;
    if (canon_status_t s = scratch_on_current_device(&ws)) return s;
    return scan_impl<double>(x, y, n, policy, param, nullptr, ws, kScratchBytes, stream);
}
