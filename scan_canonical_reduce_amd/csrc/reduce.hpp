// Launch planning for the reduction kernels (host and device shared constants).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace canon {

constexpr int kReduceThreads = 1024;  // general streaming workgroups
constexpr int kReduceWaves = kReduceThreads / 64;
constexpr int kReduceBatch = 8;        // 16-byte vectors per thread per batch
constexpr int kReduceStackDepth = 10;  // batches per wave <= 2^10
constexpr int kRowsThreads = 256;      // row-batched workgroups
constexpr int kMaxLogL = 16;
constexpr uint64_t kPartialBudget = 1ull << 16;  // partial values (P * Lp) aimed for

// Threads of the register-path streaming workgroup (one workgroup per CU),
// by layout (measured on MI355X at N = 2^28): 256 for the row-group layout
// (rows of at least 8 vectors: four waves keep about 32 KiB of loads in
// flight per CU, which streams fastest), 512 for the interleaved layouts,
// whose cross-lane swizzles want more waves to hide their latency, and 1024
// for the interleaved layout with whole vectors of lanes across all 64
// lanes (the most swizzles per element).
constexpr int pow2_reduce_threads(int logc, bool whole_vectors)
{
    return logc >= 3 ? 256 : ((logc == 0 && whole_vectors) ? 1024 : 512);
}

struct ReducePlan {
    bool pow2;       // register path (L = 2^logl, 16-byte aligned input)
    int logl;        // log2 L (pow2 path)
    int lp_log;      // log2 of L rounded up to a power of two
    uint64_t P;      // row ranges (grid.x); partial rows
    uint64_t slices; // grid.y: column slices (pow2) or lane chunks (general)
    int rw_log;      // pow2: log2 super-rows per wave
    int lw_log;      // general: log2 lanes per workgroup chunk
    int rs_log;      // general: log2 rows per thread segment
};

inline int ceil_log2(uint64_t v)
{
    int l = 0;
    while ((1ull << l) < v) ++l;
    return l;
}

// target_wg: workgroups the streaming kernel aims for (one per CU of MI355X).
inline ReducePlan plan_reduce(uint64_t n, uint32_t L, size_t elem_size, bool aligned16,
                              uint64_t target_wg)
{
    ReducePlan pl{};
    pl.lp_log = ceil_log2(L);
    const uint64_t Lp = 1ull << pl.lp_log;
    const bool is_pow2 = (Lp == L);
    pl.pow2 = is_pow2 && aligned16 && pl.lp_log <= kMaxLogL;
    pl.logl = pl.lp_log;
    if (n == 0) {
        pl.P = 0;
        pl.slices = 1;
        return pl;
    }
    uint64_t budgetP = kPartialBudget / Lp;
    if (budgetP < 1) budgetP = 1;
    if (pl.pow2) {
        const int loge = elem_size == 8 ? 1 : 2;
        const int log_sr = pl.logl > loge ? pl.logl : loge;
        const int logc = log_sr - loge;
        const int log_cw = logc < 6 ? logc : 6;
        const int logg = 6 - log_cw;
        const uint64_t GU = (uint64_t)kReduceBatch << logg;
        const uint64_t waves = pow2_reduce_threads(logc, pl.logl >= loge) / 64;
        pl.slices = 1ull << (logc - log_cw);
        const uint64_t msr = (n + (1ull << log_sr) - 1) >> log_sr;
        uint64_t pt = target_wg / pl.slices;
        if (pt < 1) pt = 1;
        if (pt > budgetP) pt = budgetP;
        uint64_t want = (msr + pt * waves - 1) / (pt * waves);
        uint64_t rw = GU;
        while (rw < want) rw *= 2;
        const uint64_t rw_max = GU << kReduceStackDepth;
        if (rw > rw_max) rw = rw_max;
        pl.rw_log = ceil_log2(rw);
        pl.P = (msr + rw * waves - 1) / (rw * waves);
    } else {
        const uint64_t m = (n + L - 1) / L;
        const uint64_t LW = Lp < (uint64_t)kReduceThreads ? Lp : (uint64_t)kReduceThreads;
        pl.lw_log = ceil_log2(LW);
        const uint64_t S = kReduceThreads / LW;
        pl.slices = (L + LW - 1) / LW;
        uint64_t pt = target_wg / pl.slices;
        if (pt < 1) pt = 1;
        if (pt > budgetP) pt = budgetP;
        uint64_t want = (m + pt * S - 1) / (pt * S);
        uint64_t rs = 1;
        while (rs < want) rs *= 2;
        const uint64_t rs_max = 8ull << kReduceStackDepth;
        if (rs > rs_max) rs = rs_max;
        pl.rs_log = ceil_log2(rs);
        pl.P = (m + rs * S - 1) / (rs * S);
    }
    return pl;
}

// Rounds per row: fewer than 2^(kRowsRoundDepth + 1).  A round holds at least
// 2^13 * S rows-of-L with L * S >= 128, so this covers rows of 2^45 elements,
// far beyond device memory; longer rows are rejected before launch.
constexpr int kRowsRoundDepth = 24;

// Rows-of-L per thread segment: the smallest power of two with rs * S >= m,
// capped so that a segment holds at most 2^kReduceStackDepth batches of 8.
__host__ __device__ inline uint64_t rows_segment_len(uint64_t m, int S)
{
    uint64_t rs = 1;
    while (rs * (uint64_t)S < m && rs < (8ull << kReduceStackDepth)) rs *= 2;
    return rs;
}

// Whether the general row kernel can reduce rows of `cols` elements (its
// round stack bounds the row length; see kRowsRoundDepth).
inline bool reduce_rows_supported(uint64_t cols, uint32_t L)
{
    int lp_log = 0;
    while ((1ull << lp_log) < L) ++lp_log;
    const int S = kRowsThreads >> (lp_log < 8 ? lp_log : 8);
    const uint64_t m = (cols + L - 1) / L;
    const uint64_t span = rows_segment_len(m, S) * S;
    return (m + span - 1) / span < (1ull << (kRowsRoundDepth + 1));
}

// Workspace of a reduction (byte offsets), for a plan with P > 0:
//   [0, 256): header; bytes 0-3 the error word, which the finishing
//     workgroup writes on every call (0, or kErrSpin when its bounded wait
//     for the other workgroups gave up);
//   [partial_off, +P * L values): the partial lane values, row p of L values
//     from row range p;
//   [flags_off, +P * slices 64-bit words): one arrival flag per streaming
//     workgroup, which holds the call's id once its partials are out.
struct ReduceWs {
    uint64_t partial_off, flags_off, bytes;
};

inline ReduceWs reduce_ws_layout(const ReducePlan& pl, uint32_t L, size_t elem_size)
{
    ReduceWs w{};
    if (pl.P == 0) return w;
    w.partial_off = 256;
    w.flags_off = w.partial_off + (pl.P * (uint64_t)L * elem_size + 255) / 256 * 256;
    w.bytes = w.flags_off + pl.P * pl.slices * 8;
    return w;
}

// n > 0.  call_id: unique to this call (never 0, never what an earlier call
// or any other data left in the flags).  POW2 = false: only the general
// streaming kernel is built; the plan must then be one for unaligned input
// (pl.pow2 false).
template <typename T, bool POW2 = true>
hipError_t launch_reduce(const T* x, uint64_t n, uint32_t L, T init, T* out, void* ws,
                         const ReducePlan& pl, uint64_t call_id, hipStream_t s);

template <typename T>
hipError_t launch_reduce_rows(const T* x, uint64_t rows, uint64_t cols, uint64_t ldx, uint32_t L,
                              T init, T* out, hipStream_t s);

}  // namespace canon
