// Canonical inclusive scan kernels, policies pairwise and block_dyadic<B>
// (gfx950).
//
// Expressions (canonical-reduce README, P4229R0 "Summary" / "Key Design
// Points"): y[i] is the value of the policy's expression over x[0..i].
//   pairwise:        PW(x[0..i]).  Writing n = i + 1 as a sum of distinct
//                    powers of two, PW over n items is the right-nested sum of
//                    the complete pairwise trees over the aligned ranges those
//                    powers mark out, largest first: T1 + (T2 + (... + Tk)).
//   block_dyadic<B>: with n = qB + t, PW(whole blocks) + PW(tail), i.e.
//                    C + W where C = PW(x[0..qB)) (the pairwise value at the
//                    previous block end) and W the pairwise prefix inside the
//                    open block; at a block end simply PW(x[0..n)).
//
// Evaluation: a Sklansky network.  Merge level lam joins aligned halves of
// 2^(lam-1) elements; every element of the upper half receives, on its left,
// the value at the end of the lower half, which is the complete pairwise tree
// of that half.  Applying levels lam = 1, 2, ... in order builds exactly the
// right-nested form above.  For block_dyadic with B = 2^b, levels lam <= b
// act on the element value as for pairwise (building W); for lam > b a block
// end keeps building its pairwise value, while every other element collects
// the received nodes in a separate carry C (same right-nested order), and
// outputs C + W.  Pairwise is the case B = 1 (every element is a block end).
//
// Levels inside a 16-byte vector, across the 64 lanes of a wave (ds_swizzle),
// across a thread's 8 vectors (readlane), across the 4 waves (LDS) and across
// tiles (published node values, below) are the same network.
//
// Across tiles (single pass): tile t publishes its tile total (its complete
// tree).  Tile-level node (k, u) covers tiles [u 2^k, (u+1) 2^k).  Tile t
// needs the nodes for the set bits k of t, node (k, (t >> k) - 1).  Nodes of
// level < 6 are rebuilt by tile t itself from the published totals of the at
// most 63 tiles before it in its aligned group of 64 (one wave, a butterfly
// in fixed lane order); nodes of level >= 6 are published by the last tile of
// their range, which climbs: node (6, t>>6) = its rebuilt low nodes plus its
// own total, and node (k+1, t>>(k+1)) = node (k, (t>>k) - 1) + node (k, t>>k)
// while bit k of t is set.  Every value is fixed by position only, never by
// arrival order.  Tile numbers come from an atomic counter, so every tile
// waited on belongs to a workgroup that is already running.
#include "device.hpp"
#include "launch.hpp"
#include "scan.hpp"

namespace canon {

// Scan state of one tile.  MODE 0: pairwise.  MODE 1: block_dyadic with
// B >= E (a 16-byte vector never straddles two blocks).  MODE 2: block_dyadic
// with B = 2 < E (float: two blocks per vector).
//
// block_dyadic keeps, per block, a carry c (nodes received at levels above
// b, right-nested) and the block end's pairwise value pe; levels <= b build
// the in-block prefix W in v.  From level b+1 on ("fork"), every level
// updates c and pe of the receiving blocks and never touches v again.
template <typename T, int MODE, int LOGV_ = 3>
struct ScanTile {
    static constexpr int E = Elem<T>::E;
    static constexpr int LOGE = Elem<T>::LOGE;
    static constexpr int LOGV = LOGV_;
    static constexpr int V = 1 << LOGV;
    static constexpr int LOG_WSPAN = LOGE + 6 + LOGV;  // elements per wave (log2)
    static constexpr int LOG_S = LOG_WSPAN + 2;        // elements per tile (log2)
    static constexpr bool BD = MODE != 0;
    static constexpr int NB = MODE == 2 ? E / 2 : 1;   // blocks per vector
    static_assert(MODE != 2 || E == 4, "two-element blocks inside a vector: float only");

    T v[V][E];
    T c[V][NB];
    T pe[V][NB];
    int b;        // log2 B
    bool forked;  // a level above b has been applied

    __device__ __forceinline__ void begin(int b_log)
    {
        b = MODE == 2 ? 1 : b_log;
        forked = false;
    }

    // value at the end of vector u's last slot: the source a receiving half
    // takes from the end of the lower half
    __device__ __forceinline__ T last(int u) const
    {
        if constexpr (BD) return forked ? pe[u][NB - 1] : v[u][E - 1];
        return v[u][E - 1];
    }

    __device__ __forceinline__ void fork()
    {
        if constexpr (BD) {
#pragma unroll
            for (int u = 0; u < V; ++u)
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    pe[u][k] = v[u][k * (E / NB) + (E / NB) - 1];
                    c[u][k] = neg_zero<T>();
                }
            forked = true;
        }
    }
    __device__ __forceinline__ void maybe_fork(int lam)
    {
        if constexpr (BD)
            if (!forked && lam > b) fork();
    }

    // Every block of vector u receives s at level lam (lam > LOGE).
    __device__ __forceinline__ void apply_vec(int lam, T s, int u)
    {
        if (!BD || lam <= b) {
#pragma unroll
            for (int e = 0; e < E; ++e) v[u][e] = s + v[u][e];
        } else {
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                c[u][k] = s + c[u][k];
                pe[u][k] = s + pe[u][k];
            }
        }
    }
    __device__ __forceinline__ void apply_all(int lam, T s)
    {
        maybe_fork(lam);
#pragma unroll
        for (int u = 0; u < V; ++u) apply_vec(lam, s, u);
    }

    // Levels inside a vector (static positions).
    __device__ __forceinline__ void slot_levels()
    {
        // level 1: odd slots receive the even slot before them
        maybe_fork(1);
#pragma unroll
        for (int u = 0; u < V; ++u)
#pragma unroll
            for (int e = 1; e < E; e += 2) v[u][e] = v[u][e - 1] + v[u][e];
        if constexpr (LOGE >= 2) {
            // level 2 (float): slots 2, 3 receive slot 1
            maybe_fork(2);
            if (MODE == 2) {
                // b = 1: the second block of the vector receives the first
#pragma unroll
                for (int u = 0; u < V; ++u) {
                    c[u][1] = pe[u][0] + c[u][1];
                    pe[u][1] = pe[u][0] + pe[u][1];
                }
            } else if (!BD || 2 <= b) {
#pragma unroll
                for (int u = 0; u < V; ++u) {
                    v[u][2] = v[u][1] + v[u][2];
                    v[u][3] = v[u][1] + v[u][3];
                }
            }
        }
    }

    template <int K>
    __device__ __forceinline__ void lane_level(int lane)
    {
        constexpr int H = 1 << K;
        const int lam = LOGE + 1 + K;
        maybe_fork(lam);
        const bool upper = (lane >> K) & 1;
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const T src = from_lower_half_end<H>(last(u));
            apply_vec(lam, upper ? src : neg_zero<T>(), u);
        }
    }

    template <int K>
    __device__ __forceinline__ void vector_level()
    {
        constexpr int H = 1 << K;
        const int lam = LOGE + 7 + K;
        maybe_fork(lam);
        T src[V];
#pragma unroll
        for (int u = 0; u < V; ++u)
            if (u & H) src[u] = readlane(last((u & ~(2 * H - 1)) + H - 1), 63);
#pragma unroll
        for (int u = 0; u < V; ++u)
            if (u & H) apply_vec(lam, src[u], u);
    }

    // All levels inside one wave's 2^LOG_WSPAN elements.
    __device__ __forceinline__ void in_wave(int lane)
    {
        slot_levels();
        lane_level<0>(lane);
        lane_level<1>(lane);
        lane_level<2>(lane);
        lane_level<3>(lane);
        lane_level<4>(lane);
        lane_level<5>(lane);
        if constexpr (LOGV >= 1) vector_level<0>();
        if constexpr (LOGV >= 2) vector_level<1>();
        if constexpr (LOGV >= 3) vector_level<2>();
        if constexpr (LOGV >= 4) vector_level<3>();
    }

    // Wave-level merges (the tile's 4 waves), given the 4 wave totals.
    __device__ __forceinline__ void across_waves(int w, T t0, T t01, T t2)
    {
        if (w & 1) apply_all(LOG_WSPAN + 1, (w & 2) ? t2 : t0);
        else maybe_fork(LOG_WSPAN + 1);
        if (w & 2) apply_all(LOG_WSPAN + 2, t01);
        else maybe_fork(LOG_WSPAN + 2);
    }

    template <bool ALIGNED>
    __device__ __forceinline__ void load(const T* __restrict__ x, uint64_t n, uint64_t g0)
    {
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const uint64_t gi = g0 + (uint64_t)u * 64 * E;
            if (ALIGNED && gi + E <= n) {
                load_vec(x + gi, v[u]);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) v[u][e] = (gi + e < n) ? x[gi + e] : neg_zero<T>();
            }
        }
    }

    template <bool ALIGNED>
    __device__ __forceinline__ void store(T* __restrict__ y, uint64_t n, uint64_t g0) const
    {
        const uint64_t bmask = (1ull << b) - 1;
#pragma unroll
        for (int u = 0; u < V; ++u) {
            T o[E];
            if (!BD || !forked) {
#pragma unroll
                for (int e = 0; e < E; ++e) o[e] = v[u][e];
            } else {
                const uint64_t gi = g0 + (uint64_t)u * 64 * E;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    constexpr int BS = E / NB;  // slots per block inside a vector
                    const int k = e / BS;
                    const bool end = (MODE == 2) ? ((e % BS) == BS - 1)
                                                 : (e == E - 1 && ((gi + E) & bmask) == 0);
                    o[e] = end ? pe[u][k] : c[u][k] + v[u][e];
                }
            }
            const uint64_t gi = g0 + (uint64_t)u * 64 * E;
            if (ALIGNED && gi + E <= n) {
                store_vec(y + gi, o);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (gi + e < n) y[gi + e] = o[e];
            }
        }
    }

    __device__ __forceinline__ void copy_values(const ScanTile& o)
    {
#pragma unroll
        for (int u = 0; u < V; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e) v[u][e] = o.v[u][e];
    }
};

// Tile-level look-back, run by one wave, in two steps.
//
// lookback_issue (right after the tile's own loads are issued): every lane
// reads, once and without waiting, the word it will need: lane j < r the
// total of tile g + j of this tile's aligned group of 64, lane j the node of
// level 6 + j when that bit of t is set.  Most of them are ready by then, so
// their latency hides behind the tile's own loads.
//
// lookback_finish (after the tile's total is published): lanes whose word was
// not ready poll it; the low nodes are rebuilt with a butterfly in fixed lane
// order; s_h[k] receives the node for every set bit k of t; and, when t closes
// an aligned group of 64 tiles, the climbing nodes are published.
//
// Latency: a group's level-6 node depends only on the 64 tile totals of that
// group and is published before this tile waits for anything else; each
// further climbing step waits only for the one left sibling it combines, so a
// node of level k depends on a chain of at most k - 6 climbing steps, never on
// earlier groups in turn.
struct LookbackWords {
    uint64_t low;   // tile total of g + lane (lane < r)
    uint64_t high;  // node of level 6 + lane (bit set)
};

template <typename T>
__device__ __forceinline__ LookbackWords lookback_issue(uint64_t t, const uint64_t* __restrict__ ws,
                                                        const ScanLayout& lay, int lane)
{
    LookbackWords w;
    const uint64_t g = t & ~63ull;
    const int r = (int)(t - g);
    const int kh = lane + kGroupLog;
    w.low = w.high = not_ready_word<T>();
    if (lane < r)
        w.low = __hip_atomic_load(ws + lay.tiles_off + g + lane, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
    if (kh < kMaxLevels && ((t >> kh) & 1))
        w.high = __hip_atomic_load(ws + lay.level_off[kh] + ((t >> kh) - 1), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    return w;
}

template <typename T>
__device__ __forceinline__ T ready_or_wait(uint64_t w, uint64_t* slot, uint32_t* err)
{
    return w != not_ready_word<T>() ? unpack_word<T>(w) : wait_word<T>(slot, err);
}

template <typename T>
__device__ __forceinline__ void lookback_finish(uint64_t t, T tile_total, LookbackWords w,
                                                uint64_t* __restrict__ ws, const ScanLayout& lay,
                                                uint32_t* err, T* s_h, int lane)
{
    const uint64_t g = t & ~63ull;
    const int r = (int)(t - g);
    T a = neg_zero<T>();
    if (lane < r) a = ready_or_wait<T>(w.low, ws + lay.tiles_off + g + lane, err);

    T node[kGroupLog];
    node[0] = (r & 1) ? readlane(a, r - 1) : neg_zero<T>();
#define CANON_BUTTERFLY(K)                                                         \
    {                                                                              \
        const T o = shfl_xor<(1 << ((K)-1))>(a);                                   \
        a = ((lane >> ((K)-1)) & 1) ? (o + a) : (a + o);                           \
        node[K] = ((r >> (K)) & 1) ? readlane(a, (r >> ((K) + 1)) << ((K) + 1))   \
                                   : neg_zero<T>();                                \
    }
    CANON_BUTTERFLY(1)
    CANON_BUTTERFLY(2)
    CANON_BUTTERFLY(3)
    CANON_BUTTERFLY(4)
    CANON_BUTTERFLY(5)
#undef CANON_BUTTERFLY

    if (r == 63) {
        // climb: node (6, t>>6), then node (k+1, t>>(k+1)) while bit k is set
        T acc = tile_total;
#pragma unroll
        for (int k = 0; k < kGroupLog; ++k) acc = node[k] + acc;
        if (lane == 0) publish(ws + lay.level_off[kGroupLog] + (t >> kGroupLog), acc);
        for (int k = kGroupLog; k < kMaxLevels - 1 && ((t >> k) & 1); ++k) {
            const T left = wait_word<T>(ws + lay.level_off[k] + ((t >> k) - 1), err);
            acc = left + acc;
            if (lane == 0) publish(ws + lay.level_off[k + 1] + (t >> (k + 1)), acc);
        }
    }

    // every node this tile applies: low ones rebuilt above, high ones polled
    const int kh = lane + kGroupLog;
    if (kh < kMaxLevels && ((t >> kh) & 1))
        s_h[kh] = ready_or_wait<T>(w.high, ws + lay.level_off[kh] + ((t >> kh) - 1), err);
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < kGroupLog; ++k) s_h[k] = node[k];
    }
}

template <typename T>
__global__ void k_scan_init(uint64_t* __restrict__ ws, uint64_t total)
{
    const uint64_t nr = not_ready_word<T>();
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (uint64_t)gridDim.x * blockDim.x)
        ws[i] = i < 32 ? 0ull : nr;
}

// Single-pass scan: one workgroup per tile; tile numbers come from an atomic
// ticket counter in the order workgroups start, so every tile waited on
// belongs to a workgroup that is already running.  The look-back words are
// read right after the tile's own loads are issued, so that their latency
// overlaps the loads.
template <typename T, int MODE, bool ALIGNED, int LOGV>
__global__ __launch_bounds__(kScanThreads) void k_scan(const T* x, T* y, uint64_t n, int b_log,
                                                       uint64_t* __restrict__ ws, ScanLayout lay)
{
    using ST = ScanTile<T, MODE, LOGV>;
    __shared__ uint32_t s_tile;
    __shared__ T s_tot[kScanWaves];
    __shared__ T s_h[kMaxLevels];
    uint32_t* err = reinterpret_cast<uint32_t*>(ws);
    uint32_t* counter = reinterpret_cast<uint32_t*>(ws + 1);

    if (threadIdx.x == 0)
        s_tile = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint64_t t = s_tile;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t g0 = (t << ST::LOG_S) + ((uint64_t)w << ST::LOG_WSPAN) + (uint64_t)lane * ST::E;

    ST st;
    st.template load<ALIGNED>(x, n, g0);
    LookbackWords lw{};
    if (w == 0 && t > 0) lw = lookback_issue<T>(t, ws, lay, lane);
    st.begin(b_log);
    st.in_wave(lane);

    if (lane == 63) s_tot[w] = st.last(ST::V - 1);
    __syncthreads();
    const T t0 = s_tot[0], t1 = s_tot[1], t2 = s_tot[2], t3 = s_tot[3];
    const T t01 = t0 + t1;
    const T tile_total = t01 + (t2 + t3);
    if (threadIdx.x == 0) publish(ws + lay.tiles_off + t, tile_total);
    st.across_waves(w, t0, t01, t2);
    if (t > 0) {
        if (w == 0) lookback_finish<T>(t, tile_total, lw, ws, lay, err, s_h, lane);
        __syncthreads();
        for (int k = 0; k < kMaxLevels && (t >> k) != 0; ++k)
            if ((t >> k) & 1) st.apply_all(ST::LOG_S + 1 + k, s_h[k]);
    }
    st.template store<ALIGNED>(y, n, g0);
}

// Row-batched scan: one workgroup per row, the row's tiles in order; the tile
// nodes come from a binary-counter stack of the row's earlier tile totals
// (held in LDS by thread 0).
template <typename T, int MODE, bool ALIGNED, int LOGV>
__global__ __launch_bounds__(kScanThreads) void k_scan_rows(const T* x, uint64_t ldx, T* y,
                                                            uint64_t ldy, uint64_t rows,
                                                            uint64_t cols, int b_log)
{
    using ST = ScanTile<T, MODE, LOGV>;
    __shared__ T s_tot[kScanWaves];
    __shared__ T s_stack[kMaxLevels];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t ntiles = (cols + (1ull << ST::LOG_S) - 1) >> ST::LOG_S;

    for (uint64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const T* xr = x + row * ldx;
        T* yr = y + row * ldy;
        for (uint64_t t = 0; t < ntiles; ++t) {
            const uint64_t g0 =
                (t << ST::LOG_S) + ((uint64_t)w << ST::LOG_WSPAN) + (uint64_t)lane * ST::E;
            ST st;
            st.template load<ALIGNED>(xr, cols, g0);
            st.begin(b_log);
            st.in_wave(lane);
            if (lane == 63) s_tot[w] = st.last(ST::V - 1);
            __syncthreads();
            const T t0 = s_tot[0], t1 = s_tot[1], t2 = s_tot[2], t3 = s_tot[3];
            const T t01 = t0 + t1;
            const T tile_total = t01 + (t2 + t3);
            st.across_waves(w, t0, t01, t2);
            for (int k = 0; k < kMaxLevels && (t >> k) != 0; ++k)
                if ((t >> k) & 1) st.apply_all(ST::LOG_S + 1 + k, s_stack[k]);
            st.template store<ALIGNED>(yr, cols, g0);
            __syncthreads();  // everyone has read s_tot and s_stack
            if (threadIdx.x == 0) {
                T acc = tile_total;
                const int merges = __builtin_ctzll(~t);
                for (int l = 0; l < merges; ++l) acc = s_stack[l] + acc;
                s_stack[merges] = acc;
            }
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------- launchers
template <typename T, int MODE, bool ALIGNED>
static hipError_t launch_scan_k(const T* x, T* y, uint64_t n, int b_log, uint64_t* ws,
                                const ScanLayout& lay, hipStream_t s)
{
    hipLaunchKernelGGL((k_scan<T, MODE, ALIGNED, scan_log_v<T>()>), dim3((unsigned)lay.ntiles),
                       dim3(kScanThreads), 0, s, x, y, n, b_log, ws, lay);
    return hipGetLastError();
}

template <typename T, int MODE>
static hipError_t launch_scan_m(const T* x, T* y, uint64_t n, int b_log, bool aligned,
                                uint64_t* ws, const ScanLayout& lay, hipStream_t s)
{
    if (aligned) return launch_scan_k<T, MODE, true>(x, y, n, b_log, ws, lay, s);
    return launch_scan_k<T, MODE, false>(x, y, n, b_log, ws, lay, s);
}

template <typename T>
hipError_t launch_scan(const T* x, T* y, uint64_t n, bool pairwise, int b_log, bool aligned,
                       uint64_t* ws, const ScanLayout& lay, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    uint64_t blocks = (lay.total_words + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL((k_scan_init<T>), dim3((unsigned)blocks), dim3(256), 0, s, ws,
                       lay.total_words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (pairwise || b_log == 0) return launch_scan_m<T, 0>(x, y, n, 0, aligned, ws, lay, s);
    if constexpr (Elem<T>::LOGE >= 2) {
        if (b_log < Elem<T>::LOGE) return launch_scan_m<T, 2>(x, y, n, b_log, aligned, ws, lay, s);
    }
    return launch_scan_m<T, 1>(x, y, n, b_log, aligned, ws, lay, s);
}

template <typename T, int MODE>
static hipError_t launch_scan_rows_m(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t rows,
                                     uint64_t cols, int b_log, bool aligned, hipStream_t s)
{
    // grid-stride over rows with about as many workgroups as fit at once
    if (aligned) {
        constexpr auto kern = k_scan_rows<T, MODE, true, scan_log_v<T>()>;
        uint64_t grid = resident_grid<kern>(kScanThreads);
        if (grid > rows) grid = rows;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kScanThreads), 0, s, x, ldx, y, ldy,
                           rows, cols, b_log);
    } else {
        constexpr auto kern = k_scan_rows<T, MODE, false, scan_log_v<T>()>;
        uint64_t grid = resident_grid<kern>(kScanThreads);
        if (grid > rows) grid = rows;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kScanThreads), 0, s, x, ldx, y, ldy,
                           rows, cols, b_log);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_scan_rows(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t rows,
                            uint64_t cols, bool pairwise, int b_log, bool aligned, hipStream_t s)
{
    if (rows == 0 || cols == 0) return hipSuccess;
    if (pairwise || b_log == 0)
        return launch_scan_rows_m<T, 0>(x, ldx, y, ldy, rows, cols, 0, aligned, s);
    if constexpr (Elem<T>::LOGE >= 2) {
        if (b_log < Elem<T>::LOGE)
            return launch_scan_rows_m<T, 2>(x, ldx, y, ldy, rows, cols, b_log, aligned, s);
    }
    return launch_scan_rows_m<T, 1>(x, ldx, y, ldy, rows, cols, b_log, aligned, s);
}

template hipError_t launch_scan<double>(const double*, double*, uint64_t, bool, int, bool,
                                        uint64_t*, const ScanLayout&, hipStream_t);
template hipError_t launch_scan<float>(const float*, float*, uint64_t, bool, int, bool, uint64_t*,
                                       const ScanLayout&, hipStream_t);
template hipError_t launch_scan_rows<double>(const double*, uint64_t, double*, uint64_t, uint64_t,
                                             uint64_t, bool, int, bool, hipStream_t);
template hipError_t launch_scan_rows<float>(const float*, uint64_t, float*, uint64_t, uint64_t,
                                            uint64_t, bool, int, bool, hipStream_t);

}  // namespace canon
