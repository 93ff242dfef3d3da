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
#include "scan.hpp"

namespace canon {

template <typename T, bool PW, bool BIGB>
struct ScanTile {
    static constexpr int E = Elem<T>::E;
    static constexpr int LOGE = Elem<T>::LOGE;
    static constexpr int V = kScanVec;
    static constexpr int LOGV = 3;
    static constexpr int LOG_WSPAN = LOGE + 6 + LOGV;  // elements per wave (log2)
    static constexpr int LOG_S = LOG_WSPAN + 2;        // elements per tile (log2)
    static constexpr int CE = BIGB ? 1 : E;            // carries per vector

    T v[V][E];
    T c[V][CE];
    uint32_t endmask;  // bit u*E+e: element (u, e) is the last one of a block
    int b;             // log2 B (block_dyadic)

    __device__ __forceinline__ void init(int b_log, uint64_t g0)
    {
        b = b_log;
        endmask = 0;
#pragma unroll
        for (int u = 0; u < V; ++u)
#pragma unroll
            for (int e = 0; e < CE; ++e) c[u][e] = neg_zero<T>();
        if (!PW) {
            const uint64_t mask = (1ull << b_log) - 1;
#pragma unroll
            for (int u = 0; u < V; ++u)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const uint64_t gi = g0 + (uint64_t)u * 64 * E + e;
                    if (((gi + 1) & mask) == 0) endmask |= 1u << (u * E + e);
                }
        }
    }
    __device__ __forceinline__ bool is_end(int u, int e) const
    {
        return (endmask >> (u * E + e)) & 1u;
    }

    // One element receives s (the end of the lower half) at level lam.
    __device__ __forceinline__ void apply_elem(int lam, T s, int u, int e)
    {
        if (PW || lam <= b) {
            v[u][e] = s + v[u][e];
        } else {
            c[u][BIGB ? 0 : e] = s + c[u][BIGB ? 0 : e];
            v[u][e] = (is_end(u, e) ? s : neg_zero<T>()) + v[u][e];
        }
    }
    // All elements of vector u receive s at level lam (lam > LOGE).
    __device__ __forceinline__ void apply_vec(int lam, T s, int u)
    {
        if (PW || lam <= b) {
#pragma unroll
            for (int e = 0; e < E; ++e) v[u][e] = s + v[u][e];
        } else if constexpr (BIGB) {
            // the whole vector lies in one block: one carry, and only the
            // last slot can be a block end
            c[u][0] = s + c[u][0];
            v[u][E - 1] = (is_end(u, E - 1) ? s : neg_zero<T>()) + v[u][E - 1];
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) apply_elem(lam, s, u, e);
        }
    }
    __device__ __forceinline__ void apply_all(int lam, T s)
    {
#pragma unroll
        for (int u = 0; u < V; ++u) apply_vec(lam, s, u);
    }

    template <int K>
    __device__ __forceinline__ void slot_level()
    {
        constexpr int H = 1 << K;
#pragma unroll
        for (int u = 0; u < V; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (e & H) apply_elem(K + 1, v[u][(e & ~(2 * H - 1)) + H - 1], u, e);
    }

    template <int K>
    __device__ __forceinline__ void lane_level(int lane)
    {
        constexpr int H = 1 << K;
        const bool upper = (lane >> K) & 1;
        T src[V];
#pragma unroll
        for (int u = 0; u < V; ++u) src[u] = from_lower_half_end<H>(v[u][E - 1]);
#pragma unroll
        for (int u = 0; u < V; ++u) apply_vec(LOGE + 1 + K, upper ? src[u] : neg_zero<T>(), u);
    }

    template <int K>
    __device__ __forceinline__ void vector_level()
    {
        constexpr int H = 1 << K;
        T src[V];
#pragma unroll
        for (int u = 0; u < V; ++u)
            if (u & H) src[u] = readlane(v[(u & ~(2 * H - 1)) + H - 1][E - 1], 63);
#pragma unroll
        for (int u = 0; u < V; ++u)
            if (u & H) apply_vec(LOGE + 7 + K, src[u], u);
    }

    // All levels inside one wave's 2^LOG_WSPAN elements.
    __device__ __forceinline__ void in_wave(int lane)
    {
        if constexpr (LOGE >= 1) slot_level<0>();
        if constexpr (LOGE >= 2) slot_level<1>();
        lane_level<0>(lane);
        lane_level<1>(lane);
        lane_level<2>(lane);
        lane_level<3>(lane);
        lane_level<4>(lane);
        lane_level<5>(lane);
        vector_level<0>();
        vector_level<1>();
        vector_level<2>();
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
    __device__ __forceinline__ void store(T* __restrict__ y, uint64_t n, uint64_t g0)
    {
#pragma unroll
        for (int u = 0; u < V; ++u) {
            T o[E];
#pragma unroll
            for (int e = 0; e < E; ++e)
                o[e] = (PW || is_end(u, e)) ? v[u][e] : c[u][BIGB ? 0 : e] + v[u][e];
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
};

// Tile-level look-back, run by one wave.  Writes into s_h[k] the node for
// every set bit k of t and publishes the climbing nodes when t closes an
// aligned group of 64 tiles.
template <typename T>
__device__ __forceinline__ void lookback(uint64_t t, T tile_total, uint64_t* __restrict__ ws,
                                         const ScanLayout& lay, uint32_t* err, T* s_h, int lane)
{
    const uint64_t g = t & ~63ull;
    const int r = (int)(t - g);
    T a = neg_zero<T>();
    if (lane < r) a = wait_word<T>(ws + lay.tiles_off + g + lane, err);
    T hv = neg_zero<T>();
    const int kh = lane + kGroupLog;
    if (kh < kMaxLevels && ((t >> kh) & 1))
        hv = wait_word<T>(ws + lay.level_off[kh] + ((t >> kh) - 1), err);

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
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < kGroupLog; ++k) s_h[k] = node[k];
    }
    if (kh < kMaxLevels) s_h[kh] = hv;

    if (r == 63) {
        T acc = tile_total;
#pragma unroll
        for (int k = 0; k < kGroupLog; ++k) acc = node[k] + acc;
        if (lane == 0) publish(ws + lay.level_off[kGroupLog] + (t >> kGroupLog), acc);
        for (int k = kGroupLog; k < kMaxLevels - 1 && ((t >> k) & 1); ++k) {
            acc = readlane(hv, k - kGroupLog) + acc;
            if (lane == 0) publish(ws + lay.level_off[k + 1] + (t >> (k + 1)), acc);
        }
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

template <typename T, bool PW, bool BIGB, bool ALIGNED>
__global__ __launch_bounds__(kScanThreads) void k_scan(const T* x, T* y, uint64_t n, int b_log,
                                                       uint64_t* __restrict__ ws, ScanLayout lay)
{
    using ST = ScanTile<T, PW, BIGB>;
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
    st.init(b_log, g0);
    st.in_wave(lane);

    if (lane == 63) s_tot[w] = st.v[ST::V - 1][ST::E - 1];
    __syncthreads();
    const T t0 = s_tot[0], t1 = s_tot[1], t2 = s_tot[2], t3 = s_tot[3];
    const T t01 = t0 + t1;
    const T tile_total = t01 + (t2 + t3);
    if (threadIdx.x == 0) publish(ws + lay.tiles_off + t, tile_total);
    if (w & 1) st.apply_all(ST::LOG_WSPAN + 1, (w & 2) ? t2 : t0);
    if (w & 2) st.apply_all(ST::LOG_WSPAN + 2, t01);

    if (t > 0) {
        if (w == 0) lookback<T>(t, tile_total, ws, lay, err, s_h, lane);
        __syncthreads();
        for (int k = 0; k < kMaxLevels && (t >> k) != 0; ++k)
            if ((t >> k) & 1) st.apply_all(ST::LOG_S + 1 + k, s_h[k]);
    }
    st.template store<ALIGNED>(y, n, g0);
}

// Row-batched scan: one workgroup per row, the row's tiles in order; the tile
// nodes come from a binary-counter stack of the row's earlier tile totals
// (held in LDS by thread 0).
template <typename T, bool PW, bool BIGB, bool ALIGNED>
__global__ __launch_bounds__(kScanThreads) void k_scan_rows(const T* x, uint64_t ldx, T* y,
                                                            uint64_t ldy, uint64_t rows,
                                                            uint64_t cols, int b_log)
{
    using ST = ScanTile<T, PW, BIGB>;
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
            st.init(b_log, g0);
            st.in_wave(lane);
            if (lane == 63) s_tot[w] = st.v[ST::V - 1][ST::E - 1];
            __syncthreads();
            const T t0 = s_tot[0], t1 = s_tot[1], t2 = s_tot[2], t3 = s_tot[3];
            const T t01 = t0 + t1;
            const T tile_total = t01 + (t2 + t3);
            if (w & 1) st.apply_all(ST::LOG_WSPAN + 1, (w & 2) ? t2 : t0);
            if (w & 2) st.apply_all(ST::LOG_WSPAN + 2, t01);
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
template <typename T, bool PW, bool BIGB>
static hipError_t launch_scan_v(const T* x, T* y, uint64_t n, int b_log, bool aligned,
                                uint64_t* ws, const ScanLayout& lay, hipStream_t s)
{
    const dim3 grid((unsigned)lay.ntiles);
    if (aligned)
        hipLaunchKernelGGL((k_scan<T, PW, BIGB, true>), grid, dim3(kScanThreads), 0, s, x, y, n,
                           b_log, ws, lay);
    else
        hipLaunchKernelGGL((k_scan<T, PW, BIGB, false>), grid, dim3(kScanThreads), 0, s, x, y, n,
                           b_log, ws, lay);
    return hipGetLastError();
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
    if (pairwise || b_log == 0) return launch_scan_v<T, true, true>(x, y, n, 0, aligned, ws, lay, s);
    if (b_log >= Elem<T>::LOGE)
        return launch_scan_v<T, false, true>(x, y, n, b_log, aligned, ws, lay, s);
    return launch_scan_v<T, false, false>(x, y, n, b_log, aligned, ws, lay, s);
}

template <typename T, bool PW, bool BIGB>
static hipError_t launch_scan_rows_v(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t rows,
                                     uint64_t cols, int b_log, bool aligned, hipStream_t s)
{
    const uint64_t grid = rows < 65536 ? rows : 65536;
    if (aligned)
        hipLaunchKernelGGL((k_scan_rows<T, PW, BIGB, true>), dim3((unsigned)grid),
                           dim3(kScanThreads), 0, s, x, ldx, y, ldy, rows, cols, b_log);
    else
        hipLaunchKernelGGL((k_scan_rows<T, PW, BIGB, false>), dim3((unsigned)grid),
                           dim3(kScanThreads), 0, s, x, ldx, y, ldy, rows, cols, b_log);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_scan_rows(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t rows,
                            uint64_t cols, bool pairwise, int b_log, bool aligned, hipStream_t s)
{
    if (rows == 0 || cols == 0) return hipSuccess;
    if (pairwise || b_log == 0)
        return launch_scan_rows_v<T, true, true>(x, ldx, y, ldy, rows, cols, 0, aligned, s);
    if (b_log >= Elem<T>::LOGE)
        return launch_scan_rows_v<T, false, true>(x, ldx, y, ldy, rows, cols, b_log, aligned, s);
    return launch_scan_rows_v<T, false, false>(x, ldx, y, ldy, rows, cols, b_log, aligned, s);
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
