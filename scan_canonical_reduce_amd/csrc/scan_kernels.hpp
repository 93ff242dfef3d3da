// Canonical inclusive scan, single pass over one sequence (gfx950):
// policies pairwise and block_dyadic<B> (canonical-reduce README, P4229R0
// "Summary" / "Key Design Points").  The in-tile network is ScanTile
// (scan_tile.hpp); this file carries values across tiles.
//
// Tile-level node (k, u) covers tiles [u 2^k, (u+1) 2^k) and is the complete
// pairwise tree over them.  Tile t needs node (k, (t >> k) - 1) for every set
// bit k of t, and applies them as merge levels above the tile.  Every value
// is fixed by position only, never by arrival order.  Tile numbers come from
// an atomic counter, so every tile waited on belongs to a workgroup that is
// already running.
#pragma once

#include "device.hpp"
#include "launch.hpp"
#include "scan.hpp"
#include "scan_tile.hpp"

namespace canon {

// Tile-level look-back.  Tile t, in group G = t >> 6 at position r = t & 63,
// needs node (k, (t >> k) - 1) for every set bit k of t.
//
//   k < 6:  rebuilt from the totals of the r tiles before t in its group
//           (wave 0: one total per lane, butterfly in fixed lane order).
//   k >= 6: the lowest such bit k0 names the node that ends at the most
//           recent group G - 1.  Nodes that end within the last two groups
//           are rebuilt from published tile totals: node (6, G-1) by wave 1
//           and node (6, G-2) by wave 2 (64 totals each).  Then
//             k0 == 6:  node (6, G-1)
//             k0 >= 7:  node (k0-1, ..) + (node (k0-2, ..) + ... +
//                       (node (7, (t >> 7) - 2) + (node (6, G-2) + node (6, G-1))))
//           i.e. the right spine of the node, whose left siblings end at least
//           two groups back and are read as published nodes (wave 3), as are
//           the nodes of the bits above k0.
// Published nodes: the workgroup of the last tile of each group G (tile
// 64 G + 63) builds node (6, G) from the group's 64 published totals right
// after that tile's front, before anything of its own look-back, and climbs:
// while the node built is a right child, parent = published left sibling +
// node.  A build waits only on other tiles' totals (a front never waits) and
// on nodes of earlier builds, never on a look-back, so a node is out about
// one front after its last tile's total and no wait is ever on a chain of
// look-backs.  The published nodes a tile reads all end before group G-1.
// Every value is fixed by position only.
//
// The words are read once right after the loads of the workgroup's next
// tile are issued (lookback_issue), so that they arrive with that data;
// words not ready then are polled in lookback_collect.
struct LookbackWords {
    uint64_t w;  // the word this lane of this wave reads (see lookback_slot)
};

// Address of the word lane `lane` of wave `wave` needs for tile t, or null.
__device__ __forceinline__ uint64_t* lookback_slot(uint64_t t, uint64_t* __restrict__ ws,
                                                   const ScanLayout& lay, int wave, int lane)
{
    const uint64_t G = t >> kGroupLog;
    const int r = (int)(t & 63);
    if (wave == 0) return lane < r ? ws + lay.tiles_off + (G << kGroupLog) + lane : nullptr;
    if (wave == 1) return G >= 1 ? ws + lay.tiles_off + ((G - 1) << kGroupLog) + lane : nullptr;
    if (wave == 2) return G >= 2 ? ws + lay.tiles_off + ((G - 2) << kGroupLog) + lane : nullptr;
    const int k = kGroupLog + lane;
    if (G == 0 || k >= kMaxLevels) return nullptr;
    const int k0 = kGroupLog + __builtin_ctzll(G);
    if (k > k0 && ((t >> k) & 1)) return ws + lay.level_off[k] + ((t >> k) - 1);
    if (k >= kGroupLog + 1 && k < k0) return ws + lay.level_off[k] + ((t >> k) - 2);
    return nullptr;
}

template <typename T>
__device__ __forceinline__ LookbackWords lookback_issue(uint64_t t, uint64_t* __restrict__ ws,
                                                        const ScanLayout& lay, int wave, int lane)
{
    LookbackWords w;
    w.w = not_ready_word<T>();
    uint64_t* slot = lookback_slot(t, ws, lay, wave, lane);
    if (slot) w.w = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return w;
}

// Complete tree over the 64 lane values, lower lanes on the left; node[k]
// receives the value of the aligned 2^k group starting at lane
// (r >> (k+1)) << (k+1) when bit k of r is set (r < 64), and the full tree
// is returned.
template <typename T>
__device__ __forceinline__ T wave_tree(T a, int lane, int r, T (&node)[kGroupLog])
{
    node[0] = (r & 1) ? readlane(a, r - 1) : neg_zero<T>();
#define CANON_BUTTERFLY(K)                                                         \
    {                                                                              \
        const T o = shfl_xor<(1 << ((K)-1))>(a);                                   \
        a = ((lane >> ((K)-1)) & 1) ? (o + a) : (a + o);                           \
        if ((K) < kGroupLog)                                                       \
            node[(K) % kGroupLog] = ((r >> (K)) & 1)                               \
                                        ? readlane(a, (r >> ((K) + 1)) << ((K) + 1)) \
                                        : neg_zero<T>();                           \
    }
    CANON_BUTTERFLY(1)
    CANON_BUTTERFLY(2)
    CANON_BUTTERFLY(3)
    CANON_BUTTERFLY(4)
    CANON_BUTTERFLY(5)
    CANON_BUTTERFLY(6)
#undef CANON_BUTTERFLY
    return readlane(a, 0);
}

// Waves 0-2 resolve their words and reduce them: s_low[0..5] = low nodes
// (wave 0), s_g6[0] = node (6, G-1) (wave 1), s_g6[1] = node (6, G-2)
// (wave 2).
template <typename T>
__device__ __forceinline__ void lookback_collect(uint64_t t, LookbackWords lw,
                                                 uint64_t* __restrict__ ws, const ScanLayout& lay,
                                                 uint32_t* err, T* s_low, T* s_g6, int wave,
                                                 int lane)
{
    uint64_t* slot = lookback_slot(t, ws, lay, wave, lane);
    const T a = slot ? ready_or_wait<T>(lw.w, slot, err) : neg_zero<T>();
    T node[kGroupLog];
    const T total = wave_tree(a, lane, wave == 0 ? (int)(t & 63) : 0, node);
    if (lane == 0) {
        if (wave == 0) {
#pragma unroll
            for (int k = 0; k < kGroupLog; ++k) s_low[k] = node[k];
        } else {
            s_g6[wave - 1] = total;
        }
    }
}

// Wave 3 resolves the published nodes (lane k - 6 for level k) into
// s_w3[k - 6].
template <typename T>
__device__ __forceinline__ void lookback_collect_high(uint64_t t, LookbackWords lw,
                                                      uint64_t* __restrict__ ws,
                                                      const ScanLayout& lay, uint32_t* err,
                                                      T* s_w3, int lane)
{
    uint64_t* slot = lookback_slot(t, ws, lay, 3, lane);
    const T a = slot ? ready_or_wait<T>(lw.w, slot, err) : neg_zero<T>();
    if (lane < kMaxLevels - kGroupLog) s_w3[lane] = a;
}

// One thread: the node of every set bit of t into s_h[k].
template <typename T>
__device__ __forceinline__ void lookback_combine(uint64_t t, const T* s_low, const T* s_g6,
                                                 const T* s_w3, T* s_h)
{
    const uint64_t G = t >> kGroupLog;
    for (int k = 0; k < kGroupLog; ++k) s_h[k] = s_low[k];
    if (G > 0) {
        const int k0 = kGroupLog + __builtin_ctzll(G);
        T acc;
        if (k0 == kGroupLog) {
            acc = s_g6[0];
        } else {
            acc = s_g6[1] + s_g6[0];
            for (int k = kGroupLog + 1; k < k0; ++k) acc = s_w3[k - kGroupLog] + acc;
        }
        s_h[k0] = acc;
        for (int k = k0 + 1; k < kMaxLevels; ++k)
            if ((t >> k) & 1) s_h[k] = s_w3[k - kGroupLog];
    }
}

// Header words zeroed but word 2, the bound of the call's waits (0: the
// default; spin_limit_of); every published word marked not ready.
template <typename T>
__global__ void k_scan_init(uint64_t* __restrict__ ws, uint64_t total, uint64_t spin_limit)
{
    const uint64_t nr = not_ready_word<T>();
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (uint64_t)gridDim.x * blockDim.x)
        ws[i] = i < 32 ? (i == 2 ? spin_limit : 0ull) : nr;
}

template <typename T>
inline void launch_scan_init(uint64_t* ws, const ScanLayout& lay, hipStream_t s)
{
    uint64_t blocks = (lay.total_words + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL((k_scan_init<T>), dim3((unsigned)blocks), dim3(256), 0, s, ws,
                       lay.total_words, g_sched_spin_limit.load(std::memory_order_relaxed));
}

// Whether tile t ends its group (its workgroup then runs group_build).
__device__ __forceinline__ bool ends_group(uint64_t t)
{
    return (t & ((1u << kGroupLog) - 1)) == (1u << kGroupLog) - 1;
}

// One wave, right after the front of tile e = 64 G + 63: node (6, G) from
// the group's 64 totals (each published by a front, so every wait here
// ends), then, while the node built is the right child of its parent
// (bit k of G set), parent = published left sibling + node.
template <typename T>
__device__ __forceinline__ void group_build(uint64_t e, uint64_t* __restrict__ ws,
                                            const ScanLayout& lay, uint32_t* err, int lane)
{
    const uint64_t G = e >> kGroupLog;
    uint64_t* slot = ws + lay.tiles_off + (G << kGroupLog) + lane;
    const uint64_t w0 = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    T node[kGroupLog];
    T acc = wave_tree(ready_or_wait<T>(w0, slot, err), lane, 0, node);
    uint64_t u = G;
    if (lane == 0) publish(ws + lay.level_off[kGroupLog] + u, acc);
    for (int k = kGroupLog; (u & 1) && k + 1 < kMaxLevels; ++k) {
        acc = wait_word<T>(ws + lay.level_off[k] + (u - 1), err) + acc;
        u >>= 1;
        if (lane == 0) publish(ws + lay.level_off[k + 1] + u, acc);
    }
}

// Every thread of the workgroup of tile t > 0: resolves the look-back into
// s_h[k] = node (k, (t >> k) - 1) for every set bit k of t.
template <typename T>
__device__ __forceinline__ void run_lookback(uint64_t t, LookbackWords lw,
                                             uint64_t* __restrict__ ws, const ScanLayout& lay,
                                             uint32_t* err, T* s_low, T* s_g6, T* s_w3, T* s_h,
                                             int w, int lane)
{
    if (w < 3)
        lookback_collect<T>(t, lw, ws, lay, err, s_low, s_g6, w, lane);
    else if (w == 3)
        lookback_collect_high<T>(t, lw, ws, lay, err, s_w3, lane);
    __syncthreads();
    if (threadIdx.x == 0) lookback_combine<T>(t, s_low, s_g6, s_w3, s_h);
    __syncthreads();
}

// Shared memory of the look-back.
template <typename T>
struct LookbackShared {
    T h[kMaxLevels];
    T low[kGroupLog];
    T g6[2];
    T w3[kMaxLevels - kGroupLog];
};

// Shared memory of a single-pass scan workgroup (the block values of
// block_dyadic with B < tile are in dynamic shared memory).
template <typename T>
struct ScanShared {
    uint32_t tile;
    T tot[kScanWaves];
    T tt;
    T wend[kScanWaves];  // last value of each wave (shifted outputs)
    LookbackShared<T> lb;
};

// What every phase of a single-pass scan workgroup needs.
template <typename T>
struct ScanCtx {
    const T* x;
    T* y;
    uint64_t n;
    int b_log;
    uint64_t* ws;
    const ScanLayout* lay;
    uint32_t* err;
    ScanShared<T>* sh;
    T* blk;  // block values (B < tile)
    int lane, w;
    T init;    // scans with an initial value (OUTX policies): init and kind
    int kind;
};

// Next tile number from the ticket counter, for the whole workgroup.  The
// shared slot is rewritten only after a later barrier of the caller.
template <typename T>
__device__ __forceinline__ uint64_t next_ticket(const ScanCtx<T>& c)
{
    if (threadIdx.x == 0)
        c.sh->tile = __hip_atomic_fetch_add(reinterpret_cast<uint32_t*>(c.ws + 1), 1u,
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    return c.sh->tile;
}

// Pairwise (MODE 0) and block_dyadic with B = 2 in float (MODE 2): the tile
// network through every level, the tile-level nodes applied to every element.
template <typename T, int MODE, bool ALIGNED, int LOGV, bool OUTX>
struct FullTile {
    using ST = ScanTile<T, MODE, LOGV>;
    struct State {
        ST st;
    };
    static constexpr int LOG_S = ST::LOG_S;
    // aligned f64 pairwise: hold the two tiles in at most 168 VGPRs (3 waves
    // per SIMD), which they fit without spilling (measured 2-10% faster;
    // float pairwise is there without the bound, and slower with it)
    static constexpr int kMinWavesPerEu =
        (MODE == 0 && ALIGNED && sizeof(T) == 8 && !kIsOpVal<T>) ? 3 : 1;

    static __device__ __forceinline__ uint64_t g0(uint64_t t, const ScanCtx<T>& c)
    {
        return (t << LOG_S) + ((uint64_t)c.w << ST::LOG_WSPAN) + (uint64_t)c.lane * ST::E;
    }
    static __device__ __forceinline__ void load(State& s, uint64_t t, const ScanCtx<T>& c)
    {
        s.st.template load<ALIGNED>(c.x, c.n, g0(t, c));
    }
    // in-tile scan; publishes and returns the tile total
    static __device__ __forceinline__ T front(State& s, uint64_t t, const ScanCtx<T>& c)
    {
        s.st.begin(c.b_log, g0(t, c));
        s.st.in_wave(c.lane);
        if (c.lane == 63) c.sh->tot[c.w] = s.st.last(ST::V - 1);
        __syncthreads();
        const T t0 = c.sh->tot[0], t1 = c.sh->tot[1], t2 = c.sh->tot[2], t3 = c.sh->tot[3];
        const T t01 = t0 + t1;
        const T total = t01 + (t2 + t3);
        if (threadIdx.x == 0) publish(c.ws + c.lay->tiles_off + t, total);
        s.st.across_waves(c.w, t0, t01, t2);
        return total;
    }
    // the tile-level nodes (in c.sh->lb.h when t > 0), then the stores;
    // with OUTX, pre collects the same nodes as a value at the position
    // just before the tile would (the pairwise value of everything before it)
    static __device__ __forceinline__ void back(State& s, uint64_t t, const ScanCtx<T>& c)
    {
        T pre = neg_zero<T>();
        for (int k = 0; k < kMaxLevels && (t >> k) != 0; ++k)
            if ((t >> k) & 1) {
                s.st.apply_all(LOG_S + 1 + k, c.sh->lb.h[k]);
                if constexpr (OUTX) pre = c.sh->lb.h[k] + pre;
            }
        if constexpr (OUTX)
            s.st.template emit<ALIGNED>(c.y, c.n, g0(t, c), c.init, c.kind, pre, c.sh->wend, c.w,
                                        c.lane, [&](int u, T(&o)[ST::E]) { s.st.final_vec(u, o); });
        else
            s.st.template store<ALIGNED>(c.y, c.n, g0(t, c));
    }
};

// Canonical inclusive pairwise scan of a tile's block totals, one value
// per block: thread tau holds blocks tau*m .. tau*m + m - 1 (m = 2^lm, at
// most 2^LMX), the same network as the elements' (levels inside a thread,
// across lanes, across the 4 waves), so a[k] ends as the pairwise value
// of the block totals up to and including its block.
template <typename T, int LMX>
struct BlockScan {
    static constexpr int M = 1 << LMX;
    T a[M];
    T tot;  // value of the thread's last block

    __device__ __forceinline__ void load(const T* s, int tau, int lm, int nblk)
    {
        const int m = 1 << lm;
#pragma unroll
        for (int k = 0; k < M; ++k) {
            const int j = tau * m + k;
            a[k] = (k < m && j < nblk) ? s[j] : neg_zero<T>();
        }
    }

    __device__ __forceinline__ void receive(T s)
    {
#pragma unroll
        for (int k = 0; k < M; ++k) a[k] = s + a[k];
        tot = s + tot;
    }

    template <int K>
    __device__ __forceinline__ void lane_level(int lane)
    {
        const T src = from_lower_half_end<(1 << K)>(tot);
        receive(((lane >> K) & 1) ? src : neg_zero<T>());
    }

    __device__ __forceinline__ void scan(int lm, int lane, int w, T* s_wt)
    {
        // levels inside the thread; entries k >= m stay -0.0
#pragma unroll
        for (int l = 1; l <= LMX; ++l) {
            if (l <= lm) {
#pragma unroll
                for (int k = 0; k < M; ++k)
                    if ((k >> (l - 1)) & 1) a[k] = a[((k >> l) << l) + (1 << (l - 1)) - 1] + a[k];
            }
        }
        tot = a[0];
#pragma unroll
        for (int l = 1; l <= LMX; ++l)
            if (l == lm) tot = a[(1 << l) - 1];
        lane_level<0>(lane);
        lane_level<1>(lane);
        lane_level<2>(lane);
        lane_level<3>(lane);
        lane_level<4>(lane);
        lane_level<5>(lane);
        if (lane == 63) s_wt[w] = tot;
        __syncthreads();
        const T w0 = s_wt[0], w1 = s_wt[1], w2 = s_wt[2];
        if (w & 1) receive((w & 2) ? w2 : w0);
        if (w & 2) receive(w0 + w1);
    }
};

// Block_dyadic with B >= E (the block sizes that LaneBlockTile and WideTile
// do not take: blocks larger than a wave's span, B >= tile, and float blocks
// of one lane's vector).  With n = qB + r, the value at a block's
// interior is C + W, C = PW(x[0..qB)) the pairwise value at the end of the
// previous block, W the pairwise prefix inside the block; at a block end it
// is the pairwise value there.  So the levels above b reduce to one pairwise
// scan over block totals:
//   B < tile (BIG false): the in-tile network stops at level b (W in every
//              element, the block total at every block end); the block totals
//              go through BlockScan (levels above b inside the tile), then the
//              tile-level nodes are added on the left of each block value
//              (right-nested, lowest level first), giving G(P_j) for every
//              block j and G(-0.0) in front of block 0; an element outputs
//              G(P_{j-1}) + W, a block end G(P_j).
//   B >= tile (BIG):  the whole tile lies in one block, the in-tile network is
//              pairwise; tile-level nodes up to level b go to every element,
//              those above b into one carry c (every element outputs c + W)
//              and, at a tile that closes a block, into its last element.
// LMX bounds log2 of the blocks each thread holds in BlockScan.
template <typename T, bool ALIGNED, int LOGV, bool BIG, int LMX, bool OUTX>
struct SplitTile {
    using ST = ScanTile<T, 3, LOGV>;
    static constexpr int E = ST::E;
    static constexpr int LOG_S = ST::LOG_S;
    static constexpr int kMinWavesPerEu = 1;  // a tighter bound spills
    struct State {
        ST st;
        BlockScan<T, LMX> bs;
    };

    static __device__ __forceinline__ int off0(const ScanCtx<T>& c)
    {
        return (c.w << ST::LOG_WSPAN) + c.lane * E;  // in the tile
    }
    static __device__ __forceinline__ uint64_t g0(uint64_t t, const ScanCtx<T>& c)
    {
        return (t << LOG_S) + (uint64_t)off0(c);
    }
    static __device__ __forceinline__ void load(State& s, uint64_t t, const ScanCtx<T>& c)
    {
        s.st.template load<ALIGNED>(c.x, c.n, g0(t, c));
    }

    static __device__ __forceinline__ T front(State& s, uint64_t t, const ScanCtx<T>& c)
    {
        s.st.begin(c.b_log, g0(t, c));
        s.st.in_wave(c.lane);  // levels <= b
        if (c.lane == 63) c.sh->tot[c.w] = s.st.last(ST::V - 1);
        __syncthreads();
        const T t0 = c.sh->tot[0], t1 = c.sh->tot[1], t2 = c.sh->tot[2], t3 = c.sh->tot[3];
        const T t01 = t0 + t1;
        s.st.across_waves(c.w, t0, t01, t2);  // levels <= b
        T total;
        if constexpr (BIG) {
            total = t01 + (t2 + t3);
        } else {
            const int nb_log = LOG_S - c.b_log;  // log2 of the blocks in the tile
            const int nblk = 1 << nb_log;
            const int lm = nb_log > 8 ? nb_log - 8 : 0;
            const int bmask = (1 << c.b_log) - 1;
            const int o0 = off0(c);
#pragma unroll
            for (int u = 0; u < ST::V; ++u) {
                const int end = o0 + u * 64 * E + E;  // one past the vector
                if ((end & bmask) == 0) c.blk[(end >> c.b_log) - 1] = s.st.v[u][E - 1];
            }
            __syncthreads();
            s.bs.load(c.blk, threadIdx.x, lm, nblk);
            s.bs.scan(lm, c.lane, c.w, c.sh->tot);
            if ((int)threadIdx.x == (nblk >> lm) - 1) c.sh->tt = s.bs.tot;  // complete tree
            __syncthreads();
            total = c.sh->tt;
        }
        if (threadIdx.x == 0) publish(c.ws + c.lay->tiles_off + t, total);
        return total;
    }

    static __device__ __forceinline__ void back(State& s, uint64_t t, const ScanCtx<T>& c)
    {
        const T* h = c.sh->lb.h;
        if constexpr (BIG) {
            T cr = neg_zero<T>();
            T wpre = neg_zero<T>();  // in-block nodes, for the value before the tile
            bool forked = false;
            const bool closes = threadIdx.x == kScanThreads - 1 &&
                                (((t + 1) << LOG_S) & ((1ull << c.b_log) - 1)) == 0;
            // levels up to b (every element), then the levels above b
            int k = 0;
#pragma unroll 1
            for (; k < kMaxLevels && (t >> k) != 0 && LOG_S + 1 + k <= c.b_log; ++k)
                if ((t >> k) & 1) {
                    s.st.apply_all(LOG_S + 1 + k, h[k]);
                    if constexpr (OUTX) wpre = h[k] + wpre;
                }
#pragma unroll 1
            for (; k < kMaxLevels && (t >> k) != 0; ++k) {
                if (!((t >> k) & 1)) continue;
                forked = true;
                cr = h[k] + cr;
                if (closes) s.st.v[ST::V - 1][E - 1] = h[k] + s.st.v[ST::V - 1][E - 1];
            }
            if constexpr (OUTX) {
                // the value before the tile: C + W, W the in-block prefix
                // before it (C alone when the tile opens a block)
                s.st.template emit<ALIGNED>(
                    c.y, c.n, g0(t, c), c.init, c.kind, cr + wpre, c.sh->wend, c.w, c.lane,
                    [&](int u, T(&o)[E]) {
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            o[e] = (!forked || (closes && u == ST::V - 1 && e == E - 1))
                                       ? s.st.v[u][e]
                                       : cr + s.st.v[u][e];
                    });
                return;
            }
            if (!forked) {
                s.st.template store<ALIGNED>(c.y, c.n, g0(t, c));
                return;
            }
#pragma unroll
            for (int u = 0; u < ST::V; ++u) {
                T o[E];
#pragma unroll
                for (int e = 0; e < E; ++e)
                    o[e] = (closes && u == ST::V - 1 && e == E - 1) ? s.st.v[u][e]
                                                                    : cr + s.st.v[u][e];
                s.st.template put<ALIGNED>(c.y, c.n, g0(t, c), u, o);
            }
        } else {
            const int nb_log = LOG_S - c.b_log;
            const int nblk = 1 << nb_log;
            const int lm = nb_log > 8 ? nb_log - 8 : 0;
            T g = neg_zero<T>();
            for (int k = 0; k < kMaxLevels && (t >> k) != 0; ++k)
                if ((t >> k) & 1) {
                    s.bs.receive(h[k]);
                    g = h[k] + g;
                }
            // c.blk[j + 1] = G(P_j), c.blk[0] = G(-0.0); every read of the
            // block totals happened before a barrier since
            const int m = 1 << lm;
#pragma unroll
            for (int k = 0; k < BlockScan<T, LMX>::M; ++k) {
                const int j = (int)threadIdx.x * m + k;
                if (k < m && j < nblk) c.blk[j + 1] = s.bs.a[k];
            }
            if (threadIdx.x == 0) c.blk[0] = g;
            __syncthreads();
            const int bmask = (1 << c.b_log) - 1;
            const int o0 = off0(c);
            // final values of vector u: C_j + W inside block j, the block's
            // pairwise value at its end
            auto fin = [&](int u, T(&o)[E]) {
                const int off = o0 + u * 64 * E;
                const int j = off >> c.b_log;
                const bool end = ((off + E) & bmask) == 0;
                const T cj = c.blk[j];
#pragma unroll
                for (int e = 0; e < E - 1; ++e) o[e] = cj + s.st.v[u][e];
                o[E - 1] = end ? c.blk[j + 1] : cj + s.st.v[u][E - 1];
            };
            if constexpr (OUTX) {
                // the value before the tile is c.blk[0] (a block end)
                s.st.template emit<ALIGNED>(c.y, c.n, g0(t, c), c.init, c.kind, g, c.sh->wend,
                                            c.w, c.lane, fin);
            } else {
#pragma unroll
                for (int u = 0; u < ST::V; ++u) {
                    T o[E];
                    fin(u, o);
                    s.st.template put<ALIGNED>(c.y, c.n, g0(t, c), u, o);
                }
            }
        }
    }
};

// block_dyadic with whole-vector blocks inside one wave: B = 64 E 2^VLOG
// with VLOG <= LOGV, so every block is 2^VLOG whole vectors of one wave and
// a block's value and its carry are the same for all 64 lanes.  The tile
// network runs the levels <= b (inside a vector, across lanes, and the
// vector levels below VLOG: the pairwise network, which needs no gating);
// each wave then moves its NBW = 2^(LOGV - VLOG) block totals into lanes
// 0..NBW-1 and runs the pairwise scan of the block totals across those
// lanes; the wave totals (the complete trees of the waves, by closure) merge
// across the 4 waves as in the pairwise network, one barrier in all.  p
// (lane j) then holds the pairwise value of the tile's blocks up to block j
// of this wave, and wpre that of the blocks before the wave.  The back adds
// the tile-level nodes on the left of both; an element outputs (value at
// the previous block end) + W, and a block end its own block's value.
template <typename T, bool ALIGNED, int LOGV, int VLOG, bool OUTX>
struct WideTile {
    using ST = ScanTile<T, 0, LOGV>;
    static constexpr int E = ST::E;
    static constexpr int LOGE = ST::LOGE;
    static constexpr int V = ST::V;
    static constexpr int LOG_S = ST::LOG_S;
    static constexpr int VPB = 1 << VLOG;             // vectors per block
    static constexpr int NBW_LOG = LOGV - VLOG;       // log2 blocks per wave
    static_assert(VLOG >= 0 && VLOG <= LOGV, "blocks of whole vectors inside one wave");
    // f64: two tiles held in at most 168 VGPRs (3 waves per SIMD), a few
    // values spilled; measured 2% faster at B = 256 (f32: no change)
    static constexpr int kMinWavesPerEu = (sizeof(T) == 8 && !kIsOpVal<T>) ? 3 : 1;
    struct State {
        ST st;
        T p;     // lane j < 2^NBW_LOG: pairwise value of the blocks up to block j of this wave
        T wpre;  // pairwise value of the tile's blocks before this wave (-0.0 for wave 0)
    };

    static __device__ __forceinline__ uint64_t g0(uint64_t t, const ScanCtx<T>& c)
    {
        return (t << LOG_S) + ((uint64_t)c.w << ST::LOG_WSPAN) + (uint64_t)c.lane * E;
    }
    static __device__ __forceinline__ void load(State& s, uint64_t t, const ScanCtx<T>& c)
    {
        s.st.template load<ALIGNED>(c.x, c.n, g0(t, c));
    }

    static __device__ __forceinline__ T front(State& s, uint64_t t, const ScanCtx<T>& c)
    {
        // levels <= b: W (the pairwise prefix inside the block) in every element
        s.st.slot_levels();
        s.st.template lane_level<0>(c.lane);
        s.st.template lane_level<1>(c.lane);
        s.st.template lane_level<2>(c.lane);
        s.st.template lane_level<3>(c.lane);
        s.st.template lane_level<4>(c.lane);
        s.st.template lane_level<5>(c.lane);
        if constexpr (VLOG >= 1) s.st.template vector_level<0>();
        if constexpr (VLOG >= 2) s.st.template vector_level<1>();
        if constexpr (VLOG >= 3) s.st.template vector_level<2>();
        if constexpr (VLOG >= 4) s.st.template vector_level<3>();
        T p = neg_zero<T>();
#pragma unroll
        for (int j = 0; j < (1 << NBW_LOG); ++j) {
            const T sj = readlane(s.st.v[(j + 1) * VPB - 1][E - 1], 63);  // block j's total
            p = c.lane == j ? sj : p;
        }
#define CANON_WIDE_LANE(K)                                                    \
    if constexpr ((K) < NBW_LOG) {                                            \
        const T src = from_lower_half_end<(1 << (K))>(p);                     \
        p = (((c.lane >> (K)) & 1) ? src : neg_zero<T>()) + p;                \
    }
        CANON_WIDE_LANE(0)
        CANON_WIDE_LANE(1)
        CANON_WIDE_LANE(2)
        CANON_WIDE_LANE(3)
        CANON_WIDE_LANE(4)
        CANON_WIDE_LANE(5)
#undef CANON_WIDE_LANE
        const T wt = readlane(p, (1 << NBW_LOG) - 1);  // complete tree of the wave
        if (c.lane == 0) c.sh->tot[c.w] = wt;
        __syncthreads();
        const T t0 = c.sh->tot[0], t1 = c.sh->tot[1], t2 = c.sh->tot[2], t3 = c.sh->tot[3];
        const T t01 = t0 + t1;
        const T total = t01 + (t2 + t3);
        if (threadIdx.x == 0) publish(c.ws + c.lay->tiles_off + t, total);
        if (c.w & 1) p = ((c.w & 2) ? t2 : t0) + p;
        if (c.w & 2) p = t01 + p;
        s.wpre = c.w == 0 ? neg_zero<T>() : c.w == 1 ? t0 : c.w == 2 ? t01 : t01 + t2;
        s.p = p;
        return total;
    }

    static __device__ __forceinline__ void back(State& s, uint64_t t, const ScanCtx<T>& c)
    {
        const T* h = c.sh->lb.h;
        T p = s.p, cw = s.wpre;
        for (int k = 0; k < kMaxLevels && (t >> k) != 0; ++k)
            if ((t >> k) & 1) {
                p = h[k] + p;
                cw = h[k] + cw;
            }
        // the value at the end of block j - 1 (cw before the wave's first
        // block) and at the end of block j, for the block of vector u
        auto fin = [&](int u, T(&o)[E]) {
            const int j = u / VPB;
            const T cj = j == 0 ? cw : readlane(p, j - 1);
#pragma unroll
            for (int e = 0; e < E - 1; ++e) o[e] = cj + s.st.v[u][e];
            if ((u + 1) % VPB == 0) {
                // read in every lane, outside the lane-63 select (compiled
                // inside the branch that lane 63 alone takes, the read gave
                // wrong values for a caller-defined operator)
                const T pj = readlane(p, j);
                o[E - 1] = c.lane == 63 ? pj : cj + s.st.v[u][E - 1];
            } else {
                o[E - 1] = cj + s.st.v[u][E - 1];
            }
        };
        if constexpr (OUTX) {
            // the element before the wave's first one ends the previous
            // wave's last block (or the tile before): its value is cw
            s.st.template emit_known<ALIGNED>(c.y, c.n, g0(t, c), c.init, c.kind, cw, c.lane, fin);
        } else {
#pragma unroll
            for (int u = 0; u < V; ++u) {
                T o[E];
                fin(u, o);
                s.st.template put<ALIGNED>(c.y, c.n, g0(t, c), u, o);
            }
        }
    }
};

// block_dyadic with blocks inside one vector row of a wave: B = E 2^Q,
// 0 <= Q <= 5, so a block is the vectors of LPB = 2^Q consecutive lanes of
// one row (64 / LPB blocks per row).  The tile network runs the levels <= b
// (inside a vector and across the block's lanes): W, the pairwise prefix
// inside the block, in every element, and the block's total at its last
// lane.  Each lane then carries one value per vector row, cur[u], through the
// pairwise scan of the block totals: across lane groups of 2 LPB .. 64 lanes,
// across the thread's rows, across the 4 waves (one barrier), lower levels
// first, each level adding the end of the lower half on the left, the same
// for every lane of a block.  At a block's last lane cur[u] is then the
// pairwise value of the tile's blocks up to that block.  The back adds the
// tile-level nodes on the left of every cur[u] and of the value before the
// wave; an element outputs the value at the end of the previous block + W,
// a block end its own block's value.  No LDS pass over the block totals and
// one barrier per tile besides the look-back's.
template <typename T, bool ALIGNED, int LOGV, int Q, bool OUTX>
struct LaneBlockTile {
    using ST = ScanTile<T, 0, LOGV>;
    static constexpr int E = ST::E;
    static constexpr int V = ST::V;
    static constexpr int LOG_S = ST::LOG_S;
    static constexpr int LPB = 1 << Q;  // lanes per block
    static_assert(Q >= 0 && Q <= 5, "blocks inside one vector row");
    static constexpr int kMinWavesPerEu = 1;
    struct State {
        ST st;
        T cur[V];  // per row u: at the block's last lane, the blocks' pairwise value up to it
        T wpre;    // pairwise value of the tile's blocks before this wave (-0.0 for wave 0)
    };

    static __device__ __forceinline__ uint64_t g0(uint64_t t, const ScanCtx<T>& c)
    {
        return (t << LOG_S) + ((uint64_t)c.w << ST::LOG_WSPAN) + (uint64_t)c.lane * E;
    }
    static __device__ __forceinline__ void load(State& s, uint64_t t, const ScanCtx<T>& c)
    {
        s.st.template load<ALIGNED>(c.x, c.n, g0(t, c));
    }

    static __device__ __forceinline__ T front(State& s, uint64_t t, const ScanCtx<T>& c)
    {
        // levels <= b: W in every element
        s.st.slot_levels();
        if constexpr (Q > 0) s.st.template lane_level<0>(c.lane);
        if constexpr (Q > 1) s.st.template lane_level<1>(c.lane);
        if constexpr (Q > 2) s.st.template lane_level<2>(c.lane);
        if constexpr (Q > 3) s.st.template lane_level<3>(c.lane);
        if constexpr (Q > 4) s.st.template lane_level<4>(c.lane);
#pragma unroll
        for (int u = 0; u < V; ++u) s.cur[u] = s.st.v[u][E - 1];
        // block levels across lane groups (sources: the last lanes of blocks)
#define CANON_LB_LANE(K)                                                              \
    if constexpr ((K) >= Q) {                                                         \
        _Pragma("unroll") for (int u = 0; u < V; ++u)                                 \
        {                                                                             \
            const T src = from_lower_half_end<(1 << (K))>(s.cur[u]);                  \
            s.cur[u] = (((c.lane >> (K)) & 1) ? src : neg_zero<T>()) + s.cur[u];      \
        }                                                                             \
    }
        CANON_LB_LANE(0)
        CANON_LB_LANE(1)
        CANON_LB_LANE(2)
        CANON_LB_LANE(3)
        CANON_LB_LANE(4)
        CANON_LB_LANE(5)
#undef CANON_LB_LANE
        // block levels across the thread's rows (sources: lane 63 of a row)
#pragma unroll
        for (int l = 0; l < LOGV; ++l) {
            const int H = 1 << l;
#pragma unroll
            for (int u = 0; u < V; ++u)
                if (u & H) s.cur[u] = readlane(s.cur[(u & ~(2 * H - 1)) + H - 1], 63) + s.cur[u];
        }
        const T wt = readlane(s.cur[V - 1], 63);  // complete tree of the wave
        if (c.lane == 0) c.sh->tot[c.w] = wt;
        __syncthreads();
        const T t0 = c.sh->tot[0], t1 = c.sh->tot[1], t2 = c.sh->tot[2], t3 = c.sh->tot[3];
        const T t01 = t0 + t1;
        const T total = t01 + (t2 + t3);
        if (threadIdx.x == 0) publish(c.ws + c.lay->tiles_off + t, total);
        if (c.w & 1) {
            const T v = (c.w & 2) ? t2 : t0;
#pragma unroll
            for (int u = 0; u < V; ++u) s.cur[u] = v + s.cur[u];
        }
        if (c.w & 2) {
#pragma unroll
            for (int u = 0; u < V; ++u) s.cur[u] = t01 + s.cur[u];
        }
        s.wpre = c.w == 0 ? neg_zero<T>() : c.w == 1 ? t0 : c.w == 2 ? t01 : t01 + t2;
        return total;
    }

    static __device__ __forceinline__ void back(State& s, uint64_t t, const ScanCtx<T>& c)
    {
        const T* h = c.sh->lb.h;
        T cw = s.wpre;
        for (int k = 0; k < kMaxLevels && (t >> k) != 0; ++k)
            if ((t >> k) & 1) {
#pragma unroll
                for (int u = 0; u < V; ++u) s.cur[u] = h[k] + s.cur[u];
                cw = h[k] + cw;
            }
        const int first = c.lane & ~(LPB - 1);  // the block's first lane
        const bool bend = (c.lane & (LPB - 1)) == LPB - 1;
        // the value at the end of the previous block: the last lane of the
        // block before in the row, else lane 63 of the row before, else cw
        // (before the wave's first block); every lane takes part in the moves
        auto fin = [&](int u, T(&o)[E]) {
            const T inrow = shfl_idx(s.cur[u], first - 1);
            const T prow = u > 0 ? readlane(s.cur[u > 0 ? u - 1 : 0], 63) : cw;
            const T prev = first > 0 ? inrow : prow;
#pragma unroll
            for (int e = 0; e < E - 1; ++e) o[e] = prev + s.st.v[u][e];
            o[E - 1] = bend ? s.cur[u] : prev + s.st.v[u][E - 1];
        };
        if constexpr (OUTX) {
            // the element before the wave's first one ends the previous
            // wave's last block (or the tile before): its value is cw
            s.st.template emit_known<ALIGNED>(c.y, c.n, g0(t, c), c.init, c.kind, cw, c.lane, fin);
        } else {
#pragma unroll
            for (int u = 0; u < V; ++u) {
                T o[E];
                fin(u, o);
                s.st.template put<ALIGNED>(c.y, c.n, g0(t, c), u, o);
            }
        }
    }
};

// One pipeline step of a persistent workgroup: tile t is in `cur` with its
// front done (total published).  Takes the next ticket and issues its loads
// into `nxt`, reads t's look-back words afresh right behind them, runs the
// next tile's front (so a tile's total never waits for another tile's
// look-back; when that tile ends its group, wave 0 then builds the group's
// node), then resolves t's look-back (its words have had the whole front
// to arrive) and finishes t.  Returns false when no tile is left.
template <class P, typename T>
__device__ __forceinline__ bool pipe_step(typename P::State& cur, typename P::State& nxt,
                                          uint64_t& t, const ScanCtx<T>& c)
{
    const uint64_t tn = next_ticket(c);
    const bool more = tn < c.lay->ntiles;
    if (more) P::load(nxt, tn, c);
    LookbackWords lw{};
    if (t > 0) lw = lookback_issue<T>(t, c.ws, *c.lay, c.w, c.lane);
    if (more) {
        P::front(nxt, tn, c);
        if (ends_group(tn) && c.w == 0) group_build<T>(tn, c.ws, *c.lay, c.err, c.lane);
    }
    if (t > 0)
        run_lookback<T>(t, lw, c.ws, *c.lay, c.err, c.sh->lb.low, c.sh->lb.g6, c.sh->lb.w3,
                        c.sh->lb.h, c.w, c.lane);
    P::back(cur, t, c);
    t = tn;
    return more;
}

// Single-pass scan kernel: a persistent grid (about as many workgroups as
// fit at once); each workgroup walks tiles in ticket order, two at a time
// (pipe_step).  Tile numbers come from an atomic ticket counter in the order
// workgroups ask, so every tile waited on belongs to a workgroup that is
// running; no front waits for anything, so every published total arrives.
template <class P, typename T>
__global__ __launch_bounds__(kScanThreads)
__attribute__((amdgpu_waves_per_eu(P::kMinWavesPerEu))) void k_scan(const T* x, T* y, uint64_t n, int b_log,
                                                       uint64_t* __restrict__ ws, ScanLayout lay,
                                                       T init, int kind)
{
    __shared__ ScanShared<T> sh;
    extern __shared__ __align__(16) unsigned char s_dyn[];
    const ScanCtx<T> c{x,
                       y,
                       n,
                       b_log,
                       ws,
                       &lay,
                       reinterpret_cast<uint32_t*>(ws),
                       &sh,
                       reinterpret_cast<T*>(s_dyn),
                       (int)(threadIdx.x & 63),
                       (int)(threadIdx.x >> 6),
                       init,
                       kind};
    uint64_t t = next_ticket(c);
    if (t >= lay.ntiles) return;
    typename P::State a, b;
    P::load(a, t, c);
    P::front(a, t, c);
    if (ends_group(t) && c.w == 0) group_build<T>(t, c.ws, lay, c.err, c.lane);
    for (;;) {
        if (!pipe_step<P, T>(a, b, t, c)) break;
        if (!pipe_step<P, T>(b, a, t, c)) break;
    }
}

// ---------------------------------------------------------------- launchers
template <class P, typename T>
static hipError_t launch_k(const T* x, T* y, uint64_t n, int b_log, uint64_t* ws,
                           const ScanLayout& lay, size_t shmem, const ScanOut<T>& out,
                           hipStream_t s)
{
    constexpr auto kern = k_scan<P, T>;
    uint64_t grid = capped_grid(resident_grid<kern>(kScanThreads, shmem));
    if (grid > lay.ntiles) grid = lay.ntiles;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kScanThreads), shmem, s, x, y, n, b_log,
                       ws, lay, out.init, out.kind);
    return hipGetLastError();
}

template <typename T, int MODE, bool OUTX>
static hipError_t launch_full(const T* x, T* y, uint64_t n, int b_log, bool aligned,
                              uint64_t* ws, const ScanLayout& lay, const ScanOut<T>& out,
                              hipStream_t s)
{
    if (aligned)
        return launch_k<FullTile<T, MODE, true, scan_log_v<T>(), OUTX>>(x, y, n, b_log, ws, lay, 0,
                                                                        out, s);
    return launch_k<FullTile<T, MODE, false, scan_log_v<T>(), OUTX>>(x, y, n, b_log, ws, lay, 0,
                                                                     out, s);
}

template <typename T, bool BIG, int LMX, bool OUTX>
static hipError_t launch_split_k(const T* x, T* y, uint64_t n, int b_log, bool aligned,
                                 uint64_t* ws, const ScanLayout& lay, const ScanOut<T>& out,
                                 hipStream_t s)
{
    constexpr int LOG_S = scan_tile_log<T>();
    const size_t shmem = BIG ? 0 : ((1ull << (LOG_S - b_log)) + 1) * sizeof(T);
    if (aligned)
        return launch_k<SplitTile<T, true, scan_log_v<T>(), BIG, LMX, OUTX>>(
            x, y, n, b_log, ws, lay, shmem, out, s);
    return launch_k<SplitTile<T, false, scan_log_v<T>(), BIG, LMX, OUTX>>(x, y, n, b_log, ws, lay,
                                                                          shmem, out, s);
}

// The WideTile kernels are instantiated in their own translation unit
// (scan_wide.hip).
template <typename T, bool OUTX>
hipError_t launch_wide(const T* x, T* y, uint64_t n, int b_log, bool aligned, uint64_t* ws,
                       const ScanLayout& lay, const ScanOut<T>& out, hipStream_t s);

// The LaneBlockTile kernels, in their own translation units (scan_lane.hip,
// scan_lane_init.hip): b_log from LOGE to LOGE + 5.  Blocks of one lane's
// vector (b_log = LOGE) only where a vector holds two values: with four, the
// six lane levels of the block scan on 16 rows spill (f32 B = 4 at 2^28:
// 613 us against 452 us for SplitTile).
template <typename T>
constexpr bool kLaneOneLaneBlocks = Elem<T>::E == 2;
template <typename T, bool OUTX>
hipError_t launch_lane_block(const T* x, T* y, uint64_t n, int b_log, bool aligned, uint64_t* ws,
                             const ScanLayout& lay, const ScanOut<T>& out, hipStream_t s);

template <typename T, bool OUTX>
hipError_t launch_lane_block_impl(const T* x, T* y, uint64_t n, int b_log, bool aligned,
                                  uint64_t* ws, const ScanLayout& lay, const ScanOut<T>& out,
                                  hipStream_t s)
{
    constexpr int LOGV = scan_log_v<T>();
#define CANON_LANE_CASE(QQ)                                                                      \
    case QQ:                                                                                     \
        if (aligned)                                                                             \
            return launch_k<LaneBlockTile<T, true, LOGV, QQ, OUTX>>(x, y, n, b_log, ws, lay, 0,  \
                                                                    out, s);                     \
        return launch_k<LaneBlockTile<T, false, LOGV, QQ, OUTX>>(x, y, n, b_log, ws, lay, 0,     \
                                                                 out, s);
    switch (b_log - Elem<T>::LOGE) {
        case 0:
            if constexpr (kLaneOneLaneBlocks<T>) {
                if (aligned)
                    return launch_k<LaneBlockTile<T, true, LOGV, 0, OUTX>>(x, y, n, b_log, ws, lay,
                                                                           0, out, s);
                return launch_k<LaneBlockTile<T, false, LOGV, 0, OUTX>>(x, y, n, b_log, ws, lay, 0,
                                                                        out, s);
            }
            return hipErrorInvalidValue;
        CANON_LANE_CASE(1)
        CANON_LANE_CASE(2)
        CANON_LANE_CASE(3)
        CANON_LANE_CASE(4)
        CANON_LANE_CASE(5)
        default: return hipErrorInvalidValue;
    }
#undef CANON_LANE_CASE
}

template <typename T, bool OUTX>
hipError_t launch_wide_impl(const T* x, T* y, uint64_t n, int b_log, bool aligned, uint64_t* ws,
                            const ScanLayout& lay, const ScanOut<T>& out, hipStream_t s)
{
    constexpr int LOGV = scan_log_v<T>();
    const int vlog = b_log - (Elem<T>::LOGE + 6);
#define CANON_WIDE_CASE(VL)                                                                  \
    case VL:                                                                                 \
        if constexpr (VL <= LOGV) {                                                          \
            if (aligned)                                                                     \
                return launch_k<WideTile<T, true, LOGV, VL, OUTX>>(x, y, n, b_log, ws, lay, 0, \
                                                                   out, s);                  \
            return launch_k<WideTile<T, false, LOGV, VL, OUTX>>(x, y, n, b_log, ws, lay, 0,    \
                                                                out, s);                     \
        }                                                                                    \
        return hipErrorInvalidValue;
    switch (vlog) {
        CANON_WIDE_CASE(0)
        CANON_WIDE_CASE(1)
        CANON_WIDE_CASE(2)
        CANON_WIDE_CASE(3)
        CANON_WIDE_CASE(4)
        default: return hipErrorInvalidValue;
    }
#undef CANON_WIDE_CASE
}

template <typename T, bool OUTX>
static hipError_t launch_split(const T* x, T* y, uint64_t n, int b_log, bool aligned,
                               uint64_t* ws, const ScanLayout& lay, const ScanOut<T>& out,
                               hipStream_t s)
{
    // blocks per thread in the block scan: 2^(log2(tile / B) - 8) when that is > 1
    constexpr int LOG_S = scan_tile_log<T>();
    if (b_log >= LOG_S)
        return launch_split_k<T, true, 0, OUTX>(x, y, n, b_log, aligned, ws, lay, out, s);
    constexpr int LOG_WSPAN = LOG_S - 2;
    if (b_log >= Elem<T>::LOGE + 6 && b_log <= LOG_WSPAN)
        return launch_wide<T, OUTX>(x, y, n, b_log, aligned, ws, lay, out, s);
    if (b_log < Elem<T>::LOGE + 6 && b_log >= Elem<T>::LOGE + (kLaneOneLaneBlocks<T> ? 0 : 1))
        return launch_lane_block<T, OUTX>(x, y, n, b_log, aligned, ws, lay, out, s);
    const int lm = LOG_S - b_log > 8 ? LOG_S - b_log - 8 : 0;
    if (lm <= 2) return launch_split_k<T, false, 2, OUTX>(x, y, n, b_log, aligned, ws, lay, out, s);
    return launch_split_k<T, false, 4, OUTX>(x, y, n, b_log, aligned, ws, lay, out, s);
}

// The single-pass scan (n >= 1).  OUTX selects the kernels with the output
// stage of a scan with an initial value (out.init, out.kind); without it the
// plain inclusive scan is written and `out` is unused.
template <typename T, bool OUTX>
hipError_t launch_scan_impl(const T* x, T* y, uint64_t n, bool pairwise, int b_log, bool aligned,
                            uint64_t* ws, const ScanLayout& lay, const ScanOut<T>& out,
                            hipStream_t s)
{
    launch_scan_init<T>(ws, lay, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (pairwise || b_log == 0)
        return launch_full<T, 0, OUTX>(x, y, n, 0, aligned, ws, lay, out, s);
    if constexpr (Elem<T>::LOGE >= 2) {
        if (b_log < Elem<T>::LOGE)
            return launch_full<T, 2, OUTX>(x, y, n, b_log, aligned, ws, lay, out, s);
    }
    return launch_split<T, OUTX>(x, y, n, b_log, aligned, ws, lay, out, s);
}

}  // namespace canon
