// Canonical scan, policy iterated_pairwise<L>, in one pass over the input
// (gfx950, register geometry: L = E * 2^j lanes, E <= L <= 512 E; element
// loads and stores where rows are off the 16-byte grid).
//
// Expression and evaluation inside a tile: as in scan_ip.hip (canonical-
// reduce README, P4229R0 "Summary"; P4016R0 "Key Design Points").  Tile t
// needs, for every lane, the pairwise value of that lane over all rows
// before the tile: the right-nested combination of node (k, (t >> k) - 1)
// for the set bits k of t, lowest level first, where node (k, u) is the
// complete per-lane pairwise tree over tiles [u 2^k, (u+1) 2^k).
//
// Across tiles, without a second read of the input and without any
// workgroup waiting before it has published what others need:
//   * each tile publishes its own per-lane totals (node (0, t)) as soon as
//     its in-tile column scan is done (the tile's "front");
//   * node (k+1, v) is formed by whichever of its two children arrives
//     second: a tile counts itself in its level-1 parent's arrival counter
//     when its loads are issued, and after publishing node (k, u), k >= 1,
//     in that node's parent's counter; the tile that counts second reads
//     the other child (waiting, if need be, for its words, which are
//     published without waiting for this tile), adds (left child on the
//     left) and publishes the parent, then tries the next level; a tile
//     counting first stops there;
//   * the tile's "back" then reads the nodes of its set bits, applies them,
//     walks its rows' lane trees and stores.
// Every node a tile waits for covers only tiles with smaller tickets, and
// the work that publishes it waits only for words already being written, so
// every wait ends.  Every value is fixed by position, never by arrival order.
// Published words are self-describing (device.hpp): polled without fences.
//
// PIPE kernels are persistent and software-pipelined like the single-pass
// scalar scan: a workgroup holds two tiles and runs the next tile's front
// before the current tile's back, so a back's reads of nodes published by
// the tiles just before it have had a whole front to arrive.
#pragma once
#include "device.hpp"
#include "launch.hpp"
#include "scan.hpp"
#include "scan_ip.hpp"
#include "scan_ip_fast.hpp"

namespace canon {

// LDS values staged per batch of look-back nodes (a multiple of kIpThreads;
// at least one node of L values).
constexpr int kIp1Stage = 1024;
// Persistent, two tiles per workgroup (else one workgroup per tile): the
// geometries whose two tiles fit the registers without spilling.
template <int LOGRV>
constexpr bool ip1_pipelined()
{
    return LOGRV <= 0;
}

// The per-level arrays of the layout, copied to LDS by every workgroup: a
// level-indexed read of the kernel argument compiles to a vector load, and
// waiting for one would also wait for every tile load issued before it.
struct Ip1Levels {
    uint64_t woff[kIpMaxLevels];
    uint64_t coff[kIpMaxLevels];
    uint64_t cnt[kIpMaxLevels];
};

__device__ __forceinline__ uint64_t* ip1_word(uint64_t* ws, const Ip1Levels& lv, uint64_t L, int k,
                                              uint64_t seg, uint64_t u, uint64_t col)
{
    return ws + lv.woff[k] + (seg * lv.cnt[k] + u) * L + col;
}

__device__ __forceinline__ uint32_t* ip1_counter(uint64_t* ws, const IpSingleLayout& lay,
                                                 const Ip1Levels& lv, int k, uint64_t seg,
                                                 uint64_t v)
{
    return reinterpret_cast<uint32_t*>(ws + lay.cbase) + lv.coff[k] + seg * lv.cnt[k] + v;
}

// Header (error word, ticket; word 2 the bound of the call's waits, 0 for
// the default), every node word not ready, counters zero.
template <typename T>
__global__ __launch_bounds__(256) void k_ip1_init(uint64_t* __restrict__ ws, IpSingleLayout lay,
                                                  uint64_t spin_limit)
{
    const uint64_t nr = not_ready_word<T>();
    const uint64_t cw = (lay.counters + 1) / 2;
    const uint64_t total = lay.cbase + cw;
    for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (uint64_t)gridDim.x * 256)
        ws[i] = i < 32 ? (i == 2 ? spin_limit : 0ull) : (i < lay.cbase ? nr : 0ull);
}

template <typename T, int LOGRV>
struct Ip1Shared {
    static constexpr int L = IpFast<T, LOGRV>::L;
    static constexpr int STAGE = L > kIp1Stage ? L : kIp1Stage;
    alignas(16) T row[4][L];  // per-wave rows exchanged between the waves
    alignas(16) T h[STAGE];   // node values of the earlier tiles, a batch at a time
    Ip1Levels lvl;
    uint32_t ticket;
};

template <typename T, int LOGRV>
struct Ip1Ctx {
    const T* x;
    uint64_t ldx;
    T* y;
    uint64_t ldy;
    uint64_t cols;
    uint64_t* ws;
    const IpSingleLayout* lay;
    uint32_t* err;
    Ip1Shared<T, LOGRV>* sh;
    int lane, w;
    T init;
    int kind;
};

// One tile in registers: vector u of thread (w, lane) holds row
// w * RW + u / RV of the tile, columns ((u % RV) * 64 + lane) * E + e.
template <typename T, int LOGRV>
struct Ip1Tile {
    T a[IpFast<T, LOGRV>::NV][Elem<T>::E];
    uint64_t item;
    uint32_t before1;  // wave 3, lane 0: the level-1 arrival count before this tile's
};

template <typename T, int LOGRV>
__device__ __forceinline__ uint64_t ip1_ticket(const Ip1Ctx<T, LOGRV>& c)
{
    if (threadIdx.x == 0)
        c.sh->ticket = __hip_atomic_fetch_add(reinterpret_cast<uint32_t*>(c.ws + 1), 1u,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    // uniform: kept in scalar registers, so that the node addresses derived
    // from it (layout arrays indexed by level) are scalar loads, which a
    // wait for them does not order behind the tile's vector loads
    const uint64_t it = __builtin_amdgcn_readfirstlane(c.sh->ticket);
    __syncthreads();  // the slot is rewritten by the next ticket
    return it;
}

// AL: rows on 16-byte boundaries (16-byte loads; else element loads).
template <bool AL, typename T, int LOGRV>
__device__ __forceinline__ void ip1_load(Ip1Tile<T, LOGRV>& s, uint64_t item,
                                         const Ip1Ctx<T, LOGRV>& c)
{
    using F = IpFast<T, LOGRV>;
    s.item = item;
    const uint64_t seg = item / c.lay->g.tps, t = item % c.lay->g.tps;
    const uint64_t row0 = t * F::R;
    const T* xs = c.x + seg * c.ldx;
    if (AL && (row0 + F::R) * F::L <= c.cols)
        ipf_load<T, LOGRV, false>(xs, c.cols, row0, c.w, c.lane, s.a);
    else
        ipf_load<T, LOGRV, true>(xs, c.cols, row0, c.w, c.lane, s.a);
    // The tile's arrival at its level-1 parent is counted now, behind its
    // loads: the count does not depend on the front, and its round trip
    // then overlaps the loads' (a tile that counts second waits, in the
    // climb, for its sibling's totals to be published, which they will be
    // without waiting for this tile).
    s.before1 = 0;
    if (c.w == 3 && c.lane == 0 && 1 < c.lay->g.levels && (t >> 1) < c.sh->lvl.cnt[1])
        s.before1 = __hip_atomic_fetch_add(ip1_counter(c.ws, *c.lay, c.sh->lvl, 1, seg, t >> 1),
                                           1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Front: the lane prefixes inside the tile, the tile's totals published,
// and the parents it completes.
template <typename T, int LOGRV>
__device__ __forceinline__ void ip1_front(Ip1Tile<T, LOGRV>& s, const Ip1Ctx<T, LOGRV>& c)
{
    using F = IpFast<T, LOGRV>;
    constexpr int E = F::E, RV = F::RV, RW = F::RW;
    const IpSingleLayout& lay = *c.lay;
    const uint64_t seg = s.item / lay.g.tps, t = s.item % lay.g.tps;
    const int lane = c.lane, w = c.w;
    // the lanes holding the wave's last rows (every lane for wide rows)
    const bool last = F::group(lane) == F::G - 1;
    auto& a = s.a;

    ipf_columns_in_wave<T, LOGRV>(a);
    if constexpr (F::G > 1) ipf_groups_in_wave<T, LOGRV>(a, lane);
    if (last) {
#pragma unroll
        for (int q = 0; q < RV; ++q) lds_store_vec(&c.sh->row[w][F::col(q, lane)], a[(RW - 1) * RV + q]);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < RV; ++q) {
        T r0[E], r1[E], r2[E];
        lds_load_vec(&c.sh->row[0][F::col(q, lane)], r0);
        lds_load_vec(&c.sh->row[1][F::col(q, lane)], r1);
        lds_load_vec(&c.sh->row[2][F::col(q, lane)], r2);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const T t0 = r0[e], t1 = r1[e], t2 = r2[e];
            if (w & 1) {
                const T v = (w & 2) ? t2 : t0;
#pragma unroll
                for (int r = 0; r < RW; ++r) a[r * RV + q][e] = v + a[r * RV + q][e];
            }
            if (w & 2) {
                const T v = t0 + t1;
#pragma unroll
                for (int r = 0; r < RW; ++r) a[r * RV + q][e] = v + a[r * RV + q][e];
            }
        }
    }
    __syncthreads();  // every wave has read row[]

    if (w == 3) {
        auto word = [&](int k, uint64_t u, uint64_t col) {
            return ip1_word(c.ws, c.sh->lvl, lay.g.L, k, seg, u, col);
        };
        T cur[RV][E];
#pragma unroll
        for (int q = 0; q < RV; ++q) {
#pragma unroll
            for (int e = 0; e < E; ++e) cur[q][e] = a[(RW - 1) * RV + q][e];
            if (last)
#pragma unroll
                for (int j = 0; j < F::NP; ++j) {
                    const T pv[2] = {cur[q][2 * j], cur[q][2 * j + 1]};
                    publish_pairs(word(0, t, F::wcol(q, j, lane)), pv);
                }
        }
        uint64_t u = t;
        for (int k = 0; k + 1 < lay.g.levels; ++k) {
            const uint64_t v = u >> 1;
            if (v >= c.sh->lvl.cnt[k + 1]) break;  // the parent covers tiles past the end
            uint32_t before = 0;
            if (k == 0)
                before = s.before1;  // counted when the tile was loaded
            else if (lane == 0)
                before = __hip_atomic_fetch_add(ip1_counter(c.ws, lay, c.sh->lvl, k + 1, seg, v),
                                                1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            before = __builtin_amdgcn_readfirstlane(before);
            if (before == 0) break;  // the sibling completes the parent
            if (last) {
                // the sibling's words: all reads issued, then waited for
                const uint64_t* sp[RV * F::NP];
#pragma unroll
                for (int q = 0; q < RV; ++q)
#pragma unroll
                    for (int j = 0; j < F::NP; ++j)
                        sp[q * F::NP + j] = word(k, u ^ 1, F::wcol(q, j, lane));
                uint64_t sw[RV * F::NP][2];
                load_pairs(sp, sw);
#pragma unroll
                for (int q = 0; q < RV; ++q) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const uint64_t col = F::wcol(q, e / 2, lane) + (e & 1);
                        const T sib = ready_or_wait<T>(sw[q * F::NP + e / 2][e & 1],
                                                       word(k, u ^ 1, col), c.err);
                        cur[q][e] = (u & 1) ? sib + cur[q][e] : cur[q][e] + sib;
                    }
#pragma unroll
                    for (int j = 0; j < F::NP; ++j) {
                        const T pv[2] = {cur[q][2 * j], cur[q][2 * j + 1]};
                        publish_pairs(word(k + 1, v, F::wcol(q, j, lane)), pv);
                    }
                }
            }
            u = v;
        }
    }
}

// Back: the nodes of the earlier tiles applied (right-nested, lowest level
// first), each row's lane tree walked, the outputs stored.
template <typename T, int LOGRV, bool OUTX, bool AL>
__device__ __forceinline__ void ip1_back(Ip1Tile<T, LOGRV>& s, const Ip1Ctx<T, LOGRV>& c)
{
    using F = IpFast<T, LOGRV>;
    using SH = Ip1Shared<T, LOGRV>;
    constexpr int E = F::E, RV = F::RV, RW = F::RW;
    // The node words are read by waves 0-2 alone: wave 3 comes to the back
    // from the front's climb, and its reads would hold up the batch.
    constexpr int RT = kIpThreads - 64;                  // reading threads
    constexpr int NB = SH::STAGE / F::L < 16 ? SH::STAGE / F::L : 16;  // nodes per batch
    constexpr int WORDS = NB * F::L;                     // words per batch
    constexpr int PER = (WORDS + RT - 1) / RT;           // words per reading thread
    const IpSingleLayout& lay = *c.lay;
    const uint64_t seg = s.item / lay.g.tps, t = s.item % lay.g.tps;
    const int lane = c.lane, w = c.w;
    auto& a = s.a;
    T* ys = c.y + seg * c.ldy;
    const uint64_t row0 = t * F::R;
    const bool full = (row0 + F::R) * F::L <= c.cols;

    // word `col` of node (k, (t >> k) - 1)
    auto node = [&](int k, int col) {
        return ip1_word(c.ws, c.sh->lvl, lay.g.L, k, seg, (t >> k) - 1, (uint64_t)col);
    };
    // The node words of up to NB set bits at a time, spread over the reading
    // threads (word idx of a batch: node idx / L, word idx % L of the node in
    // its published order, staged in that order), every read
    // issued before any is waited for, then staged in LDS.
    T b[RV][E];
#pragma unroll
    for (int q = 0; q < RV; ++q)
#pragma unroll
        for (int e = 0; e < E; ++e) b[q][e] = neg_zero<T>();
    int k = 0;
    while (k < lay.g.levels && (t >> k) != 0) {
        int lv[NB];
        int nb = 0;
        for (; k < lay.g.levels && (t >> k) != 0 && nb < NB; ++k)
            if ((t >> k) & 1) lv[nb++] = k;
        if (nb == 0) break;
        if (w < 3) {
            uint64_t wv[PER];
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int idx = i * RT + (int)threadIdx.x;
                const int m = idx / F::L, col = idx % F::L;
                wv[i] = not_ready_word<T>();
                if (idx < WORDS && m < nb)
                    wv[i] = __hip_atomic_load(node(lv[m], col), __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int idx = i * RT + (int)threadIdx.x;
                const int m = idx / F::L, col = idx % F::L;
                if (idx < WORDS && m < nb)
                    c.sh->h[idx] = ready_or_wait<T>(wv[i], node(lv[m], col), c.err);
            }
        }
        __syncthreads();
        for (int m = 0; m < nb; ++m) {
#pragma unroll
            for (int q = 0; q < RV; ++q) {
                // the node's words are staged in their published order
                T hv[E];
                if constexpr (F::NP == 1) {
                    lds_load_vec(&c.sh->h[m * F::L + F::wcol(q, 0, lane)], hv);
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        hv[e] = c.sh->h[m * F::L + F::wcol(q, e / 2, lane) + (e & 1)];
                }
#pragma unroll
                for (int e = 0; e < E; ++e) {
#pragma unroll
                    for (int r = 0; r < RW; ++r) a[r * RV + q][e] = hv[e] + a[r * RV + q][e];
                    b[q][e] = hv[e] + b[q][e];
                }
            }
        }
        __syncthreads();  // h is refilled by the next batch
    }
    // the B row of each thread's first row: the A row just above it (the
    // group before in the wave, else the last rows of the wave before)
    const int g = F::group(lane);
    if (g == F::G - 1) {
#pragma unroll
        for (int q = 0; q < RV; ++q) lds_store_vec(&c.sh->row[w][F::col(q, lane)], a[(RW - 1) * RV + q]);
    }
    __syncthreads();
    if (w > 0 && g == 0) {
#pragma unroll
        for (int q = 0; q < RV; ++q) lds_load_vec(&c.sh->row[w - 1][F::col(q, lane)], b[q]);
    }
    if constexpr (F::G > 1) {
        const int src = (lane - F::TPR) & 63;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const T up = shfl_idx(a[RW - 1][e], src);
            if (g > 0) b[0][e] = up;
        }
    }
    __syncthreads();  // row[] is rewritten by the next front

    // walk every lane up its row's tree (each row's sibling values built once)
    IpRowTree<T, LOGRV> tb;
    tb.template build<RV>(b, 0, lane);
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        IpRowTree<T, LOGRV> ta;
        ta.template build<F::NV>(a, r * RV, lane);
        T val[RV][E];
        ip_walk<T, LOGRV>(a, r * RV, ta, tb, lane, val);
        const uint64_t row = row0 + F::row(w, lane, r);
        if constexpr (OUTX) {
            if (c.kind != kScanInclusive) {
                // one position up, the value before a row's first lane being
                // the end of the previous row (the root of its B tree);
                // include_initial: the holder of element cols - 1 also
                // writes y[cols]
                if (c.kind == kScanIncludeInitial) {
#pragma unroll
                    for (int q = 0; q < RV; ++q)
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            if (row * F::L + F::col(q, lane) + e + 1 == c.cols)
                                ys[c.cols] = c.init + val[q][e];
                }
                T prev = tb.root;
#pragma unroll
                for (int q = 0; q < RV; ++q) {
                    const T up = shfl_up1(val[q][E - 1]);
                    const T before = F::sub(lane) == 0 ? prev : up;
                    prev = readlane(val[q][E - 1], 63);
#pragma unroll
                    for (int e = E - 1; e > 0; --e) val[q][e] = val[q][e - 1];
                    val[q][0] = before;
                }
            }
#pragma unroll
            for (int q = 0; q < RV; ++q)
#pragma unroll
                for (int e = 0; e < E; ++e) val[q][e] = c.init + val[q][e];
        }
#pragma unroll
        for (int q = 0; q < RV; ++q) {
            const uint64_t gi = row * F::L + F::col(q, lane);
            if (AL && (full || gi + E <= c.cols)) {
                store_vec(ys + gi, val[q]);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (gi + e < c.cols) ys[gi + e] = val[q][e];
            }
        }
        tb = ta;
    }
}

// PIPE: persistent workgroups, two tiles each (the next front before the
// current back); else one workgroup per tile.
template <typename T, int LOGRV, bool OUTX, bool PIPE, bool AL>
__global__ __launch_bounds__(kIpThreads) void k_ip_single(const T* __restrict__ x, uint64_t ldx,
                                                          T* __restrict__ y, uint64_t ldy,
                                                          uint64_t cols, uint64_t* __restrict__ ws,
                                                          IpSingleLayout lay, T init, int kind)
{
    __shared__ Ip1Shared<T, LOGRV> sh;
    const Ip1Ctx<T, LOGRV> c{x,
                             ldx,
                             y,
                             ldy,
                             cols,
                             ws,
                             &lay,
                             reinterpret_cast<uint32_t*>(ws),
                             &sh,
                             (int)(threadIdx.x & 63),
                             (int)(threadIdx.x >> 6),
                             init,
                             kind};
    const uint64_t items = lay.g.nseg * lay.g.tps;
    for (int i = (int)threadIdx.x; i < kIpMaxLevels; i += kIpThreads) {
        sh.lvl.woff[i] = lay.woff[i];
        sh.lvl.coff[i] = lay.coff[i];
        sh.lvl.cnt[i] = lay.g.cnt[i];
    }
    uint64_t it = ip1_ticket(c);  // its barrier publishes sh.lvl
    if (it >= items) return;
    Ip1Tile<T, LOGRV> A, B;
    ip1_load<AL>(A, it, c);
    ip1_front(A, c);
    if constexpr (!PIPE) {
        ip1_back<T, LOGRV, OUTX, AL>(A, c);
    } else {
        for (;;) {
            it = ip1_ticket(c);
            if (it < items) {
                ip1_load<AL>(B, it, c);
                ip1_front(B, c);
            }
            ip1_back<T, LOGRV, OUTX, AL>(A, c);
            if (it >= items) break;
            it = ip1_ticket(c);
            if (it < items) {
                ip1_load<AL>(A, it, c);
                ip1_front(A, c);
            }
            ip1_back<T, LOGRV, OUTX, AL>(B, c);
            if (it >= items) break;
        }
    }
}

template <typename T, int LOGRV, bool OUTX, bool AL>
static hipError_t launch_ip1_al(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t cols,
                                uint64_t* ws, const IpSingleLayout& lay, const ScanOut<T>& out,
                                hipStream_t s)
{
    const uint64_t items = lay.g.nseg * lay.g.tps;
    constexpr bool PIPE = ip1_pipelined<LOGRV>();
    constexpr auto kern = k_ip_single<T, LOGRV, OUTX, PIPE, AL>;
    uint64_t grid = items;
    if (PIPE) {
        const uint64_t fit = capped_grid(resident_grid<kern>(kIpThreads));
        if (grid > fit) grid = fit;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kIpThreads), 0, s, x, ldx, y, ldy, cols,
                       ws, lay, out.init, out.kind);
    return hipGetLastError();
}

template <typename T, int LOGRV, bool OUTX>
static hipError_t launch_ip1(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t cols,
                             uint64_t* ws, const IpSingleLayout& lay, const ScanOut<T>& out,
                             bool aligned, hipStream_t s)
{
    if (aligned) return launch_ip1_al<T, LOGRV, OUTX, true>(x, ldx, y, ldy, cols, ws, lay, out, s);
    return launch_ip1_al<T, LOGRV, OUTX, false>(x, ldx, y, ldy, cols, ws, lay, out, s);
}

// Narrow rows (L < 64 E), kept apart so that the plain double and float
// kernels compile in units of their own (scan_ip1_narrow_*.hip).
template <typename T, bool OUTX>
hipError_t launch_ip1_narrow(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t cols,
                             uint64_t* ws, const IpSingleLayout& lay, const ScanOut<T>& out,
                             bool al, hipStream_t s)
{
    switch (lay.g.fast_logrv) {
        case -6: return launch_ip1<T, -6, OUTX>(x, ldx, y, ldy, cols, ws, lay, out, al, s);
        case -5: return launch_ip1<T, -5, OUTX>(x, ldx, y, ldy, cols, ws, lay, out, al, s);
        case -4: return launch_ip1<T, -4, OUTX>(x, ldx, y, ldy, cols, ws, lay, out, al, s);
        case -3: return launch_ip1<T, -3, OUTX>(x, ldx, y, ldy, cols, ws, lay, out, al, s);
        case -2: return launch_ip1<T, -2, OUTX>(x, ldx, y, ldy, cols, ws, lay, out, al, s);
        case -1: return launch_ip1<T, -1, OUTX>(x, ldx, y, ldy, cols, ws, lay, out, al, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, bool OUTX>
static hipError_t launch_ip1_o(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t cols,
                               uint64_t* ws, const IpSingleLayout& lay, const ScanOut<T>& out,
                               bool al, hipStream_t s)
{
    if (lay.g.fast_logrv < 0)
        return launch_ip1_narrow<T, OUTX>(x, ldx, y, ldy, cols, ws, lay, out, al, s);
    switch (lay.g.fast_logrv) {
        case 0: return launch_ip1<T, 0, OUTX>(x, ldx, y, ldy, cols, ws, lay, out, al, s);
        case 1: return launch_ip1<T, 1, OUTX>(x, ldx, y, ldy, cols, ws, lay, out, al, s);
        case 2: return launch_ip1<T, 2, OUTX>(x, ldx, y, ldy, cols, ws, lay, out, al, s);
        case 3: return launch_ip1<T, 3, OUTX>(x, ldx, y, ldy, cols, ws, lay, out, al, s);
        default: return hipErrorInvalidValue;
    }
}

// One pass; the caller has checked cols > 0, lay.g.fast_logrv >= 0 and that
// the items fit one launch (nseg * tps < 2^31).
template <typename T, bool PLAIN>
hipError_t launch_scan_ip_single(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t cols,
                                 uint64_t* ws, const IpSingleLayout& lay, const ScanOut<T>* out,
                                 bool aligned, hipStream_t s)
{
    const uint64_t words = lay.cbase + (lay.counters + 1) / 2;
    uint64_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL((k_ip1_init<T>), dim3((unsigned)blocks), dim3(256), 0, s, ws, lay,
                       g_sched_spin_limit.load(std::memory_order_relaxed));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (out) return launch_ip1_o<T, true>(x, ldx, y, ldy, cols, ws, lay, *out, aligned, s);
    if constexpr (PLAIN)
        return launch_ip1_o<T, false>(x, ldx, y, ldy, cols, ws, lay, ScanOut<T>{}, aligned, s);
    return hipErrorInvalidValue;
}

}  // namespace canon
