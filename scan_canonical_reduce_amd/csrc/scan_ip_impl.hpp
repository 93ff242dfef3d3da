// Canonical inclusive scan, policy iterated_pairwise<L> (gfx950).
//
// Expression (canonical-reduce README, P4229R0 "Summary"; the P4016R0
// two-stage expression of "Key Design Points" observed on every prefix):
// y[i] = CR_L(x[0..i]).  View x as rows of L lanes, element i at row
// k = i / L, lane r = i % L.  With
//   A_j = PW of lane j over rows 0..k   (the pairwise prefix of the lane),
//   B_j = PW of lane j over rows 0..k-1 (absent when k = 0),
// y[kL + r] = PW(A_0, ..., A_r, B_{r+1}, ..., B_{L-1}).
//
// PW over the lane values, padded with -0.0 to Lp = 2^ceil(log2 L) lanes, is
// a complete binary tree.  For lane r, walk from leaf r to the root: at each
// level the sibling subtree lies either entirely left of r (all its lanes
// hold A values) or entirely right (all B values).  So
//   val = A_r;  for each level: val = pureA(left sibling) + val
//                               or val = val + pureB(right sibling)
// where pureA / pureB are the subtree values of the trees over row k's A
// values and row k-1's A values (= row k's B values).
//
// This file holds the general path (any L up to the LDS budget, any
// alignment); the register geometry (L = 64 E 2^j, aligned rows) runs in one
// pass (scan_ip1.hip).  Three kernels, no waiting between workgroups:
//   1. tile totals: tile t = R consecutive rows; per lane, the complete
//      pairwise tree over the tile's R rows (an L-vector per tile);
//   2. node levels: node (k, u) = node (k-1, 2u) + node (k-1, 2u+1), built
//      a few levels per launch, per lane;
//   3. scan: per tile, per lane: the pairwise prefix of the lane inside the
//      tile (shift-reduce stack), then the nodes for the set bits k of t
//      applied in increasing k (right-nested, as the pairwise prefix of the
//      lane requires); the B row of the tile's first row is the right-nested
//      value of those nodes alone.  Then the per-row trees in LDS and the
//      walk above for every element.
// Row-batched scans run the same kernels with one segment per row.
#pragma once
#include "device.hpp"
#include "launch.hpp"
#include "scan.hpp"
#include "scan_ip.hpp"

namespace canon {

template <typename T>
__device__ __forceinline__ T* ip_node(T* nodes, const IpLayout& lay, int k, uint64_t seg,
                                      uint64_t u)
{
    return nodes + lay.off[k] + (seg * lay.cnt[k] + u) * (uint64_t)lay.L;
}

// Value of lane j at row `row` of segment `seg` (row-major, L lanes per row),
// or -0.0 past the segment's end.
template <typename T>
__device__ __forceinline__ T ip_load(const T* __restrict__ xs, uint64_t cols, uint32_t L,
                                     uint64_t row, uint64_t j)
{
    const uint64_t gi = row * L + j;
    return (j < L && gi < cols) ? xs[gi] : neg_zero<T>();
}

// Kernel 1: tile totals into node level 0.
template <typename T>
__global__ __launch_bounds__(kIpThreads) void k_ip_totals(const T* __restrict__ x, uint64_t ldx,
                                                          uint64_t cols, uint32_t* __restrict__ err,
                                                          T* __restrict__ nodes, IpLayout lay)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) err[0] = 0u;  // nothing here can time out
    const uint64_t items = lay.nseg * lay.tps;
    const int R = 1 << lay.r_log;
    for (uint64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const uint64_t seg = item / lay.tps, t = item % lay.tps;
        const T* xs = x + seg * ldx;
        for (uint64_t j = threadIdx.x; j < lay.L; j += kIpThreads) {
            TreeStack<T, 1, kIpMaxRLog> st;
            T v[1];
            for (int r = 0; r < R; ++r) {
                v[0] = ip_load(xs, cols, lay.L, t * R + r, j);
                st.push(r, v);
            }
            st.collapse(R, v);
            ip_node(nodes, lay, 0, seg, t)[j] = v[0];
        }
    }
}

// Kernel 2: node levels k0+1 .. k0+kIpLevelsPerPass from level k0.  Item =
// (segment, block of 2^kIpLevelsPerPass level-k0 nodes); only complete nodes
// are written.
template <typename T>
__global__ __launch_bounds__(kIpThreads) void k_ip_nodes(T* __restrict__ nodes, IpLayout lay,
                                                         int k0)
{
    constexpr int NB = 1 << kIpLevelsPerPass;
    const uint64_t cnt0 = lay.cnt[k0];
    const uint64_t blocks = (cnt0 + NB - 1) / NB;
    const uint64_t items = lay.nseg * blocks;
    for (uint64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const uint64_t seg = item / blocks, b = item % blocks;
        for (uint64_t j = threadIdx.x; j < lay.L; j += kIpThreads) {
            T v[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const uint64_t u = b * NB + i;
                v[i] = u < cnt0 ? ip_node(nodes, lay, k0, seg, u)[j] : neg_zero<T>();
            }
#pragma unroll
            for (int l = 1; l <= kIpLevelsPerPass; ++l) {
                const int k = k0 + l;
#pragma unroll
                for (int i = 0; i < (NB >> l); ++i) {
                    v[i] = v[2 * i] + v[2 * i + 1];
                    const uint64_t u = b * (NB >> l) + i;
                    if (k < lay.levels && u < lay.cnt[k]) ip_node(nodes, lay, k, seg, u)[j] = v[i];
                }
            }
        }
    }
}

// Kernel 3: the scan.  LDS holds one tree per row for rows -1 .. R-1 of the
// tile: tree ri (row ri - 1) has Lp leaves at [ri * 2Lp, ri * 2Lp + Lp) and
// level l at offset 2Lp - (2Lp >> l).
template <typename T, bool OUTX>
__global__ __launch_bounds__(kIpThreads) void k_ip_scan(const T* __restrict__ x, uint64_t ldx,
                                                        T* __restrict__ y, uint64_t ldy,
                                                        uint64_t cols, const T* __restrict__ nodes,
                                                        IpLayout lay, T init, int kind)
{
    extern __shared__ unsigned char ip_smem[];
    T* tree = reinterpret_cast<T*>(ip_smem);
    const int R = 1 << lay.r_log;
    const uint64_t Lp = 1ull << lay.lp_log;
    const uint64_t L = lay.L;
    const uint64_t items = lay.nseg * lay.tps;
    auto lvl = [&](int ri, int l) -> T* { return tree + (uint64_t)ri * 2 * Lp + (2 * Lp - ((2 * Lp) >> l)); };

    for (uint64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const uint64_t seg = item / lay.tps, t = item % lay.tps;
        const T* xs = x + seg * ldx;
        T* ys = y + seg * ldy;

        // lane prefixes inside the tile, then the nodes of the earlier tiles
        for (uint64_t j = threadIdx.x; j < Lp; j += kIpThreads) {
            TreeStack<T, 1, kIpMaxRLog> st;
            T v[1];
            for (int r = 0; r < R; ++r) {
                v[0] = ip_load(xs, cols, (uint32_t)L, t * R + r, j);
                st.push(r, v);
                st.collapse(r + 1, v);
                lvl(r + 1, 0)[j] = v[0];
            }
            T b = neg_zero<T>();
            for (int k = 0; k < lay.levels && (t >> k) != 0; ++k) {
                if (!((t >> k) & 1)) continue;
                const T h = j < L ? ip_node(nodes, lay, k, seg, (t >> k) - 1)[j] : neg_zero<T>();
                for (int r = 0; r < R; ++r) lvl(r + 1, 0)[j] = h + lvl(r + 1, 0)[j];
                b = h + b;
            }
            lvl(0, 0)[j] = b;
        }
        __syncthreads();

        // subtree values of every row's tree
        for (int l = 1; l <= lay.lp_log; ++l) {
            const uint64_t width = Lp >> l;
            const uint64_t total = (uint64_t)(R + 1) * width;
            for (uint64_t e = threadIdx.x; e < total; e += kIpThreads) {
                const int ri = (int)(e / width);
                const uint64_t u = e % width;
                lvl(ri, l)[u] = lvl(ri, l - 1)[2 * u] + lvl(ri, l - 1)[2 * u + 1];
            }
            __syncthreads();
        }

        // the walk from each lane to the root
        auto walk = [&](int r, uint64_t i) {
            T val = lvl(r + 1, 0)[i];
            for (int l = 1; l <= lay.lp_log; ++l) {
                const uint64_t pos = i >> (l - 1);
                const uint64_t sib = pos ^ 1;
                if (pos & 1) val = lvl(r + 1, l - 1)[sib] + val;  // left sibling: A values
                else val = val + lvl(r, l - 1)[sib];              // right sibling: B values
            }
            return val;
        };
        const uint64_t elems = (uint64_t)R * L;
        for (uint64_t e = threadIdx.x; e < elems; e += kIpThreads) {
            const int r = (int)(e / L);
            const uint64_t i = e % L;
            const uint64_t gi = (t * R + r) * L + i;
            if (gi >= cols) continue;
            if constexpr (!OUTX) {
                ys[gi] = walk(r, i);
            } else if (kind == kScanInclusive) {
                ys[gi] = init + walk(r, i);
            } else {
                // the value before element (r, i): lane i - 1 of the same
                // row, or at lane 0 the end of the previous row, which is the
                // root of that row's tree (the B tree of row r; -0.0 before
                // the first element)
                ys[gi] = init + (i > 0 ? walk(r, i - 1) : lvl(r, lay.lp_log)[0]);
                if (kind == kScanIncludeInitial && gi + 1 == cols) ys[cols] = init + walk(r, i);
            }
        }
        __syncthreads();  // the trees are rebuilt for the next tile
    }
}

// ============================================================================
// Chunked rows (Lp > kIpWholeRowMaxL).  A row's lane tree is too large for
// LDS, so its lanes are cut into chunks of C = 2^chunk_log; a chunk's lanes
// hold the complete subtrees of level chunk_log.  The walk of lane r climbs
// first inside r's chunk (the chunk's trees in LDS, as k_ip_scan), then
// above it, where every sibling is a whole aligned group of chunks: pure A
// (left) or pure B (right) values of the tree over the row's chunk totals,
// which the workspace holds per row (A: the row's, B: the row above's).
//   3a. chunk totals: per (tile, chunk), the chunk's A values of every row
//       of the tile and their complete tree's root;
//   3b. chunk trees: per row, the levels above the chunk totals;
//   3c. the scan: per (tile, chunk), the chunk's trees again and the walk.
// ============================================================================

// Chunk tree of row `row` of segment `seg` (2 nchunks values).
template <typename T>
__device__ __forceinline__ T* ip_chunk_tree(T* nodes, const IpLayout& lay, uint64_t seg,
                                            uint64_t row)
{
    const uint64_t nc = 1ull << (lay.lp_log - lay.chunk_log);
    return nodes + lay.cl_off + (seg * lay.rows + row) * 2 * nc;
}

// The leaves of the per-row trees of one chunk of one tile, as k_ip_scan
// builds them for a whole row: tree ri (row ri - 1 of the tile; ri = 0 is
// the row above the tile) at lvl(ri, 0)[jj] for the chunk's lanes
// jj = j - c C; lanes past L are -0.0.
template <typename T, class Lvl>
__device__ __forceinline__ void ip_chunk_leaves(const T* __restrict__ xs, uint64_t cols,
                                                const T* __restrict__ nodes, const IpLayout& lay,
                                                uint64_t seg, uint64_t t, uint64_t c, Lvl lvl)
{
    const int R = 1 << lay.r_log;
    const uint64_t C = 1ull << lay.chunk_log;
    const uint64_t L = lay.L;
    for (uint64_t jj = threadIdx.x; jj < C; jj += kIpThreads) {
        const uint64_t j = c * C + jj;
        TreeStack<T, 1, kIpMaxRLog> st;
        T v[1];
        for (int r = 0; r < R; ++r) {
            v[0] = ip_load(xs, cols, (uint32_t)L, t * R + r, j);
            st.push(r, v);
            st.collapse(r + 1, v);
            lvl(r + 1, 0)[jj] = v[0];
        }
        T b = neg_zero<T>();
        for (int k = 0; k < lay.levels && (t >> k) != 0; ++k) {
            if (!((t >> k) & 1)) continue;
            const T h = j < L ? ip_node(nodes, lay, k, seg, (t >> k) - 1)[j] : neg_zero<T>();
            for (int r = 0; r < R; ++r) lvl(r + 1, 0)[jj] = h + lvl(r + 1, 0)[jj];
            b = h + b;
        }
        lvl(0, 0)[jj] = b;
    }
}

// Levels 1 .. chunk_log of trees ri0 .. R of the chunk (complete subtrees,
// lower lanes on the left); ends with a barrier.
template <typename T, class Lvl>
__device__ __forceinline__ void ip_chunk_levels(const IpLayout& lay, int ri0, Lvl lvl)
{
    const int R = 1 << lay.r_log;
    const uint64_t C = 1ull << lay.chunk_log;
    for (int l = 1; l <= lay.chunk_log; ++l) {
        const uint64_t width = C >> l;
        const uint64_t total = (uint64_t)(R + 1 - ri0) * width;
        for (uint64_t e = threadIdx.x; e < total; e += kIpThreads) {
            const int ri = ri0 + (int)(e / width);
            const uint64_t u = e % width;
            lvl(ri, l)[u] = lvl(ri, l - 1)[2 * u] + lvl(ri, l - 1)[2 * u + 1];
        }
        __syncthreads();
    }
}

// Kernel 3a: the chunk totals of every row of every tile (level 0 of the
// rows' chunk trees).
template <typename T>
__global__ __launch_bounds__(kIpThreads) void k_ip_chunk_totals(const T* __restrict__ x,
                                                                uint64_t ldx, uint64_t cols,
                                                                T* __restrict__ nodes,
                                                                IpLayout lay)
{
    extern __shared__ unsigned char ip_smem[];
    T* tree = reinterpret_cast<T*>(ip_smem);
    const int R = 1 << lay.r_log;
    const uint64_t C = 1ull << lay.chunk_log;
    const uint64_t nc = 1ull << (lay.lp_log - lay.chunk_log);
    const uint64_t items = lay.nseg * lay.tps * nc;
    auto lvl = [&](int ri, int l) -> T* { return tree + (uint64_t)ri * 2 * C + (2 * C - ((2 * C) >> l)); };
    for (uint64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const uint64_t seg = item / (lay.tps * nc), rem = item % (lay.tps * nc);
        const uint64_t t = rem / nc, c = rem % nc;
        ip_chunk_leaves<T>(x + seg * ldx, cols, nodes, lay, seg, t, c, lvl);
        __syncthreads();
        ip_chunk_levels<T>(lay, 1, lvl);
        for (int r = (int)threadIdx.x; r < R; r += kIpThreads) {
            const uint64_t row = t * R + r;
            if (row < lay.rows) ip_chunk_tree(nodes, lay, seg, row)[c] = lvl(r + 1, lay.chunk_log)[0];
        }
        __syncthreads();  // the trees are rebuilt for the next item
    }
}

// Kernel 3b: levels 1 .. log2(nchunks) of every row's chunk tree, one
// thread per row.
template <typename T>
__global__ __launch_bounds__(kIpThreads) void k_ip_chunk_rows(T* __restrict__ nodes, IpLayout lay)
{
    const int lc = lay.lp_log - lay.chunk_log;
    const uint64_t nc = 1ull << lc;
    const uint64_t items = lay.nseg * lay.rows;
    for (uint64_t item = (uint64_t)blockIdx.x * kIpThreads + threadIdx.x; item < items;
         item += (uint64_t)gridDim.x * kIpThreads) {
        T* ct = ip_chunk_tree(nodes, lay, item / lay.rows, item % lay.rows);
        for (int l = 1; l <= lc; ++l) {
            T* lo = ct + (2 * nc - ((2 * nc) >> (l - 1)));
            T* hi = ct + (2 * nc - ((2 * nc) >> l));
            for (uint64_t u = 0; u < (nc >> l); ++u) hi[u] = lo[2 * u] + lo[2 * u + 1];
        }
    }
}

// Kernel 3c: the scan of one chunk of one tile at a time.
template <typename T, bool OUTX>
__global__ __launch_bounds__(kIpThreads) void k_ip_scan_chunked(const T* __restrict__ x,
                                                                uint64_t ldx, T* __restrict__ y,
                                                                uint64_t ldy, uint64_t cols,
                                                                T* __restrict__ nodes,
                                                                IpLayout lay, T init, int kind)
{
    extern __shared__ unsigned char ip_smem[];
    T* tree = reinterpret_cast<T*>(ip_smem);
    const int R = 1 << lay.r_log;
    const uint64_t C = 1ull << lay.chunk_log;
    const int lc = lay.lp_log - lay.chunk_log;
    const uint64_t nc = 1ull << lc;
    const uint64_t L = lay.L;
    const uint64_t items = lay.nseg * lay.tps * nc;
    auto lvl = [&](int ri, int l) -> T* { return tree + (uint64_t)ri * 2 * C + (2 * C - ((2 * C) >> l)); };

    for (uint64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const uint64_t seg = item / (lay.tps * nc), rem = item % (lay.tps * nc);
        const uint64_t t = rem / nc, c = rem % nc;
        T* ys = y + seg * ldy;
        ip_chunk_leaves<T>(x + seg * ldx, cols, nodes, lay, seg, t, c, lvl);
        __syncthreads();
        ip_chunk_levels<T>(lay, 0, lvl);

        // above the chunk: level lv of the chunk tree of row `row` (A side)
        // or of the row above (B side; -0.0 above the segment's first row)
        auto above = [&](int r, uint64_t i, T val) {
            const uint64_t row = t * R + r;
            const T* a = ip_chunk_tree(nodes, lay, seg, row);
            const T* b = row > 0 ? ip_chunk_tree(nodes, lay, seg, row - 1) : nullptr;
            for (int l = lay.chunk_log + 1; l <= lay.lp_log; ++l) {
                const int lv = l - 1 - lay.chunk_log;
                const uint64_t pos = i >> (l - 1);
                const uint64_t sib = (pos ^ 1) + (2 * nc - ((2 * nc) >> lv));
                if (pos & 1) val = a[sib] + val;                 // left sibling: A values
                else val = val + (b ? b[sib] : neg_zero<T>());   // right sibling: B values
            }
            return val;
        };
        // the walk from lane i (in chunk c) to the root
        auto walk = [&](int r, uint64_t i) {
            const uint64_t jj = i - c * C;
            T val = lvl(r + 1, 0)[jj];
            for (int l = 1; l <= lay.chunk_log; ++l) {
                const uint64_t pos = jj >> (l - 1);
                const uint64_t sib = pos ^ 1;
                if (pos & 1) val = lvl(r + 1, l - 1)[sib] + val;
                else val = val + lvl(r, l - 1)[sib];
            }
            return above(r, i, val);
        };
        const uint64_t lo = c * C, hi = (c + 1) * C < L ? (c + 1) * C : L;
        const uint64_t elems = (uint64_t)R * (hi > lo ? hi - lo : 0);
        for (uint64_t e = threadIdx.x; e < elems; e += kIpThreads) {
            const int r = (int)(e / (hi - lo));
            const uint64_t i = lo + e % (hi - lo);
            const uint64_t gi = (t * R + r) * L + i;
            if (gi >= cols) continue;
            if constexpr (!OUTX) {
                ys[gi] = walk(r, i);
            } else if (kind == kScanInclusive) {
                ys[gi] = init + walk(r, i);
            } else {
                // the value before element (r, i): lane i - 1 of the same row
                // (at a chunk's first lane, the last lane of the chunk before,
                // whose walk inside its chunk gives that chunk's A total), or
                // at lane 0 the end of the row above, the root of its chunk
                // tree (-0.0 before the segment's first element)
                T before;
                if (i > lo) {
                    before = walk(r, i - 1);
                } else if (i > 0) {
                    before = above(r, i - 1, ip_chunk_tree(nodes, lay, seg, t * R + r)[c - 1]);
                } else {
                    const uint64_t row = t * R + r;
                    before = row > 0 ? ip_chunk_tree(nodes, lay, seg, row - 1)[2 * nc - 2]
                                     : neg_zero<T>();
                }
                ys[gi] = init + before;
                if (kind == kScanIncludeInitial && gi + 1 == cols) ys[cols] = init + walk(r, i);
            }
        }
        __syncthreads();  // the trees are rebuilt for the next item
    }
}

template <typename T>
static hipError_t launch_ip_nodes(T* nodes, const IpLayout& lay, hipStream_t s)
{
    for (int k0 = 0; k0 + 1 < lay.levels; k0 += kIpLevelsPerPass) {
        const uint64_t blocks = (lay.cnt[k0] + (1u << kIpLevelsPerPass) - 1) >> kIpLevelsPerPass;
        const uint64_t nit = lay.nseg * blocks;
        const unsigned g = (unsigned)capped_grid(nit < kIpMaxGrid ? nit : kIpMaxGrid);
        hipLaunchKernelGGL((k_ip_nodes<T>), dim3(g), dim3(kIpThreads), 0, s, nodes, lay, k0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------- launcher
template <typename T, bool OUTX>
static hipError_t launch_ip(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t cols,
                            uint32_t* err, T* nodes, const IpLayout& lay, const ScanOut<T>& out,
                            hipStream_t s)
{
    if (lay.fast_logrv >= 0) return hipErrorInvalidValue;  // the single pass serves it
    const uint64_t items = lay.nseg * lay.tps;
    const unsigned grid = (unsigned)capped_grid(items < kIpMaxGrid ? items : kIpMaxGrid);
    hipLaunchKernelGGL((k_ip_totals<T>), dim3(grid), dim3(kIpThreads), 0, s, x, ldx, cols, err,
                       nodes, lay);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_ip_nodes<T>(nodes, lay, s);
    if (e != hipSuccess) return e;
    const size_t lds = ip_lds_bytes(lay, sizeof(T));
    if (lay.chunk_log < lay.lp_log) {
        const uint64_t citems = items << (lay.lp_log - lay.chunk_log);
        const unsigned cgrid = (unsigned)capped_grid(citems < kIpMaxGrid ? citems : kIpMaxGrid);
        hipLaunchKernelGGL((k_ip_chunk_totals<T>), dim3(cgrid), dim3(kIpThreads), lds, s, x, ldx,
                           cols, nodes, lay);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const uint64_t rows = lay.nseg * lay.rows;
        uint64_t rgrid = (rows + kIpThreads - 1) / kIpThreads;
        if (rgrid > 4096) rgrid = 4096;
        hipLaunchKernelGGL((k_ip_chunk_rows<T>), dim3((unsigned)capped_grid(rgrid)),
                           dim3(kIpThreads), 0, s, nodes, lay);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((k_ip_scan_chunked<T, OUTX>), dim3(cgrid), dim3(kIpThreads), lds, s, x,
                           ldx, y, ldy, cols, nodes, lay, out.init, out.kind);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_ip_scan<T, OUTX>), dim3(grid), dim3(kIpThreads), lds, s, x, ldx, y, ldy,
                       cols, nodes, lay, out.init, out.kind);
    return hipGetLastError();
}

template <typename T, bool PLAIN>
hipError_t launch_scan_ip(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t nseg,
                          uint64_t cols, uint32_t* err, T* nodes, const IpLayout& lay,
                          const ScanOut<T>* out, hipStream_t s)
{
    if (nseg == 0) return hipSuccess;
    if (cols == 0) {
        if (out && out->kind == kScanIncludeInitial)
            return launch_put_column(y, ldy, nseg, out->init, s);
        return hipSuccess;
    }
    if (out) return launch_ip<T, true>(x, ldx, y, ldy, cols, err, nodes, lay, *out, s);
    if constexpr (PLAIN)
        return launch_ip<T, false>(x, ldx, y, ldy, cols, err, nodes, lay, ScanOut<T>{}, s);
    return hipErrorInvalidValue;
}

}  // namespace canon
