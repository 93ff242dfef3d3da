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
// Three kernels, no waiting between workgroups:
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
#include "device.hpp"
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

template <typename T>
static hipError_t launch_ip_nodes(T* nodes, const IpLayout& lay, hipStream_t s)
{
    for (int k0 = 0; k0 + 1 < lay.levels; k0 += kIpLevelsPerPass) {
        const uint64_t blocks = (lay.cnt[k0] + (1u << kIpLevelsPerPass) - 1) >> kIpLevelsPerPass;
        const uint64_t nit = lay.nseg * blocks;
        const unsigned g = (unsigned)(nit < kIpMaxGrid ? nit : kIpMaxGrid);
        hipLaunchKernelGGL((k_ip_nodes<T>), dim3(g), dim3(kIpThreads), 0, s, nodes, lay, k0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ============================================================================
// Fast path: L = 64 * E * RV with RV = 2^LOGRV in {1, ..., 8} (a row is RV
// wave-wide 16-byte loads), 16-byte aligned rows.  A tile is 64 / RV rows;
// each thread holds 16 vectors: wave w owns rows w*RW .. w*RW + RW-1
// (RW = 16 / RV), vector u = row-in-wave u / RV, row-vector q = u % RV, lanes
// (q * 64 + lane) * E + e.  The lane tree of a row has three kinds of levels:
// inside a vector (static), across the 64 lanes (xor butterfly), across the
// RV vectors of the row (in the thread).
// ============================================================================
template <typename T, int LOGRV>
struct IpFast {
    static constexpr int E = Elem<T>::E;
    static constexpr int LOGE = Elem<T>::LOGE;
    static constexpr int RV = 1 << LOGRV;
    static constexpr int NV = 16;
    static constexpr int RW = NV / RV;
    static constexpr int LOGRW = 4 - LOGRV;
    static constexpr int R = 4 * RW;  // rows per tile
    static constexpr int L = 64 * E * RV;
};

// butterfly partner value of `v` held by lane ^ 2^K
template <int K, typename T>
__device__ __forceinline__ T xor_lane(T v)
{
    return shfl_xor<(1 << K)>(v);
}

template <typename T, int LOGRV, bool GUARD>
__device__ __forceinline__ void ipf_load(const T* __restrict__ xs, uint64_t cols, uint64_t row0,
                                         int w, int lane, T (&a)[16][Elem<T>::E])
{
    using F = IpFast<T, LOGRV>;
#pragma unroll
    for (int u = 0; u < F::NV; ++u) {
        const uint64_t row = row0 + (uint64_t)w * F::RW + u / F::RV;
        const uint64_t gi = row * F::L + (uint64_t)((u % F::RV) * 64 + lane) * F::E;
        if (!GUARD || gi + F::E <= cols) {
            load_vec(xs + gi, a[u]);
        } else {
#pragma unroll
            for (int e = 0; e < F::E; ++e) a[u][e] = gi + e < cols ? xs[gi + e] : neg_zero<T>();
        }
    }
}

// In-wave pairwise prefix down each lane over the wave's RW rows (Sklansky
// over rows; the upper half receives the end of the lower half).
template <typename T, int LOGRV>
__device__ __forceinline__ void ipf_columns_in_wave(T (&a)[16][Elem<T>::E])
{
    using F = IpFast<T, LOGRV>;
#pragma unroll
    for (int h = 1; h < F::RW; h *= 2)
#pragma unroll
        for (int r = 0; r < F::RW; ++r)
            if (r & h)
#pragma unroll
                for (int q = 0; q < F::RV; ++q)
#pragma unroll
                    for (int e = 0; e < F::E; ++e)
                        a[r * F::RV + q][e] = a[((r & ~(2 * h - 1)) + h - 1) * F::RV + q][e] +
                                              a[r * F::RV + q][e];
}

// The sibling values one row contributes to the walks of the lanes of a
// row (its own, as the A side, or the next one, as the B side), per 16-byte
// vector q of the row held by this thread:
//   sv[l][q][s]: the complete subtree of 2^l slots starting at slot s 2^l
//                (inside the vector, l < log2 E);
//   o[K][q]:     the partner lane's subtree at lane level K (lane ^ 2^K);
//   pv[l][q]:    this thread's subtree of vector q at vector level l.
template <typename T, int LOGRV>
struct IpRowTree {
    static constexpr int E = Elem<T>::E, LOGE = Elem<T>::LOGE, RV = 1 << LOGRV;
    T sv[LOGE][RV][E];
    T o[6][RV];
    T pv[LOGRV > 0 ? LOGRV : 1][RV];
    T root;  // the complete tree over the whole row (the same in every lane)

    // row = vectors rows[v0 .. v0 + RV)
    template <int NV>
    __device__ __forceinline__ void build(const T (&rows)[NV][E], int v0, int lane)
    {
        T p[RV];
#pragma unroll
        for (int q = 0; q < RV; ++q) {
            T cur[E];
#pragma unroll
            for (int e = 0; e < E; ++e) cur[e] = rows[v0 + q][e];
#pragma unroll
            for (int l = 0; l < LOGE; ++l) {
#pragma unroll
                for (int s2 = 0; s2 < (E >> l); ++s2) sv[l][q][s2] = cur[s2];
#pragma unroll
                for (int s2 = 0; s2 < (E >> (l + 1)); ++s2) cur[s2] = cur[2 * s2] + cur[2 * s2 + 1];
            }
            p[q] = cur[0];
        }
#define CANON_IP_TREE_LANE(K)                                                           \
    {                                                                                   \
        const bool right = (lane >> (K)) & 1;                                           \
        _Pragma("unroll") for (int q = 0; q < RV; ++q)                                  \
        {                                                                               \
            o[K][q] = xor_lane<K>(p[q]);                                                \
            p[q] = right ? (o[K][q] + p[q]) : (p[q] + o[K][q]);                         \
        }                                                                               \
    }
        CANON_IP_TREE_LANE(0)
        CANON_IP_TREE_LANE(1)
        CANON_IP_TREE_LANE(2)
        CANON_IP_TREE_LANE(3)
        CANON_IP_TREE_LANE(4)
        CANON_IP_TREE_LANE(5)
#undef CANON_IP_TREE_LANE
#pragma unroll
        for (int l = 0; l < LOGRV; ++l) {
            const int h = 1 << l;
#pragma unroll
            for (int q = 0; q < RV; ++q) pv[l][q] = p[q];
#pragma unroll
            for (int i = 0; i < RV / (2 * h); ++i) p[2 * i * h] = p[2 * i * h] + p[(2 * i + 1) * h];
        }
        root = p[0];
    }
};

// val[q][e]: the walk of every lane of row vectors rows[v0 .. v0 + RV) from
// its leaf to the root: at each level the sibling subtree lies wholly left
// (A row, added on the left) or wholly right (B row, added on the right).
template <typename T, int LOGRV, int NV>
__device__ __forceinline__ void ip_walk(const T (&rows)[NV][Elem<T>::E], int v0,
                                        const IpRowTree<T, LOGRV>& A,
                                        const IpRowTree<T, LOGRV>& B, int lane,
                                        T (&val)[1 << LOGRV][Elem<T>::E])
{
    constexpr int E = Elem<T>::E, LOGE = Elem<T>::LOGE, RV = 1 << LOGRV;
#pragma unroll
    for (int q = 0; q < RV; ++q)
#pragma unroll
        for (int e = 0; e < E; ++e) val[q][e] = rows[v0 + q][e];
#pragma unroll
    for (int l = 0; l < LOGE; ++l)
#pragma unroll
        for (int q = 0; q < RV; ++q)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int node = e >> l, sib = node ^ 1;
                val[q][e] = (node & 1) ? A.sv[l][q][sib] + val[q][e] : val[q][e] + B.sv[l][q][sib];
            }
#pragma unroll
    for (int K = 0; K < 6; ++K) {
        const bool right = (lane >> K) & 1;
#pragma unroll
        for (int q = 0; q < RV; ++q)
#pragma unroll
            for (int e = 0; e < E; ++e)
                val[q][e] = right ? (A.o[K][q] + val[q][e]) : (val[q][e] + B.o[K][q]);
    }
#pragma unroll
    for (int l = 0; l < LOGRV; ++l) {
        const int h = 1 << l;
#pragma unroll
        for (int q = 0; q < RV; ++q) {
            const int node = q >> l, sib = node ^ 1;
#pragma unroll
            for (int e = 0; e < E; ++e)
                val[q][e] = (node & 1) ? A.pv[l][sib * h] + val[q][e] : val[q][e] + B.pv[l][sib * h];
        }
    }
}

// Kernel 1 (fast): tile totals, lane by lane, into node level 0.
template <typename T, int LOGRV>
__global__ __launch_bounds__(kIpThreads) void k_ip_totals_fast(const T* __restrict__ x,
                                                               uint64_t ldx, uint64_t cols,
                                                               uint32_t* __restrict__ err,
                                                               T* __restrict__ nodes, IpLayout lay)
{
    using F = IpFast<T, LOGRV>;
    __shared__ T s_tot[4][F::L];
    if (blockIdx.x == 0 && threadIdx.x == 0) err[0] = 0u;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t items = lay.nseg * lay.tps;
    for (uint64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const uint64_t seg = item / lay.tps, t = item % lay.tps;
        const T* xs = x + seg * ldx;
        T a[F::NV][F::E];
        const uint64_t row0 = t * F::R;
        if ((row0 + F::R) * F::L <= cols) ipf_load<T, LOGRV, false>(xs, cols, row0, w, lane, a);
        else ipf_load<T, LOGRV, true>(xs, cols, row0, w, lane, a);
        // complete tree over the wave's rows, per lane
#pragma unroll
        for (int h = 1; h < F::RW; h *= 2)
#pragma unroll
            for (int r = 0; r < F::RW; r += 2 * h)
#pragma unroll
                for (int q = 0; q < F::RV; ++q)
#pragma unroll
                    for (int e = 0; e < F::E; ++e)
                        a[r * F::RV + q][e] = a[r * F::RV + q][e] + a[(r + h) * F::RV + q][e];
#pragma unroll
        for (int q = 0; q < F::RV; ++q)
#pragma unroll
            for (int e = 0; e < F::E; ++e) s_tot[w][(q * 64 + lane) * F::E + e] = a[q][e];
        __syncthreads();
        T* dst = ip_node(nodes, lay, 0, seg, t);
        for (int j = threadIdx.x; j < F::L; j += kIpThreads)
            dst[j] = (s_tot[0][j] + s_tot[1][j]) + (s_tot[2][j] + s_tot[3][j]);
        __syncthreads();
    }
}

// Kernel 3 (fast): the scan.
template <typename T, int LOGRV, bool OUTX>
__global__ __launch_bounds__(kIpThreads) void k_ip_scan_fast(const T* __restrict__ x, uint64_t ldx,
                                                             T* __restrict__ y, uint64_t ldy,
                                                             uint64_t cols,
                                                             const T* __restrict__ nodes,
                                                             IpLayout lay, T init, int kind)
{
    using F = IpFast<T, LOGRV>;
    constexpr int E = F::E, RV = F::RV, RW = F::RW;
    __shared__ T s_row[4][F::L];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t items = lay.nseg * lay.tps;

    for (uint64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const uint64_t seg = item / lay.tps, t = item % lay.tps;
        const T* xs = x + seg * ldx;
        T* ys = y + seg * ldy;
        const uint64_t row0 = t * F::R;
        const bool full = (row0 + F::R) * F::L <= cols;
        T a[F::NV][E];
        if (full) ipf_load<T, LOGRV, false>(xs, cols, row0, w, lane, a);
        else ipf_load<T, LOGRV, true>(xs, cols, row0, w, lane, a);

        // lane prefixes: inside the wave, across the 4 waves, then the nodes
        // of the earlier tiles (right-nested, lowest level first)
        ipf_columns_in_wave<T, LOGRV>(a);
#pragma unroll
        for (int q = 0; q < RV; ++q)
#pragma unroll
            for (int e = 0; e < E; ++e)
                s_row[w][(q * 64 + lane) * E + e] = a[(RW - 1) * RV + q][e];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < RV; ++q)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int j = (q * 64 + lane) * E + e;
                const T t0 = s_row[0][j], t1 = s_row[1][j], t2 = s_row[2][j];
                if (w & 1) {
                    const T s = (w & 2) ? t2 : t0;
#pragma unroll
                    for (int r = 0; r < RW; ++r) a[r * RV + q][e] = s + a[r * RV + q][e];
                }
                if (w & 2) {
                    const T s = t0 + t1;
#pragma unroll
                    for (int r = 0; r < RW; ++r) a[r * RV + q][e] = s + a[r * RV + q][e];
                }
            }
        T b[RV][E];
#pragma unroll
        for (int q = 0; q < RV; ++q)
#pragma unroll
            for (int e = 0; e < E; ++e) b[q][e] = neg_zero<T>();
        for (int k = 0; k < lay.levels && (t >> k) != 0; ++k) {
            if (!((t >> k) & 1)) continue;
            const T* h = ip_node(nodes, lay, k, seg, (t >> k) - 1);
#pragma unroll
            for (int q = 0; q < RV; ++q) {
                T hv[E];
                load_vec(h + (q * 64 + lane) * E, hv);
#pragma unroll
                for (int e = 0; e < E; ++e) {
#pragma unroll
                    for (int r = 0; r < RW; ++r) a[r * RV + q][e] = hv[e] + a[r * RV + q][e];
                    b[q][e] = hv[e] + b[q][e];
                }
            }
        }
        // the B row of each wave's first row: the A row just above it
        __syncthreads();  // s_row is reused
#pragma unroll
        for (int q = 0; q < RV; ++q)
#pragma unroll
            for (int e = 0; e < E; ++e)
                s_row[w][(q * 64 + lane) * E + e] = a[(RW - 1) * RV + q][e];
        __syncthreads();
        if (w > 0) {
#pragma unroll
            for (int q = 0; q < RV; ++q)
#pragma unroll
                for (int e = 0; e < E; ++e) b[q][e] = s_row[w - 1][(q * 64 + lane) * E + e];
        }

        // walk every lane up its row's tree.  For row r: A = a[row r],
        // B = a[row r-1] (b for the wave's first row).  The sibling subtree
        // values a walk needs depend only on the row, so each row's are
        // built once (IpRowTree) and serve as its A side and as the next
        // row's B side.
        IpRowTree<T, LOGRV> tb;
        tb.template build<RV>(b, 0, lane);
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            IpRowTree<T, LOGRV> ta;
            ta.template build<F::NV>(a, r * RV, lane);
            T val[RV][E];
            ip_walk<T, LOGRV>(a, r * RV, ta, tb, lane, val);
            // store row r
            const uint64_t row = row0 + (uint64_t)w * RW + r;
            if constexpr (OUTX) {
                if (kind != kScanInclusive) {
                    // one position up: the value before lane slot 0 of a
                    // vector comes from lane - 1, from lane 63 of the
                    // previous vector, or, at the row's start, from the end
                    // of the previous row (the root of the B tree; -0.0
                    // before the first element)
                    if (kind == kScanIncludeInitial) {
#pragma unroll
                        for (int q = 0; q < RV; ++q)
#pragma unroll
                            for (int e = 0; e < E; ++e)
                                if (row * F::L + (uint64_t)(q * 64 + lane) * E + e + 1 == cols)
                                    ys[cols] = init + val[q][e];
                    }
                    T prev = tb.root;
#pragma unroll
                    for (int q = 0; q < RV; ++q) {
                        const T up = shfl_up1(val[q][E - 1]);
                        const T before = lane == 0 ? prev : up;
                        prev = readlane(val[q][E - 1], 63);
#pragma unroll
                        for (int e = E - 1; e > 0; --e) val[q][e] = val[q][e - 1];
                        val[q][0] = before;
                    }
                }
#pragma unroll
                for (int q = 0; q < RV; ++q)
#pragma unroll
                    for (int e = 0; e < E; ++e) val[q][e] = init + val[q][e];
            }
#pragma unroll
            for (int q = 0; q < RV; ++q) {
                const uint64_t gi = row * F::L + (uint64_t)(q * 64 + lane) * E;
                if (full || gi + E <= cols) {
                    store_vec(ys + gi, val[q]);
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        if (gi + e < cols) ys[gi + e] = val[q][e];
                }
            }
            tb = ta;
        }
        __syncthreads();  // s_row is rewritten by the next tile
    }
}

// ---------------------------------------------------------------- launcher
template <typename T, int LOGRV, bool OUTX>
static hipError_t launch_ip_fast(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t cols,
                                 uint32_t* err, T* nodes, const IpLayout& lay,
                                 const ScanOut<T>& out, hipStream_t s)
{
    const uint64_t items = lay.nseg * lay.tps;
    const unsigned grid = (unsigned)(items < kIpMaxGrid ? items : kIpMaxGrid);
    hipLaunchKernelGGL((k_ip_totals_fast<T, LOGRV>), dim3(grid), dim3(kIpThreads), 0, s, x, ldx,
                       cols, err, nodes, lay);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_ip_nodes<T>(nodes, lay, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_ip_scan_fast<T, LOGRV, OUTX>), dim3(grid), dim3(kIpThreads), 0, s, x,
                       ldx, y, ldy, cols, nodes, lay, out.init, out.kind);
    return hipGetLastError();
}

template <typename T, bool OUTX>
static hipError_t launch_ip(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t cols,
                            uint32_t* err, T* nodes, const IpLayout& lay, const ScanOut<T>& out,
                            hipStream_t s)
{
    if (lay.fast_logrv >= 0) {
        switch (lay.fast_logrv) {
            case 0: return launch_ip_fast<T, 0, OUTX>(x, ldx, y, ldy, cols, err, nodes, lay, out, s);
            case 1: return launch_ip_fast<T, 1, OUTX>(x, ldx, y, ldy, cols, err, nodes, lay, out, s);
            case 2: return launch_ip_fast<T, 2, OUTX>(x, ldx, y, ldy, cols, err, nodes, lay, out, s);
            default:
                return launch_ip_fast<T, 3, OUTX>(x, ldx, y, ldy, cols, err, nodes, lay, out, s);
        }
    }
    const uint64_t items = lay.nseg * lay.tps;
    const unsigned grid = (unsigned)(items < kIpMaxGrid ? items : kIpMaxGrid);
    hipLaunchKernelGGL((k_ip_totals<T>), dim3(grid), dim3(kIpThreads), 0, s, x, ldx, cols, err,
                       nodes, lay);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_ip_nodes<T>(nodes, lay, s);
    if (e != hipSuccess) return e;
    const size_t lds = ip_lds_bytes(lay, sizeof(T));
    hipLaunchKernelGGL((k_ip_scan<T, OUTX>), dim3(grid), dim3(kIpThreads), lds, s, x, ldx, y, ldy,
                       cols, nodes, lay, out.init, out.kind);
    return hipGetLastError();
}

template <typename T>
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
    return launch_ip<T, false>(x, ldx, y, ldy, cols, err, nodes, lay, ScanOut<T>{}, s);
}

template hipError_t launch_scan_ip<double>(const double*, uint64_t, double*, uint64_t, uint64_t,
                                           uint64_t, uint32_t*, double*, const IpLayout&,
                                           const ScanOut<double>*, hipStream_t);
template hipError_t launch_scan_ip<float>(const float*, uint64_t, float*, uint64_t, uint64_t,
                                          uint64_t, uint32_t*, float*, const IpLayout&,
                                          const ScanOut<float>*, hipStream_t);

}  // namespace canon
