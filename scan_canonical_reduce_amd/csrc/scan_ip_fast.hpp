// Register geometry and lane trees of the iterated_pairwise scan's
// single-pass kernel.
#pragma once

#include "device.hpp"
#include "scan_ip.hpp"

namespace canon {

// ============================================================================
// Register geometry: L = E * 2^(6 + LOGRV) lanes, LOGRV in {-6, ..., 3},
// 16-byte aligned rows; each thread holds 16 vectors of 16 bytes.
//   LOGRV >= 0 (wide rows): a row is RV = 2^LOGRV wave-wide vectors; wave w
//     owns rows w*RW .. w*RW + RW-1 (RW = 16 / RV), vector u = row-in-wave
//     u / RV, row-vector q = u % RV, lanes (q * 64 + lane) * E + e.
//   LOGRV < 0 (narrow rows): a row is the vectors of TPR = 2^(6 + LOGRV)
//     consecutive lanes; the wave's lanes form G = 64 / TPR groups, group g
//     (lanes g*TPR ..) owning 16 consecutive rows, so a wave holds 16 G rows
//     and vector u of a thread is row (w*G + g)*16 + u, lanes
//     (lane % TPR) * E + e.
// A tile is 4 waves' rows (64 G / RV rows, 4096 E elements).  The lane tree
// of a row has three kinds of levels: inside a vector (static), across the
// TPR lanes of the row (xor butterfly), across the RV vectors of the row
// (in the thread).
// ============================================================================
template <typename T, int LOGRV>
struct IpFast {
    static_assert(LOGRV >= -6 && LOGRV <= 3, "register geometry");
    static constexpr int E = Elem<T>::E;
    static constexpr int LOGE = Elem<T>::LOGE;
    static constexpr int LOGT = LOGRV >= 0 ? 6 : 6 + LOGRV;  // lanes of a row vector
    static constexpr int TPR = 1 << LOGT;
    static constexpr int G = 64 / TPR;                        // row groups per wave
    static constexpr int LOGV = LOGRV >= 0 ? LOGRV : 0;       // vectors per row
    static constexpr int RV = 1 << LOGV;
    static constexpr int NV = 16;
    static constexpr int RW = NV / RV;  // rows per thread
    static constexpr int LOGRW = 4 - LOGV;
    static constexpr int R = 4 * G * RW;  // rows per tile
    static constexpr int L = TPR * E * RV;

    // (constants for wide rows: one group, the column is the lane)
    __device__ static int group(int lane) { return G == 1 ? 0 : lane >> LOGT; }
    __device__ static int sub(int lane) { return TPR == 64 ? lane : lane & (TPR - 1); }
    // first lane of the row held by vector q of a row of this thread, and
    // the tile row of this thread's row-in-thread r (64-bit, so that the
    // addresses of a thread's vectors stay one base and constant offsets)
    __device__ static uint64_t col(int q, int lane) { return ((uint64_t)q * TPR + sub(lane)) * E; }
    __device__ static uint64_t row(int w, int lane, int r)
    {
        return ((uint64_t)w * G + group(lane)) * RW + r;
    }
    // Index inside a published node (L words, one a column) of the word of
    // value 2j of vector q of this thread's row; value 2j+1's word follows
    // it.  Pair-major, so that one 16-byte store or load per pair covers
    // whole lines across the lanes; with two values a vector it is col.
    static constexpr int NP = E / 2;  // pairs a vector
    __device__ static uint64_t wcol(int q, int j, int lane)
    {
        return (((uint64_t)q * NP + j) * TPR + sub(lane)) * 2;
    }
};

// butterfly partner value of `v` held by lane ^ 2^K (VALU lane moves: the
// row trees are a chain of log2 TPR dependent exchanges per row)
template <int K, typename T>
__device__ __forceinline__ T xor_lane(T v)
{
    return shfl_xor_valu<(1 << K)>(v);
}

template <typename T, int LOGRV, bool GUARD>
__device__ __forceinline__ void ipf_load(const T* __restrict__ xs, uint64_t cols, uint64_t row0,
                                         int w, int lane, T (&a)[16][Elem<T>::E])
{
    using F = IpFast<T, LOGRV>;
#pragma unroll
    for (int u = 0; u < F::NV; ++u) {
        const uint64_t row = row0 + F::row(w, lane, u / F::RV);
        const uint64_t gi = row * F::L + F::col(u % F::RV, lane);
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

// Narrow rows: the pairwise prefix down each lane continued across the
// wave's G row groups (Sklansky over groups, lower blocks first as inside
// the thread): a group in the upper half of an aligned block of 2h groups
// receives, on the left of every row, the end of the lower half, held by
// the same column of group (g & ~(2h-1)) + h - 1.
template <typename T, int LOGRV>
__device__ __forceinline__ void ipf_groups_in_wave(T (&a)[16][Elem<T>::E], int lane)
{
    using F = IpFast<T, LOGRV>;
    static_assert(F::RV == 1, "narrow rows only");
    const int g = F::group(lane);
#pragma unroll
    for (int h = 1; h < F::G; h *= 2) {
        const int src = (((g & ~(2 * h - 1)) + h - 1) << F::LOGT) | F::sub(lane);
        T v[F::E];
#pragma unroll
        for (int e = 0; e < F::E; ++e) v[e] = shfl_idx(a[F::RW - 1][e], src);
        if (g & h) {
#pragma unroll
            for (int r = 0; r < F::RW; ++r)
#pragma unroll
                for (int e = 0; e < F::E; ++e) a[r][e] = v[e] + a[r][e];
        }
    }
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
    using F = IpFast<T, LOGRV>;
    static constexpr int E = F::E, LOGE = F::LOGE, RV = F::RV, LOGT = F::LOGT, LOGV = F::LOGV;
    T sv[LOGE][RV][E];
    T o[LOGT > 0 ? LOGT : 1][RV];
    T pv[LOGV > 0 ? LOGV : 1][RV];
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
    if constexpr ((K) < LOGT) {                                                         \
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
        for (int l = 0; l < LOGV; ++l) {
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
                                        T (&val)[IpFast<T, LOGRV>::RV][Elem<T>::E])
{
    using F = IpFast<T, LOGRV>;
    constexpr int E = F::E, LOGE = F::LOGE, RV = F::RV, LOGT = F::LOGT, LOGV = F::LOGV;
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
    for (int K = 0; K < LOGT; ++K) {
        const bool right = (lane >> K) & 1;
#pragma unroll
        for (int q = 0; q < RV; ++q)
#pragma unroll
            for (int e = 0; e < E; ++e)
                val[q][e] = right ? (A.o[K][q] + val[q][e]) : (val[q][e] + B.o[K][q]);
    }
#pragma unroll
    for (int l = 0; l < LOGV; ++l) {
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

}  // namespace canon
