// One tile of the canonical inclusive scan, policies pairwise and
// block_dyadic<B> (gfx950): the in-tile part shared by the single-pass and the
// row-batched scan kernels.
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
// across a thread's V vectors (readlane), across the 4 waves (LDS) and across
// tiles (by the kernels) are the same network.
//
#pragma once

#include "device.hpp"
#include "scan.hpp"

namespace canon {

// Scan state of one tile.  MODE 0: pairwise.  MODE 1: block_dyadic with
// B >= E (a 16-byte vector never straddles two blocks), carries kept per
// vector.  MODE 2: block_dyadic with B = 2 < E (float: two blocks per
// vector).  MODE 3: block_dyadic with B >= E, levels <= b only: the levels
// above b are left to the kernel, which runs them on the block totals.
//
// Levels <= b build the in-block prefix W in v.  From level b+1 on ("fork"),
// the elements of a block share one carry c, the nodes received at levels
// above b combined right-nested, and output c + W; only the block's last
// element keeps adding what it receives to its own value, which thereby
// becomes the pairwise value of the prefix ending there, its output.  Above
// b the end of a lower half is always a block end, so the value a receiving
// half takes is always the last element's value.
template <typename T, int MODE, int LOGV_>
struct ScanTile {
    static constexpr int E = Elem<T>::E;
    static constexpr int LOGE = Elem<T>::LOGE;
    static constexpr int LOGV = LOGV_;
    static constexpr int V = 1 << LOGV;
    static constexpr int LOG_WSPAN = LOGE + 6 + LOGV;  // elements per wave (log2)
    static constexpr int LOG_S = LOG_WSPAN + 2;        // elements per tile (log2)
    static constexpr bool BD = MODE == 1 || MODE == 2;  // carries per vector
    static constexpr int NB = MODE == 2 ? E / 2 : 1;   // blocks per vector
    static_assert(MODE != 2 || E == 4, "two-element blocks inside a vector: float only");
    static_assert(V <= 32, "block-end mask holds one bit per vector");

    T v[V][E];
    T c[V][NB];
    uint32_t endm;  // MODE 1: bit u set when slot E-1 of vector u ends a block
    int b;          // log2 B
    bool forked;    // a level above b has been applied

    // g0: sequence index of the thread's first element in the tile
    __device__ __forceinline__ void begin(int b_log, uint64_t g0)
    {
        b = MODE == 2 ? 1 : b_log;
        forked = false;
        endm = 0;
        if constexpr (MODE == 1) {
            const uint64_t bmask = (1ull << b) - 1;
#pragma unroll
            for (int u = 0; u < V; ++u)
                if (((g0 + (uint64_t)u * 64 * E + E) & bmask) == 0) endm |= 1u << u;
        }
    }

    // level lam merges two halves of one block (lam <= b); b is uniform, so
    // every such test is a scalar branch
    __device__ __forceinline__ bool in_block(int lam) const { return lam <= b; }

    // value at the end of vector u's last slot: the source a receiving half
    // takes from the end of the lower half
    __device__ __forceinline__ T last(int u) const { return v[u][E - 1]; }

    __device__ __forceinline__ void fork()
    {
        if constexpr (BD) {
#pragma unroll
            for (int u = 0; u < V; ++u)
#pragma unroll
                for (int k = 0; k < NB; ++k) c[u][k] = neg_zero<T>();
            forked = true;
        }
    }
    __device__ __forceinline__ void maybe_fork(int lam)
    {
        if constexpr (BD)
            if (!forked && !in_block(lam)) fork();
    }

    // Every block of vector u receives s at level lam (lam > LOGE).
    __device__ __forceinline__ void apply_vec(int lam, T s, int u)
    {
        if constexpr (MODE == 3)
            if (!in_block(lam)) return;
        if (!BD || in_block(lam)) {
#pragma unroll
            for (int e = 0; e < E; ++e) v[u][e] = s + v[u][e];
        } else if constexpr (MODE == 1) {
            c[u][0] = s + c[u][0];
            const T t = s + v[u][E - 1];
            v[u][E - 1] = ((endm >> u) & 1) ? t : v[u][E - 1];
        } else {
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                c[u][k] = s + c[u][k];
                v[u][2 * k + 1] = s + v[u][2 * k + 1];
            }
        }
    }
    __device__ __forceinline__ void apply_all(int lam, T s)
    {
        maybe_fork(lam);
#pragma unroll
        for (int u = 0; u < V; ++u) apply_vec(lam, s, u);
    }

    // Makes the compiler finish a level's additions before the next level:
    // otherwise it defers those whose results feed no later level to the
    // end, holding every received value in registers until then.
    __device__ __forceinline__ void pin()
    {
#pragma unroll
        for (int u = 0; u < V; ++u) {
#pragma unroll
            for (int e = 0; e < E; ++e) pin_reg(v[u][e]);
            if constexpr (BD) {
#pragma unroll
                for (int k = 0; k < NB; ++k) pin_reg(c[u][k]);
            }
        }
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
                // b = 1: the second block of the vector receives the end of
                // the first
#pragma unroll
                for (int u = 0; u < V; ++u) {
                    c[u][1] = v[u][1] + c[u][1];
                    v[u][3] = v[u][1] + v[u][3];
                }
            } else if (!BD || in_block(2)) {
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
        if constexpr (MODE == 3)
            if (!in_block(lam)) return;
        maybe_fork(lam);
        const bool upper = (lane >> K) & 1;
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const T src = from_lower_half_end<H>(last(u));
            apply_vec(lam, upper ? src : neg_zero<T>(), u);
        }
        pin();
    }

    template <int K>
    __device__ __forceinline__ void vector_level()
    {
        constexpr int H = 1 << K;
        const int lam = LOGE + 7 + K;
        if constexpr (MODE == 3)
            if (!in_block(lam)) return;
        maybe_fork(lam);
        T src[V];
#pragma unroll
        for (int u = 0; u < V; ++u)
            if (u & H) src[u] = readlane(last((u & ~(2 * H - 1)) + H - 1), 63);
#pragma unroll
        for (int u = 0; u < V; ++u)
            if (u & H) apply_vec(lam, src[u], u);
        pin();
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

    // Writes vector u's outputs o[0..E) at sequence index g0 + u*64*E.
    template <bool ALIGNED>
    __device__ __forceinline__ void put(T* __restrict__ y, uint64_t n, uint64_t g0, int u,
                                        const T (&o)[E]) const
    {
        const uint64_t gi = g0 + (uint64_t)u * 64 * E;
        if (ALIGNED && gi + E <= n) {
            store_vec(y + gi, o);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (gi + e < n) y[gi + e] = o[e];
        }
    }

    // Final inclusive values o[0..E) of vector u (block_dyadic: C + W off
    // the block ends).
    __device__ __forceinline__ void final_vec(int u, T (&o)[E]) const
    {
        if (!BD || !forked) {
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = v[u][e];
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                constexpr int BS = E / NB;  // slots per block inside a vector
                const int k = e / BS;
                const bool end = (MODE == 2) ? ((e % BS) == BS - 1)
                                             : (e == E - 1 && ((endm >> u) & 1));
                o[e] = end ? v[u][e] : c[u][k] + v[u][e];
            }
        }
    }

    template <bool ALIGNED>
    __device__ __forceinline__ void store(T* __restrict__ y, uint64_t n, uint64_t g0) const
    {
#pragma unroll
        for (int u = 0; u < V; ++u) {
            T o[E];
            final_vec(u, o);
            put<ALIGNED>(y, n, g0, u, o);
        }
    }

    // Output stage of a scan with an initial value.  fin(u, o) gives the
    // final inclusive values S of vector u (sequence indices g0 + u*64*E +
    // e).  kind 0 writes y[i] = init + S_i.  Kinds 1 and 2 write y[i] = init
    // + S_{i-1}: the value before a thread's first element comes from lane
    // l - 1, from lane 63 of the previous vector, from the previous wave's
    // last element (exchanged in s_wend) or, for the tile's first element,
    // `pre`, the value of the element before the tile (-0.0, the empty
    // prefix, before the sequence's first element, so that y[0] = init +
    // -0.0 = init).  Every write stays inside the tile's own positions
    // (clipped to n), so the scan may run in place; with kind 2 the holder of
    // element n - 1 also writes y[n] = init + S_{n-1}.  Every thread of the
    // workgroup calls this (one barrier inside for kinds 1 and 2).
    template <bool ALIGNED, class F>
    __device__ __forceinline__ void emit(T* __restrict__ y, uint64_t n, uint64_t g0, T init,
                                         int kind, T pre, T* s_wend, int w, int lane,
                                         F&& fin) const
    {
        if (kind == 0) {
            emit_inclusive<ALIGNED>(y, n, g0, init, fin);
            return;
        }
        {
            T o[E];
            fin(V - 1, o);
            if (lane == 63) s_wend[w] = o[E - 1];
        }
        __syncthreads();
        emit_shifted<ALIGNED>(y, n, g0, init, kind, w == 0 ? pre : s_wend[w - 1], lane, fin);
    }

    // The same when the caller already knows the value before the wave's
    // first element (`before`): no exchange, no barrier.
    template <bool ALIGNED, class F>
    __device__ __forceinline__ void emit_known(T* __restrict__ y, uint64_t n, uint64_t g0, T init,
                                               int kind, T before, int lane, F&& fin) const
    {
        if (kind == 0) emit_inclusive<ALIGNED>(y, n, g0, init, fin);
        else emit_shifted<ALIGNED>(y, n, g0, init, kind, before, lane, fin);
    }

    template <bool ALIGNED, class F>
    __device__ __forceinline__ void emit_inclusive(T* __restrict__ y, uint64_t n, uint64_t g0,
                                                   T init, F&& fin) const
    {
#pragma unroll
        for (int u = 0; u < V; ++u) {
            T o[E];
            fin(u, o);
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = init + o[e];
            put<ALIGNED>(y, n, g0, u, o);
        }
    }

    // Kinds 1 and 2, given `carry`, the value before the wave's first element.
    template <bool ALIGNED, class F>
    __device__ __forceinline__ void emit_shifted(T* __restrict__ y, uint64_t n, uint64_t g0,
                                                 T init, int kind, T carry, int lane,
                                                 F&& fin) const
    {
#pragma unroll
        for (int u = 0; u < V; ++u) {
            T o[E];
            fin(u, o);
            const T up = shfl_up1(o[E - 1]);
            T s[E];
            s[0] = init + (lane == 0 ? carry : up);
#pragma unroll
            for (int e = 1; e < E; ++e) s[e] = init + o[e - 1];
            carry = readlane(o[E - 1], 63);
            if (kind == 2) {
                const uint64_t gi = g0 + (uint64_t)u * 64 * E;
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (gi + e == n - 1) y[n] = init + o[e];
            }
            put<ALIGNED>(y, n, g0, u, s);
        }
    }
};

}  // namespace canon
