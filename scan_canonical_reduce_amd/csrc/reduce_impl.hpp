// Canonical reduction kernels (gfx950).
//
// Expression (canonical-reduce README, P4016R0 "Key Design Points"): element
// i goes to lane i mod L; every lane is reduced by the iterative pairwise
// tree PW in index order; the L lane values are combined by PW in lane order;
// init is added once, on the left, at the end.
//
// View the input as a row-major matrix with L columns ("lanes"); row r holds
// x[rL .. rL+L).  Because PW over a sequence equals PW over the values of its
// aligned power-of-two chunks (bottom-up pairing never pairs across an
// aligned chunk boundary before the chunk is complete), the lane trees can be
// evaluated chunk by chunk in any schedule: every partial value below is the
// complete subtree of an aligned power-of-two range of rows, padded at the
// end with -0.0 where the input stops (exact: x + -0.0 == x).
//
// One kernel per call: workgroup p computes, for every lane, the subtree
// over its aligned range of rows and writes partial[p][lane]; the last
// workgroup (highest index) then waits for every other workgroup's arrival
// flag and finishes: PW over the partials of each lane in range order, PW
// over lanes, then init + R.
#pragma once
#include "device.hpp"
#include "launch.hpp"
#include "reduce.hpp"

namespace canon {

// What the finishing workgroup needs (the workspace layout of reduce.hpp).
template <typename T>
struct ReduceFin {
    T* partial;       // P rows of L values
    uint64_t* flags;  // one per streaming workgroup
    uint32_t* err;    // the error word
    uint64_t call_id;
    uint64_t P;
    uint32_t L;
    int lp_log;
    T init;
    T* out;
    long spin_limit;  // polls of the finishing workgroup's wait
};

// Partial values move between workgroups with device-coherent accesses
// (relaxed device-scope atomics): they are performed at the device's
// coherence point, so neither the writer's cache nor the reader's needs a
// write-back or an invalidation.
template <typename T>
__device__ __forceinline__ void store_coherent(T* p, T v)
{
    using U = typename std::conditional<sizeof(T) == 8, uint64_t, uint32_t>::type;
    __hip_atomic_store(reinterpret_cast<U*>(p), __builtin_bit_cast(U, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ T load_coherent(const T* p)
{
    using U = typename std::conditional<sizeof(T) == 8, uint64_t, uint32_t>::type;
    return __builtin_bit_cast(
        T, __hip_atomic_load(reinterpret_cast<const U*>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT));
}

// PW over partial[q0..q1)[j] (rows in range order), batches of 8 merged with
// a binary-counter stack; B batches' loads are in flight at a time.
template <typename T, int B>
__device__ __forceinline__ T pw_partials(const T* __restrict__ partial, uint64_t L, uint64_t j,
                                         uint64_t q0, uint64_t q1)
{
    TreeStack<T, 1, kReduceStackDepth> st;
    T v[1];
    const uint64_t nb = q1 > q0 ? (q1 - q0 + 7) / 8 : 0;
    for (uint64_t k0 = 0; k0 < nb; k0 += B) {
        T a[B][8];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint64_t q = q0 + (k0 + b) * 8 + u;
                a[b][u] = q < q1 ? load_coherent(partial + q * L + j) : neg_zero<T>();
            }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (k0 + b >= nb) break;
#pragma unroll
            for (int h = 1; h < 8; h *= 2)
#pragma unroll
                for (int u = 0; u < 8; u += 2 * h) a[b][u] = a[b][u] + a[b][u + h];
            v[0] = a[b][0];
            st.push(k0 + b, v);
        }
    }
    st.collapse(nb, v);
    return v[0];
}

// The finish, by one workgroup of FT threads: lane value = PW over the
// partials of the lane; R = PW over lanes 0..L-1 (padded to Lp = 2^lp_log
// with -0.0 lanes); out = init + R.
//   Lp <= FT: S = FT / Lp threads per lane, each over an aligned power-of-
//     two segment of the partials; segments and then lanes merged in LDS.
//   Lp > FT: thread t owns lanes [t*K, (t+1)*K), K = Lp / FT.
template <typename T, int FT>
__device__ __forceinline__ void finish_block(const ReduceFin<T>& f, T* s_v)
{
    constexpr int PB = 4;  // batches of partials in flight per thread
    const int t = threadIdx.x;
    const uint64_t Lp = 1ull << f.lp_log;
    const uint64_t P = f.P, L = f.L;
    if (Lp <= (uint64_t)FT) {
        const int S = FT >> f.lp_log;
        const uint64_t j = t & (Lp - 1);
        const int s = t >> f.lp_log;
        uint64_t ps = 1;
        while (ps * S < P) ps *= 2;
        const uint64_t q0 = s * ps, q1 = (q0 + ps) < P ? (q0 + ps) : P;
        s_v[t] = (j < L) ? pw_partials<T, PB>(f.partial, L, j, q0, q1) : neg_zero<T>();
        __syncthreads();
        for (int h = 1; h < S; h *= 2) {
            if (s % (2 * h) == 0) s_v[t] = s_v[t] + s_v[t + h * (int)Lp];
            __syncthreads();
        }
        // lanes 0..Lp-1 now at s_v[0..Lp)
        for (uint64_t h = 1; h < Lp; h *= 2) {
            if ((uint64_t)t < Lp && t % (2 * h) == 0) s_v[t] = s_v[t] + s_v[t + h];
            __syncthreads();
        }
    } else {
        const uint64_t K = Lp / FT;
        TreeStack<T, 1, kMaxLogL + 1> st;
        T v[1];
        for (uint64_t k = 0; k < K; ++k) {
            const uint64_t j = t * K + k;
            v[0] = (j < L) ? pw_partials<T, PB>(f.partial, L, j, 0, P) : neg_zero<T>();
            st.push(k, v);
        }
        st.collapse(K, v);
        s_v[t] = v[0];
        __syncthreads();
        for (int h = 1; h < FT; h *= 2) {
            if (t % (2 * h) == 0) s_v[t] = s_v[t] + s_v[t + h];
            __syncthreads();
        }
    }
    if (t == 0) f.out[0] = f.init + s_v[0];
}

// After a streaming workgroup has written its partials (store_coherent;
// every thread calls this): every wave waits until its stores are performed,
// then the workgroup's flag is set to the call id; the last workgroup
// instead waits (bounded) for every other flag, finishes, and writes the
// error word.  Only the last workgroup waits, and only for workgroups that
// never wait, so the wait ends whatever the grid and however many
// workgroups are resident.
template <typename T, int FT>
__device__ __forceinline__ void arrive_or_finish(const ReduceFin<T>& f, T* s_v)
{
    const uint64_t nwg = (uint64_t)gridDim.x * gridDim.y;
    const uint64_t me = (uint64_t)blockIdx.y * gridDim.x + blockIdx.x;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores performed
    __syncthreads();
    if (me + 1 < nwg) {
        if (threadIdx.x == 0)
            __hip_atomic_store(f.flags + me, f.call_id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    int late = 0;
    for (uint64_t i = threadIdx.x; i + 1 < nwg && !late; i += FT) {
        long it = 0;
        while (__hip_atomic_load(f.flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
               f.call_id) {
            if (++it > f.spin_limit) {
                late = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    late = __syncthreads_or(late);
    finish_block<T, FT>(f, s_v);
    if (threadIdx.x == 0) *f.err = late ? kErrSpin : 0u;
}

// ============================================================================
// Streaming kernel for L = 2^LOGL and 16-byte aligned input.
//
// A "super-row" is max(L, E) consecutive elements (E = elements per 16-byte
// vector): one row when L >= E, else E/L rows whose lanes are first reduced
// inside the vector.  A wave instruction loads 64 vectors; CW = vectors of a
// super-row handled by one wave (<= 64), G = 64 / CW super-rows per
// instruction.  Rows wider than 64 vectors are split into column slices
// (grid.y).  Each thread loads U = 8 vectors per batch; a batch covers G*U
// aligned super-rows.  Within a batch:
//   row-group layout (super-row >= 128 B): thread g holds super-rows
//     g*U .. g*U+7: tree over them in registers, then across lanes g;
//   interleaved layout (super-row < 128 B): instruction u covers super-rows
//     u*G .. u*G+G-1 contiguously: tree across lanes first, then over u.
// Batches of a wave are merged with a binary-counter stack; the 16 waves of
// the workgroup are merged through LDS as a complete tree.
// ============================================================================
template <typename T, int LOGL>
struct Pow2Geom {
    static constexpr int E = Elem<T>::E;
    static constexpr int LOGE = Elem<T>::LOGE;
    static constexpr int VE = LOGL < LOGE ? (1 << LOGL) : E;  // lane values per vector
    static constexpr int LOG_SR = LOGL > LOGE ? LOGL : LOGE;  // log2 elements per super-row
    static constexpr int LOGC = LOG_SR - LOGE;                // log2 vectors per super-row
    static constexpr int LOG_CW = LOGC < 6 ? LOGC : 6;
    static constexpr int CW = 1 << LOG_CW;
    static constexpr int LOGG = 6 - LOG_CW;
    static constexpr int G = 1 << LOGG;
    static constexpr int U = kReduceBatch;
    static constexpr int GU = G * U;
    static constexpr bool INTERLEAVED = LOGC < 3;
    static constexpr int SW = CW * VE;  // lanes of one column slice
    static constexpr int THREADS = pow2_reduce_threads(LOGC, VE == E);
    static constexpr int WAVES = THREADS / 64;
    static_assert(SW <= THREADS, "one thread per lane of a column slice in the wave merge");
};

// Reduce the E elements of one vector to VE lane values: the vector holds E/VE
// rows of VE lanes; rows are paired bottom-up, lower row on the left.
template <typename T, int VE>
__device__ __forceinline__ void in_vector_rows(T (&w)[Elem<T>::E], T (&out)[VE])
{
    constexpr int E = Elem<T>::E;
#pragma unroll
    for (int rows = E / VE; rows > 1; rows /= 2) {
#pragma unroll
        for (int r = 0; r < rows / 2; ++r)
#pragma unroll
            for (int j = 0; j < VE; ++j) w[r * VE + j] = w[2 * r * VE + j] + w[(2 * r + 1) * VE + j];
    }
#pragma unroll
    for (int j = 0; j < VE; ++j) out[j] = w[j];
}

// Complete tree across the G lane groups (lanes l, l^CW, l^2CW, ...); lower
// group on the left.  Every lane of a column ends with the same value.
template <typename T, int VE, int LOG_CW, int LOGG>
__device__ __forceinline__ void tree_across_groups(T (&v)[VE], int g)
{
#pragma unroll
    for (int k = 0; k < LOGG; ++k) {
        constexpr int dummy = 0;
        (void)dummy;
        T o[VE];
#pragma unroll
        for (int i = 0; i < VE; ++i) {
            switch (LOG_CW + k) {
                case 0: o[i] = shfl_xor<1>(v[i]); break;
                case 1: o[i] = shfl_xor<2>(v[i]); break;
                case 2: o[i] = shfl_xor<4>(v[i]); break;
                case 3: o[i] = shfl_xor<8>(v[i]); break;
                case 4: o[i] = shfl_xor<16>(v[i]); break;
                default: o[i] = shfl_xor<32>(v[i]); break;
            }
        }
        const bool upper = (g >> k) & 1;
#pragma unroll
        for (int i = 0; i < VE; ++i) v[i] = upper ? (o[i] + v[i]) : (v[i] + o[i]);
    }
}

template <typename T, int LOGL, bool GUARD>
__device__ __forceinline__ void pow2_batch(const T* __restrict__ x, uint64_t n, uint64_t sr_base,
                                           int slice, int c, int g,
                                           T (&out)[Pow2Geom<T, LOGL>::VE])
{
    using GM = Pow2Geom<T, LOGL>;
    constexpr int E = GM::E, VE = GM::VE, U = GM::U;
    T a[U][VE];
    T w[U][E];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t sr = GM::INTERLEAVED ? sr_base + (uint64_t)u * GM::G + g
                                            : sr_base + (uint64_t)g * U + u;
        const uint64_t el = (sr << GM::LOG_SR) + (uint64_t)(slice * GM::CW + c) * E;
        if (!GUARD || el + E <= n) {
            load_vec(x + el, w[u]);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) w[u][e] = (el + e < n) ? x[el + e] : neg_zero<T>();
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) in_vector_rows<T, VE>(w[u], a[u]);
    if constexpr (GM::INTERLEAVED) {
#pragma unroll
        for (int u = 0; u < U; ++u) tree_across_groups<T, VE, GM::LOG_CW, GM::LOGG>(a[u], g);
    }
#pragma unroll
    for (int h = 1; h < U; h *= 2)
#pragma unroll
        for (int u = 0; u < U; u += 2 * h)
#pragma unroll
            for (int i = 0; i < VE; ++i) a[u][i] = a[u][i] + a[u + h][i];
    if constexpr (!GM::INTERLEAVED) tree_across_groups<T, VE, GM::LOG_CW, GM::LOGG>(a[0], g);
#pragma unroll
    for (int i = 0; i < VE; ++i) out[i] = a[0][i];
}

template <typename T, int LOGL>
__global__ __launch_bounds__((Pow2Geom<T, LOGL>::THREADS)) void k_reduce_pow2(
    const T* __restrict__ x, uint64_t n, int rw_log, ReduceFin<T> f)
{
    using GM = Pow2Geom<T, LOGL>;
    constexpr int VE = GM::VE;
    constexpr uint64_t L = 1ull << LOGL;
    __shared__ T s_wave[GM::WAVES][GM::SW];
    __shared__ T s_fin[GM::THREADS];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & (GM::CW - 1), g = lane >> GM::LOG_CW;
    const uint64_t p = blockIdx.x;
    const int slice = blockIdx.y;
    const uint64_t rw = 1ull << rw_log;  // super-rows per wave (multiple of GU)
    const uint64_t sr0 = (p * GM::WAVES + wave) * rw;
    const uint64_t msr = (n + (1ull << GM::LOG_SR) - 1) >> GM::LOG_SR;

    uint64_t nb = 0, nfull = 0;  // batches holding data / entirely inside x
    if (sr0 < msr) {
        const uint64_t span = (msr - sr0) < rw ? (msr - sr0) : rw;
        nb = (span + GM::GU - 1) / GM::GU;
        const uint64_t full_rows = (n >> GM::LOG_SR) > sr0 ? (n >> GM::LOG_SR) - sr0 : 0;
        nfull = full_rows / GM::GU;
        if (nfull > nb) nfull = nb;
    }
    TreeStack<T, VE, kReduceStackDepth> st;
    T v[VE];
    for (uint64_t k = 0; k < nfull; ++k) {
        pow2_batch<T, LOGL, false>(x, n, sr0 + k * GM::GU, slice, c, g, v);
        st.push(k, v);
    }
    for (uint64_t k = nfull; k < nb; ++k) {
        pow2_batch<T, LOGL, true>(x, n, sr0 + k * GM::GU, slice, c, g, v);
        st.push(k, v);
    }
    st.collapse(nb, v);

    if (g == 0) {
#pragma unroll
        for (int i = 0; i < VE; ++i) s_wave[wave][c * VE + i] = v[i];
    }
    __syncthreads();
    if (threadIdx.x < GM::SW) {
        T t[GM::WAVES];
#pragma unroll
        for (int w = 0; w < GM::WAVES; ++w) t[w] = s_wave[w][threadIdx.x];
#pragma unroll
        for (int h = 1; h < GM::WAVES; h *= 2)
#pragma unroll
            for (int w = 0; w < GM::WAVES; w += 2 * h) t[w] = t[w] + t[w + h];
        store_coherent(f.partial + p * L + (uint64_t)slice * GM::SW + threadIdx.x, t[0]);
    }
    arrive_or_finish<T, GM::THREADS>(f, s_fin);
}

// ============================================================================
// Streaming kernel for any L and any alignment.  Thread (j, s): lane j of a
// chunk of LW lanes (grid.y picks the chunk), segment s of S aligned
// segments of the workgroup's row range; it walks 2^rs_log rows of lane j
// (element loads, coalesced across j), merging batches of 8 rows with a
// binary-counter stack; the S segments are merged through LDS.
// ============================================================================
template <typename T>
__global__ __launch_bounds__(kReduceThreads) void k_reduce_general(const T* __restrict__ x,
                                                                   uint64_t n, uint32_t L,
                                                                   int lw_log, int rs_log,
                                                                   ReduceFin<T> f)
{
    __shared__ T s_seg[kReduceThreads];
    const int LW = 1 << lw_log, S = kReduceThreads >> lw_log;
    const int jl = threadIdx.x & (LW - 1), s = threadIdx.x >> lw_log;
    const uint64_t j = (uint64_t)blockIdx.y * LW + jl;
    const uint64_t p = blockIdx.x;
    const uint64_t rs = 1ull << rs_log;
    const uint64_t r0 = (p * S + s) * rs, r1 = r0 + rs;
    const uint64_t m = (n + L - 1) / L;  // rows

    T v[1];
    uint64_t nb = 0;
    TreeStack<T, 1, kReduceStackDepth> st;
    if (j < L && r0 < m) {
        const uint64_t rend = r1 < m ? r1 : m;
        nb = (rend - r0 + 7) / 8;
        for (uint64_t k = 0; k < nb; ++k) {
            T a[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint64_t r = r0 + k * 8 + u;
                const uint64_t el = r * L + j;
                a[u] = (r < r1 && el < n) ? x[el] : neg_zero<T>();
            }
#pragma unroll
            for (int h = 1; h < 8; h *= 2)
#pragma unroll
                for (int u = 0; u < 8; u += 2 * h) a[u] = a[u] + a[u + h];
            v[0] = a[0];
            st.push(k, v);
        }
    }
    st.collapse(nb, v);
    s_seg[threadIdx.x] = v[0];
    __syncthreads();
    // complete tree over the S segments of each lane (segment s at s*LW + jl)
    for (int h = 1; h < S; h *= 2) {
        if (s % (2 * h) == 0) s_seg[threadIdx.x] = s_seg[threadIdx.x] + s_seg[threadIdx.x + h * LW];
        __syncthreads();
    }
    if (s == 0 && j < L) store_coherent(f.partial + p * L + j, s_seg[jl]);
    __syncthreads();  // s_seg is the finish's LDS
    arrive_or_finish<T, kReduceThreads>(f, s_seg);
}

// ============================================================================
// Row-batched reduce: one workgroup per row.  Lanes are processed in chunks
// of LW = min(Lp, 256); S = 256 / LW threads share a lane, each over an
// aligned segment of rs rows-of-L (rs a power of two, at most
// 8 << kReduceStackDepth so that a segment's batches fit its stack).  The S
// segments of a "round" (rs * S aligned rows) are merged in LDS to the
// round's complete subtree per lane; LONG rows (more than one round) merge
// their rounds, per lane, with a second binary-counter stack.  Lane values of
// a chunk are then merged in LDS to the chunk's complete subtree, and chunk
// values across chunks with a binary-counter stack (the cross-lane PW over
// aligned chunks of lanes).
// ============================================================================
template <typename T>
__device__ __forceinline__ T rows_segment(const T* __restrict__ xr, uint64_t cols, uint32_t L,
                                          uint64_t j, uint64_t m, uint64_t r0, uint64_t r1)
{
    T v[1];
    uint64_t nb = 0;
    TreeStack<T, 1, kReduceStackDepth> st;
    if (j < L && r0 < m) {
        const uint64_t rend = r1 < m ? r1 : m;
        nb = (rend - r0 + 7) / 8;
        for (uint64_t k = 0; k < nb; ++k) {
            T a[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint64_t r = r0 + k * 8 + u;
                const uint64_t el = r * L + j;
                a[u] = (r < r1 && el < cols) ? xr[el] : neg_zero<T>();
            }
#pragma unroll
            for (int h = 1; h < 8; h *= 2)
#pragma unroll
                for (int u = 0; u < 8; u += 2 * h) a[u] = a[u] + a[u + h];
            v[0] = a[0];
            st.push(k, v);
        }
    }
    st.collapse(nb, v);
    return v[0];
}

template <typename T, bool LONG>
__global__ __launch_bounds__(kRowsThreads) void k_reduce_rows(const T* __restrict__ x,
                                                              uint64_t rows, uint64_t cols,
                                                              uint64_t ldx, uint32_t L, int lw_log,
                                                              T init, T* __restrict__ out)
{
    __shared__ T s_v[kRowsThreads];
    const int t = threadIdx.x;
    const int LW = 1 << lw_log, S = kRowsThreads >> lw_log;
    const int jl = t & (LW - 1), s = t >> lw_log;
    const uint64_t m = (cols + L - 1) / L;
    const uint64_t rs = rows_segment_len(m, S);
    const uint64_t span = rs * S;  // rows of one round
    const uint64_t nrounds = LONG ? (m + span - 1) / span : 1;
    const uint64_t nchunks = (L + LW - 1) / LW;

    for (uint64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const T* xr = x + row * ldx;
        TreeStack<T, 1, 17> cst;
        T cv[1];
        for (uint64_t ch = 0; ch < nchunks; ++ch) {
            const uint64_t j = ch * LW + jl;
            TreeStack<T, 1, LONG ? kRowsRoundDepth : 0> rst;
            T rv[1];
            for (uint64_t rd = 0; rd < nrounds; ++rd) {
                const uint64_t r0 = rd * span + s * rs;
                s_v[t] = rows_segment(xr, cols, L, j, m, r0, r0 + rs);
                __syncthreads();
                for (int h = 1; h < S; h *= 2) {
                    if (s % (2 * h) == 0) s_v[t] = s_v[t] + s_v[t + h * LW];
                    __syncthreads();
                }
                if constexpr (LONG) {
                    // the round's subtree of lane j, at s_v[jl]
                    rv[0] = s_v[jl];
                    rst.push(rd, rv);
                    __syncthreads();  // s_v is rewritten by the next round
                }
            }
            if constexpr (LONG) {
                rst.collapse(nrounds, rv);
                if (s == 0) s_v[t] = rv[0];
                __syncthreads();
            }
            for (int h = 1; h < LW; h *= 2) {
                if (t < LW && t % (2 * h) == 0) s_v[t] = s_v[t] + s_v[t + h];
                __syncthreads();
            }
            cv[0] = s_v[0];
            __syncthreads();
            cst.push(ch, cv);
        }
        cst.collapse(nchunks, cv);
        if (t == 0) out[row] = (cols == 0) ? init : init + cv[0];
    }
}

// ============================================================================
// Row-batched reduce, register path: L = 2^LOGL with a row of L at most one
// wave-wide load (L <= 64 E), 16-byte aligned rows, at most
// 2^kRowsStackDepth batches per row.  One wave per row: the wave walks the
// row's batches in order (pow2_batch, as the streaming kernel) with a
// binary-counter stack, which leaves the row's L lane values in lanes
// 0 .. CW-1 (VE each); the complete tree over the lanes is taken in the
// thread and then across those lanes, and init is added on the left.
// ============================================================================
constexpr int kRowsStackDepth = 6;

template <typename T, int LOGL>
__global__ __launch_bounds__(kRowsThreads) void k_reduce_rows_pow2(const T* __restrict__ x,
                                                                   uint64_t rows, uint64_t cols,
                                                                   uint64_t ldx, T init,
                                                                   T* __restrict__ out)
{
    using GM = Pow2Geom<T, LOGL>;
    static_assert(GM::LOGC <= 6, "a row of L fits one wave-wide load");
    constexpr int VE = GM::VE;
    const int lane = threadIdx.x & 63;
    const int c = lane & (GM::CW - 1), g = lane >> GM::LOG_CW;
    const uint64_t waves = (uint64_t)gridDim.x * (kRowsThreads / 64);
    const uint64_t msr = (cols + (1ull << GM::LOG_SR) - 1) >> GM::LOG_SR;
    const uint64_t nb = (msr + GM::GU - 1) / GM::GU;
    const uint64_t nfull = ((cols >> GM::LOG_SR) / GM::GU) < nb ? (cols >> GM::LOG_SR) / GM::GU : nb;
    for (uint64_t row = (uint64_t)blockIdx.x * (kRowsThreads / 64) + (threadIdx.x >> 6); row < rows;
         row += waves) {
        const T* xr = x + row * ldx;
        TreeStack<T, VE, kRowsStackDepth> st;
        T v[VE];
        for (uint64_t k = 0; k < nfull; ++k) {
            pow2_batch<T, LOGL, false>(xr, cols, k * GM::GU, 0, c, g, v);
            st.push(k, v);
        }
        for (uint64_t k = nfull; k < nb; ++k) {
            pow2_batch<T, LOGL, true>(xr, cols, k * GM::GU, 0, c, g, v);
            st.push(k, v);
        }
        st.collapse(nb, v);
        // lanes c * VE + i: the tree over the thread's VE lanes, then across
        // the CW threads holding the row's lanes (lower lanes on the left)
#pragma unroll
        for (int h = 1; h < VE; h *= 2)
#pragma unroll
            for (int i = 0; i < VE; i += 2 * h) v[i] = v[i] + v[i + h];
        T r = v[0];
#pragma unroll
        for (int k = 0; k < GM::LOG_CW; ++k) {
            T o;
            switch (k) {
                case 0: o = shfl_xor<1>(r); break;
                case 1: o = shfl_xor<2>(r); break;
                case 2: o = shfl_xor<4>(r); break;
                case 3: o = shfl_xor<8>(r); break;
                case 4: o = shfl_xor<16>(r); break;
                default: o = shfl_xor<32>(r); break;
            }
            r = ((lane >> k) & 1) ? (o + r) : (r + o);
        }
        if (lane == 0) out[row] = (cols == 0) ? init : init + r;
    }
}

template <typename T, int LOGL>
static hipError_t launch_rows_pow2(const T* x, uint64_t rows, uint64_t cols, uint64_t ldx, T init,
                                   T* out, hipStream_t s)
{
    constexpr int RPB = kRowsThreads / 64;  // rows per workgroup
    // at most one workgroup per CU, each wave walking rows grid-stride: four
    // waves per CU keep about 32 KiB of loads in flight, where streaming
    // reads are fastest (16384 x 4096 f64, L = 16: 86 -> 81 us)
    uint64_t grid = (rows + RPB - 1) / RPB;
    const uint64_t cus = device_cus();
    if (grid > cus) grid = cus;
    grid = capped_grid(grid);
    hipLaunchKernelGGL((k_reduce_rows_pow2<T, LOGL>), dim3((unsigned)grid), dim3(kRowsThreads), 0,
                       s, x, rows, cols, ldx, init, out);
    return hipGetLastError();
}

template <typename T, int LOGL>
static hipError_t launch_rows_pow2_dispatch(int logl, const T* x, uint64_t rows, uint64_t cols,
                                            uint64_t ldx, T init, T* out, hipStream_t s)
{
    if constexpr (LOGL > Elem<T>::LOGE + 6) {
        return hipErrorInvalidValue;
    } else {
        if (logl == LOGL) return launch_rows_pow2<T, LOGL>(x, rows, cols, ldx, init, out, s);
        return launch_rows_pow2_dispatch<T, LOGL + 1>(logl, x, rows, cols, ldx, init, out, s);
    }
}

// ============================================================================
// Host-side launchers (called from api.cpp).
// ============================================================================
template <typename T, int LOGL>
static hipError_t launch_pow2_one(const T* x, uint64_t n, const ReducePlan& pl,
                                  const ReduceFin<T>& f, hipStream_t s)
{
    dim3 grid((unsigned)pl.P, (unsigned)pl.slices);
    hipLaunchKernelGGL((k_reduce_pow2<T, LOGL>), grid, dim3(Pow2Geom<T, LOGL>::THREADS), 0, s, x,
                       n, pl.rw_log, f);
    return hipGetLastError();
}

template <typename T, int LOGL>
static hipError_t launch_pow2_dispatch(int logl, const T* x, uint64_t n, const ReducePlan& pl,
                                       const ReduceFin<T>& f, hipStream_t s)
{
    if constexpr (LOGL > kMaxLogL) {
        return hipErrorInvalidValue;
    } else {
        if (logl == LOGL) return launch_pow2_one<T, LOGL>(x, n, pl, f, s);
        return launch_pow2_dispatch<T, LOGL + 1>(logl, x, n, pl, f, s);
    }
}

template <typename T, bool POW2>
hipError_t launch_reduce(const T* x, uint64_t n, uint32_t L, T init, T* out, void* ws,
                         const ReducePlan& pl, uint64_t call_id, hipStream_t s)
{
    if (pl.P == 0) return hipErrorInvalidValue;
    const ReduceWs w = reduce_ws_layout(pl, L, sizeof(T));
    unsigned char* b = static_cast<unsigned char*>(ws);
    const uint64_t lim = g_sched_spin_limit.load(std::memory_order_relaxed);
    const ReduceFin<T> f{reinterpret_cast<T*>(b + w.partial_off),
                         reinterpret_cast<uint64_t*>(b + w.flags_off),
                         reinterpret_cast<uint32_t*>(b),
                         call_id,
                         pl.P,
                         L,
                         pl.lp_log,
                         init,
                         out,
                         lim ? (long)lim : kSpinLimit};
    if (pl.pow2) {
        if constexpr (POW2) return launch_pow2_dispatch<T, 0>(pl.logl, x, n, pl, f, s);
        return hipErrorInvalidValue;
    }
    dim3 grid((unsigned)pl.P, (unsigned)pl.slices);
    hipLaunchKernelGGL((k_reduce_general<T>), grid, dim3(kReduceThreads), 0, s, x, n, L, pl.lw_log,
                       pl.rs_log, f);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_reduce_rows(const T* x, uint64_t rows, uint64_t cols, uint64_t ldx, uint32_t L,
                              T init, T* out, hipStream_t s)
{
    int lp_log = 0;
    while ((1ull << lp_log) < L) ++lp_log;
    // register path: power-of-two L of at most one wave-wide load per row of
    // L, 16-byte aligned rows, and rows short enough for its stack
    const uint64_t batch_elems = 64ull * kReduceBatch * Elem<T>::E;
    const bool aligned = ((uintptr_t)x % 16 == 0) && ((ldx * sizeof(T)) % 16 == 0);
    if ((1ull << lp_log) == L && lp_log <= Elem<T>::LOGE + 6 && aligned &&
        cols <= (batch_elems << kRowsStackDepth))
        return launch_rows_pow2_dispatch<T, 0>(lp_log, x, rows, cols, ldx, init, out, s);
    const int lw_log = lp_log < 8 ? lp_log : 8;
    const int S = kRowsThreads >> lw_log;
    const uint64_t m = (cols + L - 1) / L;
    // one workgroup per row (the kernel strides over rows past the grid limit)
    const uint64_t grid = capped_grid(rows < 0x7FFFFFFFull ? rows : 0x7FFFFFFFull);
    if (rows_segment_len(m, S) * S >= m)
        hipLaunchKernelGGL((k_reduce_rows<T, false>), dim3((unsigned)grid), dim3(kRowsThreads), 0,
                           s, x, rows, cols, ldx, L, lw_log, init, out);
    else
        hipLaunchKernelGGL((k_reduce_rows<T, true>), dim3((unsigned)grid), dim3(kRowsThreads), 0,
                           s, x, rows, cols, ldx, L, lw_log, init, out);
    return hipGetLastError();
}

}  // namespace canon
