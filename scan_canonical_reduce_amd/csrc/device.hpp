// Device-side helpers shared by the libcanon kernels (gfx950, wave64).
//
// Everything here is plain data movement: 16-byte loads and stores, wave64
// cross-lane moves, and agent-scope atomics for the scan's published values.
// The only arithmetic the kernels perform on data is IEEE addition, always
// written as (left + right) with `left` covering the lower input indices.
//
// "Absent" values are represented by -0.0: x + (-0.0) == x for every x
// (including +0.0, -0.0, infinities and NaN), and -0.0 + -0.0 == -0.0, so
// padding a sequence with trailing -0.0 never changes its pairwise value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace canon {

constexpr int kWave = 64;

template <typename T> struct Elem;
template <> struct Elem<double> {
    using base_t = double;
    using bits_t = uint64_t;
    static constexpr int E = 2;     // elements per 16-byte vector
    static constexpr int LOGE = 1;
    typedef double vec_t __attribute__((ext_vector_type(2)));
};
template <> struct Elem<float> {
    using base_t = float;
    using bits_t = uint32_t;
    static constexpr int E = 4;
    static constexpr int LOGE = 2;
    typedef float vec_t __attribute__((ext_vector_type(4)));
};

// ------------------------------------------------------------- operators
// The expression is the same for any binary operator.  Kernels are written
// with `a + b` on their value type T; for an operator other than IEEE
// addition T is OpVal<B, Op>, a B-sized wrapper whose `+` applies Op (left
// operand on the left), so every kernel evaluates the identical tree.  Op:
//   OpMul  multiplication, absent value 1.0
//   OpMin  IEEE 754-2019 minimum (NaN if either operand is NaN, -0.0 below
//          +0.0), absent value +inf
//   OpMax  IEEE 754-2019 maximum, absent value -inf
// The absent value is the operator's exact identity (op(x, absent) == x for
// every x, NaN payloads aside), as -0.0 is for addition.
struct OpMul {
    template <typename B>
    static __host__ __device__ __forceinline__ B f(B a, B b) { return a * b; }
    template <typename B>
    static __host__ __device__ __forceinline__ B identity() { return B(1.0); }
};
// minimum / maximum: the compiler's IEEE 754-2019 minimum / maximum (one
// v_minimum3_f32 / v_maximum3_f32 on gfx950; v_min_f64 / v_max_f64 with the
// NaN case selected in double).
struct OpMin {
    template <typename B>
    static __host__ __device__ __forceinline__ B f(B a, B b)
    {
        return __builtin_elementwise_minimum(a, b);
    }
    template <typename B>
    static __host__ __device__ __forceinline__ B identity() { return B(__builtin_inf()); }
};
struct OpMax {
    template <typename B>
    static __host__ __device__ __forceinline__ B f(B a, B b)
    {
        return __builtin_elementwise_maximum(a, b);
    }
    template <typename B>
    static __host__ __device__ __forceinline__ B identity() { return B(-__builtin_inf()); }
};

template <typename B, class Op>
struct OpVal {
    B v;
};
template <typename B, class Op>
__host__ __device__ __forceinline__ OpVal<B, Op> operator+(OpVal<B, Op> a, OpVal<B, Op> b)
{
    return OpVal<B, Op>{Op::template f<B>(a.v, b.v)};
}
template <typename B, class Op> struct Elem<OpVal<B, Op>> : Elem<B> {};

// T is an OpVal wrapper (an operator other than addition).
template <typename T>
constexpr bool kIsOpVal = !std::is_same<T, typename Elem<T>::base_t>::value;

// The absent value of T's operator.
template <typename T> struct Absent {
    static __device__ __forceinline__ T value() { return T(-0.0); }
};
template <typename B, class Op> struct Absent<OpVal<B, Op>> {
    static __device__ __forceinline__ OpVal<B, Op> value()
    {
        return OpVal<B, Op>{Op::template identity<B>()};
    }
};
template <typename T> __device__ __forceinline__ T neg_zero() { return Absent<T>::value(); }

// Keeps a value in a VGPR at this point (an empty asm operand): the compiler
// may not move the operations that produce it past here.
template <typename T> __device__ __forceinline__ void pin_reg(T& x) { asm volatile("" : "+v"(x)); }
// A copy of the per-lane value v that the compiler cannot relate to v: the
// addresses of a tile's stores derived from it are computed where they are
// used, instead of being kept live from the tile's loads (one 64-bit address
// per vector of the thread).
template <typename T> __device__ __forceinline__ T fresh_copy(T v)
{
    asm volatile("" : "+v"(v));
    return v;
}
template <typename B, class Op> __device__ __forceinline__ void pin_reg(OpVal<B, Op>& x)
{
    asm volatile("" : "+v"(x.v));
}

// ---------------------------------------------------------------- 16-byte I/O
// (T is double / float or an OpVal wrapper of one: same bits either way.)
template <typename T>
__device__ __forceinline__ void load_vec(const T* p, T (&v)[Elem<T>::E])
{
    using V = typename Elem<T>::vec_t;
    V x = __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
#pragma unroll
    for (int e = 0; e < Elem<T>::E; ++e) {
        // through a scalar: a bit cast of the vector element itself reads
        // element 0 (seen with this compiler)
        const typename Elem<T>::base_t b = x[e];
        v[e] = __builtin_bit_cast(T, b);
    }
}

template <typename T>
__device__ __forceinline__ void store_vec(T* p, const T (&v)[Elem<T>::E])
{
    using V = typename Elem<T>::vec_t;
    V x;
#pragma unroll
    for (int e = 0; e < Elem<T>::E; ++e) {
        const typename Elem<T>::base_t b = __builtin_bit_cast(typename Elem<T>::base_t, v[e]);
        x[e] = b;
    }
    __builtin_nontemporal_store(x, reinterpret_cast<V*>(p));
}

// 16 bytes from / to LDS in one access (element e of lane l at l * E + e:
// one element at a time would hit the same banks from neighbouring lanes).
template <typename T>
__device__ __forceinline__ void lds_load_vec(const T* p, T (&v)[Elem<T>::E])
{
    using V = typename Elem<T>::vec_t;
    const V x = *reinterpret_cast<const V*>(p);
#pragma unroll
    for (int e = 0; e < Elem<T>::E; ++e) {
        const typename Elem<T>::base_t b = x[e];
        v[e] = __builtin_bit_cast(T, b);
    }
}

template <typename T>
__device__ __forceinline__ void lds_store_vec(T* p, const T (&v)[Elem<T>::E])
{
    using V = typename Elem<T>::vec_t;
    V x;
#pragma unroll
    for (int e = 0; e < Elem<T>::E; ++e) {
        const typename Elem<T>::base_t b = __builtin_bit_cast(typename Elem<T>::base_t, v[e]);
        x[e] = b;
    }
    *reinterpret_cast<V*>(p) = x;
}

// ------------------------------------------------------- wave64 lane moves
// ds_swizzle in bit mode: source lane = ((lane & AND) | OR) ^ XOR within each
// group of 32 lanes.  PAT = AND | OR << 5 | XOR << 10.
template <int PAT>
__device__ __forceinline__ uint32_t swz32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, PAT);
}

template <int PAT>
__device__ __forceinline__ double swz(double v)
{
    uint64_t b = __builtin_bit_cast(uint64_t, v);
    uint32_t lo = swz32<PAT>((uint32_t)b), hi = swz32<PAT>((uint32_t)(b >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
template <int PAT>
__device__ __forceinline__ float swz(float v)
{
    return __builtin_bit_cast(float, swz32<PAT>(__builtin_bit_cast(uint32_t, v)));
}

__device__ __forceinline__ double readlane(double v, int lane)
{
    uint64_t b = __builtin_bit_cast(uint64_t, v);
    uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ float readlane(float v, int lane)
{
    return __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_readlane(
                                         (int)__builtin_bit_cast(uint32_t, v), lane));
}

template <int PAT, typename B, class Op>
__device__ __forceinline__ OpVal<B, Op> swz(OpVal<B, Op> v)
{
    return OpVal<B, Op>{swz<PAT>(v.v)};
}
template <typename B, class Op>
__device__ __forceinline__ OpVal<B, Op> readlane(OpVal<B, Op> v, int lane)
{
    return OpVal<B, Op>{readlane(v.v, lane)};
}

// One 32-bit lane move through DPP (the source operand of a VALU move read
// from another lane of the same row of 16): lanes outside the row and bank
// masks keep `old`.
template <int CTRL, int ROWS = 0xF, int BANKS = 0xF>
__device__ __forceinline__ uint32_t dpp32(uint32_t old, uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWS, BANKS, false);
}

// Apply a 32-bit lane move to each half of a 64-bit value, or to a 32-bit one.
template <typename T, typename F>
__device__ __forceinline__ T per_dword(T v, T old, F f)
{
    if constexpr (sizeof(T) == 8) {
        const uint64_t b = __builtin_bit_cast(uint64_t, v), o = __builtin_bit_cast(uint64_t, old);
        const uint32_t lo = f((uint32_t)o, (uint32_t)b);
        const uint32_t hi = f((uint32_t)(o >> 32), (uint32_t)(b >> 32));
        return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
    } else {
        return __builtin_bit_cast(T, f(__builtin_bit_cast(uint32_t, old), __builtin_bit_cast(uint32_t, v)));
    }
}

// The 32-bit value held by lane (lane ^ MASK), MASK a power of two below 64,
// without an LDS round trip: DPP quad permutations for 1 and 2, two
// bank-masked row shifts for 4 and 8, the gfx950 lane-swap instructions
// (v_permlane16_swap / v_permlane32_swap) for 16 and 32.
template <int MASK>
__device__ __forceinline__ uint32_t xor32(uint32_t v)
{
    if constexpr (MASK == 1) {
        return dpp32<0xB1>(0u, v);  // quad_perm [1,0,3,2]
    } else if constexpr (MASK == 2) {
        return dpp32<0x4E>(0u, v);  // quad_perm [2,3,0,1]
    } else if constexpr (MASK == 4) {
        // lanes with bit 2 clear read lane + 4 (row_shl:4), the others lane - 4
        return dpp32<0x114, 0xF, 0xA>(dpp32<0x104, 0xF, 0x5>(0u, v), v);
    } else if constexpr (MASK == 8) {
        return dpp32<0x118, 0xF, 0xC>(dpp32<0x108, 0xF, 0x3>(0u, v), v);
    } else if constexpr (MASK == 16) {
        // swap of rows 1, 3 of the first operand with rows 0, 2 of the second
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (__lane_id() & 16) ? r[0] : r[1];
    } else {
        // swap of the upper half of the first operand with the lower half of the second
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (__lane_id() & 32) ? r[0] : r[1];
    }
}

// Value of `v` held by lane (lane ^ MASK) through xor32 (VALU lane moves;
// shfl_xor below goes through the LDS crossbar and keeps fewer registers
// live, which the kernels held to a fixed occupancy rely on).
template <int MASK, typename T>
__device__ __forceinline__ T shfl_xor_valu(T v)
{
    static_assert(MASK > 0 && MASK < 64 && (MASK & (MASK - 1)) == 0, "xor mask");
    return per_dword(v, v, [](uint32_t, uint32_t x) { return xor32<MASK>(x); });
}

// Value of `v` held by lane (lane ^ MASK), MASK a power of two below 64.
template <int MASK, typename T>
__device__ __forceinline__ T shfl_xor(T v)
{
    static_assert(MASK > 0 && MASK < 64 && (MASK & (MASK - 1)) == 0, "xor mask");
    if constexpr (MASK < 32) {
        return swz<0x1F | (MASK << 10)>(v);
    } else {
        const int addr = (int)((__lane_id() ^ 32u) << 2);
        if constexpr (sizeof(T) == 8) {
            uint64_t b = __builtin_bit_cast(uint64_t, v);
            uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)b);
            uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)(b >> 32));
            return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
        } else {
            return __builtin_bit_cast(
                T, (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)__builtin_bit_cast(uint32_t, v)));
        }
    }
}

// Value of `v` held by lane (lane - 1); lane 0 receives lane 63's value.
template <typename T>
__device__ __forceinline__ T shfl_up1(T v)
{
    const int addr = (int)(((__lane_id() - 1u) & 63u) << 2);
    if constexpr (sizeof(T) == 8) {
        uint64_t b = __builtin_bit_cast(uint64_t, v);
        uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)b);
        uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)(b >> 32));
        return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
    } else {
        return __builtin_bit_cast(
            T, (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)__builtin_bit_cast(uint32_t, v)));
    }
}

// Value of `v` held by lane `src` (0 .. 63), through the LDS crossbar.
template <typename T>
__device__ __forceinline__ T shfl_idx(T v, int src)
{
    const int addr = (int)(((uint32_t)src & 63u) << 2);
    if constexpr (sizeof(T) == 8) {
        uint64_t b = __builtin_bit_cast(uint64_t, v);
        uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)b);
        uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)(b >> 32));
        return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
    } else {
        return __builtin_bit_cast(
            T, (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)__builtin_bit_cast(uint32_t, v)));
    }
}

// Value of `v` held by the last lane of the lower half of this lane's aligned
// group of 2*H lanes: lane ((lane & ~(2H-1)) | (H-1)).  H in {1,...,32}.
template <int H, typename T>
__device__ __forceinline__ T from_lower_half_end(T v)
{
    static_assert(H >= 1 && H <= 32 && (H & (H - 1)) == 0, "half size");
    if constexpr (H < 32) {
        constexpr int AND = 0x1F & ~(2 * H - 1);
        constexpr int OR = H - 1;
        return swz<AND | (OR << 5)>(v);
    } else {
        return readlane(v, 31);
    }
}

// ----------------------------------------------- published 64-bit words
// Values published between workgroups of one kernel are single 64-bit words,
// stored and polled with agent-scope relaxed atomics: the word itself says
// whether it is ready, so no ordering with other memory is needed.
//   f64: the value's bits; "not ready" is a signalling-NaN pattern that no
//        addition can produce (published values are canonicalised first).
//   f32: the value's bits in the low half and 1 in the high half; "not
//        ready" is 0.
constexpr uint64_t kNotReady64 = 0x7FF4DEADBEEF0001ull;
constexpr uint64_t kNotReady32 = 0ull;
constexpr uint32_t kErrSpin = 1u;
constexpr long kSpinLimit = 1l << 20;

template <typename T> __device__ __forceinline__ uint64_t not_ready_word()
{
    return sizeof(T) == 8 ? kNotReady64 : kNotReady32;
}

__device__ __forceinline__ uint64_t pack_word(double v)
{
    return __builtin_bit_cast(uint64_t, __builtin_canonicalize(v));
}
__device__ __forceinline__ uint64_t pack_word(float v)
{
    return (1ull << 32) | (uint64_t)__builtin_bit_cast(uint32_t, v);
}
template <typename B, class Op>
__device__ __forceinline__ uint64_t pack_word(OpVal<B, Op> v)
{
    return pack_word(v.v);
}
// The value of a ready word (double / float, or their OpVal wrappers).
template <typename T> __device__ __forceinline__ T unpack_word(uint64_t w)
{
    if constexpr (sizeof(T) == 8)
        return __builtin_bit_cast(T, w);
    else
        return __builtin_bit_cast(T, (uint32_t)w);
}

template <typename T>
__device__ __forceinline__ void publish(uint64_t* slot, T v)
{
    __hip_atomic_store(slot, pack_word(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The words of values v[0 .. N) published to slot[0 .. N) (16-byte aligned,
// N even) two at a time, each pair in one 16-byte store with the coherence of
// a relaxed agent-scope atomic store (sc1: written through this XCD's L2 to
// memory).  One store per pair, where a store per word would leave every
// written line half-filled twice: the lanes of a wave then write whole lines.
// An aligned 16-byte store never splits an 8-byte word, so a reader's 64-bit
// load sees a word either not ready or whole.  A store of more than 8 bytes
// must be followed by two wait states before a VALU instruction may write
// its data registers (the compiler inserts them after its own stores, not
// after one written in asm): the s_nop 1 in the same asm block.
template <int N, typename T>
__device__ __forceinline__ void publish_pairs(uint64_t* slot, const T (&v)[N])
{
    static_assert(N % 2 == 0, "pairs of words");
    using u32x4 = unsigned int __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < N; i += 2) {
        const uint64_t a = pack_word(v[i]), b = pack_word(v[i + 1]);
        const u32x4 d = {(unsigned)a, (unsigned)(a >> 32), (unsigned)b, (unsigned)(b >> 32)};
        asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1"
                     :
                     : "v"(slot + i), "v"(d)
                     : "memory");
    }
}

// Words slot[q][0 .. N) (each 16-byte aligned, N even) read two at a time,
// each pair in one 16-byte load with the coherence of a relaxed agent-scope
// atomic load (sc1: from memory, not this XCD's L2): the counterpart of
// publish_pairs, so that the lanes of a wave read each line once.  Every load
// is issued, then one wait for all of them; each result register is then
// passed through an empty asm, so that nothing uses (or reuses) it before the
// wait.  The loads are as ordered as the atomic loads they replace: relaxed.
template <int Q, int N>
__device__ __forceinline__ void load_pairs(const uint64_t* const (&slot)[Q], uint64_t (&w)[Q][N])
{
    static_assert(N % 2 == 0, "pairs of words");
    using u32x4 = unsigned int __attribute__((ext_vector_type(4)));
    u32x4 d[Q][N / 2];
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int i = 0; i < N / 2; ++i)
            asm volatile("global_load_dwordx4 %0, %1, off sc1"
                         : "=&v"(d[q][i])
                         : "v"(slot[q] + 2 * i)
                         : "memory");
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            asm volatile("" : "+v"(d[q][i]));
            w[q][2 * i] = ((uint64_t)d[q][i][1] << 32) | d[q][i][0];
            w[q][2 * i + 1] = ((uint64_t)d[q][i][3] << 32) | d[q][i][2];
        }
}

// The bound of a wait: header word 2 of the workspace whose error word is
// `err` (its first 32 bits), written by the call's init kernel (0: the
// default, kSpinLimit).
__device__ __forceinline__ long spin_limit_of(const uint32_t* err)
{
    const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(err) + 2,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return v ? (long)v : kSpinLimit;
}

// Poll a published word until it is ready.  The wait is bounded: after the
// call's bound (spin_limit_of(err), at least 64 polls), or as soon as another
// wave has recorded an error, the kernel's error word gets kErrSpin and -0.0
// is returned, so that every wave still runs to completion and the host can
// report the failure.  Both are checked every 64 polls only: the header words
// share a cache line with the ticket counter, and loads of that line by every
// short wait slowed the tickets of the whole grid.
template <typename T>
__device__ __forceinline__ T wait_word(uint64_t* slot, uint32_t* err)
{
    const uint64_t nr = not_ready_word<T>();
    uint64_t w = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    long it = 0, limit = kSpinLimit;
    while (w == nr) {
        ++it;
        if ((it & 63) == 0) {
            if (it == 64) limit = spin_limit_of(err);
            if (it > limit ||
                __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
                __hip_atomic_fetch_or(err, kErrSpin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return neg_zero<T>();
            }
        }
        __builtin_amdgcn_s_sleep(2);
        w = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return unpack_word<T>(w);
}

// The value of a word read earlier, or, when it was not ready then, the
// value once it is (wait_word).
template <typename T>
__device__ __forceinline__ T ready_or_wait(uint64_t w, uint64_t* slot, uint32_t* err)
{
    return w != not_ready_word<T>() ? unpack_word<T>(w) : wait_word<T>(slot, err);
}

// Binary-counter ("shift-reduce") stack of complete pairwise subtrees, one
// entry per level, each entry a small vector of W values.  push(k, v) adds the
// k-th (0-based) subtree of equal size; after n pushes, collapse(n) returns
// the right-to-left combination s_top + ... (s_1 + s_0), i.e. the pairwise
// value over all pushed items.  k and n are uniform across the wave, so every
// branch is scalar and every register index static.
template <typename T, int W, int D>
struct TreeStack {
    T s[D + 1][W];

    __device__ __forceinline__ void push(uint64_t k, T (&v)[W])
    {
        // merges = number of trailing one bits of k; the merged subtree then
        // lands at level `merges`.  Static indices only (no break), so the
        // stack stays in registers.
        const int merges = __builtin_ctzll(~k);
#pragma unroll
        for (int l = 0; l < D; ++l) {
            if (l < merges) {
#pragma unroll
                for (int i = 0; i < W; ++i) v[i] = s[l][i] + v[i];
            }
        }
#pragma unroll
        for (int l = 0; l <= D; ++l) {
            const bool here = (l == merges);
#pragma unroll
            for (int i = 0; i < W; ++i) s[l][i] = here ? v[i] : s[l][i];
        }
    }

    // n pushes; returns -0.0 ("absent") when n == 0.  Requires n <= 2^D.
    __device__ __forceinline__ void collapse(uint64_t n, T (&out)[W]) const
    {
#pragma unroll
        for (int i = 0; i < W; ++i) out[i] = neg_zero<T>();
#pragma unroll
        for (int l = 0; l <= D; ++l) {
            if ((n >> l) & 1) {
#pragma unroll
                for (int i = 0; i < W; ++i) out[i] = s[l][i] + out[i];
            }
        }
    }
};

}  // namespace canon
