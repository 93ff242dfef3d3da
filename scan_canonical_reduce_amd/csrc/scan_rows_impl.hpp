// Canonical inclusive scan of many independent rows (gfx950): policies
// pairwise and block_dyadic<B> (canonical-reduce README, P4229R0 "Summary" /
// "Key Design Points").  The in-tile network is ScanTile (scan_tile.hpp).
#pragma once
#include "device.hpp"
#include "launch.hpp"
#include "scan.hpp"
#include "scan_tile.hpp"

namespace canon {

// Row-batched scan: one workgroup per row, the row's tiles in order; the tile
// nodes come from a binary-counter stack of the row's earlier tile totals
// (held in LDS by thread 0).  OUTX: scan with an initial value (init, kind),
// see ScanTile::emit.
template <typename T, int MODE, bool ALIGNED, int LOGV, bool OUTX>
__global__ __launch_bounds__(kScanThreads) void k_scan_rows(const T* x, uint64_t ldx, T* y,
                                                            uint64_t ldy, uint64_t rows,
                                                            uint64_t cols, int b_log, T init,
                                                            int kind)
{
    using ST = ScanTile<T, MODE, LOGV>;
    __shared__ T s_tot[kScanWaves];
    __shared__ T s_stack[kMaxLevels];
    __shared__ T s_wend[kScanWaves];
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
            st.begin(b_log, g0);
            st.in_wave(lane);
            if (lane == 63) s_tot[w] = st.last(ST::V - 1);
            __syncthreads();
            const T t0 = s_tot[0], t1 = s_tot[1], t2 = s_tot[2], t3 = s_tot[3];
            const T t01 = t0 + t1;
            const T tile_total = t01 + (t2 + t3);
            st.across_waves(w, t0, t01, t2);
            // OUTX: the value just before the tile, C + W, where W collects
            // the nodes of levels <= b (inside the open block) and C those
            // above b, each right-nested; C alone at a block end
            T pc = neg_zero<T>(), pw = neg_zero<T>();
            for (int k = 0; k < kMaxLevels && (t >> k) != 0; ++k)
                if ((t >> k) & 1) {
                    st.apply_all(ST::LOG_S + 1 + k, s_stack[k]);
                    if constexpr (OUTX) {
                        if (st.in_block(ST::LOG_S + 1 + k)) pw = s_stack[k] + pw;
                        else pc = s_stack[k] + pc;
                    }
                }
            // the stores' offset as a fresh copy: otherwise the compiler keeps
            // the address of every vector from its load to its store (f64
            // block_dyadic: 104 VGPRs and 4 waves per SIMD, against 90 and 5)
            const uint64_t gs = fresh_copy(g0);
            if constexpr (OUTX)
                st.template emit<ALIGNED>(yr, cols, gs, init, kind, pc + pw, s_wend, w, lane,
                                          [&](int u, T(&o)[ST::E]) { st.final_vec(u, o); });
            else
                st.template store<ALIGNED>(yr, cols, gs);
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
template <typename T, int MODE, bool ALIGNED, bool OUTX>
static hipError_t launch_scan_rows_k(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t rows,
                                     uint64_t cols, int b_log, const ScanOut<T>& out,
                                     hipStream_t s)
{
    constexpr auto kern = k_scan_rows<T, MODE, ALIGNED, scan_rows_log_v<T>(), OUTX>;
    // one workgroup per row (the kernel strides over rows past the grid limit)
    const uint64_t grid = capped_grid(rows < 0x7FFFFFFFull ? rows : 0x7FFFFFFFull);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kScanThreads), 0, s, x, ldx, y, ldy, rows,
                       cols, b_log, out.init, out.kind);
    return hipGetLastError();
}

template <typename T, int MODE, bool PLAIN>
static hipError_t launch_scan_rows_m(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t rows,
                                     uint64_t cols, int b_log, bool aligned, const ScanOut<T>* out,
                                     hipStream_t s)
{
    const ScanOut<T> o = out ? *out : ScanOut<T>{};
    if (!PLAIN && !out) return hipErrorInvalidValue;
    if (!PLAIN || out) {
        if (aligned)
            return launch_scan_rows_k<T, MODE, true, true>(x, ldx, y, ldy, rows, cols, b_log, o, s);
        return launch_scan_rows_k<T, MODE, false, true>(x, ldx, y, ldy, rows, cols, b_log, o, s);
    }
    if constexpr (PLAIN) {
        if (aligned)
            return launch_scan_rows_k<T, MODE, true, false>(x, ldx, y, ldy, rows, cols, b_log, o,
                                                            s);
        return launch_scan_rows_k<T, MODE, false, false>(x, ldx, y, ldy, rows, cols, b_log, o, s);
    }
    return hipErrorInvalidValue;
}

// Plain inclusive row scan when out is null, else the scan with an initial
// value that *out describes (cols == 0 then still writes init for
// include_initial, into every row).
template <typename T, bool PLAIN, bool PW_ONLY>
hipError_t launch_scan_rows(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t rows,
                            uint64_t cols, bool pairwise, int b_log, bool aligned,
                            const ScanOut<T>* out, hipStream_t s)
{
    if (rows == 0) return hipSuccess;
    if (cols == 0) {
        if (out && out->kind == kScanIncludeInitial) return launch_put_column(y, ldy, rows, out->init, s);
        return hipSuccess;
    }
    if (pairwise || b_log == 0)
        return launch_scan_rows_m<T, 0, PLAIN>(x, ldx, y, ldy, rows, cols, 0, aligned, out, s);
    if constexpr (PW_ONLY) {
        return hipErrorInvalidValue;
    } else {
        if constexpr (Elem<T>::LOGE >= 2) {
            if (b_log < Elem<T>::LOGE)
                return launch_scan_rows_m<T, 2, PLAIN>(x, ldx, y, ldy, rows, cols, b_log, aligned,
                                                       out, s);
        }
        return launch_scan_rows_m<T, 1, PLAIN>(x, ldx, y, ldy, rows, cols, b_log, aligned, out,
                                               s);
    }
}

}  // namespace canon
