// Launch planning for the scan kernels (host and device shared constants).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace canon {

constexpr int kScanThreads = 256;  // 4 waves
constexpr int kScanWaves = kScanThreads / 64;
constexpr int kScanVec = 8;        // 16-byte vectors per thread per tile
constexpr int kGroupLog = 6;       // tile nodes up to this level are rebuilt from tile totals
constexpr int kMaxLevels = 48;

// Workspace layout of a single-pass scan (offsets in 64-bit words).
//   word 0: error word (low 32 bits); word 1: tile counter (low 32 bits)
//   [tiles_off, +ntiles): published tile totals (tile-level 0 nodes)
//   [level_off[k], +ceil(ntiles / 2^k)): published tile-level k nodes,
//       k >= kGroupLog
// Each published word holds one value (one lane value for the
// iterated_pairwise scan, whose nodes are vectors of L words).
struct ScanLayout {
    uint64_t ntiles;
    uint64_t width;  // words per node (1, or L for iterated_pairwise)
    uint64_t tiles_off;
    uint64_t level_off[kMaxLevels];
    uint64_t total_words;
};

inline ScanLayout make_scan_layout(uint64_t ntiles, uint64_t width)
{
    ScanLayout l{};
    l.ntiles = ntiles;
    l.width = width;
    l.tiles_off = 32;  // 256 bytes of header
    uint64_t off = l.tiles_off + ntiles * width;
    for (int k = 0; k < kMaxLevels; ++k) {
        l.level_off[k] = off;
        if (k >= kGroupLog) off += ((ntiles + (1ull << k) - 1) >> k) * width;
    }
    l.total_words = off;
    return l;
}

// log2 of the 16-byte vectors each thread of the single-pass scan holds:
// 256 bytes of the tile per thread for both types (measured best on MI355X:
// fewer bytes per tile leave more tiles, each with its look-back round trip;
// more cost occupancy)
template <typename T>
constexpr int scan_log_v()
{
    return 4;
}

// The same for the row-batched scan, whose tiles hold 128 bytes per thread
// in double (a 4096-element row is one tile).
template <typename T>
constexpr int scan_rows_log_v()
{
    return sizeof(T) == 8 ? 3 : 4;
}

template <typename T>
constexpr int scan_tile_log()
{
    return (sizeof(T) == 8 ? 1 : 2) + 6 + scan_log_v<T>() + 2;  // log2(E * 64 * V * waves)
}

// Output of a scan with an initial value.  S_i is the policy's value on
// x[0..i] and S_{-1} the empty prefix:
//   kScanInclusive       y[i] = init + S_i        (n outputs)
//   kScanExclusive       y[i] = init + S_{i-1}    (n outputs; y[0] = init)
//   kScanIncludeInitial  the same for i <= n      (n + 1 outputs)
enum ScanKind : int { kScanInclusive = 0, kScanExclusive = 1, kScanIncludeInitial = 2 };

template <typename T>
struct ScanOut {
    T init;
    int kind;
};

template <typename T>
hipError_t launch_scan(const T* x, T* y, uint64_t n, bool pairwise, int b_log, bool aligned,
                       uint64_t* ws, const ScanLayout& lay, hipStream_t s);

template <typename T>
hipError_t launch_scan_with_init(const T* x, T* y, uint64_t n, bool pairwise, int b_log,
                                 bool aligned, uint64_t* ws, const ScanLayout& lay,
                                 const ScanOut<T>& out, hipStream_t s);

template <typename T>
hipError_t launch_scan_order_free(const T* x, T* y, uint64_t n, bool aligned, uint64_t* ws,
                                  const ScanLayout& lay, const ScanOut<T>& out, hipStream_t s);

// y[r * ldy] = v for r < rows, on stream s.
template <typename T>
hipError_t launch_put_column(T* y, uint64_t ldy, uint64_t rows, T v, hipStream_t s);

// out == null: the plain inclusive scan of every row; else the scan with an
// initial value that *out describes.
// PLAIN = false: only the kernels with an output stage are built (out must
// not be null).  PW_ONLY: only the pairwise kernels are built.
template <typename T, bool PLAIN = true, bool PW_ONLY = false>
hipError_t launch_scan_rows(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t rows,
                            uint64_t cols, bool pairwise, int b_log, bool aligned,
                            const ScanOut<T>* out, hipStream_t s);


}  // namespace canon
