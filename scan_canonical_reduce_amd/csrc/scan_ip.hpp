// Planning for the iterated_pairwise<L> scan (host and device shared).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace canon {

constexpr int kIpThreads = 256;
constexpr int kIpMaxRLog = 6;         // LDS path: at most 64 rows per tile
constexpr int kIpNoFast = -100;       // IpLayout::fast_logrv of the LDS path
constexpr int kIpLevelsPerPass = 4;   // node levels built per launch
constexpr int kIpMaxLevels = 48;
constexpr uint64_t kIpMaxGrid = 0x7FFFFFFFull;  // one workgroup per item
constexpr uint32_t kIpMaxL = 65536;   // largest lane count of the scan
// Lane counts above kIpWholeRowMaxL keep only chunks of 2^kIpChunkLog lanes'
// trees in LDS; the trees above the chunks live in the workspace.
constexpr uint32_t kIpWholeRowMaxL = 2048;
constexpr int kIpChunkLog = 9;

// Geometry of an iterated_pairwise scan over nseg independent segments of
// `cols` elements (one segment for a plain scan, one per row for the row
// scan), and the layout of the node arrays in the workspace (in elements):
// level k holds, per segment, cnt[k] nodes of L values: the complete
// pairwise trees, lane by lane, over tiles [u 2^k, (u+1) 2^k).
// Chunked geometry (Lp > kIpWholeRowMaxL): the lanes of a row form
// nchunks = Lp / C chunks of C = 2^chunk_log lanes; after the nodes, the
// workspace holds per segment and row the tree over that row's chunk totals
// (2 nchunks values: level 0, the chunk totals, at [0, nchunks), level l at
// 2 nchunks - (2 nchunks >> l)).
struct IpLayout {
    uint32_t L;
    int lp_log;     // Lp = 2^lp_log >= L
    int r_log;      // R = 2^r_log rows of L lanes per tile
    int chunk_log;  // lanes per chunk (== lp_log: the whole row is one chunk)
    uint64_t nseg;
    uint64_t rows;  // rows of L per segment
    uint64_t tps;   // tiles per segment
    int levels;     // node levels with at least one node
    uint64_t cnt[kIpMaxLevels];
    uint64_t off[kIpMaxLevels];
    uint64_t cl_off;  // chunked: offset of the chunk trees (elements)
    uint64_t total;   // elements of node (and chunk tree) storage
    int fast_logrv;   // register path with L = E * 2^(6 + fast_logrv), -6 .. 3; else kIpNoFast
};

// LDS budget (elements) for the per-row trees of one tile: (R + 1) * 2 * Lp
inline uint64_t ip_lds_elems(size_t elem_size) { return elem_size == 8 ? 8192 : 16384; }

// `aligned`: rows start on 16-byte boundaries (x, y and both pitches).
inline IpLayout make_ip_layout(uint64_t nseg, uint64_t cols, uint32_t L, size_t elem_size,
                               bool aligned)
{
    IpLayout lay{};
    lay.L = L;
    int lp = 0;
    while ((1ull << lp) < L) ++lp;
    lay.lp_log = lp;
    const uint64_t Lp = 1ull << lp;
    const int loge = elem_size == 8 ? 1 : 2;
    lay.fast_logrv = kIpNoFast;
    lay.chunk_log = lp;
    int rl;
    if (aligned && Lp == L && lp >= loge && lp <= loge + 9) {
        lay.fast_logrv = lp - loge - 6;
        rl = 6 - lay.fast_logrv;  // 4096 E / L rows per tile
    } else {
        if (Lp > kIpWholeRowMaxL) lay.chunk_log = kIpChunkLog;
        const uint64_t Lc = 1ull << lay.chunk_log;
        rl = kIpMaxRLog;
        while (rl > 0 && ((1ull << rl) + 1) * 2 * Lc > ip_lds_elems(elem_size)) --rl;
    }
    lay.r_log = rl;
    lay.nseg = nseg;
    const uint64_t rows = (cols + L - 1) / L;
    lay.rows = rows;
    lay.tps = (rows + (1ull << rl) - 1) >> rl;
    uint64_t off = 0;
    lay.levels = 0;
    for (int k = 0; k < kIpMaxLevels; ++k) {
        lay.cnt[k] = k == 0 ? lay.tps : (lay.tps >> k);
        lay.off[k] = off;
        if (lay.cnt[k] > 0) lay.levels = k + 1;
        off += nseg * lay.cnt[k] * L;
    }
    lay.cl_off = off;
    if (lay.chunk_log < lay.lp_log) off += nseg * rows * 2 * (Lp >> lay.chunk_log);
    lay.total = off;
    return lay;
}

// Workspace of the single-pass iterated_pairwise scan (fast geometry, any
// segment count), in 64-bit words from the workspace start:
//   word 0: error word (low 32 bits); word 1: ticket counter (low 32 bits);
//   [woff[k], +nseg * cnt[k] * L): node level k, one published word per lane
//     (node (k, u) of segment s at woff[k] + (s * cnt[k] + u) * L, its words
//     in pairs of adjacent columns: IpFast::wcol);
//   [cbase, ...): 32-bit arrival counters, level k >= 1 at coff[k] (in
//     32-bit units from cbase): one per node, counting its finished children.
struct IpSingleLayout {
    IpLayout g;
    uint64_t woff[kIpMaxLevels];
    uint64_t coff[kIpMaxLevels];
    uint64_t cbase;
    uint64_t counters;
    uint64_t total_words;
};

inline IpSingleLayout make_ip_single_layout(const IpLayout& g)
{
    IpSingleLayout s{};
    s.g = g;
    uint64_t off = 32;  // 256 bytes of header
    uint64_t c = 0;
    for (int k = 0; k < kIpMaxLevels; ++k) {
        s.woff[k] = off;
        off += g.nseg * g.cnt[k] * g.L;
        s.coff[k] = c;
        if (k >= 1) c += g.nseg * g.cnt[k];
    }
    s.cbase = off;
    s.counters = c;
    s.total_words = off + (c + 1) / 2;
    return s;
}

inline size_t ip_lds_bytes(const IpLayout& lay, size_t elem_size)
{
    return (size_t)((1ull << lay.r_log) + 1) * 2 * (1ull << lay.chunk_log) * elem_size;
}

// out == null: the plain inclusive scan; else the scan with an initial
// value that *out describes (ScanOut, scan.hpp).
template <typename T>
struct ScanOut;

// PLAIN = false (both launchers): only the kernels with an output stage are
// built (out must not be null).  The single-pass launcher takes the layout
// of the register geometry whatever the alignment; `aligned` (rows on
// 16-byte boundaries: x, y and both pitches) selects 16-byte loads and
// stores, else element loads and stores.
template <typename T, bool PLAIN = true>
hipError_t launch_scan_ip_single(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t cols,
                                 uint64_t* ws, const IpSingleLayout& lay, const ScanOut<T>* out,
                                 bool aligned, hipStream_t s);

template <typename T, bool PLAIN = true>
hipError_t launch_scan_ip(const T* x, uint64_t ldx, T* y, uint64_t ldy, uint64_t nseg,
                          uint64_t cols, uint32_t* err, T* nodes, const IpLayout& lay,
                          const ScanOut<T>* out, hipStream_t s);

}  // namespace canon
