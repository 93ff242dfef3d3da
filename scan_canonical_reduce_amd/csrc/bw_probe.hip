// Streaming bandwidth probes for the benchmark (not part of libcanon's ABI):
// the practical HBM read and copy ceilings of the part, i.e. what a kernel
// that only moves the bytes reaches.  Workgroups of 256 threads take tiles
// of V 16-byte vectors per thread (every wave instruction 1 KiB contiguous,
// non-temporal loads and stores), either one tile per workgroup ("one-shot",
// grid = tiles) or a fixed grid striding over the tiles.  Dynamic LDS that
// the kernels never touch (allocated at launch all the same) caps the
// workgroups per CU (160 KiB / shmem).
// Measured on MI355X: copies peak with small one-shot tiles and few
// workgroups per CU (8 KiB tiles, 4 per CU: about 32 KiB in flight per CU);
// reads with a grid of 2 workgroups per CU.  The benchmark times a few such
// variants and reports the best of each kind.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Reads nvec 16-byte vectors; a workgroup whose data XOR to `magic` writes
// it to sink[blockIdx.x] (never in practice: the store keeps the loads).
template <int V>
__global__ __launch_bounds__(kThreads) void k_probe_read(const u32x4* __restrict__ x,
                                                         uint64_t nvec, uint64_t ntiles,
                                                         uint32_t magic,
                                                         uint32_t* __restrict__ sink)
{
    uint32_t acc = 0;
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint64_t base = t * ((uint64_t)kThreads * V) + threadIdx.x;
        u32x4 v[V];
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const uint64_t i = base + (uint64_t)u * kThreads;
            v[u] = i < nvec ? __builtin_nontemporal_load(x + i) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < V; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == magic) sink[blockIdx.x] = acc;
}

template <int V>
__global__ __launch_bounds__(kThreads) void k_probe_copy(const u32x4* __restrict__ x,
                                                         u32x4* __restrict__ y, uint64_t nvec,
                                                         uint64_t ntiles)
{
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint64_t base = t * ((uint64_t)kThreads * V) + threadIdx.x;
        u32x4 v[V];
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const uint64_t i = base + (uint64_t)u * kThreads;
            if (i < nvec) v[u] = __builtin_nontemporal_load(x + i);
        }
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const uint64_t i = base + (uint64_t)u * kThreads;
            if (i < nvec) __builtin_nontemporal_store(v[u], y + i);
        }
    }
}

uint64_t ntiles_of(uint64_t nvec, int v) { return (nvec + (uint64_t)kThreads * v - 1) / ((uint64_t)kThreads * v); }

unsigned grid_of(uint64_t ntiles, unsigned grid)
{
    return (grid == 0 || grid > ntiles) ? (unsigned)ntiles : grid;
}

template <int V>
int read_v(const void* x, uint64_t nvec, unsigned grid, unsigned shmem, void* sink, void* stream)
{
    const uint64_t nt = ntiles_of(nvec, V);
    hipLaunchKernelGGL((k_probe_read<V>), dim3(grid_of(nt, grid)), dim3(kThreads), shmem,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(x), nvec, nt,
                       0x9E3779B9u, static_cast<uint32_t*>(sink));
    return (int)hipGetLastError();
}

template <int V>
int copy_v(const void* x, void* y, uint64_t nvec, unsigned grid, unsigned shmem, void* stream)
{
    const uint64_t nt = ntiles_of(nvec, V);
    hipLaunchKernelGGL((k_probe_copy<V>), dim3(grid_of(nt, grid)), dim3(kThreads), shmem,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(x),
                       static_cast<u32x4*>(y), nvec, nt);
    return (int)hipGetLastError();
}

}  // namespace

// Streaming read of `bytes` (a multiple of 16) from the 16-byte aligned
// device buffer x: `vecs` vectors per thread and tile (1, 2, 4, 8 or 16),
// `grid` workgroups (0: one per tile), `shmem` bytes of unused dynamic LDS
// per workgroup (0 .. 65536).  sink: one 32-bit word per workgroup.
// Enqueued on `stream`; returns the HIP error code (-1: bad vecs).
extern "C" int canon_probe_read(const void* x, size_t bytes, int vecs, unsigned grid,
                                unsigned shmem, void* sink, void* stream)
{
    const uint64_t nvec = bytes / 16;
    if (nvec == 0) return 0;
    switch (vecs) {
        case 1: return read_v<1>(x, nvec, grid, shmem, sink, stream);
        case 2: return read_v<2>(x, nvec, grid, shmem, sink, stream);
        case 4: return read_v<4>(x, nvec, grid, shmem, sink, stream);
        case 8: return read_v<8>(x, nvec, grid, shmem, sink, stream);
        case 16: return read_v<16>(x, nvec, grid, shmem, sink, stream);
        default: return -1;
    }
}

// Streaming copy of `bytes` from x to y (both 16-byte aligned, not
// overlapping); arguments as canon_probe_read.
extern "C" int canon_probe_copy(const void* x, void* y, size_t bytes, int vecs, unsigned grid,
                                unsigned shmem, void* stream)
{
    const uint64_t nvec = bytes / 16;
    if (nvec == 0) return 0;
    switch (vecs) {
        case 1: return copy_v<1>(x, y, nvec, grid, shmem, stream);
        case 2: return copy_v<2>(x, y, nvec, grid, shmem, stream);
        case 4: return copy_v<4>(x, y, nvec, grid, shmem, stream);
        case 8: return copy_v<8>(x, y, nvec, grid, shmem, stream);
        case 16: return copy_v<16>(x, y, nvec, grid, shmem, stream);
        default: return -1;
    }
}
