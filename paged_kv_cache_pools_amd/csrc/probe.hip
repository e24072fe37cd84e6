// probe.hip -- a plain streaming read of a device buffer, the measured
// denominator beside the nominal 8 TB/s: what one kernel of 16-byte
// nontemporal loads reads per second from HBM on this GPU.  Not part of the
// attention path; bench.py times it over a buffer far larger than the caches.
//
// The access pattern is decode's: each wave reads whole 4 KiB tiles, one
// contiguous KiB per load instruction, all four loads in flight before any is
// used, and the tiles are dealt round-robin over the waves of the grid.
// Measured over 4 GiB on MI355X: 6.70-6.81 TB/s with 1024-4096 workgroups,
// against 5.9-6.0 TB/s for consecutive threads striding over the buffer in
// 16-byte chunks.  Each thread folds what it read into one word, written only
// when the word equals a fixed pattern (data-dependent, so the loads cannot be
// dropped, and in practice the probe writes nothing).
#include <hip/hip_runtime.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kTileLoads = 4;                // 16-byte loads per lane per tile
constexpr int kTileChunks = 64 * kTileLoads;  // 16-byte chunks per tile (4 KiB)
constexpr size_t kMaxProbeGrid = 4096;
constexpr uint32_t kProbePattern = 0x9E3779B9u;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4 *__restrict__ buf,
                                                                   size_t chunks,
                                                                   uint32_t *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const size_t wave = (size_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
    const size_t waves = (size_t)gridDim.x * (kProbeThreads / 64);
    const size_t tiles = chunks / kTileChunks;
    uint32_t acc = 0;
    for (size_t t = wave; t < tiles; t += waves) {
        const u32x4 *p = buf + t * kTileChunks + lane;
        u32x4 x[kTileLoads];
#pragma unroll
        for (int u = 0; u < kTileLoads; ++u) x[u] = __builtin_nontemporal_load(p + u * 64);
#pragma unroll
        for (int u = 0; u < kTileLoads; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    }
    // the chunks past the last whole tile
    for (size_t i = tiles * kTileChunks + wave * 64 + lane; i < chunks; i += waves * 64) acc ^= buf[i].x;
    if (acc == kProbePattern) sink[0] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
    const size_t chunks = bytes / 16;
    if (chunks == 0) return hipSuccess;
    // one tile per wave at most, kMaxProbeGrid workgroups at most
    size_t grid = (chunks + (size_t)kTileChunks * 4 - 1) / ((size_t)kTileChunks * 4);
    if (grid > kMaxProbeGrid) grid = kMaxProbeGrid;
    read_probe_kernel<<<dim3((unsigned)grid), kProbeThreads, 0, stream>>>(
        static_cast<const u32x4 *>(buf), chunks, sink);
    return hipGetLastError();
}

}  // namespace pkv
