// copy.hip -- whole-block copies between physical blocks of the pools, the
// device half of copy-on-write: when a sequence appends into a block it shares
// with another (after a fork), it moves to a fresh block that must first hold
// the shared block's contents ("Nano-vLLM engine deep-dive", section 2.2;
// "LLM basics primer" part 4, section 17.7).  One block id addresses every
// layer's K and V pools ("Nano-vLLM Part 2", section 05.2), so one logical copy
// moves the block in every pool passed.
//
// Geometry: a workgroup of 256 threads moves one chunk of one block of one
// pool, U 16-byte moves per thread with every load issued before the first
// store; grid.x runs over (pair, chunk), grid.y over the pools of this launch.
// Large copies use U = 4 (16 KiB chunks) with nontemporal loads and stores:
// measured on MI355X over 256 blocks x 64 pools of 32 KiB, 6.28 TB/s of
// read + write against 5.72 TB/s with ordinary accesses and 5.26 TB/s for a
// plain device-to-device hipMemcpy of the same bytes.  A launch of under 2048
// such workgroups (one fork's copy) uses U = 1 (4 KiB chunks) to spread the
// few kilobytes over more compute units.  Pool pointers travel by value in
// the kernel arguments, kMaxCopyPools per launch.
#include <hip/hip_runtime.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct PoolPtrs {
    unsigned char *p[kMaxCopyPools];
};

template <int U, bool NT>
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(PoolPtrs pools, size_t block_bytes,
                                                               int32_t num_blocks,
                                                               const int32_t *__restrict__ copies,
                                                               int32_t chunks_per_block) {
    const int pair = blockIdx.x / chunks_per_block;
    const int chunk = blockIdx.x % chunks_per_block;
    const int32_t src = copies[2 * pair];
    const int32_t dst = copies[2 * pair + 1];
    // uniform over the workgroup: an invalid pair copies nothing
    PKV_DEBUG_CHECK(((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks) &&
                        chunk == 0 && blockIdx.y == 0 && threadIdx.x == 0,
                    kDbgCopy, (unsigned)src >= (unsigned)num_blocks ? src : dst, pair);
    if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks || src == dst)
        return;
    unsigned char *pool = pools.p[blockIdx.y];
    const u32x4 *from = reinterpret_cast<const u32x4 *>(pool + (size_t)src * block_bytes);
    u32x4 *to = reinterpret_cast<u32x4 *>(pool + (size_t)dst * block_bytes);
    const size_t n16 = block_bytes / 16;
    const size_t base = (size_t)chunk * (kThreads * U) + threadIdx.x;
    u32x4 v[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const size_t e = base + (size_t)i * kThreads;
        if (e < n16) v[i] = NT ? __builtin_nontemporal_load(from + e) : from[e];
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const size_t e = base + (size_t)i * kThreads;
        if (e < n16) {
            if (NT)
                __builtin_nontemporal_store(v[i], to + e);
            else
                to[e] = v[i];
        }
    }
}

template <int U, bool NT>
hipError_t launch_pools(const CopyArgs &a, const PoolPtrs &ptrs, int32_t count) {
    const size_t chunk_bytes = (size_t)kThreads * U * 16;
    const size_t chunks = (a.block_bytes + chunk_bytes - 1) / chunk_bytes;
    dim3 grid((unsigned)(chunks * (size_t)a.num_copies), (unsigned)count);
    copy_blocks_kernel<U, NT><<<grid, kThreads, 0, a.stream>>>(ptrs, a.block_bytes, a.num_blocks,
                                                              a.copies, (int32_t)chunks);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_copy_blocks(const CopyArgs &a) {
    const size_t big_chunks = (a.block_bytes + 16383) / 16384;
    for (int32_t first = 0; first < a.num_pools; first += kMaxCopyPools) {
        const int32_t count = a.num_pools - first < kMaxCopyPools ? a.num_pools - first
                                                                   : kMaxCopyPools;
        PoolPtrs ptrs{};
        for (int32_t i = 0; i < count; ++i)
            ptrs.p[i] = static_cast<unsigned char *>(a.pools[first + i]);
        const bool small = big_chunks * (size_t)a.num_copies * (size_t)count < 2048;
        const hipError_t e = small ? launch_pools<1, false>(a, ptrs, count)
                                   : launch_pools<4, true>(a, ptrs, count);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

PKV_DEBUG_WORD_ACCESS(copy)

}  // namespace pkv
