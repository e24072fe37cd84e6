// store.hip -- slot-mapping scatter of new tokens' K/V into the paged pools.
//
// Each new token's K and V are appended to the cache at the slot the block
// manager assigned (Nano-vLLM engine deep-dive, §2.1: each step appends the
// new token's K/V to the cache; §2.2: the cache is addressed per block and
// per slot; Nano-vLLM Part 2, §05.3: a kernel writes the new K/V into the
// cache).  A pure bit copy, bound by HBM bandwidth.
//
// One thread moves one 16-byte chunk (8 bf16) of K and the matching chunk of
// V.  Source rows [token][kv_head][head_dim] and destination rows
// [block][kv_head][offset][head_dim] are both contiguous in head_dim, so a
// wavefront reads and writes whole 128/256-byte rows.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

__global__ __launch_bounds__(256) void store_kernel(const uint4 *__restrict__ k,
                                                    const uint4 *__restrict__ v,
                                                    const int32_t *__restrict__ slots,
                                                    int32_t num_tokens, uint4 *__restrict__ kc,
                                                    uint4 *__restrict__ vc, int32_t num_blocks,
                                                    int32_t num_kv_heads, int32_t chunks) {
    // total < 2^31 is checked on the host, so the index arithmetic stays 32-bit.
    const int32_t per_token = num_kv_heads * chunks;
    const int32_t total = num_tokens * per_token;
    const int32_t stride = gridDim.x * blockDim.x;
    for (int32_t idx = blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
        const int32_t t = idx / per_token;
        const int32_t rem = idx - t * per_token;
        // The data loads do not depend on the slot, so all three are issued
        // together and a decode-sized store costs one memory round trip, not
        // two.  The empty asm on the skip path uses the data there too, which
        // keeps the compiler from sinking the loads below the slot test.
        const uint4 kk = k[idx];
        const uint4 vv = v[idx];
        const int32_t slot = slots[t];
        const int32_t block = slot / kBlockTokens;
        // slot < 0 is a padding token; a block past the pool is never written
        if (slot < 0 || block >= num_blocks) {
            PKV_DEBUG_CHECK(slot >= 0 && rem == 0, kDbgSlot, slot, t);
            asm volatile("" ::"v"(kk.x), "v"(kk.y), "v"(kk.z), "v"(kk.w), "v"(vv.x), "v"(vv.y),
                         "v"(vv.z), "v"(vv.w));
            continue;
        }
        const int32_t offset = slot % kBlockTokens;
        const int32_t h = rem / chunks;
        const int32_t c = rem - h * chunks;
        const int64_t dst =
            (((int64_t)block * num_kv_heads + h) * kBlockTokens + offset) * chunks + c;
        kc[dst] = kk;
        vc[dst] = vv;
    }
}

// ---- FP8 cache: OCP E4M3 codes with one fp32 scale per (token, KV head),
// quantized by quantize8 (pkv_device.h) ----

template <int D>
__global__ __launch_bounds__(256) void store_fp8_kernel(
    const uint4 *__restrict__ k, const uint4 *__restrict__ v, const int32_t *__restrict__ slots,
    int32_t num_tokens, uint2 *__restrict__ kc, uint2 *__restrict__ vc, float *__restrict__ ks,
    float *__restrict__ vs, int32_t num_blocks, int32_t num_kv_heads) {
    constexpr int LPR = D / 8;  // lanes per (token, head) row
    const int32_t rows = num_tokens * num_kv_heads;
    const int32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
    const int32_t row = gid / LPR;
    const int c = threadIdx.x % LPR;
    const bool in_range = row < rows;  // no early exit: the whole group shuffles
    const int32_t r = in_range ? row : 0;
    const int32_t t = r / num_kv_heads, h = r % num_kv_heads;
    const uint4 kk = k[(size_t)r * LPR + c];
    const uint4 vv = v[(size_t)r * LPR + c];
    const int32_t slot = slots[t];
    float ksc, vsc;
    const uint2 kq = quantize8<LPR>(kk, ksc);
    const uint2 vq = quantize8<LPR>(vv, vsc);
    // slot < 0 is a padding token; a block past the pool is never written
    PKV_DEBUG_CHECK(in_range && slot >= 0 && slot / kBlockTokens >= num_blocks && h == 0 && c == 0,
                    kDbgSlot, slot, t);
    if (!in_range || slot < 0 || slot / kBlockTokens >= num_blocks) return;
    const size_t dst_row = ((size_t)(slot / kBlockTokens) * num_kv_heads + h) * kBlockTokens +
                           slot % kBlockTokens;
    kc[dst_row * LPR + c] = kq;
    vc[dst_row * LPR + c] = vq;
    if (c == 0) {
        ks[dst_row] = ksc;
        vs[dst_row] = vsc;
    }
}

hipError_t launch_store_fp8(const StoreFp8Args &a, hipStream_t stream) {
    if (a.num_tokens == 0) return hipSuccess;
    const int64_t threads_total = (int64_t)a.num_tokens * a.num_kv_heads * (a.head_dim / 8);
    const int threads = 256;
    const unsigned blocks = (unsigned)((threads_total + threads - 1) / threads);
    if (a.head_dim == 64)
        hipLaunchKernelGGL(store_fp8_kernel<64>, dim3(blocks), dim3(threads), 0, stream,
                           (const uint4 *)a.k, (const uint4 *)a.v, a.slots, a.num_tokens,
                           (uint2 *)a.k_cache, (uint2 *)a.v_cache, a.k_scale, a.v_scale,
                           a.num_blocks, a.num_kv_heads);
    else
        hipLaunchKernelGGL(store_fp8_kernel<128>, dim3(blocks), dim3(threads), 0, stream,
                           (const uint4 *)a.k, (const uint4 *)a.v, a.slots, a.num_tokens,
                           (uint2 *)a.k_cache, (uint2 *)a.v_cache, a.k_scale, a.v_scale,
                           a.num_blocks, a.num_kv_heads);
    return hipGetLastError();
}

PKV_DEBUG_WORD_ACCESS(store)

hipError_t launch_store(const StoreArgs &a, hipStream_t stream) {
    if (a.num_tokens == 0) return hipSuccess;
    const int chunks = a.head_dim / 8;
    const int64_t total = (int64_t)a.num_tokens * a.num_kv_heads * chunks;
    const int threads = 256;
    int64_t blocks = (total + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
    hipLaunchKernelGGL(store_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const uint4 *)a.k, (const uint4 *)a.v, a.slots, a.num_tokens,
                       (uint4 *)a.k_cache, (uint4 *)a.v_cache, a.num_blocks, a.num_kv_heads,
                       chunks);
    return hipGetLastError();
}

}  // namespace pkv
