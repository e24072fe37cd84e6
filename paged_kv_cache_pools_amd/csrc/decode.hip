// decode.hip -- the decode kernels (gfx950): split-KV partitions plus a merge
// pass, and the single-pass kernel that merges its waves in LDS.  The
// attention itself -- scaled dot-product attention of one query token per
// sequence over its paged K/V cache, grouped-query heads sharing a KV head --
// is in decode_wave.h.
#include <algorithm>
#include <mutex>

#include "decode_fp8_mfma.h"

namespace pkv {

// Library-owned scratch for the entry point that allocates nothing
// (pkv_decode_attn_noalloc): the split-KV partials live here instead of in a
// caller's workspace.  Every GPU the library runs on holds its own copy of
// this array until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): it
// passes the device address noalloc_scratch() looks up.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

PKV_DEBUG_WORD_ACCESS(decode)

hipError_t noalloc_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {  // once per device, with that device current
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// The fused store's new token in the cache's own format: bf16 rows, or FP8
// codes plus their scales (k_store / v_store are the code pools then, and
// ks_store / vs_store the scale arrays).
template <int D, bool FP8>
__device__ __forceinline__ NewToken make_new_token(const uint16_t *k_new, const uint16_t *v_new,
                                                   const int32_t *slots, void *k_store,
                                                   void *v_store, float *ks_store, float *vs_store,
                                                   const int32_t *bt_row, int32_t num_blocks,
                                                   int32_t num_kv_heads, int s, int kvh, int ctx) {
    if constexpr (FP8)
        return new_token_fp8<D>(k_new, v_new, slots, (uint8_t *)k_store, (uint8_t *)v_store,
                                ks_store, vs_store, bt_row, num_blocks, num_kv_heads, s, kvh, ctx);
    else
        return new_token<D>(k_new, v_new, slots, (uint16_t *)k_store, (uint16_t *)v_store, bt_row,
                            num_blocks, num_kv_heads, s, kvh, ctx);
}

// Split-KV decode: one wavefront per (sequence, KV head, partition of
// partition_tokens tokens).  A sequence that fits one partition is written
// directly; otherwise each partition writes (m, l, acc) for the merge pass.
//
// The grid is one-dimensional with the KV head innermost, then the sequence,
// then the group of partitions one workgroup holds.  Workgroups are dealt to
// the 8 XCDs round-robin by linear id, so every XCD receives the same mix of
// sequences and partition groups; with the partition group innermost instead,
// an XCD would receive one partition group only -- all of the work for group
// 0, hardly any for the late groups that only long contexts reach (measured:
// a batch of 256 short contexts ran 2.1x slower that way).
template <int D, int G, bool FP8>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const uint16_t *__restrict__ q, const void *k_cache, const void *v_cache,
    const float *k_scale, const float *v_scale, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t num_blocks, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t partition_tokens, int32_t max_parts, float scale_log2, uint16_t *__restrict__ out,
    float *__restrict__ ws_out,
    float *__restrict__ ws_ml, const uint16_t *__restrict__ k_new,
    const uint16_t *__restrict__ v_new, const int32_t *__restrict__ slots, void *k_store,
    void *v_store, float *ks_store, float *vs_store, const float *__restrict__ rope_table,
    int32_t rope_positions) {
    constexpr int LPR = D / 8, TPL = 64 / LPR;
    const int lane = threadIdx.x & 63;
    int kvh = blockIdx.x % num_kv_heads;
    int s = (blockIdx.x / num_kv_heads) % num_seqs;
    const int part = (blockIdx.x / (num_kv_heads * num_seqs)) * (blockDim.x >> 6) + wave_id_uniform();
    if constexpr (FP8)  // within each group of partitions
        pair_kv_heads(blockIdx.x % (num_kv_heads * num_seqs), num_kv_heads * num_seqs,
                      num_kv_heads, s, kvh);
    const int row = lane / LPR;
    const int c = lane % LPR;
    const int h0 = kvh * G;

    const int ctx = clamp_context(context_lens[s], max_context_len, max_blocks_per_seq,
                                  kvh == 0 && part == 0 && lane == 0, s);
    const int32_t *bt_row = block_tables + (size_t)s * max_blocks_per_seq;
    if (ctx <= 0) {
        if (part == 0) {
            write_zero_rows<D, G>(out, num_q_heads, s, kvh);
            store_only<D>(make_new_token<D, FP8>(k_new, v_new, slots, k_store, v_store, ks_store,
                                                 vs_store, bt_row, num_blocks, num_kv_heads, s,
                                                 kvh, ctx),
                          rope_at<D>(rope_table, rope_positions, ctx));
        }
        return;
    }
    const int t_begin = part * partition_tokens;
    if (t_begin >= ctx) return;
    const int t_end = min(t_begin + partition_tokens, ctx);
    const int nparts = (ctx + partition_tokens - 1) / partition_tokens;
    // the partition holding the last position carries the fused store
    NewToken nt;
    if (t_end == ctx)
        nt = make_new_token<D, FP8>(k_new, v_new, slots, k_store, v_store, ks_store, vs_store,
                                    bt_row, num_blocks, num_kv_heads, s, kvh, ctx);

    if constexpr (FP8) {
        if (ctx > kExactDecodeKeys) {  // uniform: the matrix-core path
            extern __shared__ float smem[];  // [waves] rings of Fp8Mma<D>::WAVE_BYTES
            using Mma = Fp8Mma<D>;
            unsigned char *ring =
                reinterpret_cast<unsigned char *>(smem) + wave_id_uniform() * Mma::WAVE_BYTES;
            f32x4_t o[Mma::MT];
            float mr, lr;
            wave_attend_fp8_mfma<D, G>(q + (size_t)s * num_q_heads * D,
                                       static_cast<const uint8_t *>(k_cache),
                                       static_cast<const uint8_t *>(v_cache), k_scale, v_scale,
                                       bt_row, num_blocks, num_q_heads, num_kv_heads, scale_log2,
                                       kvh, t_begin, t_end, nt, ring, o, mr, lr);
            const int col = lane & 15, grp = lane >> 4;  // head, dimensions 16m + 4grp ..
            if (col < G) {
                const size_t hrow = (size_t)s * num_q_heads + h0 + col;
                if (nparts == 1) {
                    const float inv = 1.f / lr;
                    uint16_t *dst = out + hrow * D + 4 * grp;
#pragma unroll
                    for (int m = 0; m < Mma::MT; ++m)
                        *reinterpret_cast<uint2 *>(dst + 16 * m) =
                            make_uint2(pack_bf16x2(o[m][0] * inv, o[m][1] * inv),
                                       pack_bf16x2(o[m][2] * inv, o[m][3] * inv));
                } else {
                    const size_t r = hrow * max_parts + part;
#pragma unroll
                    for (int m = 0; m < Mma::MT; ++m)
                        *reinterpret_cast<float4 *>(ws_out + r * D + 16 * m + 4 * grp) =
                            make_float4(o[m][0], o[m][1], o[m][2], o[m][3]);
                    if (grp == 0) {
                        ws_ml[r * 2 + 0] = mr;
                        ws_ml[r * 2 + 1] = lr;
                    }
                }
            }
            return;
        }
    }
    float acc[G][8], mg[G], lg[G];
    wave_attend<D, G, FP8>(q, k_cache, v_cache, k_scale, v_scale, bt_row, num_blocks, num_q_heads,
                           num_kv_heads, scale_log2, s, kvh, t_begin, t_end, nt,
                           rope_at<D>(rope_table, rope_positions, ctx), acc, mg, lg);

    if (nparts == 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (g % TPL == row) {
                float o[8];
                const float inv = 1.f / lg[g];
#pragma unroll
                for (int x = 0; x < 8; ++x) o[x] = acc[g][x] * inv;
                reinterpret_cast<uint4 *>(out + ((size_t)s * num_q_heads + h0 + g) * D)[c] = pack8(o);
            }
        }
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (g % TPL == row) {
                const size_t r = ((size_t)s * num_q_heads + h0 + g) * max_parts + part;
                float4 *dst = reinterpret_cast<float4 *>(ws_out + r * D + c * 8);
                dst[0] = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
                dst[1] = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
                if (c == 0) {
                    ws_ml[r * 2 + 0] = mg[g];
                    ws_ml[r * 2 + 1] = lg[g];
                }
            }
        }
    }
}

// Single-pass decode: one workgroup of W wavefronts per (sequence, KV head).
// The sequence's blocks are split evenly among the waves; each wave runs
// wave_attend over its share and the waves merge their (m, l, acc) through
// LDS, so no workspace and no second kernel are needed.
template <int D, int G, bool FP8>
__global__ __launch_bounds__(512) void decode_fused_kernel(
    const uint16_t *__restrict__ q, const void *k_cache, const void *v_cache,
    const float *k_scale, const float *v_scale, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t num_blocks, int32_t num_q_heads, int32_t num_kv_heads, float scale_log2,
    uint16_t *__restrict__ out, const uint16_t *__restrict__ k_new,
    const uint16_t *__restrict__ v_new, const int32_t *__restrict__ slots, void *k_store,
    void *v_store, float *ks_store, float *vs_store, const float *__restrict__ rope_table,
    int32_t rope_positions) {
    // [W][G][D] acc, then [W][G] m, then [W][G] l; FP8: [W] rings of
    // Fp8Mma<D>::WAVE_BYTES (the matrix-core path)
    extern __shared__ float smem[];
    int kvh = blockIdx.x;
    int s = blockIdx.y;
    // KV heads 2k and 2k + 1 of a sequence back to back on one XCD: FP8 scale
    // rows of the two share 128-byte lines; bf16 or FP8, their tiles of a block
    // are adjacent in the pool (measured 0.3-0.6% faster for bf16 too)
    pair_kv_heads(blockIdx.y * num_kv_heads + blockIdx.x, num_kv_heads * (int)gridDim.y,
                  num_kv_heads, s, kvh);
    const int ctx = clamp_context(context_lens[s], max_context_len, max_blocks_per_seq,
                                  kvh == 0 && threadIdx.x == 0, s);
    const int32_t *bt_row = block_tables + (size_t)s * max_blocks_per_seq;
    const size_t row = (size_t)s * num_q_heads * D;
    if constexpr (FP8) {
        if (ctx > kExactDecodeKeys) {  // uniform over the workgroup: the matrix-core path
            attend_unit_fp8_mfma<D, G>(
                q + row, static_cast<const uint8_t *>(k_cache),
                static_cast<const uint8_t *>(v_cache), k_scale, v_scale, bt_row, ctx, num_blocks,
                num_q_heads, num_kv_heads, scale_log2, out + row, kvh, blockDim.x >> 6,
                reinterpret_cast<unsigned char *>(smem), [&]() {
                    return make_new_token<D, FP8>(k_new, v_new, slots, k_store, v_store,
                                                  ks_store, vs_store, bt_row, num_blocks,
                                                  num_kv_heads, s, kvh, ctx);
                });
            return;
        }
    }
    attend_unit<D, G, FP8>(
        q + row, k_cache, v_cache, k_scale, v_scale, bt_row, ctx, num_blocks, num_q_heads,
        num_kv_heads, scale_log2, out + row, kvh, blockDim.x >> 6, smem,
        [&]() {
            return make_new_token<D, FP8>(k_new, v_new, slots, k_store, v_store, ks_store,
                                          vs_store, bt_row, num_blocks, num_kv_heads, s, kvh, ctx);
        },
        rope_at<D>(rope_table, rope_positions, ctx));
}

// Second pass: merge the partitions of every (sequence, query head) that had
// more than one.  One wavefront per (sequence, query head).
template <int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(
    const int32_t *__restrict__ context_lens, int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t num_seqs, int32_t num_q_heads, int32_t partition_tokens, int32_t max_parts,
    const float *__restrict__ ws_out, const float *__restrict__ ws_ml, uint16_t *__restrict__ out) {
    constexpr int E = D / 64;  // elements per lane
    const int lane = threadIdx.x & 63;
    const int row_id = blockIdx.x * (blockDim.x >> 6) + wave_id_uniform();
    if (row_id >= num_seqs * num_q_heads) return;
    const int s = row_id / num_q_heads;
    const int ctx = clamp_context(context_lens[s], max_context_len, max_blocks_per_seq, false, s);
    if (ctx <= 0) return;
    const int nparts = (ctx + partition_tokens - 1) / partition_tokens;
    if (nparts <= 1) return;

    const float *ml = ws_ml + (size_t)row_id * max_parts * 2;
    float M = -INFINITY;
    for (int p = lane; p < nparts; p += 64) M = fmaxf(M, ml[p * 2]);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d));

    float a[E];
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] = 0.f;
    float L = 0.f;
    const float *po = ws_out + (size_t)row_id * max_parts * D + lane * E;
    for (int p = 0; p < nparts; ++p) {
        const float w = fast_exp2(ml[p * 2] - M);
        L = fmaf(w, ml[p * 2 + 1], L);
#pragma unroll
        for (int e = 0; e < E; ++e) a[e] = fmaf(w, po[(size_t)p * D + e], a[e]);
    }
    const float inv = 1.f / L;
    uint16_t *o = out + (size_t)row_id * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = (uint16_t)f32_to_bf16_rne(a[e] * inv);
}

template <int D, int G, bool FP8>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
    const float scale_log2 = a.scale * 1.4426950408889634f;
    if (a.fused_waves > 0) {
        const int W = a.fused_waves;
        size_t lds = (size_t)W * G * (D + 2) * sizeof(float);
        // (HIP on this GPU launches up to the 160 KiB of LDS a compute unit
        // has without a per-kernel attribute: 8 FP8 rings take 132 KiB)
        if constexpr (FP8) lds = std::max(lds, (size_t)W * Fp8Mma<D>::WAVE_BYTES);
        hipLaunchKernelGGL((decode_fused_kernel<D, G, FP8>), dim3(a.num_kv_heads, a.num_seqs),
                           dim3(64 * W), lds, stream, (const uint16_t *)a.q, a.k_cache, a.v_cache,
                           a.k_scale, a.v_scale, a.block_tables, a.context_lens, a.max_blocks_per_seq,
                           a.max_context_len, a.num_blocks, a.num_q_heads, a.num_kv_heads,
                           scale_log2, (uint16_t *)a.out, (const uint16_t *)a.k_new,
                           (const uint16_t *)a.v_new, a.slots, a.k_store, a.v_store,
                           a.k_scale_store, a.v_scale_store, a.rope_table, a.rope_positions);
        return hipGetLastError();
    }
    const int waves = a.max_parts >= 4 ? 4 : (a.max_parts >= 2 ? 2 : 1);
    const unsigned groups = (unsigned)((a.max_parts + waves - 1) / waves);
    const dim3 grid(groups * (unsigned)a.num_kv_heads * (unsigned)a.num_seqs);
    const size_t split_lds = FP8 ? (size_t)waves * Fp8Mma<D>::WAVE_BYTES : 0;
    hipLaunchKernelGGL((decode_split_kernel<D, G, FP8>), grid, dim3(64 * waves), split_lds, stream,
                       (const uint16_t *)a.q, a.k_cache, a.v_cache, a.k_scale, a.v_scale,
                       a.block_tables, a.context_lens,
                       a.max_blocks_per_seq, a.max_context_len, a.num_blocks, a.num_seqs,
                       a.num_q_heads, a.num_kv_heads, a.partition_tokens, a.max_parts, scale_log2,
                       (uint16_t *)a.out, a.ws_out, a.ws_ml, (const uint16_t *)a.k_new,
                       (const uint16_t *)a.v_new, a.slots, a.k_store, a.v_store,
                       a.k_scale_store, a.v_scale_store, a.rope_table, a.rope_positions);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_parts <= 1) return e;
    const int rows = a.num_seqs * a.num_q_heads;
    hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3((rows + 3) / 4), dim3(256), 0, stream,
                       a.context_lens, a.max_blocks_per_seq, a.max_context_len, a.num_seqs,
                       a.num_q_heads, a.partition_tokens, a.max_parts, a.ws_out, a.ws_ml,
                       (uint16_t *)a.out);
    return hipGetLastError();
}

template <int D, bool FP8>
static hipError_t launch_decode_d(const DecodeArgs &a, hipStream_t stream) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_decode_t<D, 1, FP8>(a, stream);
        case 2: return launch_decode_t<D, 2, FP8>(a, stream);
        case 4: return launch_decode_t<D, 4, FP8>(a, stream);
        case 8: return launch_decode_t<D, 8, FP8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    if (a.fp8)
        return a.head_dim == 64 ? launch_decode_d<64, true>(a, stream)
                                : launch_decode_d<128, true>(a, stream);
    return a.head_dim == 64 ? launch_decode_d<64, false>(a, stream)
                            : launch_decode_d<128, false>(a, stream);
}

}  // namespace pkv
