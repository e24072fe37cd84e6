// prefill.hip -- the chunked causal prefill kernel (gfx950): one workgroup
// per (prompt, KV head, block of query tokens), each running the MFMA query
// tile of prefill_tile.h, over a bf16 cache or an FP8 one (codes + scales).
#include "prefill_tile.h"

namespace pkv {

// Waves per workgroup: 8 at head_dim 128 (two per SIMD, one workgroup per
// compute unit; every staged key chunk feeds 256 query columns), 4 at 64.
template <int D>
constexpr int prefill_waves() { return D == 128 ? 8 : 4; }

template <int D, int G, bool FP8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const float *__restrict__ k_scale,
    const float *__restrict__ v_scale, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ cu_new_lens, const int32_t *__restrict__ context_lens,
    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_blocks, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t num_qblocks, float scale_log2,
    uint16_t *__restrict__ out) {
    using Geo = PrefillGeom<D, G, prefill_waves<D>(), FP8>;
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * Geo::BUF];

    // ---- work unit.  Workgroups are dealt to the 8 XCDs round-robin by their
    // linear id; the id is remapped so that each XCD receives a contiguous
    // range of units ordered (KV head, prompt, query block from the last):
    // the workgroups an XCD runs together share one prompt's K/V in its L2,
    // and the longest query blocks of a prompt start first.
    const int units = num_kv_heads * num_seqs * num_qblocks;
    int unit;
    {
        const int L = blockIdx.x;
        const int xcd = L & 7, slot = L >> 3;
        const int per = units >> 3, rem = units & 7;
        unit = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
    }
    const int qb = num_qblocks - 1 - unit % num_qblocks;
    const int p = (unit / num_qblocks) % num_seqs;
    const int kvh = unit / (num_qblocks * num_seqs);
    prefill_unit<D, G, false, false, prefill_waves<D>(), FP8>(
        q, k_cache, v_cache, block_tables, cu_new_lens, context_lens, max_blocks_per_seq,
        max_context_len, num_blocks, num_q_heads, num_kv_heads, scale_log2, out, p, qb, kvh, lds,
        SplitSlot{}, CrossGeom{}, k_scale, v_scale);
}

PKV_DEBUG_WORD_ACCESS(prefill)

template <int D, int G, bool FP8>
static hipError_t launch_prefill_f(const PrefillArgs &a, hipStream_t stream) {
    using Geo = PrefillGeom<D, G, prefill_waves<D>(), FP8>;
    const int nqb = (a.max_new_len + Geo::TWG - 1) / Geo::TWG;
    const int64_t units = (int64_t)nqb * a.num_kv_heads * a.num_seqs;
    const float scale_log2 = a.scale * 1.4426950408889634f;
    hipLaunchKernelGGL((prefill_kernel<D, G, FP8>), dim3((unsigned)units), dim3(Geo::THREADS), 0,
                       stream, (const uint16_t *)a.q, (const uint16_t *)a.k_cache,
                       (const uint16_t *)a.v_cache, a.k_scale, a.v_scale, a.block_tables,
                       a.cu_new_lens, a.context_lens, a.max_blocks_per_seq, a.max_context_len,
                       a.num_blocks, a.num_seqs, a.num_q_heads, a.num_kv_heads, nqb, scale_log2,
                       (uint16_t *)a.out);
    return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t stream) {
    return a.fp8 ? launch_prefill_f<D, G, true>(a, stream) : launch_prefill_f<D, G, false>(a, stream);
}

template <int D>
static hipError_t launch_prefill_d(const PrefillArgs &a, hipStream_t stream) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_prefill_t<D, 1>(a, stream);
        case 2: return launch_prefill_t<D, 2>(a, stream);
        case 4: return launch_prefill_t<D, 4>(a, stream);
        case 8: return launch_prefill_t<D, 8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
    if (a.num_seqs == 0 || a.max_new_len == 0) return hipSuccess;
    return a.head_dim == 64 ? launch_prefill_d<64>(a, stream) : launch_prefill_d<128>(a, stream);
}

}  // namespace pkv
