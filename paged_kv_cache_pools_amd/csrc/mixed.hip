// mixed.hip -- one launch for a continuous-batching iteration: the decode
// sequences (one new token each) and the prefill chunks of newly admitted or
// partly processed prompts attend together.
//
// Iteration-level scheduling puts the running sequences' next tokens and the
// newly admitted requests into one batch and one forward pass (Nano-vLLM
// engine deep-dive §5.1-5.2; LLM primer part 4 §17.5).  Attention is the same
// definition for every sequence: its new tokens sit at positions c .. c+n-1
// after c cached ones and new token i sees keys 0 .. c+i (deep-dive §3.2;
// primer §22); a decode token is the case n = 1.  The two kinds of work
// differ in what bounds them: a decode token streams its whole K/V once for G
// multiply-adds per element (HBM-bound), a prefill chunk reuses each K/V
// element for TWG query tokens on the matrix cores (MFMA-bound).
//
// One grid holds both kinds of workgroup (256 threads each):
//  * decode unit = (decode sequence, KV head): the single-pass decode of
//    decode_wave.h with its 4 waves splitting the sequence's blocks and
//    merging in LDS;
//  * prefill unit = (prefill sequence, KV head, query block): the MFMA query
//    tile of prefill_tile.h.
// Order of dispatch.  A prefill unit's run time grows with the keys it
// attends to, and the longest ones set the launch's length, so prefill units
// go heaviest first: prompts by context length, longest first (ranked in the
// kernel when there are at most 64 prompts), then query block from the last,
// then segment, with the KV head innermost.  Workgroups are dealt to the 8
// XCDs round-robin, so with 8 KV heads every XCD works on one head: the query
// blocks of a (prompt, KV head) that re-read its K/V meet in one XCD's L2.
// The decode and prefill lists are interleaved in groups of 8 workgroups
// (decode, prefill, decode, ...) while both last, which keeps that alignment
// and gives every XCD both kinds, so bandwidth-bound and compute-bound work
// overlap on each.  When the whole launch is resident at once (at most two
// workgroups per compute unit) and the prefill units are split by key range
// (so the decode units are the longest), the decode list goes first instead:
// an XCD's dispatcher fills its compute units breadth first, walking its
// shader engines in turn, so the period-2 interleave would put two decode
// units on each compute unit of half the engines; decode first gives each
// compute unit at most one (measured on 32 x 4096 decode + one split 64-token
// chunk: 103 against 124-128 us).  Unsplit, the few long prefill units are
// the longest, and the interleave serves them better (185 against 224 us).
//
// A prefill unit may run as several workgroups, each over a contiguous
// segment of its key chunks (prefill_tile.h, SPLIT): a chunk of a prompt with
// a long cached context is otherwise one workgroup's serial walk over every
// key, which outlasts the rest of the launch.  The unit's segments are
// adjacent in the dispatch order and write partial results; a second, small
// launch merges them (the kernel boundary makes them visible; handing them
// over inside the launch would take an L2 write-back per segment on this
// GPU's per-XCD caches, which measured far slower).
//
// Sequences 0 .. num_decode-1 are the decode sequences: one new token each.
// One with more new tokens is still computed in full (its workgroup for a KV
// head runs every query block of it in turn); one with none writes nothing.
//
// Over an FP8 cache (codes + per-(token, KV head) scales) each kind runs the
// FP8 form of its own launch: the decode units the FP8 decode's (matrix cores
// above 128 keys, its LDS rings inside this kernel's LDS), the prefill units
// the FP8 query tile.
#include "decode_fp8_mfma.h"
#include "decode_wave.h"
#include "prefill_tile.h"

namespace pkv {

// The prefill prompt (0-based among the prefill sequences) of rank `rank` by
// context length, longest first, ties by order: with at most 64 prompts lane
// i ranks prompt i and the wave finds the lane holding `rank`; with more,
// prompts keep the caller's order.  Every lane of the wave must call.
__device__ __forceinline__ int prompt_of_rank(const int32_t *__restrict__ context_lens,
                                              int num_decode, int num_prefill, int rank) {
    if (num_prefill > 64) return rank;
    const int lane = threadIdx.x & 63;
    const int mine = lane < num_prefill ? context_lens[num_decode + lane] : -1;
    int r = 0;
    for (int j = 0; j < num_prefill; ++j) {
        const int other = __shfl(mine, j);
        r += (other > mine) || (other == mine && j < lane);
    }
    const unsigned long long hit = __ballot(lane < num_prefill && r == rank);
    return __ffsll((long long)hit) - 1;
}

template <int D, int G, bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mixed_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const float *__restrict__ k_scale,
    const float *__restrict__ v_scale, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ cu_new_lens, const int32_t *__restrict__ context_lens,
    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_blocks, int32_t num_decode,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t num_qblocks,
    float scale_log2, uint16_t *__restrict__ out, float *partials, int32_t seg_slots) {
    using Geo = PrefillGeom<D, G, 4, FP8>;
    static_assert(kMixedWaves * G * (D + 2) * sizeof(float) <= 2 * Geo::BUF, "decode merge fits the LDS");
    static_assert(!FP8 || kMixedWaves * Fp8Mma<D>::WAVE_BYTES <= 2 * Geo::BUF,
                  "the FP8 decode rings fit the LDS");
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * Geo::BUF];

    const int num_prefill = num_seqs - num_decode;
    const int dec_units = num_decode * num_kv_heads;
    const int pf_units = num_prefill * num_kv_heads * num_qblocks * seg_slots;  // workgroups
    const int unit = blockIdx.x;
    // when every workgroup of the launch is resident at once and the prefill
    // units are split into short segments, the decode units -- then the
    // longest -- go first: the dispatcher gives each compute unit one before
    // any gets a second workgroup, so no decode unit shares a compute unit
    // with another
    const int m8 = (seg_slots > 1 && dec_units + pf_units <= kResidentWorkgroups)
                       ? 0
                       : min(dec_units, pf_units) / 8 * 8;  // units of each list interleaved
    bool is_decode;
    int idx;
    if (unit < 2 * m8) {
        const int g = unit >> 3;
        is_decode = (g & 1) == 0;
        idx = (g >> 1) * 8 + (unit & 7);
    } else {
        const int r = unit - 2 * m8;
        is_decode = r < dec_units - m8;
        idx = m8 + (is_decode ? r : r - (dec_units - m8));
    }

    if (!is_decode) {
        // idx = ((rank * num_qblocks + qb from the last) * seg_slots + seg) * H_kv + kvh
        const int kvh = idx % num_kv_heads;
        idx /= num_kv_heads;
        SplitSlot split;
        split.seg = idx % seg_slots;
        split.slots = seg_slots;
        idx /= seg_slots;
        const int qb = num_qblocks - 1 - idx % num_qblocks;
        const int rank = idx / num_qblocks;
        const int unit = idx * num_kv_heads + kvh;  // the unit's partials
        if (seg_slots > 1)
            split.partials = partials + (size_t)unit * seg_slots * prefill_partial_floats<D, G>();
        const int p = prompt_of_rank(context_lens, num_decode, num_prefill, rank);
        prefill_unit<D, G, true, false, 4, FP8>(
            q, k_cache, v_cache, block_tables, cu_new_lens, context_lens, max_blocks_per_seq,
            max_context_len, num_blocks, num_q_heads, num_kv_heads, scale_log2, out,
            num_decode + p, qb, kvh, lds, split, CrossGeom{}, k_scale, v_scale);
        return;
    }

    const int s = idx / num_kv_heads;
    const int kvh = idx % num_kv_heads;
    const int row0 = cu_new_lens[s];
    const int n = cu_new_lens[s + 1] - row0;
    const int ctx = clamp_context(context_lens[s], max_context_len, max_blocks_per_seq,
                                  kvh == 0 && threadIdx.x == 0, s);
    if (n == 1 && ctx >= 1) {
        const size_t row = (size_t)row0 * num_q_heads * D;
        const int32_t *bt_row = block_tables + (size_t)s * max_blocks_per_seq;
        if constexpr (FP8) {
            if (ctx > kExactDecodeKeys) {  // uniform: the FP8 decode's matrix-core path
                attend_unit_fp8_mfma<D, G>(q + row, reinterpret_cast<const uint8_t *>(k_cache),
                                           reinterpret_cast<const uint8_t *>(v_cache), k_scale,
                                           v_scale, bt_row, ctx, num_blocks, num_q_heads,
                                           num_kv_heads, scale_log2, out + row, kvh, kMixedWaves,
                                           lds, []() { return NewToken{}; });
                return;
            }
        }
        attend_unit<D, G, FP8>(q + row, k_cache, v_cache, k_scale, v_scale, bt_row, ctx,
                               num_blocks, num_q_heads, num_kv_heads, scale_log2, out + row, kvh,
                               kMixedWaves, reinterpret_cast<float *>(lds),
                               []() { return NewToken{}; }, Rope{});
        return;
    }
    // not a single token: the prefill tiles of the whole sequence, in turn
    const int nq = (min(n, ctx) + Geo::TWG - 1) / Geo::TWG;
    for (int qb = nq - 1; qb >= 0; --qb) {
        __syncthreads();  // the previous tile's last LDS reads are done
        prefill_unit<D, G, false, false, 4, FP8>(
            q, k_cache, v_cache, block_tables, cu_new_lens, context_lens, max_blocks_per_seq,
            max_context_len, num_blocks, num_q_heads, num_kv_heads, scale_log2, out, s, qb, kvh,
            lds, SplitSlot{}, CrossGeom{}, k_scale, v_scale);
    }
}

// Second launch of a split mixed step: prefill_merge_parts workgroups per
// prefill unit, in the mixed kernel's unit order, merging the segments of the
// units that split.
template <int D, int G>
__global__ __launch_bounds__(256) void mixed_merge_kernel(
    const int32_t *__restrict__ cu_new_lens, const int32_t *__restrict__ context_lens,
    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_decode, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t num_qblocks, uint16_t *__restrict__ out,
    const float *__restrict__ partials, int32_t seg_slots) {
    const int num_prefill = num_seqs - num_decode;
    constexpr int PARTS = prefill_merge_parts<D, G>();
    static_assert(PARTS <= kMaxSegments, "the host's grid bound covers the merge launch");
    const int unit = blockIdx.x / PARTS;  // (rank * num_qblocks + qb from the last) * H_kv + kvh
    const int kvh = unit % num_kv_heads;
    const int qb = num_qblocks - 1 - (unit / num_kv_heads) % num_qblocks;
    const int rank = unit / (num_kv_heads * num_qblocks);
    const int p = prompt_of_rank(context_lens, num_decode, num_prefill, rank);
    prefill_merge<D, G>(cu_new_lens, context_lens, max_blocks_per_seq, max_context_len,
                        num_q_heads, out, num_decode + p, qb, kvh,
                        partials + (size_t)unit * seg_slots * prefill_partial_floats<D, G>(),
                        seg_slots, blockIdx.x % PARTS);
}

template <int D, int G, bool FP8>
static hipError_t launch_mixed_f(const MixedArgs &a, hipStream_t stream) {
    using Geo = PrefillGeom<D, G, 4, FP8>;
    const int nqb = a.num_seqs > a.num_decode ? (a.max_new_len + Geo::TWG - 1) / Geo::TWG : 0;
    const int64_t units = (int64_t)a.num_decode * a.num_kv_heads +
                          (int64_t)(a.num_seqs - a.num_decode) * a.num_kv_heads * nqb * a.seg_slots;
    if (units == 0) return hipSuccess;
    const float scale_log2 = a.scale * 1.4426950408889634f;
    hipLaunchKernelGGL((mixed_kernel<D, G, FP8>), dim3((unsigned)units), dim3(Geo::THREADS), 0,
                       stream, (const uint16_t *)a.q, (const uint16_t *)a.k_cache,
                       (const uint16_t *)a.v_cache, a.k_scale, a.v_scale, a.block_tables,
                       a.cu_new_lens, a.context_lens,
                       a.max_blocks_per_seq, a.max_context_len, a.num_blocks, a.num_decode,
                       a.num_seqs, a.num_q_heads, a.num_kv_heads, nqb, scale_log2,
                       (uint16_t *)a.out, a.partials, a.seg_slots);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.seg_slots <= 1) return e;
    const int64_t pf_units = (int64_t)(a.num_seqs - a.num_decode) * a.num_kv_heads * nqb;
    hipLaunchKernelGGL((mixed_merge_kernel<D, G>), dim3((unsigned)(pf_units * prefill_merge_parts<D, G>())),
                       dim3(256), 0,
                       stream, a.cu_new_lens, a.context_lens, a.max_blocks_per_seq,
                       a.max_context_len, a.num_decode, a.num_seqs, a.num_q_heads, a.num_kv_heads,
                       nqb, (uint16_t *)a.out, a.partials, a.seg_slots);
    return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_mixed_t(const MixedArgs &a, hipStream_t stream) {
    return a.fp8 ? launch_mixed_f<D, G, true>(a, stream) : launch_mixed_f<D, G, false>(a, stream);
}

PKV_DEBUG_WORD_ACCESS(mixed)

static_assert(PrefillGeom<128, 1>::WAVES == kTileWaves && PrefillGeom<128, 1>::COLS == kTileCols,
              "the host sizes the mixed launch for this tile");
static_assert(mixed_partial_bytes(64) == prefill_partial_floats<64, 1>() * sizeof(float) &&
                  mixed_partial_bytes(128) == prefill_partial_floats<128, 1>() * sizeof(float),
              "partial result size");

template <int D>
static hipError_t launch_mixed_d(const MixedArgs &a, hipStream_t stream) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_mixed_t<D, 1>(a, stream);
        case 2: return launch_mixed_t<D, 2>(a, stream);
        case 4: return launch_mixed_t<D, 4>(a, stream);
        case 8: return launch_mixed_t<D, 8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mixed(const MixedArgs &a, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    return a.head_dim == 64 ? launch_mixed_d<64>(a, stream) : launch_mixed_d<128>(a, stream);
}

}  // namespace pkv
