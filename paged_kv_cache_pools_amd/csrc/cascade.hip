// cascade.hip -- decode attention for a batch whose sequences share prompt
// prefixes through identical physical blocks.
//
// Requests that share a system prompt point their block tables at the same
// physical blocks, so the prefix is stored once ("Nano-vLLM engine
// deep-dive", section 2.2; "LLM basics primer" part 4, sections 17.6-17.7).
// Plain decode still reads those blocks once per sequence.  Here a group's
// decode queries attend to its shared prefix together, reading it once: for a
// group of n sequences and one KV head, the n x G query rows against the
// prefix keys form a small matrix product, run as the MFMA query tile of
// prefill_tile.h in its cross-attention mode (no causal mask: the prefix
// precedes every query).  Each sequence's own tail -- its tokens after the
// prefix -- runs as split-KV decode units (decode_wave.h).  Both write
// unnormalised partial results (O, m, l) into one workspace row per
// (sequence, query head), and a second launch merges them:
//   out = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p,
// the merge of split-KV decode, so the result is the sequence's attention
// over its whole context up to fp32 rounding.
//
// Groups are ranges of consecutive sequences: group g is sequences
// group_starts[g] .. group_starts[g + 1] - 1, sharing their first
// prefix_lens[g] tokens (whole blocks); a sequence outside every group, or in
// a group of prefix 0, is all tail.
//
// Tails, balanced.  The tails of all (sequence, KV head) units, block after
// block in (sequence, KV head) order, form one list of T blocks, and the NW
// waves of the tail workgroups each take one contiguous run of it: wave w the
// blocks [floor(w T / NW), floor((w + 1) T / NW)).  Every wave streams the same
// number of blocks whatever the lengths of the tails, in long runs (a fixed
// split into partitions leaves the last round of waves part-filled and makes
// every short partition pay the start of a stream); where a run crosses from
// one unit to the next it writes the first unit's partial result and starts
// afresh.  A run is at least partition_tokens tokens (NW is lowered for short
// lists), so a unit has at most ceil(tail / partition_tokens) + 1 pieces.
// Every tail workgroup computes the units' offsets in the list (a scan over
// the sequences' tail lengths) in LDS; the first also writes them to the
// workspace for the merge.  The split depends only on the inputs and the
// grid, so results are reproducible.
//
// Workspace row of (sequence s, query head h), slots = max_parts + kMaxSegments:
// slots 0 .. max_parts - 1 hold the tail pieces of the unit in list order,
// slots max_parts .. the prefix segments (the prefix tile splits its keys into
// up to kMaxSegments ranges of at least 512 keys).  After the rows: the list's
// wave count NW, then the offsets, for the merge.
//
// Dispatch order: all prefix tiles first, then the tail workgroups (the host
// sizes their number: two per compute unit, as many as can be resident, or
// several rounds of shorter runs).  The dispatcher hands an XCD's
// workgroups to its compute units breadth first, so as long as at most 256
// tiles have keys to read (they lead the grid) no compute unit runs two of
// them, and the tail workgroups that find no slot start as the tiles finish.
// (With the key segment innermost instead, a 2048-token prefix's four live
// segments of eight put two busy tiles on half the compute units and none on
// the others; the step was 1-3% slower.)  (Alternating the kinds in
// short runs instead aliases with the dispatcher's walk over the shader
// engines and piles the tiles onto half of them -- measured.  Shorter runs for
// the workgroups that start late measured slower: 219-250 against 204 us.)
// Over an FP8 cache (codes + per-(token, KV head) scales) the prefix tiles
// are the FP8 query tile; a tail wave runs the FP8 decode's matrix-core path,
// with its LDS ring, when the list's offsets fit in the LDS after the four
// waves' rings (batches of up to a few hundred sequences) and the sequence
// holds more than kExactDecodeKeys keys, else the FP8 decode's VALU path.
#include <mutex>

#include "decode_fp8_mfma.h"
#include "decode_wave.h"
#include "prefill_tile.h"

namespace pkv {

namespace {

struct GroupView {
    int begin, end, prefix;  // sequences [begin, end), shared prefix tokens (0 for none)
};

// Group g with its range clamped to [0, num_seqs] and its prefix to whole
// blocks within ctx_cap.
__device__ __forceinline__ GroupView group_view(const int32_t *__restrict__ group_starts,
                                                const int32_t *__restrict__ prefix_lens, int g,
                                                int num_seqs, int ctx_cap) {
    GroupView v;
    v.begin = min(max(group_starts[g], 0), num_seqs);
    v.end = min(max(group_starts[g + 1], v.begin), num_seqs);
    v.prefix = min(max(prefix_lens[g], 0), ctx_cap) / kBlockTokens * kBlockTokens;
    return v;
}

// The group holding sequence s (the last g with group_starts[g] <= s, by
// binary search, checked against the group's end), or a view of prefix 0
// when no group does.  Per thread.
__device__ __forceinline__ GroupView group_of(const int32_t *__restrict__ group_starts,
                                              const int32_t *__restrict__ prefix_lens,
                                              int num_groups, int num_seqs, int ctx_cap, int s) {
    if (num_groups <= 0) return GroupView{s, s + 1, 0};
    int lo = 0, hi = num_groups - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (group_starts[mid] <= s)
            lo = mid;
        else
            hi = mid - 1;
    }
    GroupView v = group_view(group_starts, prefix_lens, lo, num_seqs, ctx_cap);
    if (s < v.begin || s >= v.end) v = GroupView{s, s + 1, 0};
    return v;
}

// The tail of sequence s: tokens [prefix, ctx) in `blocks` whole or partial
// blocks (none when the context does not pass the prefix).
struct TailView {
    int prefix, ctx, blocks;
};

__device__ __forceinline__ TailView tail_of(const int32_t *__restrict__ context_lens,
                                            const int32_t *__restrict__ group_starts,
                                            const int32_t *__restrict__ prefix_lens,
                                            int num_groups, int num_seqs, int ctx_cap, int s) {
    TailView t;
    t.ctx = min(context_lens[s], ctx_cap);
    t.prefix = group_of(group_starts, prefix_lens, num_groups, num_seqs, ctx_cap, s).prefix;
    t.blocks = t.ctx > t.prefix
                   ? (t.ctx + kBlockTokens - 1) / kBlockTokens - t.prefix / kBlockTokens
                   : 0;
    return t;
}

// The wave of a list of T blocks split among nw waves that holds block x.
__device__ __forceinline__ int tail_wave_of(int x, int total, int nw) {
    return (int)(((int64_t)(x + 1) * nw - 1) / total);
}

constexpr int kTailWaves = 4;  // waves of a tail workgroup
constexpr int kTailThreads = 64 * kTailWaves;

// Prefix tiles split their keys into segments of at least this many 64-key
// chunks (512 keys), up to kMaxSegments.
constexpr int kPrefixSegmentChunks = 8;

// Key segments of a prefix of `keys` tokens (0 without one): the split the
// prefix tile makes of its 64-key chunks.
__device__ __forceinline__ int prefix_segments(int keys) {
    return keys > 0 ? prefill_segments((keys + 63) / 64, kMaxSegments, kPrefixSegmentChunks) : 0;
}

}  // namespace

template <int D, int G, bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void cascade_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const float *__restrict__ k_scale,
    const float *__restrict__ v_scale, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t num_blocks, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    const int32_t *__restrict__ group_starts, const int32_t *__restrict__ prefix_lens,
    int32_t num_groups, int32_t prefix_qblocks, int32_t partition_tokens, int32_t max_parts,
    float scale_log2, float *__restrict__ ws_out, float *__restrict__ ws_ml,
    int32_t *__restrict__ ws_list) {
    using Geo = PrefillGeom<D, G, 4, FP8>;
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * Geo::BUF];
    static_assert(2 * Geo::BUF >= (kMaxPrefixSeqs + 1 + kTailWaves) * (int)sizeof(int32_t),
                  "a tail workgroup's list fits the tile's LDS");
    const int slots = max_parts + kMaxSegments;
    const int ctx_cap = min(max_context_len, max_blocks_per_seq * kBlockTokens);
    const int pf_units = num_groups * prefix_qblocks * kMaxSegments * num_kv_heads;

    if ((int)blockIdx.x < pf_units) {
        // a prefix tile: idx = ((seg * num_groups + g) * prefix_qblocks + qb) * H_kv + kvh.
        // The key segment is outermost: a prefix has fewer segments than
        // kMaxSegments unless it is long, and the tiles past its last return at
        // once, so the tiles with keys to read come first in the grid and the
        // dispatcher spreads them over distinct compute units.
        int idx = blockIdx.x;
        const int kvh = idx % num_kv_heads;
        idx /= num_kv_heads;
        const int qb = idx % prefix_qblocks;
        idx /= prefix_qblocks;
        const int g = idx % num_groups;
        SplitSlot split;
        split.seg = idx / num_groups;
        split.slots = kMaxSegments;
        split.min_chunks = kPrefixSegmentChunks;
        split.ws_out = ws_out;
        split.ws_ml = ws_ml;
        split.ws_slots = slots;
        split.slot0 = max_parts;
        const GroupView v = group_view(group_starts, prefix_lens, g, num_seqs, ctx_cap);
        CrossGeom cross;
        cross.row0 = v.begin;
        cross.n = v.end - v.begin;
        cross.keys = v.prefix;
        cross.bt = block_tables + (size_t)v.begin * max_blocks_per_seq;
        prefill_unit<D, G, true, true, 4, FP8>(
            q, k_cache, v_cache, block_tables, nullptr, nullptr, max_blocks_per_seq,
            max_context_len, num_blocks, num_q_heads, num_kv_heads, scale_log2, nullptr, 0, qb, kvh,
            lds, split, cross, k_scale, v_scale);
        return;
    }

    // a tail workgroup.  First the list: tail_off[s] = H x the tail blocks of
    // the sequences before s (each thread counts a run of sequences, then an
    // exclusive scan of the runs' totals).
    const int tw = blockIdx.x - pf_units;  // tail workgroup
    // [num_seqs + 1] list offsets, then the 4 waves' sums (in the tile's LDS).
    // FP8: at the end of the LDS, so that when the list is short enough the
    // waves' rings of the matrix-core decode path fit before it
    constexpr int kLdsBytes = 2 * Geo::BUF;
    const int list_at = FP8 ? ((kLdsBytes - (num_seqs + 1 + kTailWaves) * 4) & ~15) : 0;
    int32_t *tail_off = reinterpret_cast<int32_t *>(lds + list_at);
    const bool rings = FP8 && list_at >= kTailWaves * Fp8Mma<D>::WAVE_BYTES;  // uniform
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int S = num_seqs, H = num_kv_heads;
    const int per = (S + kTailThreads - 1) / kTailThreads;
    const int s_lo = min(S, tid * per), s_hi = min(S, s_lo + per);
    int run = 0;
    for (int s = s_lo; s < s_hi; ++s) {
        PKV_DEBUG_CHECK(tw == 0 && (context_lens[s] < 0 || context_lens[s] > ctx_cap),
                        kDbgContext, context_lens[s], s);
        const int b = tail_of(context_lens, group_starts, prefix_lens, num_groups, S, ctx_cap, s)
                          .blocks;
        tail_off[s] = b;
        run += b;
    }
    int incl = run;  // inclusive scan within the wave, then across the 4 waves
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    int32_t *wsum = tail_off + S + 1;
    if (lane == 63) wsum[tid >> 6] = incl;
    __syncthreads();
    int before = 0;
    for (int u = 0; u < (tid >> 6); ++u) before += wsum[u];
    int at = before + incl - run;
    for (int s = s_lo; s < s_hi; ++s) {
        const int b = tail_off[s];
        tail_off[s] = at * H;
        at += b;
    }
    if (tid == kTailThreads - 1) tail_off[S] = (before + incl) * H;
    __syncthreads();
    const int total = tail_off[S];  // T
    const int nw_all = ((int)gridDim.x - pf_units) * kTailWaves;
    const int min_run = max(1, partition_tokens / kBlockTokens);
    const int nw = max(1, min(nw_all, total / min_run));
    if (tw == 0) {  // the list, for the merge
        for (int s = tid; s <= S; s += kTailThreads) ws_list[1 + s] = tail_off[s];
        if (tid == 0) ws_list[0] = nw;
    }

    const int w = tw * kTailWaves + wave_id_uniform();
    if (w >= nw || total == 0) return;  // uniform: no run for this wave
    const int r1 = (int)((int64_t)(w + 1) * total / nw);
    int x = (int)((int64_t)w * total / nw);
    // the sequence holding block x: the last s with tail_off[s] <= x
    int s = 0;
    for (int lo = 0, hi = S - 1; lo <= hi;) {
        const int mid = (lo + hi) >> 1;
        if (tail_off[mid] <= x) {
            s = mid;
            lo = mid + 1;
        } else {
            hi = mid - 1;
        }
    }
    constexpr int LPR = D / 8, TPL = 64 / LPR;
    const int row = lane / LPR;
    const int c = lane % LPR;
    unsigned char *const ring = lds + wave_id_uniform() * Fp8Mma<D>::WAVE_BYTES;
    while (x < r1) {
        while (tail_off[s + 1] <= x) ++s;  // past sequences with no tail
        const int nb = (tail_off[s + 1] - tail_off[s]) / H;
        const int rel = x - tail_off[s];
        const int kvh = rel / nb, j0 = rel - kvh * nb;
        const int take = min(nb - j0, r1 - x);
        // the tail is the last nb blocks of the context: one load, no group lookup
        TailView tv;
        tv.ctx = min(context_lens[s], ctx_cap);
        tv.blocks = nb;
        tv.prefix = ((tv.ctx + kBlockTokens - 1) / kBlockTokens - nb) * kBlockTokens;
        const int t_begin = tv.prefix + j0 * kBlockTokens;
        const int t_end = min(tv.prefix + (j0 + take) * kBlockTokens, tv.ctx);
        // the unit's piece: waves before this one that hold blocks of it
        const int ustart = tail_off[s] + kvh * nb;
        const int piece = w - tail_wave_of(ustart, total, nw);
        if constexpr (FP8) {
            // a sequence of more than kExactDecodeKeys keys: the FP8 decode's
            // matrix-core path, as the plain FP8 decode takes it (uniform)
            if (rings && tv.ctx > kExactDecodeKeys) {
                f32x4_t o[Fp8Mma<D>::MT];
                float mr, lr;
                wave_attend_fp8_mfma<D, G>(
                    q + (size_t)s * num_q_heads * D, reinterpret_cast<const uint8_t *>(k_cache),
                    reinterpret_cast<const uint8_t *>(v_cache), k_scale, v_scale,
                    block_tables + (size_t)s * max_blocks_per_seq, num_blocks, num_q_heads,
                    num_kv_heads, scale_log2, kvh, t_begin, t_end, NewToken{}, ring, o, mr, lr);
                const int col = lane & 15, grp = lane >> 4;  // head, dimensions 16m + 4grp ..
                if (col < G) {
                    const size_t r = ((size_t)s * num_q_heads + kvh * G + col) * slots + piece;
#pragma unroll
                    for (int m = 0; m < Fp8Mma<D>::MT; ++m)
                        *reinterpret_cast<float4 *>(ws_out + r * D + 16 * m + 4 * grp) =
                            make_float4(o[m][0], o[m][1], o[m][2], o[m][3]);
                    if (grp == 0) {
                        ws_ml[r * 2 + 0] = mr;
                        ws_ml[r * 2 + 1] = lr;
                    }
                }
                x += take;
                continue;
            }
        }
        float acc[G][8], mg[G], lg[G];
        wave_attend<D, G, FP8>(q, k_cache, v_cache, k_scale, v_scale,
                               block_tables + (size_t)s * max_blocks_per_seq, num_blocks,
                               num_q_heads, num_kv_heads, scale_log2, s, kvh, t_begin, t_end,
                               NewToken{}, Rope{}, acc, mg, lg);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (g % TPL == row) {
                const size_t r = ((size_t)s * num_q_heads + kvh * G + g) * slots + piece;
                float4 *dst = reinterpret_cast<float4 *>(ws_out + r * D + c * 8);
                dst[0] = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
                dst[1] = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
                if (c == 0) {
                    ws_ml[r * 2 + 0] = mg[g];
                    ws_ml[r * 2 + 1] = lg[g];
                }
            }
        }
        x += take;
    }
}

// Merge the partial results of every (sequence, query head): one wavefront
// each, its tail partitions then its prefix segments, in slot order.  A row
// whose inputs break the call's preconditions -- a prefix longer than the
// sequence's context, or a group member past the prefix_rows the launch's
// tiles cover -- is written as NaN.
template <int D>
__global__ __launch_bounds__(256) void cascade_reduce_kernel(
    const int32_t *__restrict__ context_lens, int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    const int32_t *__restrict__ group_starts, const int32_t *__restrict__ prefix_lens,
    int32_t num_groups, int32_t prefix_rows, int32_t max_parts, const float *__restrict__ ws_out,
    const float *__restrict__ ws_ml, const int32_t *__restrict__ ws_list,
    uint16_t *__restrict__ out) {
    constexpr int E = D / 64;  // elements per lane
    const int lane = threadIdx.x & 63;
    const int row_id = blockIdx.x * (blockDim.x >> 6) + wave_id_uniform();
    if (row_id >= num_seqs * num_q_heads) return;
    const int s = row_id / num_q_heads;
    const int slots = max_parts + kMaxSegments;
    const int ctx_cap = min(max_context_len, max_blocks_per_seq * kBlockTokens);
    const int ctx = min(context_lens[s], ctx_cap);
    const GroupView v = group_of(group_starts, prefix_lens, num_groups, num_seqs, ctx_cap, s);
    const int prefix = v.prefix;
    uint16_t *o = out + (size_t)row_id * D + lane * E;
    if (prefix > 0 && (prefix > ctx || s - v.begin >= prefix_rows)) {
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = 0x7fc0;  // bf16 NaN: undefined for these inputs
        return;
    }
    if (ctx <= 0) {  // an empty context is 0
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = 0;
        return;
    }
    // the unit's tail pieces: the waves of the tail list that hold its blocks
    const int H = num_kv_heads, kvh = (row_id % num_q_heads) / (num_q_heads / H);
    const int nw = ws_list[0], total = ws_list[1 + num_seqs];
    const int off = ws_list[1 + s], nb = (ws_list[2 + s] - off) / H;
    int nparts = 0;
    if (nb > 0) {
        const int ustart = off + kvh * nb;
        nparts = tail_wave_of(ustart + nb - 1, total, nw) - tail_wave_of(ustart, total, nw) + 1;
    }
    const int n = nparts + prefix_segments(prefix);
    auto slot_of = [&](int i) { return i < nparts ? i : max_parts + (i - nparts); };

    // online over batches of 8 slots: every load of a batch is issued before
    // the first is used; the running maximum M rescales what came before
    const float *ml = ws_ml + (size_t)row_id * slots * 2;
    const float *po = ws_out + (size_t)row_id * slots * D + lane * E;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    float M = -INFINITY, L = 0.f;
    for (int i0 = 0; i0 < n; i0 += 8) {
        float m8[8], l8[8], v8[8][E];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int sl = slot_of(min(i0 + j, n - 1));
            m8[j] = i0 + j < n ? ml[sl * 2] : -INFINITY;
            l8[j] = ml[sl * 2 + 1];
#pragma unroll
            for (int e = 0; e < E; ++e) v8[j][e] = po[(size_t)sl * D + e];
        }
        float Mn = M;
#pragma unroll
        for (int j = 0; j < 8; ++j) Mn = fmaxf(Mn, m8[j]);
        const float r = (Mn == -INFINITY) ? 1.f : fast_exp2(M - Mn);
        L *= r;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] *= r;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float w = (m8[j] == -INFINITY) ? 0.f : fast_exp2(m8[j] - Mn);
            L = fmaf(w, l8[j], L);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = fmaf(w, v8[j][e], acc[e]);
        }
        M = Mn;
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = (uint16_t)f32_to_bf16_rne(acc[e] * inv);
}

int32_t compute_units() {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static int32_t cus[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

template <int D, int G, bool FP8>
static hipError_t launch_cascade_f(const CascadeArgs &a, hipStream_t stream) {
    using Geo = PrefillGeom<D, G, 4, FP8>;
    const int prefix_qblocks = cascade_prefix_qblocks(a.max_group_size, G);
    static_assert(Geo::THREADS == kTailThreads, "tail workgroups are tile-sized");
    const int64_t pf_units = (int64_t)a.num_groups * prefix_qblocks * kMaxSegments * a.num_kv_heads;
    const int64_t tail_units = a.tail_workgroups;
    const float scale_log2 = a.scale * 1.4426950408889634f;
    hipLaunchKernelGGL((cascade_kernel<D, G, FP8>), dim3((unsigned)(pf_units + tail_units)),
                       dim3(Geo::THREADS), 0, stream, (const uint16_t *)a.q,
                       (const uint16_t *)a.k_cache, (const uint16_t *)a.v_cache, a.k_scale,
                       a.v_scale, a.block_tables,
                       a.context_lens, a.max_blocks_per_seq, a.max_context_len, a.num_blocks,
                       a.num_seqs, a.num_q_heads, a.num_kv_heads, a.group_starts, a.prefix_lens,
                       a.num_groups, prefix_qblocks, a.partition_tokens, a.max_parts, scale_log2,
                       a.ws_out, a.ws_ml, a.ws_list);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int rows = a.num_seqs * a.num_q_heads;
    hipLaunchKernelGGL((cascade_reduce_kernel<D>), dim3((rows + 3) / 4), dim3(256), 0, stream,
                       a.context_lens, a.max_blocks_per_seq, a.max_context_len, a.num_seqs,
                       a.num_q_heads, a.num_kv_heads, a.group_starts, a.prefix_lens, a.num_groups,
                       prefix_qblocks * Geo::TWG, a.max_parts, a.ws_out, a.ws_ml, a.ws_list,
                       (uint16_t *)a.out);
    return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_cascade_t(const CascadeArgs &a, hipStream_t stream) {
    return a.fp8 ? launch_cascade_f<D, G, true>(a, stream) : launch_cascade_f<D, G, false>(a, stream);
}

template <int D>
static hipError_t launch_cascade_d(const CascadeArgs &a, hipStream_t stream) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_cascade_t<D, 1>(a, stream);
        case 2: return launch_cascade_t<D, 2>(a, stream);
        case 4: return launch_cascade_t<D, 4>(a, stream);
        case 8: return launch_cascade_t<D, 8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_cascade(const CascadeArgs &a, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    return a.head_dim == 64 ? launch_cascade_d<64>(a, stream) : launch_cascade_d<128>(a, stream);
}

// Query blocks of the prefix tiles: a tile holds 4 waves x 32 / G sequences.

PKV_DEBUG_WORD_ACCESS(cascade)

}  // namespace pkv
