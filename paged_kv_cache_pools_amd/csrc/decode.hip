// decode.hip -- split-KV single-query paged attention for decode (gfx950).
//
// Computes, for each sequence s and query head h,
//   out[s][h] = softmax(scale * q[s][h] . K^T) V
// over the sequence's cached tokens 0 .. ctx-1 of KV head h / G, where token t
// lives in physical block block_tables[s][t / 16] at offset t % 16.  This is
// the scaled dot-product attention of the Nano-vLLM engine deep-dive (§3: in
// decode q is one token, K and V are the whole cache) and of the LLM primer
// part 4 (§21.1), with grouped-query heads sharing a KV head (primer §21.1)
// and the cache paged through a block table (deep-dive §2.2, primer §17.7).
//
// Decode reads every cached K and V once and does G multiply-adds per value
// read, so it is bound by HBM bandwidth, not arithmetic; the matrix cores are
// not used.  Design for CDNA4 (64-wide wavefronts):
//  * Work unit = (sequence, KV head, partition of P tokens) = one wavefront.
//    The wave serves all G query heads of the KV head, so each K/V byte is
//    read from HBM exactly once for the whole group.
//  * A (block, KV head) tile is one contiguous 16 x head_dim bf16 run.  Load j
//    of a block moves bytes [1024 j, 1024 j + 1024) of the tile, 16 bytes per
//    lane: lane l sees token j*TPL + l/LPR, elements 8*(l%LPR) .. +8.  Every
//    load instruction is one fully coalesced 1 KiB request.
//  * The lanes sharing a token ("row" r = l / LPR) own all head_dim elements
//    of the row's tokens, so each row runs its own online softmax over the
//    tokens r, TPL+r, 2 TPL+r, ... and rows merge once at the end of the
//    partition.  The per-token partial dot products of one lane are summed
//    across its row by a butterfly that halves the number of live values per
//    step (reduce-scatter), so a lane ends with whole scores for 1..2 of the
//    row's (head, token) pairs instead of duplicating every sum.
//  * Softmax is online and in fp32 with exp2 (log2 e is folded into the
//    scale): running max m, running sum l, accumulator rescaled by
//    exp2(m_old - m_new) -- the max subtraction of the deep-dive's §3.2.
//  * The next block's K and V are loaded while the current block computes.
//  * Partitions write (m, l, unnormalised acc) to the workspace and a second
//    kernel merges them: out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
//    A sequence that fits in one partition is written directly.
//  * Tokens past the context (tail of the last block) are removed by select,
//    never by multiplying with a zero weight, so NaN bits there cannot leak.
#include <math.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

template <int D, int G>
struct DecodeGeom {
    static constexpr int LPR = D / 8;                     // lanes per token row
    static constexpr int TPL = 64 / LPR;                  // tokens per wave-wide load (rows)
    static constexpr int NL = kBlockTokens / TPL;         // loads per block per lane
    static constexpr int NV = NL * G;                     // partial dots per lane per block
    static constexpr int K = NV >= LPR ? NV / LPR : 1;    // whole scores a lane keeps
    static constexpr int REP = NV >= LPR ? 1 : LPR / NV;  // lanes holding the same score
    static constexpr int LPH = LPR / G;                   // lanes of a row holding one head
    static_assert(D == 64 || D == 128, "head_dim");
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
    // score index i = g * NL + j (head g, load j) is kept by lane-in-row
    // holder(i), register slot(i)
    static constexpr int holder(int i) { return NV >= LPR ? i / K : i * REP; }
    static constexpr int slot(int i) { return NV >= LPR ? i % K : 0; }
};

// Butterfly reduce-scatter of N values over the `Width` lanes of a row,
// continuing as an all-reduce once one value is left.  Lane-in-row c keeps
// indices [c*N/Width, (c+1)*N/Width) when N >= Width, else index c / (Width/N).
template <int Width, int N>
__device__ __forceinline__ void row_reduce_scatter(float (&v)[N], int c) {
    constexpr int kMax = N;
    int n = kMax;
#pragma unroll
    for (int delta = Width / 2; delta >= 1; delta >>= 1) {
        if (n > 1) {
            const bool upper = (c & delta) != 0;
            const int h = n / 2;
#pragma unroll
            for (int k = 0; k < kMax / 2; ++k) {
                if (k < h) {
                    const float send = upper ? v[k] : v[h + k];
                    const float keep = upper ? v[h + k] : v[k];
                    v[k] = keep + __shfl_xor(send, delta);
                }
            }
            n = h;
        } else {
            v[0] += __shfl_xor(v[0], delta);
        }
    }
}

template <int D, int G>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t num_blocks, int32_t num_q_heads, int32_t num_kv_heads, int32_t partition_tokens,
    int32_t max_parts, float scale_log2, uint16_t *__restrict__ out, float *__restrict__ ws_out,
    float *__restrict__ ws_ml) {
    using Geo = DecodeGeom<D, G>;
    constexpr int LPR = Geo::LPR, TPL = Geo::TPL, NL = Geo::NL, NV = Geo::NV, K = Geo::K;
    constexpr int LPH = Geo::LPH, REP = Geo::REP;
    const float kNegInf = -INFINITY;

    const int lane = threadIdx.x & 63;
    const int part = blockIdx.x * (blockDim.x >> 6) + wave_id_uniform();
    const int kvh = blockIdx.y;
    const int s = blockIdx.z;
    const int row = lane / LPR;
    const int c = lane % LPR;
    const int row_base = row * LPR;

    int ctx = context_lens[s];
    ctx = min(ctx, min(max_context_len, max_blocks_per_seq * kBlockTokens));
    const int h0 = kvh * G;
    if (ctx <= 0) {
        if (part == 0) {  // empty context: the output is defined as 0
#pragma unroll
            for (int g = 0; g < G; ++g)
                if (g % TPL == row) {
                    uint4 z = {0u, 0u, 0u, 0u};
                    reinterpret_cast<uint4 *>(out + ((size_t)s * num_q_heads + h0 + g) * D)[c] = z;
                }
        }
        return;
    }
    const int t_begin = part * partition_tokens;
    if (t_begin >= ctx) return;
    const int t_end = min(t_begin + partition_tokens, ctx);
    const int nparts = (ctx + partition_tokens - 1) / partition_tokens;

    // this lane's 8 elements of each query head of the group
    float qf[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const uint4 u = reinterpret_cast<const uint4 *>(q + ((size_t)s * num_q_heads + h0 + g) * D)[c];
        unpack8(u, qf[g]);
    }

    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[g][x] = 0.f;
    float m = kNegInf;  // running max of this row for head g(lane), log2 domain
    float l = 0.f;      // running sum of this lane's own weights

    const int32_t *bt = block_tables + (size_t)s * max_blocks_per_seq;
    const size_t tile = (size_t)kBlockTokens * D;  // elements of one (block, head) tile
    const int b_begin = t_begin / kBlockTokens;
    const int b_end = (t_end + kBlockTokens - 1) / kBlockTokens;

    auto tile_ptr = [&](const uint16_t *base, int b) -> const uint4 * {
        int pb = bt[b];
        // an out-of-range id is a caller error; read block 0 instead of faulting
        pb = ((unsigned)pb < (unsigned)num_blocks) ? pb : 0;
        return reinterpret_cast<const uint4 *>(base + ((size_t)pb * num_kv_heads + kvh) * tile) +
               lane;
    };

    uint4 kcur[NL], vcur[NL];
    {
        const uint4 *kp = tile_ptr(k_cache, b_begin);
        const uint4 *vp = tile_ptr(v_cache, b_begin);
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            kcur[j] = kp[j * 64];
            vcur[j] = vp[j * 64];
        }
    }

    for (int b = b_begin; b < b_end; ++b) {
        uint4 knext[NL], vnext[NL];
        if (b + 1 < b_end) {
            const uint4 *kp = tile_ptr(k_cache, b + 1);
            const uint4 *vp = tile_ptr(v_cache, b + 1);
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                knext[j] = kp[j * 64];
                vnext[j] = vp[j * 64];
            }
        }
        const int tb = b * kBlockTokens;
        const bool partial = tb + kBlockTokens > t_end;

        // ---- scores: partial dot products, then the row butterfly
        float v[NV];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            float kf[8];
            unpack8(kcur[j], kf);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = 0.f;
#pragma unroll
                for (int x = 0; x < 8; ++x) d = fmaf(qf[g][x], kf[x], d);
                v[g * NL + j] = d;
            }
        }
        row_reduce_scatter<LPR, NV>(v, c);

        float sc[K];
        float bmax = kNegInf;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            sc[k] = v[k] * scale_log2;
            if (partial) {
                const int i = (NV >= LPR) ? c * K + k : c / REP;
                const int t = tb + (i % NL) * TPL + row;
                sc[k] = (t < t_end) ? sc[k] : kNegInf;
            }
            bmax = fmaxf(bmax, sc[k]);
        }
#pragma unroll
        for (int d = 1; d < LPH; d <<= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, d));

        const float m_new = fmaxf(m, bmax);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;  // no live token yet
        const float alpha = exp2f(m - m_use);
        float p[K];
        float psum = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            p[k] = exp2f(sc[k] - m_use);
            psum += p[k];
        }
        if (REP > 1 && (c % REP) != 0) psum = 0.f;  // a replica: counted once per head
        l = l * alpha + psum;
        m = m_new;

        // ---- rescale the accumulators, then add P V for this row's tokens
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float a = __shfl(alpha, row_base + g * LPH);
#pragma unroll
            for (int x = 0; x < 8; ++x) acc[g][x] *= a;
        }
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            float vf[8];
            unpack8(vcur[j], vf);
            if (partial) {
                const bool live = tb + j * TPL + row < t_end;
#pragma unroll
                for (int x = 0; x < 8; ++x) vf[x] = live ? vf[x] : 0.f;
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int i = g * NL + j;
                const float pg = __shfl(p[Geo::slot(i)], row_base + Geo::holder(i));
#pragma unroll
                for (int x = 0; x < 8; ++x) acc[g][x] = fmaf(pg, vf[x], acc[g][x]);
            }
        }

#pragma unroll
        for (int j = 0; j < NL; ++j) {
            kcur[j] = knext[j];
            vcur[j] = vnext[j];
        }
    }

    // ---- merge the rows: each row holds (m, l, acc) over its own tokens
#pragma unroll
    for (int d = 1; d < LPH; d <<= 1) l += __shfl_xor(l, d);
    float mg[G], lg[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float mr = __shfl(m, row_base + g * LPH);
        const float lr = __shfl(l, row_base + g * LPH);
        float M = mr;
#pragma unroll
        for (int d = LPR; d < 64; d <<= 1) M = fmaxf(M, __shfl_xor(M, d));
        const float f = (mr == kNegInf) ? 0.f : exp2f(mr - M);
        float L = lr * f;
#pragma unroll
        for (int d = LPR; d < 64; d <<= 1) L += __shfl_xor(L, d);
#pragma unroll
        for (int x = 0; x < 8; ++x) {
            float a = acc[g][x] * f;
#pragma unroll
            for (int d = LPR; d < 64; d <<= 1) a += __shfl_xor(a, d);
            acc[g][x] = a;
        }
        mg[g] = M;
        lg[g] = L;
    }

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
    int ctx = context_lens[s];
    ctx = min(ctx, min(max_context_len, max_blocks_per_seq * kBlockTokens));
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
        const float w = exp2f(ml[p * 2] - M);
        L = fmaf(w, ml[p * 2 + 1], L);
#pragma unroll
        for (int e = 0; e < E; ++e) a[e] = fmaf(w, po[(size_t)p * D + e], a[e]);
    }
    const float inv = 1.f / L;
    uint16_t *o = out + (size_t)row_id * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = (uint16_t)f32_to_bf16_rne(a[e] * inv);
}

template <int D, int G>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
    const int waves = a.max_parts >= 4 ? 4 : (a.max_parts >= 2 ? 2 : 1);
    dim3 grid((a.max_parts + waves - 1) / waves, a.num_kv_heads, a.num_seqs);
    const float scale_log2 = a.scale * 1.4426950408889634f;
    hipLaunchKernelGGL((decode_split_kernel<D, G>), grid, dim3(64 * waves), 0, stream,
                       (const uint16_t *)a.q, (const uint16_t *)a.k_cache,
                       (const uint16_t *)a.v_cache, a.block_tables, a.context_lens,
                       a.max_blocks_per_seq, a.max_context_len, a.num_blocks, a.num_q_heads,
                       a.num_kv_heads, a.partition_tokens, a.max_parts, scale_log2,
                       (uint16_t *)a.out, a.ws_out, a.ws_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_parts <= 1) return e;
    const int rows = a.num_seqs * a.num_q_heads;
    hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3((rows + 3) / 4), dim3(256), 0, stream,
                       a.context_lens, a.max_blocks_per_seq, a.max_context_len, a.num_seqs,
                       a.num_q_heads, a.partition_tokens, a.max_parts, a.ws_out, a.ws_ml,
                       (uint16_t *)a.out);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs &a, hipStream_t stream) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_decode_t<D, 1>(a, stream);
        case 2: return launch_decode_t<D, 2>(a, stream);
        case 4: return launch_decode_t<D, 4>(a, stream);
        case 8: return launch_decode_t<D, 8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    return a.head_dim == 64 ? launch_decode_d<64>(a, stream) : launch_decode_d<128>(a, stream);
}

}  // namespace pkv
