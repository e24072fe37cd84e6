// prefill.hip -- chunked causal prefill attention over the paged cache, on
// the gfx950 matrix cores.
//
// Prompt p has c cached tokens and n new ones (their K/V already stored).  New
// token i sits at position c + i and attends to keys 0 .. c + i inclusive:
// itself and what precedes it, never a later token (Nano-vLLM engine
// deep-dive §3.2, lower-triangular causal mask; LLM primer part 4 §22 steps
// 6-8, where the masked weight is exactly 0).  Prefill does O(n * ctx * d)
// work on O(ctx * d) bytes, so unlike decode it is compute-bound (primer
// §17.1) and Q K^T and P V run as bf16 MFMA with fp32 accumulation.
//
// Formulation (chosen for CDNA4's MFMA register layouts):
//   S^T = K Q^T  with A = K rows (keys x d) and B = Q^T (d x query columns),
//   O^T = V^T P^T with A = V^T (d x keys)  and B = P^T (keys x columns).
// In the 16x16 accumulator layout each lane holds 4 consecutive rows of one
// column, so every score a lane holds belongs to ONE query column: the online
// softmax state (max m, sum l) and the rescale of O^T are lane-local, and the
// exponentiated scores become the B operand of the P V product without any
// cross-lane shuffle (the order of the contraction index inside an MFMA is
// free, so both operands use the same key permutation sigma below).
//
// Work split: a workgroup (4 wavefronts) owns one (prompt, KV head, block of
// query tokens); each wave owns 64 query columns = 64/G tokens x the G query
// heads that share the KV head, so every K/V fragment read from LDS feeds 4
// MFMAs.  Keys stream in chunks of 64 (4 cache blocks) gathered through the
// block table into LDS: K row-major (one padded row per key), V transposed
// (one padded row per head_dim element) so the A operand of P V is two 8-byte
// LDS reads.  Padding (16 B per row) keeps the 16-lane LDS reads conflict-free.
// Keys at or past the context end are zero in LDS (V) or masked by select (S),
// so NaN bits in unused slots never reach the output.
#include <math.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4 &a, const uint4 &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Split two finite fp32 softmax weights into bf16 hi and lo parts with
// p == hi + lo to about 2^-16 relative: hi is p truncated to bf16 (its upper
// half), lo is the exact remainder p - hi rounded to bf16.  Using both in the
// P V product keeps the weights' rounding far below the bf16 output rounding.
__device__ __forceinline__ void split2_bf16(float p0, float p1, uint32_t &hi, uint32_t &lo) {
    const uint32_t b0 = __float_as_uint(p0), b1 = __float_as_uint(p1);
    hi = __builtin_amdgcn_perm(b1, b0, 0x07060302u);  // (b0 >> 16) | (b1 & 0xffff0000)
    const float r0 = p0 - __uint_as_float(b0 & 0xffff0000u);
    const float r1 = p1 - __uint_as_float(b1 & 0xffff0000u);
    uint32_t c0 = __float_as_uint(r0), c1 = __float_as_uint(r1);
    c0 += 0x7fffu + ((c0 >> 16) & 1u);
    c1 += 0x7fffu + ((c1 >> 16) & 1u);
    lo = __builtin_amdgcn_perm(c1, c0, 0x07060302u);
}

template <int D, int G>
struct PrefillGeom {
    static constexpr int WAVES = 4;
    static constexpr int COLS = 64;              // query columns per wave
    static constexpr int TW = COLS / G;          // query tokens per wave
    static constexpr int TWG = WAVES * TW;       // query tokens per workgroup
    static constexpr int KC = 64;                // keys per chunk (4 cache blocks)
    static constexpr int KSTEPS = D / 32;        // MFMA k-steps over head_dim
    static constexpr int MT = D / 16;            // head_dim tiles of O^T
    static constexpr int KROW = D * 2 + 16;      // bytes per K row in LDS
    static constexpr int VROW = KC * 2 + 16;     // bytes per V^T row in LDS
    static constexpr int KBYTES = KC * KROW;
    static constexpr int VBYTES = D * VROW;
    static_assert(D == 64 || D == 128, "head_dim");
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
};

template <int D, int G>
__global__ __launch_bounds__(256) void prefill_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ cu_new_lens, const int32_t *__restrict__ context_lens,
    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_blocks, int32_t num_q_heads,
    int32_t num_kv_heads, float scale_log2, uint16_t *__restrict__ out) {
    using Geo = PrefillGeom<D, G>;
    constexpr int TW = Geo::TW, TWG = Geo::TWG, KC = Geo::KC, KSTEPS = Geo::KSTEPS;
    constexpr int MT = Geo::MT, KROW = Geo::KROW, VROW = Geo::VROW;
    const float kNegInf = -INFINITY;

    __shared__ __attribute__((aligned(16))) unsigned char lds_k[Geo::KBYTES];
    __shared__ __attribute__((aligned(16))) unsigned char lds_v[Geo::VBYTES];

    const int p = blockIdx.z;
    const int kvh = blockIdx.y;
    const int qb = gridDim.x - 1 - blockIdx.x;  // late (longest) query blocks start first
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = wave_id_uniform();
    const int a = lane >> 4;   // 16-lane group
    const int col = lane & 15; // column within an N-tile

    const int row0 = cu_new_lens[p];
    int ctx = context_lens[p];
    ctx = min(ctx, min(max_context_len, max_blocks_per_seq * kBlockTokens));
    const int n = min(cu_new_lens[p + 1] - row0, ctx);
    const int c = ctx - n;
    const int T0 = qb * TWG;
    if (n <= 0 || T0 >= n) return;
    const int kend = c + min(T0 + TWG, n);  // keys [0, kend) are visible to someone here

    // ---- Q^T fragments (B operand): column j = nt*16 + col of this wave is
    // token  T0 + w*TW + j / G,  query head  kvh*G + j % G
    uint4 qf[4][KSTEPS];
    int pos[4];  // absolute position of each N-tile's column for this lane
    bool live[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int j = nt * 16 + col;
        const int tok = T0 + w * TW + j / G;
        const int h = kvh * G + j % G;
        live[nt] = tok < n;
        pos[nt] = c + tok;
        const uint4 *src =
            reinterpret_cast<const uint4 *>(q + ((size_t)(row0 + min(tok, n - 1)) * num_q_heads + h) * D);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            uint4 u = src[ks * 4 + a];
            if (!live[nt]) u = make_uint4(0u, 0u, 0u, 0u);
            qf[nt][ks] = u;
        }
    }

    f32x4_t o[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) o[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m[4], l[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        m[nt] = kNegInf;
        l[nt] = 0.f;
    }
    // smallest position among this wave's live columns: chunks wholly below it
    // need no causal mask
    const int wave_min_pos = c + T0 + w * TW;

    const int32_t *bt = block_tables + (size_t)p * max_blocks_per_seq;
    const size_t tile = (size_t)kBlockTokens * D;

    for (int k0 = 0; k0 < kend; k0 += KC) {
        __syncthreads();  // the previous chunk's LDS reads are done
        // ---- stage K rows: 16-byte chunks, one whole cache block per pass
        {
            constexpr int CPB = kBlockTokens * D / 8;  // 16-byte chunks per block tile
            constexpr int ITEMS = KC * D / 8;
#pragma unroll
            for (int it = 0; it < ITEMS / 256; ++it) {
                const int id = it * 256 + tid;
                const int blk = id / CPB;
                const int within = id % CPB;
                const int tok = within / (D / 8);
                const int dc = within % (D / 8);
                const int lb = k0 / kBlockTokens + blk;  // logical block
                uint4 u = make_uint4(0u, 0u, 0u, 0u);
                if (lb * kBlockTokens < ctx) {
                    int pb = bt[lb];
                    pb = ((unsigned)pb < (unsigned)num_blocks) ? pb : 0;
                    u = reinterpret_cast<const uint4 *>(
                        k_cache + ((size_t)pb * num_kv_heads + kvh) * tile)[within];
                }
                *reinterpret_cast<uint4 *>(lds_k + (blk * kBlockTokens + tok) * KROW + dc * 16) = u;
            }
        }
        // ---- stage V transposed: a thread takes 2 consecutive keys x 8
        // elements and writes 8 (key, key+1) pairs into V^T rows
        {
            constexpr int ITEMS = (KC / 2) * (D / 8);
#pragma unroll
            for (int it = 0; it < (ITEMS + 255) / 256; ++it) {
                const int id = it * 256 + tid;
                if (id < ITEMS) {
                    const int pair = id % (KC / 2);
                    const int dc = id / (KC / 2);
                    const int key = k0 + 2 * pair;
                    uint4 u0 = make_uint4(0u, 0u, 0u, 0u), u1 = u0;
                    if (key < ctx) {
                        int pb = bt[key / kBlockTokens];
                        pb = ((unsigned)pb < (unsigned)num_blocks) ? pb : 0;
                        const uint16_t *base = v_cache + ((size_t)pb * num_kv_heads + kvh) * tile;
                        u0 = reinterpret_cast<const uint4 *>(base + (key % kBlockTokens) * D)[dc];
                        if (key + 1 < ctx)  // same block: key is even, blocks hold 16
                            u1 = reinterpret_cast<const uint4 *>(base + (key % kBlockTokens + 1) * D)[dc];
                    }
                    const uint32_t w0[4] = {u0.x, u0.y, u0.z, u0.w};
                    const uint32_t w1[4] = {u1.x, u1.y, u1.z, u1.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t lo = (w0[e] & 0xffffu) | (w1[e] << 16);
                        const uint32_t hi = (w0[e] >> 16) | (w1[e] & 0xffff0000u);
                        *reinterpret_cast<uint32_t *>(lds_v + (dc * 8 + 2 * e) * VROW + pair * 4) = lo;
                        *reinterpret_cast<uint32_t *>(lds_v + (dc * 8 + 2 * e + 1) * VROW + pair * 4) = hi;
                    }
                }
            }
        }
        __syncthreads();

        // ---- S^T = K Q^T over the chunk's 4 key tiles
        f32x4_t s[4][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) s[kt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const uint4 kf = *reinterpret_cast<const uint4 *>(
                    lds_k + (kt * 16 + col) * KROW + (ks * 32 + a * 8) * 2);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) s[kt][nt] = mfma16x16x32(kf, qf[nt][ks], s[kt][nt]);
            }
        }

        // ---- online softmax per column; s[kt][nt][r] is key k0 + 16 kt + 4 a + r
        const bool need_mask = (k0 + KC > wave_min_pos) || (k0 + KC > ctx);
        uint4 ph[2][4], pl[2][4];  // P^T (hi and lo parts) as the B operand, per 32-key step and N-tile
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            float bm = kNegInf;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = s[kt][nt][r] * scale_log2;
                    if (need_mask) {
                        const int key = k0 + kt * 16 + a * 4 + r;
                        v = (key < ctx && key <= pos[nt]) ? v : kNegInf;
                    }
                    s[kt][nt][r] = v;
                    bm = fmaxf(bm, v);
                }
            bm = fmaxf(bm, __shfl_xor(bm, 16));
            bm = fmaxf(bm, __shfl_xor(bm, 32));
            const float m_new = fmaxf(m[nt], bm);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;
            const float alpha = exp2f(m[nt] - m_use);
            m[nt] = m_new;
            float psum = 0.f;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = exp2f(s[kt][nt][r] - m_use);
                    s[kt][nt][r] = e;
                    psum += e;
                }
            l[nt] = l[nt] * alpha + psum;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) o[mt][nt] *= alpha;
            // key permutation sigma: MFMA k-slot (a, 0..3) <- keys 4a..4a+3 of
            // the step's first 16, k-slot (a, 4..7) <- keys 16+4a..16+4a+3
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                split2_bf16(s[2 * kk][nt][0], s[2 * kk][nt][1], ph[kk][nt].x, pl[kk][nt].x);
                split2_bf16(s[2 * kk][nt][2], s[2 * kk][nt][3], ph[kk][nt].y, pl[kk][nt].y);
                split2_bf16(s[2 * kk + 1][nt][0], s[2 * kk + 1][nt][1], ph[kk][nt].z, pl[kk][nt].z);
                split2_bf16(s[2 * kk + 1][nt][2], s[2 * kk + 1][nt][3], ph[kk][nt].w, pl[kk][nt].w);
            }
        }

        // ---- O^T += V^T P^T
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const unsigned char *vrow = lds_v + (mt * 16 + col) * VROW;
                const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + (kk * 32 + a * 4) * 2);
                const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + (kk * 32 + 16 + a * 4) * 2);
                const uint4 vf = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    o[mt][nt] = mfma16x16x32(vf, ph[kk][nt], o[mt][nt]);
                    o[mt][nt] = mfma16x16x32(vf, pl[kk][nt], o[mt][nt]);
                }
            }
        }
    }

    // ---- normalise and write: o[mt][nt][r] is O^T[d = 16 mt + 4 a + r][column]
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        float lt = l[nt];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        if (!live[nt]) continue;
        const float inv = 1.f / lt;
        const int j = nt * 16 + col;
        const int tok = T0 + w * TW + j / G;
        const int h = kvh * G + j % G;
        uint16_t *dst = out + ((size_t)(row0 + tok) * num_q_heads + h) * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            uint2 pk;
            pk.x = pack_bf16x2(o[mt][nt][0] * inv, o[mt][nt][1] * inv);
            pk.y = pack_bf16x2(o[mt][nt][2] * inv, o[mt][nt][3] * inv);
            *reinterpret_cast<uint2 *>(dst + mt * 16 + a * 4) = pk;
        }
    }
}

template <int D, int G>
static hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t stream) {
    using Geo = PrefillGeom<D, G>;
    dim3 grid((a.max_new_len + Geo::TWG - 1) / Geo::TWG, a.num_kv_heads, a.num_seqs);
    const float scale_log2 = a.scale * 1.4426950408889634f;
    hipLaunchKernelGGL((prefill_kernel<D, G>), grid, dim3(256), 0, stream, (const uint16_t *)a.q,
                       (const uint16_t *)a.k_cache, (const uint16_t *)a.v_cache, a.block_tables,
                       a.cu_new_lens, a.context_lens, a.max_blocks_per_seq, a.max_context_len,
                       a.num_blocks, a.num_q_heads, a.num_kv_heads, scale_log2, (uint16_t *)a.out);
    return hipGetLastError();
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
