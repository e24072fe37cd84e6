// decode_wave.h -- the wavefront-level decode attention shared by the decode
// kernels (decode.hip) and the mixed prefill + decode kernel (mixed.hip).
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
//  * K and V stream through registers two blocks ahead of the compute.
//  * Partitions write (m, l, unnormalised acc) to the workspace and a second
//    kernel merges them: out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
//    A sequence that fits in one partition is written directly.
//  * Tokens past the context (tail of the last block) are removed by select,
//    never by multiplying with a zero weight, so NaN bits there cannot leak.
#pragma once

#include <math.h>

#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// DPP lane-permutation controls (GFX9 encoding).  Each of the first four is
// an involution within a row of 16 lanes that pairs lanes differing in one bit
// b and every lower bit: row_mirror (i <-> 15-i, b = 3), row_half_mirror
// (i <-> i^7 within 8 lanes, b = 2), quad_perm [3,2,1,0] (i <-> i^3, b = 1),
// quad_perm [1,0,3,2] (i <-> i^1, b = 0).  Their xor masks 15, 7, 3, 1 span
// GF(2)^4, so applying a prefix of them sums over a coset of lanes: a butterfly.
constexpr int kDppRowMirror = 0x140;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppQuadRev = 0x1B;
constexpr int kDppQuadSwap = 0xB1;
constexpr int kDppRowBcast = 0x150;  // + k: every lane of a row reads lane k of the row

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// FP8 decode of a context of at most this many keys runs wave_attend (fp32
// weights); longer ones run on the matrix cores with bf16 weights
// (decode_fp8_mfma.h), where a few comparable keys could otherwise leave much
// of the 1e-2 absolute budget to the weights' rounding.
constexpr int kExactDecodeKeys = 128;

// a.lo * b.lo + a.hi * b.hi + c on two packed bf16 pairs (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Cache-policy operand of a buffer load: the nontemporal hint.  Cached K/V is
// streamed through once per launch, so marking the loads nontemporal keeps them
// from displacing reusable lines on their way through the cache hierarchy; on
// the 4 KiB random tile gather of decode it raises the achieved HBM read rate
// by about a tenth.
constexpr int kNontemporal = 2;

// Buffer resource for `bytes` bytes at `base` (raw, 32-bit elements; reads
// past `bytes` return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kNontemporal));
}

__device__ __forceinline__ uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, kNontemporal));
}

__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// Eight OCP E4M3 codes (bytes of u, in order) to four packed bf16 pairs:
// every E4M3 value, subnormals included, is exactly a bf16 value.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}

__device__ __forceinline__ uint4 fp8x8_to_bf16(const uint2 &u) {
    return make_uint4(fp8x2_to_bf16<false>(u.x), fp8x2_to_bf16<true>(u.x),
                      fp8x2_to_bf16<false>(u.y), fp8x2_to_bf16<true>(u.y));
}

// Eight OCP E4M3 codes to fp32.
__device__ __forceinline__ void fp8x8_to_f32(const uint2 &u, float (&f)[8]) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)u.x, false);
    const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)u.x, true);
    const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)u.y, false);
    const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8((int)u.y, true);
    f[0] = a.x;
    f[1] = a.y;
    f[2] = b.x;
    f[3] = b.y;
    f[4] = c.x;
    f[5] = c.y;
    f[6] = d.x;
    f[7] = d.y;
}

// 2^x with the hardware instruction: exact at 0 (2^0 = 1), 0 at -inf, and
// results below the normal range flush to 0 -- all that a softmax weight needs
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// f(integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

template <int D, int G>
struct DecodeGeom {
    static constexpr int LPR = D / 8;              // lanes per token row (16 B each)
    static constexpr int LOG_LPR = ilog2(LPR);
    static constexpr int TPL = 64 / LPR;           // token rows per wave (tokens per load)
    static constexpr int NL = kBlockTokens / TPL;  // loads per block per lane
    static constexpr int M = ilog2(G);             // butterfly steps that split heads
    static constexpr int LPH = LPR / G;            // lanes of a row that end with one head
    static_assert(D == 64 || D == 128, "head_dim");
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
    static_assert(M <= LOG_LPR, "group larger than a row");
    // butterfly step k (0-based) of a row
    static constexpr int ctrl(int k) {
        return LPR == 16 ? (k == 0 ? kDppRowMirror
                                   : k == 1 ? kDppHalfMirror : k == 2 ? kDppQuadRev : kDppQuadSwap)
                         : (k == 0 ? kDppHalfMirror : k == 1 ? kDppQuadRev : kDppQuadSwap);
    }
};

// Step k splitting N head positions of NL tokens each: keep the first half,
// receive the partner's copy of it.  Lane c's list holds, at position p, head
// g(c) ^ p (g(c) = the head the lane ends with); the partner flips bit k of the
// head and every later one, so the partner's entry for my position q sits at
// its position N-1-q -- a fixed register for every lane, hence no selects.
template <int CTRL, int N, int NL, int TOTAL>
__device__ __forceinline__ void head_split_step(float (&v)[TOTAL]) {
#pragma unroll
    for (int q = 0; q < N / 2; ++q)
#pragma unroll
        for (int j = 0; j < NL; ++j) v[q * NL + j] += dpp<CTRL>(v[(N - 1 - q) * NL + j]);
}

template <typename Geo, int K, int TOTAL>
__device__ __forceinline__ void row_butterfly(float (&v)[TOTAL]) {
    if constexpr (K < Geo::LOG_LPR) {
        constexpr int CTRL = Geo::ctrl(K);
        if constexpr (K < Geo::M) {
            head_split_step<CTRL, ((TOTAL / Geo::NL) >> K), Geo::NL>(v);
        } else {
#pragma unroll
            for (int j = 0; j < Geo::NL; ++j) v[j] += dpp<CTRL>(v[j]);
        }
        row_butterfly<Geo, K + 1>(v);
    }
}

// Value of x held by lane `src` of this lane's token row.
template <typename Geo, int SRC>
__device__ __forceinline__ float row_bcast(float x, int row_base) {
    if constexpr (Geo::LPR == 16) {
        return dpp<kDppRowBcast + SRC>(x);
    } else {
        return __shfl(x, row_base + SRC);
    }
}

// The new token of a fused store + decode, as seen by the one wavefront whose
// span holds the sequence's last position: `src_k`/`src_v` point at the
// token's K/V row for this KV head (null when nothing is stored), `dst_k`/
// `dst_v` at its cache row (null when the slot is skipped), and `pos` is the
// position whose cached K/V the row replaces in this wave's arithmetic (-1
// when the slot is not that position's).
// Most wavefronts a decode workgroup has (the single-pass kernel's bound).
constexpr int kMaxDecodeWaves = 8;

struct NewToken {
    const uint4 *src_k = nullptr, *src_v = nullptr;
    uint4 *dst_k = nullptr, *dst_v = nullptr;
    int pos = -1;
    // FP8 cache: the row's code destinations (8 codes per lane) and its scale
    // slots; the row is quantized as the FP8 store does
    uint2 *dst_kq = nullptr, *dst_vq = nullptr;
    float *dst_ks = nullptr, *dst_vs = nullptr;
};

// Rotary position embedding of a sequence's new token: the fp32 table row
// (cos for elements i < d/2, then sin) of its position, or null for none.
struct Rope {
    const float *row = nullptr;
};

// Rotate this lane's 8 elements (8c .. 8c+7) of a head row by the table row:
// elements i and i + d/2 form a pair, held by lanes c and c ^ (LPR/2) of the
// same token row.  `pair` is what this lane hands its partner: the register
// that holds, in the partner, the same head as `u` does here (u itself when
// both lanes hold one head's row).  First half: x1 c - x2 s; second half:
// x2 c + x1 s; each product and sum rounded in fp32 (no fused multiply-add),
// the result rounded to bf16.  Every lane of the wave must call it (it
// shuffles).
template <int D>
__device__ __forceinline__ uint4 rope8(const uint4 &u, const uint4 &pair, const float *row,
                                       int c) {
    constexpr int LPR = D / 8, HALF = LPR / 2;
    const bool first = c < HALF;
    const int i0 = 8 * (c % HALF);
    const float4 c0 = reinterpret_cast<const float4 *>(row + i0)[0];
    const float4 c1 = reinterpret_cast<const float4 *>(row + i0)[1];
    const float4 s0 = reinterpret_cast<const float4 *>(row + D / 2 + i0)[0];
    const float4 s1 = reinterpret_cast<const float4 *>(row + D / 2 + i0)[1];
    const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    const uint4 w = make_uint4(__shfl_xor(pair.x, HALF), __shfl_xor(pair.y, HALF),
                               __shfl_xor(pair.z, HALF), __shfl_xor(pair.w, HALF));
    float x[8], y[8], o[8];
    unpack8(u, x);
    unpack8(w, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float a = __fmul_rn(x[e], cs[e]);
        const float b = __fmul_rn(y[e], sn[e]);
        o[e] = first ? __fsub_rn(a, b) : __fadd_rn(a, b);
    }
    return pack8(o);
}

// FP8 patch of a loaded block: the token row that holds the new token (load
// `load`, lanes with `here_row`) takes the codes and scales staged in LDS
// (codes[0] K, codes[1] V, 8 per lane of the row's LPR lanes).
template <int NL, int LPR>
__device__ __forceinline__ void patch_fp8_row(uint2 (&kt)[NL], uint2 (&vt)[NL], float (&ks)[NL],
                                              float (&vs)[NL], const uint2 (&codes)[2][LPR],
                                              const float (&scales)[2], int load, bool here_row) {
    const int c = (threadIdx.x & 63) % LPR;
    const uint2 kq = codes[0][c], vq = codes[1][c];
    const float ksc = scales[0], vsc = scales[1];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const bool here = j == load && here_row;
        kt[j].x = here ? kq.x : kt[j].x;
        kt[j].y = here ? kq.y : kt[j].y;
        vt[j].x = here ? vq.x : vt[j].x;
        vt[j].y = here ? vq.y : vt[j].y;
        ks[j] = here ? ksc : ks[j];
        vs[j] = here ? vsc : vs[j];
    }
}

// One wavefront's attention over tokens [t_begin, t_end) (t_begin < t_end,
// t_begin a multiple of 16) of sequence s for the G query heads of KV head
// kvh.  On return every lane holds, for each head g of the group, the wave's
// running max mg[g] (log2 domain), weight sum lg[g] and the unnormalised
// output acc[g][0..7] for head_dim elements 8c .. 8c+7 (c = lane % LPR).
//
// FP8 = true reads an FP8 cache (OCP E4M3 codes, one fp32 scale per token and
// KV head in k_scale / v_scale [block][kv head][16]).  The lane layout is the
// bf16 one -- 8 elements per lane per load, 8-byte loads of 512 bytes per
// instruction -- and the K codes become bf16 pairs for the same dot products;
// a token's K scale multiplies its scores, its V scale its weights.
template <int D, int G, bool FP8 = false>
__device__ __forceinline__ void wave_attend(
    const uint16_t *__restrict__ q, const void *k_cache, const void *v_cache,
    const float *k_scale, const float *v_scale, const int32_t *__restrict__ bt,
    int32_t num_blocks, int32_t num_q_heads, int32_t num_kv_heads, float scale_log2, int s,
    int kvh, int t_begin, int t_end, const NewToken &nt, const Rope &rope, float (&acc)[G][8],
    float (&mg)[G], float (&lg)[G]) {
    using Geo = DecodeGeom<D, G>;
    using Tile = typename std::conditional<FP8, uint2, uint4>::type;  // one lane's 8 elements
    constexpr uint32_t EB = FP8 ? 1 : 2;                               // bytes per element
    constexpr int LPR = Geo::LPR, TPL = Geo::TPL, NL = Geo::NL, LPH = Geo::LPH;
    const float kNegInf = -INFINITY;

    const int lane = threadIdx.x & 63;
    const int row = lane / LPR;
    const int c = lane % LPR;
    const int row_base = row * LPR;
    const int my_head = c / LPH;  // the head whose scores this lane ends with
    const int h0 = kvh * G;

    // this lane's 8 elements (4 bf16 pairs) of each query head, in the lane's
    // butterfly order: position p holds head my_head ^ p
    uint4 qp[G];
#pragma unroll
    for (int p = 0; p < G; ++p) {
        const int h = h0 + (my_head ^ p);
        qp[p] = reinterpret_cast<const uint4 *>(q + ((size_t)s * num_q_heads + h) * D)[c];
    }
    if (rope.row != nullptr) {  // uniform: q rotated at the sequence's last position
        // the partner lane c ^ (LPR/2) ends with head my_head ^ (G/2), so its
        // position p ^ (G/2) holds the head this lane's position p holds
        uint4 qr[G];
#pragma unroll
        for (int p = 0; p < G; ++p) qr[p] = rope8<D>(qp[p], qp[p ^ (G / 2)], rope.row, c);
#pragma unroll
        for (int p = 0; p < G; ++p) qp[p] = qr[p];
    }

#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[g][x] = 0.f;
    float m = kNegInf;  // running max of this row's scores for my_head (log2 domain)
    float l = 0.f;      // running sum of this row's weights for my_head

    const size_t tile = (size_t)kBlockTokens * D * EB;  // bytes of one (block, head) tile
    const int b_begin = t_begin / kBlockTokens;
    const int b_end = (t_end + kBlockTokens - 1) / kBlockTokens;

    // Tiles are read with buffer loads: a scalar descriptor per tile (base =
    // the tile, size = one tile) plus a fixed per-lane offset, so the loads
    // need no per-block vector address arithmetic, and a read can never leave
    // the tile.
    const uint32_t lane_off = lane * 8u * EB;
    const int b_last = b_end - 1;
    // Prefetches run up to two blocks past the span; those get an empty
    // buffer range, so they still count as issued loads (the waits stay
    // static) but fetch nothing and return zeros.  Token row r of load j is
    // token j * TPL + r of the block; with FP8 its two scales come along.
    auto load = [&](Tile (&kb)[NL], Tile (&vb)[NL], float (&ks)[NL], float (&vs)[NL], int b) {
        int pb = bt[min(b, b_last)];
        // an out-of-range id is a caller error; read block 0 instead of faulting
        PKV_DEBUG_CHECK((unsigned)pb >= (unsigned)num_blocks && lane == 0, kDbgBlockId, pb,
                        min(b, b_last));
        pb = ((unsigned)pb < (unsigned)num_blocks) ? pb : 0;
        const size_t unit = (size_t)pb * num_kv_heads + kvh;
        const uint32_t bytes = b <= b_last ? (uint32_t)tile : 0u;
        const auto kr = tile_rsrc(static_cast<const char *>(k_cache) + unit * tile, bytes);
        const auto vr = tile_rsrc(static_cast<const char *>(v_cache) + unit * tile, bytes);
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            if constexpr (FP8) {
                kb[j] = buffer_load8(kr, lane_off + j * 512u);
                vb[j] = buffer_load8(vr, lane_off + j * 512u);
            } else {
                kb[j] = buffer_load16(kr, lane_off + j * 1024u);
                vb[j] = buffer_load16(vr, lane_off + j * 1024u);
            }
        }
        if constexpr (FP8) {
            const uint32_t sbytes = b <= b_last ? kBlockTokens * 4u : 0u;
            const auto ksr = tile_rsrc(k_scale + unit * kBlockTokens, sbytes);
            const auto vsr = tile_rsrc(v_scale + unit * kBlockTokens, sbytes);
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                ks[j] = buffer_load_f32(ksr, (j * TPL + row) * 4u);
                vs[j] = buffer_load_f32(vsr, (j * TPL + row) * 4u);
            }
        }
    };

    // fused store: this wave holds the sequence's last position, so it writes
    // the new token's row to its cache slot and, when that slot is the last
    // position's, uses the row in place of what it loads from there (nothing
    // in this launch reads the slot after the write)
    // (uint4 is a struct: its selects are written per 32-bit word, which keeps
    // everything in registers)
    const int patch_block = nt.pos >= 0 ? nt.pos / kBlockTokens : -1;
    const int patch_load = (nt.pos % kBlockTokens) / TPL;
    const bool patch_row = row == (nt.pos % kBlockTokens) % TPL;
    uint4 kn = make_uint4(0u, 0u, 0u, 0u), vn = kn;
    // FP8: the new row's codes and scales wait in LDS for the patch, one slot
    // per wave, instead of holding registers through the loop.  Every token
    // row of the wave quantizes the same row (the group shuffles stay within
    // a row), so every lane writes the slot word it later reads itself.
    __shared__ uint2 nt_codes[FP8 ? kMaxDecodeWaves : 1][2][LPR];
    __shared__ float nt_scales[FP8 ? kMaxDecodeWaves : 1][2];
    if (nt.src_k != nullptr) {  // uniform: only the wave holding the last position
        if constexpr (FP8) {
            if (nt.dst_kq != nullptr) {
                float ksc, vsc;
                const uint2 kq = quantize8<LPR>(nt.src_k[c], ksc);
                const uint2 vq = quantize8<LPR>(nt.src_v[c], vsc);
                if (row == 0) {  // row 0 stores it
                    nt.dst_kq[c] = kq;
                    nt.dst_vq[c] = vq;
                    if (c == 0) {
                        *nt.dst_ks = ksc;
                        *nt.dst_vs = vsc;
                    }
                }
                const int w = wave_id_uniform();
                nt_codes[w][0][c] = kq;
                nt_codes[w][1][c] = vq;
                nt_scales[w][0] = ksc;
                nt_scales[w][1] = vsc;
            }
        } else {
            kn = nt.src_k[c];
            vn = nt.src_v[c];
            if (rope.row != nullptr) kn = rope8<D>(kn, kn, rope.row, c);  // rotated before it is stored
            if (nt.dst_k != nullptr && row == 0) {
                nt.dst_k[c] = kn;
                nt.dst_v[c] = vn;
            }
        }
    }
    auto patch = [&](uint4 &x, const uint4 &y, bool here) {
        x.x = here ? y.x : x.x;
        x.y = here ? y.y : x.y;
        x.z = here ? y.z : x.z;
        x.w = here ? y.w : x.w;
    };

    // (the scales are written only by the FP8 patch; bf16 keeps const arrays)
    using Scales = typename std::conditional<FP8, float[NL], const float[NL]>::type;
    auto process = [&](Tile (&kt)[NL], Tile (&vt)[NL], Scales &ks, Scales &vs, int b) {
        const int tb = b * kBlockTokens;
        const bool partial = tb + kBlockTokens > t_end;
        uint4 kb[NL];  // K as bf16 pairs
        if constexpr (FP8) {
            // (this names no variable the bf16 branch does not name first:
            // the closure's capture order, and with it the bf16 kernels'
            // register allocation, stays as it is without the FP8 patch)
            if (b == patch_block)  // uniform
                patch_fp8_row<NL>(kt, vt, ks, vs, nt_codes[wave_id_uniform()],
                                  nt_scales[wave_id_uniform()], patch_load, patch_row);
#pragma unroll
            for (int j = 0; j < NL; ++j) kb[j] = fp8x8_to_bf16(kt[j]);
        } else {
#pragma unroll
            for (int j = 0; j < NL; ++j) kb[j] = kt[j];
            if (b == patch_block) {
#pragma unroll
                for (int j = 0; j < NL; ++j) {
                    const bool here = j == patch_load && patch_row;
                    patch(kb[j], kn, here);
                    patch(vt[j], vn, here);
                }
            }
        }
        // partial dot products: v[p * NL + j] = q(head at position p) . K(token j)
        // over my 8 elements (bf16 pair dot products accumulate in fp32; bf16 x
        // bf16 products are exact)
        float v[G * NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
#pragma unroll
            for (int p = 0; p < G; ++p) {
                float d = dot2_bf16(qp[p].w, kb[j].w, 0.f);
                d = dot2_bf16(qp[p].z, kb[j].z, d);
                d = dot2_bf16(qp[p].y, kb[j].y, d);
                d = dot2_bf16(qp[p].x, kb[j].x, d);
                v[p * NL + j] = d;
            }
        }
        row_butterfly<Geo, 0>(v);  // v[j] = full score of (my_head, token j of this row)

        float sc[NL];
        float bm = kNegInf;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            sc[j] = (FP8 ? v[j] * ks[j] : v[j]) * scale_log2;
            if (partial) sc[j] = (tb + j * TPL + row < t_end) ? sc[j] : kNegInf;
            bm = fmaxf(bm, sc[j]);
        }
        const float m_new = fmaxf(m, bm);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;  // no live token yet
        const float alpha = fast_exp2(m - m_use);
        float pr[NL];
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            pr[j] = fast_exp2(sc[j] - m_use);
            psum += pr[j];
        }
        l = l * alpha + psum;
        m = m_new;

        // rescale only when some row's maximum moved (alpha != 1 somewhere)
        if (!__all(alpha == 1.f)) {
            static_for<G>([&](auto gc) {
                constexpr int g = decltype(gc)::value;
                const float a = row_bcast<Geo, g * LPH>(alpha, row_base);
#pragma unroll
                for (int x = 0; x < 8; ++x) acc[g][x] *= a;
            });
        }
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            float vf[8];
            float pj = pr[j];  // the weight, times the token's V scale for FP8
            if constexpr (FP8) {
                fp8x8_to_f32(vt[j], vf);
                pj *= vs[j];
            } else {
                unpack8(vt[j], vf);
            }
            if (partial) {  // rows past the end: NaN codes, scales or bits stay out
                const bool live = tb + j * TPL + row < t_end;
#pragma unroll
                for (int x = 0; x < 8; ++x) vf[x] = live ? vf[x] : 0.f;
                pj = live ? pj : 0.f;
            }
            static_for<G>([&](auto gc) {
                constexpr int g = decltype(gc)::value;
                const float pg = row_bcast<Geo, g * LPH>(pj, row_base);
#pragma unroll
                for (int x = 0; x < 8; ++x) acc[g][x] = fmaf(pg, vf[x], acc[g][x]);
            });
        }
    };

    // stream the blocks through three register buffers, loading two blocks
    // ahead of the one being computed.  The prefetches are unconditional (past
    // the end they fetch nothing), so the wait before each block covers only
    // the loads issued before it.
    Tile k0[NL], v0[NL], k1[NL], v1[NL], k2[NL], v2[NL];
    float ks0[NL], vs0[NL], ks1[NL], vs1[NL], ks2[NL], vs2[NL];  // FP8 scales (else unused)
    load(k0, v0, ks0, vs0, b_begin);
    load(k1, v1, ks1, vs1, b_begin + 1);
    for (int b = b_begin;;) {
        load(k2, v2, ks2, vs2, b + 2);
        process(k0, v0, ks0, vs0, b);
        if (++b >= b_end) break;
        load(k0, v0, ks0, vs0, b + 2);
        process(k1, v1, ks1, vs1, b);
        if (++b >= b_end) break;
        load(k1, v1, ks1, vs1, b + 2);
        process(k2, v2, ks2, vs2, b);
        if (++b >= b_end) break;
    }

    // ---- merge the rows: row r holds (m, l, acc) over its own tokens
    static_for<G>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        const float mr = row_bcast<Geo, g * LPH>(m, row_base);
        const float lr = row_bcast<Geo, g * LPH>(l, row_base);
        float M = mr;
#pragma unroll
        for (int d = LPR; d < 64; d <<= 1) M = fmaxf(M, __shfl_xor(M, d));
        const float f = (mr == kNegInf) ? 0.f : fast_exp2(mr - M);
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
    });
}

// Zero output rows of a sequence with an empty context (defined as 0).
template <int D, int G>
__device__ __forceinline__ void write_zero_rows(uint16_t *out, int num_q_heads, int s, int kvh) {
    constexpr int LPR = D / 8, TPL = 64 / LPR;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int g = 0; g < G; ++g)
        if (g % TPL == lane / LPR) {
            const uint4 z = {0u, 0u, 0u, 0u};
            reinterpret_cast<uint4 *>(out + ((size_t)s * num_q_heads + kvh * G + g) * D)[lane % LPR] = z;
        }
}

// The fused store's new token for (sequence s, KV head kvh) of a sequence
// with ctx cached tokens (the new one included): its K/V rows, its cache row
// when slots[s] names a slot in the pool, and the position it stands for when
// that slot is where the block table puts position ctx - 1.  Empty when the
// launch stores nothing (slots == null).
template <int D>
__device__ __forceinline__ NewToken new_token(const uint16_t *k_new, const uint16_t *v_new,
                                              const int32_t *slots, uint16_t *k_cache,
                                              uint16_t *v_cache, const int32_t *bt_row,
                                              int32_t num_blocks, int32_t num_kv_heads, int s,
                                              int kvh, int ctx) {
    NewToken t;
    if (slots == nullptr) return t;
    const size_t src = ((size_t)s * num_kv_heads + kvh) * D;
    t.src_k = reinterpret_cast<const uint4 *>(k_new + src);
    t.src_v = reinterpret_cast<const uint4 *>(v_new + src);
    const int slot = slots[s];
    PKV_DEBUG_CHECK(slot >= 0 && slot / kBlockTokens >= num_blocks && kvh == 0 &&
                        (threadIdx.x & 63) == 0,
                    kDbgSlot, slot, s);
    if (slot < 0 || slot / kBlockTokens >= num_blocks) return t;  // skipped: nothing written
    const size_t dst =
        (((size_t)(slot / kBlockTokens) * num_kv_heads + kvh) * kBlockTokens + slot % kBlockTokens) * D;
    t.dst_k = reinterpret_cast<uint4 *>(k_cache + dst);
    t.dst_v = reinterpret_cast<uint4 *>(v_cache + dst);
    if (ctx > 0) {
        const int last = ctx - 1;
        if ((int64_t)bt_row[last / kBlockTokens] * kBlockTokens + last % kBlockTokens == slot)
            t.pos = last;
    }
    return t;
}

// The new token of a fused FP8 store + decode: as new_token, with the
// destinations in the FP8 code pools (one byte per element) and their scale
// arrays [block][kv head][16].
template <int D>
__device__ __forceinline__ NewToken new_token_fp8(const uint16_t *k_new, const uint16_t *v_new,
                                                  const int32_t *slots, uint8_t *k_codes,
                                                  uint8_t *v_codes, float *k_scale, float *v_scale,
                                                  const int32_t *bt_row, int32_t num_blocks,
                                                  int32_t num_kv_heads, int s, int kvh, int ctx) {
    NewToken t;
    if (slots == nullptr) return t;
    const size_t src = ((size_t)s * num_kv_heads + kvh) * D;
    t.src_k = reinterpret_cast<const uint4 *>(k_new + src);
    t.src_v = reinterpret_cast<const uint4 *>(v_new + src);
    const int slot = slots[s];
    PKV_DEBUG_CHECK(slot >= 0 && slot / kBlockTokens >= num_blocks && kvh == 0 &&
                        (threadIdx.x & 63) == 0,
                    kDbgSlot, slot, s);
    if (slot < 0 || slot / kBlockTokens >= num_blocks) return t;  // skipped: nothing written
    const size_t row =
        ((size_t)(slot / kBlockTokens) * num_kv_heads + kvh) * kBlockTokens + slot % kBlockTokens;
    t.dst_kq = reinterpret_cast<uint2 *>(k_codes + row * D);
    t.dst_vq = reinterpret_cast<uint2 *>(v_codes + row * D);
    t.dst_ks = k_scale + row;
    t.dst_vs = v_scale + row;
    if (ctx > 0) {
        const int last = ctx - 1;
        if ((int64_t)bt_row[last / kBlockTokens] * kBlockTokens + last % kBlockTokens == slot)
            t.pos = last;
    }
    return t;
}

// The rotation for a sequence whose context (the new token included) holds
// ctx tokens: the table row of position ctx - 1, clamped into the table (a
// position past it is a caller error).  Empty when the launch has no table.
template <int D>
__device__ __forceinline__ Rope rope_at(const float *table, int32_t positions, int ctx) {
    Rope r;
    if (table != nullptr) r.row = table + (size_t)min(max(ctx - 1, 0), positions - 1) * D;
    return r;
}

// Write the new token's rows (fused store of a sequence with an empty context).
template <int D>
__device__ __forceinline__ void store_only(const NewToken &t, const Rope &rope) {
    const int lane = threadIdx.x & 63;
    const int c = lane % (D / 8);
    if (t.src_k == nullptr) return;  // uniform
    uint4 kk = t.src_k[c];
    if (t.dst_kq != nullptr) {  // uniform: an FP8 cache; every lane shuffles in quantize8
        float ksc, vsc;
        const uint2 kq = quantize8<D / 8>(kk, ksc);
        const uint2 vq = quantize8<D / 8>(t.src_v[c], vsc);
        if (lane < D / 8) {
            t.dst_kq[lane] = kq;
            t.dst_vq[lane] = vq;
            if (lane == 0) {
                *t.dst_ks = ksc;
                *t.dst_vs = vsc;
            }
        }
        return;
    }
    if (rope.row != nullptr) kk = rope8<D>(kk, kk, rope.row, c);  // all lanes shuffle
    if (t.dst_k != nullptr && lane < D / 8) {
        t.dst_k[lane] = kk;
        t.dst_v[lane] = t.src_v[lane];
    }
}

// One (sequence, KV head) of single-pass decode, run by the W waves of the
// calling workgroup (every thread of it must call): the sequence's blocks are
// split evenly among the waves, each wave runs wave_attend over its share,
// and the waves merge their (m, l, acc) through `smem` (W * G * (D + 2)
// floats).  q and out point at the sequence's [num_q_heads][D] rows; ctx is
// its clamped context length.  make_new_token() gives the fused store's new
// token for this (sequence, KV head) (empty when nothing is stored); it is
// called only by the wave holding the last block.  An empty context writes
// zero rows (and stores its token).
template <int D, int G, bool FP8, typename MakeNewToken>
__device__ __forceinline__ void attend_unit(
    const uint16_t *__restrict__ q, const void *k_cache, const void *v_cache,
    const float *k_scale, const float *v_scale, const int32_t *__restrict__ bt_row, int ctx,
    int32_t num_blocks, int32_t num_q_heads, int32_t num_kv_heads, float scale_log2,
    uint16_t *__restrict__ out, int kvh, int W, float *smem, MakeNewToken make_new_token,
    const Rope &rope) {
    constexpr int LPR = D / 8, TPL = 64 / LPR;
    const int w = wave_id_uniform();
    const int lane = threadIdx.x & 63;
    const int row = lane / LPR;
    const int c = lane % LPR;

    if (ctx <= 0) {
        if (w == 0) {
            write_zero_rows<D, G>(out, num_q_heads, 0, kvh);
            store_only<D>(make_new_token(), rope);
        }
        return;  // uniform over the workgroup: no barrier is skipped
    }
    const int nb = (ctx + kBlockTokens - 1) / kBlockTokens;
    const int b0 = (w * nb) / W, b1 = ((w + 1) * nb) / W;
    // the wave holding the last block carries the fused store
    NewToken nt;
    if (b0 < b1 && b1 == nb) nt = make_new_token();

    float *lds_acc = smem;
    float *lds_m = smem + W * G * D;
    float *lds_l = lds_m + W * G;
    if (b0 < b1) {
        float acc[G][8], mg[G], lg[G];
        wave_attend<D, G, FP8>(q, k_cache, v_cache, k_scale, v_scale, bt_row, num_blocks,
                               num_q_heads, num_kv_heads, scale_log2, 0, kvh, b0 * kBlockTokens,
                               min(b1 * kBlockTokens, ctx), nt, rope, acc, mg, lg);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (g % TPL == row) {
                float4 *dst = reinterpret_cast<float4 *>(lds_acc + (w * G + g) * D + c * 8);
                dst[0] = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
                dst[1] = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
            }
        }
        if (lane < G) {
            // every lane holds every head's totals; lane g publishes head g
            float mv = mg[0], lv = lg[0];
#pragma unroll
            for (int g = 1; g < G; ++g) {
                mv = (lane == g) ? mg[g] : mv;
                lv = (lane == g) ? lg[g] : lv;
            }
            lds_m[w * G + lane] = mv;
            lds_l[w * G + lane] = lv;
        }
    } else if (lane < G) {  // no blocks for this wave: it contributes nothing
        lds_m[w * G + lane] = -INFINITY;
        lds_l[w * G + lane] = 0.f;
    }
    __syncthreads();

    // merge: thread t produces output elements t, t + 64W, ... of the G x D tile
    for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
        const int g = e / D;
        float M = -INFINITY;
        for (int u = 0; u < W; ++u) M = fmaxf(M, lds_m[u * G + g]);
        float num = 0.f, den = 0.f;
        for (int u = 0; u < W; ++u) {
            const float mu = lds_m[u * G + g];
            if (mu == -INFINITY) continue;  // an idle wave (its acc slot is unwritten)
            const float f = fast_exp2(mu - M);
            num = fmaf(f, lds_acc[(u * G + g) * D + (e % D)], num);
            den = fmaf(f, lds_l[u * G + g], den);
        }
        out[((size_t)kvh * G + g) * D + (e % D)] =
            (uint16_t)f32_to_bf16_rne(num / den);
    }
}


}  // namespace pkv
