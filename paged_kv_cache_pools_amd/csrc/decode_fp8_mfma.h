// decode_fp8_mfma.h -- decode attention over an FP8 cache on the matrix cores
// (gfx950), for spans longer than kExactDecodeKeys keys.
//
// One wavefront computes the attention of the G query heads of one KV head
// over a span of cached tokens whose K and V are OCP E4M3 codes with one fp32
// scale per (token, KV head).  Every E4M3 value is exactly a bf16 value, so
// codes become bf16 MFMA operands without rounding, and both products run on
// v_mfma_f32_16x16x32_bf16 (fp32 accumulation):
//
//   scores   S^T[token][head] = K[token][:] . q[head][:]: A = the block's 16
//            K rows, B = the G query rows (columns G..15 are zero), D/32
//            k-steps.  Lane l ends with tokens 4(l/16) .. 4(l/16)+3 of head
//            l % 16, which it multiplies by their K scales.
//   weights  p = 2^(score - m) per lane, then times the token's V scale and
//            rounded to bf16; the weight sum is taken from the same rounded
//            weights divided by the V scale, so the result is a convex
//            combination of cached V rows (code x scale) whose weights are
//            off by at most 2^-9 relative.
//   output   O^T[dim][head] += V^T[dim][token] . P^T[token][head] over a pair
//            of blocks: the C layout of a block's scores gives each lane 4
//            tokens of one head, and a pair's 4 + 4 are the 8 k-values a lane
//            holds in the B operand of a 32-token product, so the weights need
//            no data movement.  The A operand, 16 dimensions x the same 32
//            tokens, comes from LDS through the transposing read
//            ds_read_b64_tr_b8: within each 16-lane group it hands lane i
//            byte (i % 8) of the 8-byte chunks addressed by lanes 2c + i/8,
//            c = 0..7, so lanes 2c and 2c+1 address token c's two 8-byte
//            halves of a 16-dimension chunk and lane i receives dimension i of
//            the 8 tokens.
//
// The running maximum m of a head is shared by the four lanes holding its
// column and is raised only when some score exceeds it by more than 2^8
// (kFp8RescaleLog2): weights then stay below 2^8, the output (a ratio) does
// not depend on m, and the cross-lane maximum and the rescale of the
// accumulators are skipped for almost every block.
//
// Staging: a block's K codes, V codes and its two rows of 16 scales go from
// global memory straight to LDS (buffer loads with the LDS bit), into a ring
// of four slots per wave with three blocks in flight.  A token row's 16-byte
// chunks sit XOR-swizzled by token (chunk q of row t at position q ^ (t mod
// D/16)), which keeps the K fragment reads and the transposing V reads free of
// bank conflicts.  Every vector-memory instruction of the loop is such a load,
// OPS per block in a fixed order, so "block b has landed" is the immediate
// wait vmcnt <= 2 OPS (the two later blocks' loads) and holds for any span:
// prefetches past the span's end use an empty buffer range and fetch nothing.
#pragma once

#include "decode_wave.h"

#ifndef PKV_FP8_RING
#define PKV_FP8_RING 4
#endif

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_t mfma_bf16_16x16x32(const uint4 &a, const uint4 &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// two fp32 -> packed bf16 (hardware convert, round to nearest even)
__device__ __forceinline__ uint32_t cvt_pk_bf16_rne(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){lo, hi}, bf16x2_t));
}

// a score may exceed its head's running maximum by this much (log2 domain)
// before the maximum is raised
constexpr float kFp8RescaleLog2 = 8.f;

template <int D>
struct Fp8Mma {
    static constexpr int CH = D / 16;                    // 16-byte chunks per token row
    static constexpr int TILE = kBlockTokens * D;        // bytes of a block's K (or V) codes
    static constexpr int SLOT = 2 * TILE + 2 * kBlockTokens * 4;  // K, V, 16 K + 16 V scales
    static constexpr int RING = PKV_FP8_RING;            // slots per wave (even)
    static constexpr int WAVE_BYTES = RING * SLOT;       // LDS per wave
    static constexpr int DMA = TILE / 1024;              // 1 KiB loads per code tile
    static constexpr int OPS = 2 * DMA + 2;              // vector-memory instructions per block
    static constexpr int KS = D / 32;                    // k-steps of the scores
    static constexpr int MT = D / 16;                    // 16-dimension tiles of the output
    static_assert(RING % 2 == 0 && (RING - 2) * OPS < 64, "ring");
    // LDS offset, within a code tile, of chunk q of token row t
    static __device__ __forceinline__ int chunk(int t, int q) {
        return (t * CH + (q ^ (t & (CH - 1)))) * 16;
    }
};

// s_waitcnt immediates (expcnt and the counters not named left at their maxima)
constexpr int waitcnt_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }  // vmcnt <= n < 64
constexpr int kWaitLgkm0 = 0xC07F;                       // lgkmcnt == 0

template <int AUX = kNontemporal>
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, unsigned char *lds,
                                          uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void *)lds, 16, voff, 0, 0, AUX);
}

__device__ __forceinline__ uint2 ds_read_tr8(const unsigned char *p) {
    const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) i32x2_t *)(p));
    return make_uint2((uint32_t)v.x, (uint32_t)v.y);
}

// Two KV heads' scale rows (16 fp32 each) share a 128-byte line.  Units
// (sequence, KV head) are numbered L = s * H + kvh; this gives the workgroup
// with linear id L (one of U = S * H in order) the unit that puts heads 2k and
// 2k + 1 of a sequence on one XCD, back to back: workgroups are dealt to the 8
// XCDs round-robin by linear id, and ids 16a + 8h + x take pair 8a + x, member
// h, so the second head reads the line from its XCD's L2 instead of HBM.  Ids
// past the last whole group of 16, and odd H, keep their unit.
__device__ __forceinline__ void pair_kv_heads(int L, int U, int H, int &s, int &kvh) {
    if ((H & 1) == 0 && L < (U & ~15)) {
        const int pair = 8 * (L >> 4) + (L & 7), h = (L >> 3) & 1;
        s = pair / (H >> 1);
        kvh = 2 * (pair % (H >> 1)) + h;
    }
}

// The wave's attention over tokens [t_begin, t_end) (t_begin a multiple of 16,
// t_begin < t_end) of one sequence: q points at the sequence's [num_q_heads][D]
// query rows, bt at its block-table row, ring at WAVE_BYTES of LDS owned by
// this wave.  On return lane l holds, for head h = l % 16 (meaningful for
// h < G): o[m][r] = the unnormalised output for dimension 16m + 4(l/16) + r,
// m_run = the head's reference maximum (log2 domain) and l_run = its weight
// sum (all four lanes of the head agree on both).  nt is the fused store's new
// token (empty unless this wave holds the sequence's last position).
template <int D, int G>
__device__ __forceinline__ void wave_attend_fp8_mfma(
    const uint16_t *__restrict__ q, const uint8_t *k_cache, const uint8_t *v_cache,
    const float *k_scale, const float *v_scale, const int32_t *__restrict__ bt,
    int32_t num_blocks, int32_t num_q_heads, int32_t num_kv_heads, float scale_log2, int kvh,
    int t_begin, int t_end, const NewToken &nt, unsigned char *ring,
    f32x4_t (&o)[Fp8Mma<D>::MT], float &m_run, float &l_run) {
    using Geo = Fp8Mma<D>;
    constexpr int CH = Geo::CH, TILE = Geo::TILE, SLOT = Geo::SLOT, KS = Geo::KS,
                  MT = Geo::MT, DMA = Geo::DMA, OPS = Geo::OPS;
    constexpr int LPR = D / 8;  // lanes of a row in the store's quantization layout
    const float kNegInf = -INFINITY;
    static_assert(G >= 1 && G <= 16, "group size");

    const int lane = threadIdx.x & 63;
    const int col = lane & 15;  // head of the scores / output; token of a K fragment
    const int grp = lane >> 4;  // k-group: tokens 4grp .. 4grp + 3 of a block

    // query fragments: k-step s, k-value e of group grp is dimension
    // 64(s/2) + 16grp + 8(s%2) + e -- the dimensions a K fragment holds there
    uint4 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int d0 = 64 * (s >> 1) + 16 * grp + 8 * (s & 1);
        qf[s] = col < G ? *reinterpret_cast<const uint4 *>(q + (size_t)(kvh * G + col) * D + d0)
                        : make_uint4(0u, 0u, 0u, 0u);
    }

    // fused store: quantize the new token's row (every lane shuffles), write
    // it from the first row group, and keep it for the patch of its slot
    uint2 kq = make_uint2(0u, 0u), vq = kq;
    float ksc = 0.f, vsc = 0.f;
    if (nt.src_k != nullptr && nt.dst_kq != nullptr) {  // uniform
        const int c = lane % LPR;
        kq = quantize8<LPR>(nt.src_k[c], ksc);
        vq = quantize8<LPR>(nt.src_v[c], vsc);
        if (lane < LPR) {
            nt.dst_kq[c] = kq;
            nt.dst_vq[c] = vq;
            if (lane == 0) {
                *nt.dst_ks = ksc;
                *nt.dst_vs = vsc;
            }
        }
    }
    const int patch_block = nt.pos >= 0 ? nt.pos / kBlockTokens : -1;
    const int patch_tok = nt.pos % kBlockTokens;

#pragma unroll
    for (int m = 0; m < MT; ++m) o[m] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    m_run = kNegInf;
    l_run = 0.f;

    // per-lane LDS offsets, fixed for the whole loop
    uint32_t dma_off[DMA];  // global byte offset in a tile of this lane's 16-byte chunk
#pragma unroll
    for (int i = 0; i < DMA; ++i) {
        const int p = 64 * i + lane;  // LDS chunk position the load writes
        const int t = p / CH, pos = p % CH;
        dma_off[i] = (uint32_t)(t * D + (pos ^ (t & (CH - 1))) * 16);
    }
    int k_off[KS / 2];  // K fragment reads: token col, chunk 4i + grp
#pragma unroll
    for (int i = 0; i < KS / 2; ++i) k_off[i] = Geo::chunk(col, 4 * i + grp);
    // transposing V reads: lane 16grp + 2c + h addresses half h of token
    // 4grp + c % 4 of the pair's first (c < 4) or second block
    const int tr_c = col >> 1, tr_tok = 4 * grp + (tr_c & 3);
    const int tr_base = (tr_c >= 4 ? SLOT : 0) + TILE + 8 * (col & 1);
    int v_off[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) v_off[m] = tr_base + Geo::chunk(tr_tok, m);

    const int b_begin = t_begin / kBlockTokens;
    const int b_end = (t_end + kBlockTokens - 1) / kBlockTokens;
    const int b_last = b_end - 1;
    const int nblk = b_end - b_begin;

    // one block's loads into ring slot `slot`: K codes, V codes, K scales, V
    // scales (past the span: an empty range, nothing fetched, counts kept)
    auto issue = [&](int b, int slot) {
        int pb = bt[min(b, b_last)];
        // an out-of-range id is a caller error; read block 0 instead of faulting
        PKV_DEBUG_CHECK((unsigned)pb >= (unsigned)num_blocks && lane == 0, kDbgBlockId, pb,
                        min(b, b_last));
        pb = ((unsigned)pb < (unsigned)num_blocks) ? pb : 0;
        const size_t unit = (size_t)pb * num_kv_heads + kvh;
        const bool live = b <= b_last;
        unsigned char *sl = ring + slot * SLOT;
        const auto kr = tile_rsrc(k_cache + unit * TILE, live ? (uint32_t)TILE : 0u);
        const auto vr = tile_rsrc(v_cache + unit * TILE, live ? (uint32_t)TILE : 0u);
#pragma unroll
        for (int i = 0; i < DMA; ++i) lds_dma16(kr, sl + 1024 * i, dma_off[i]);
#pragma unroll
        for (int i = 0; i < DMA; ++i) lds_dma16(vr, sl + TILE + 1024 * i, dma_off[i]);
        const auto ksr = tile_rsrc(k_scale + unit * kBlockTokens, live ? 64u : 0u);
        const auto vsr = tile_rsrc(v_scale + unit * kBlockTokens, live ? 64u : 0u);
        if (lane < 4) {  // 4 lanes x 16 bytes per scale row
            // (cached normally: the neighbouring KV head reads the same lines)
            lds_dma16<0>(ksr, sl + 2 * TILE, lane * 16u);
            lds_dma16<0>(vsr, sl + 2 * TILE + 64, lane * 16u);
        }
    };

    // the new token's row replaces what its slot's block holds (the loads
    // may have read the slot before or after the store above)
    auto patch = [&](int b, const unsigned char *slc) {
        if (b != patch_block) return;  // uniform
        unsigned char *sl = const_cast<unsigned char *>(slc);
        if (lane < LPR) {
            const int off = Geo::chunk(patch_tok, lane >> 1) + 8 * (lane & 1);
            *reinterpret_cast<uint2 *>(sl + off) = kq;
            *reinterpret_cast<uint2 *>(sl + TILE + off) = vq;
        }
        if (lane == 0) {
            reinterpret_cast<float *>(sl + 2 * TILE)[patch_tok] = ksc;
            reinterpret_cast<float *>(sl + 2 * TILE + 64)[patch_tok] = vsc;
        }
    };

    // scores and weights of block b (slot at sl): this lane's 4 weights
    // (tokens 4grp .. 4grp + 3, head col) in fp32, times their V scales, and
    // the reciprocal V scales.  They stay fp32 until the pair's P V: a raised
    // maximum rescales the accumulators and the weight sum, and `pending`
    // (the pair's first block's weights, when this is its second) with them.
    struct Weights {
        float w[4], rv[4];
    };
    auto scores = [&](int b, const unsigned char *sl, Weights *pending) {
        uint4 kf[KS];
#pragma unroll
        for (int i = 0; i < KS / 2; ++i) {
            const uint4 raw = *reinterpret_cast<const uint4 *>(sl + k_off[i]);
            kf[2 * i] = fp8x8_to_bf16(make_uint2(raw.x, raw.y));
            kf[2 * i + 1] = fp8x8_to_bf16(make_uint2(raw.z, raw.w));
        }
        f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) sacc = mfma_bf16_16x16x32(kf[s], qf[s], sacc);
        const float4 ks = *reinterpret_cast<const float4 *>(sl + 2 * TILE + 16 * grp);
        const float4 vs = *reinterpret_cast<const float4 *>(sl + 2 * TILE + 64 + 16 * grp);
        const float ksa[4] = {ks.x, ks.y, ks.z, ks.w}, vsa[4] = {vs.x, vs.y, vs.z, vs.w};
        const int t0 = b * kBlockTokens + 4 * grp;  // this lane's first token
        const bool partial = (b + 1) * kBlockTokens > t_end;  // uniform
        float sc[4];
        float lm = kNegInf;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sc[r] = sacc[r] * ksa[r] * scale_log2;
            if (partial) sc[r] = (t0 + r < t_end) ? sc[r] : kNegInf;
            lm = fmaxf(lm, sc[r]);
        }
        if (__any(lm > m_run + kFp8RescaleLog2)) {  // raise the head's maximum
            float mx = fmaxf(lm, __shfl_xor(lm, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mn = fmaxf(m_run, mx);
            const float alpha = (mn == kNegInf) ? 1.f : fast_exp2(m_run - mn);
            m_run = mn;
            l_run *= alpha;
#pragma unroll
            for (int m = 0; m < MT; ++m) o[m] *= alpha;
            if (pending != nullptr) {
#pragma unroll
                for (int r = 0; r < 4; ++r) pending->w[r] *= alpha;
            }
        }
        const float mu = (m_run == kNegInf) ? 0.f : m_run;
        Weights out;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            out.w[r] = fast_exp2(sc[r] - mu) * vsa[r];
            out.rv[r] = __builtin_amdgcn_rcpf(vsa[r]);
            if (partial) {  // tokens past the end: NaN scales stay out
                const bool live = t0 + r < t_end;
                out.w[r] = live ? out.w[r] : 0.f;
                out.rv[r] = live ? out.rv[r] : 0.f;
            }
        }
        return out;
    };
    // a block's weights rounded to bf16 as P V uses them, their sum (the
    // rounded weights over the V scales) added to the head's
    auto round_weights = [&](const Weights &x) {
        const uint2 wb = make_uint2(cvt_pk_bf16_rne(x.w[0], x.w[1]),
                                    cvt_pk_bf16_rne(x.w[2], x.w[3]));
        l_run = fmaf(bf16_lo(wb.x), x.rv[0], l_run);
        l_run = fmaf(bf16_hi(wb.x), x.rv[1], l_run);
        l_run = fmaf(bf16_lo(wb.y), x.rv[2], l_run);
        l_run = fmaf(bf16_hi(wb.y), x.rv[3], l_run);
        return wb;
    };

    // P V over a pair of blocks (slots at pair, pair + SLOT): bx the first
    // block, has_y whether the second exists
    auto pv = [&](const unsigned char *pair, int bx, bool has_y, uint2 wx, uint2 wy) {
        const uint4 pf = make_uint4(wx.x, wx.y, wy.x, wy.y);
        // tokens past the end, and a missing second block: their codes (NaN
        // fill, or a stale slot) stay out
        const bool mask = !has_y || (bx + 2) * kBlockTokens > t_end;  // uniform
        uint32_t mx = ~0u, my = ~0u;
        if (mask) {
            const int tx = bx * kBlockTokens + 4 * grp, ty = tx + kBlockTokens;
            mx = my = 0u;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                mx |= (tx + c < t_end) ? (0xFFu << (8 * c)) : 0u;
                my |= (has_y && ty + c < t_end) ? (0xFFu << (8 * c)) : 0u;
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            uint2 raw = ds_read_tr8(pair + v_off[m]);
            if (mask) {
                raw.x &= mx;
                raw.y &= my;
            }
            o[m] = mfma_bf16_16x16x32(fp8x8_to_bf16(raw), pf, o[m]);
        }
    };

    // ring: block b_begin + k in slot k % RING; RING - 1 blocks in flight
    constexpr int RING = Geo::RING, AHEAD = (RING - 2) * OPS;
#pragma unroll
    for (int k = 0; k < RING - 1; ++k) issue(b_begin + k, k);
    auto pair_step = [&](int i, auto s0c) {
        constexpr int S0 = decltype(s0c)::value;  // slot of the pair's first block
        const int bx = b_begin + i;
        const bool has_y = i + 1 < nblk;  // uniform
        unsigned char *sx = ring + S0 * SLOT;
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(AHEAD));  // block bx has landed
        patch(bx, sx);
        Weights px = scores(bx, sx, nullptr);
        issue(bx + RING - 1, (S0 + RING - 1) % RING);  // the previous pair's second slot
        uint2 wy = make_uint2(0u, 0u);
        if (has_y) {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(AHEAD));  // block bx + 1 has landed
            patch(bx + 1, sx + SLOT);
            const Weights py = scores(bx + 1, sx + SLOT, &px);
            wy = round_weights(py);
        }
        const uint2 wx = round_weights(px);
        pv(sx, bx, has_y, wx, wy);
        if (has_y) {
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // this pair's reads are done
            issue(bx + RING, S0);
        }
    };
    for (int i = 0; i < nblk; i += RING) {
        bool done = false;
        static_for<RING / 2>([&](auto pc) {
            constexpr int P = decltype(pc)::value;
            if (done || i + 2 * P >= nblk) {
                done = true;
                return;
            }
            pair_step(i + 2 * P, std::integral_constant<int, 2 * P>{});
        });
        if (done) break;
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // no load left in flight into the ring

    // the head's weight sum over the four lanes of its column
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
}

// One (sequence, KV head) of single-pass FP8 decode on the matrix cores, run by
// the W waves of the calling workgroup (every thread must call): as
// attend_unit, with smem = W * Fp8Mma<D>::WAVE_BYTES bytes of LDS; each wave's
// (m, l, acc) goes to the start of its own ring after its loop, then the
// workgroup merges them.  ctx > 0.
template <int D, int G, typename MakeNewToken>
__device__ __forceinline__ void attend_unit_fp8_mfma(
    const uint16_t *__restrict__ q, const uint8_t *k_cache, const uint8_t *v_cache,
    const float *k_scale, const float *v_scale, const int32_t *__restrict__ bt_row, int ctx,
    int32_t num_blocks, int32_t num_q_heads, int32_t num_kv_heads, float scale_log2,
    uint16_t *__restrict__ out, int kvh, int W, unsigned char *smem,
    MakeNewToken make_new_token) {
    using Geo = Fp8Mma<D>;
    const int w = wave_id_uniform();
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, grp = lane >> 4;
    const int nb = (ctx + kBlockTokens - 1) / kBlockTokens;
    const int b0 = (w * nb) / W, b1 = ((w + 1) * nb) / W;
    // the wave holding the last block carries the fused store
    NewToken nt;
    if (b0 < b1 && b1 == nb) nt = make_new_token();

    unsigned char *ring = smem + w * Geo::WAVE_BYTES;
    float *res = reinterpret_cast<float *>(ring);  // [G][D] acc, [G] m, [G] l
    if (b0 < b1) {
        f32x4_t o[Geo::MT];
        float mr, lr;
        wave_attend_fp8_mfma<D, G>(q, k_cache, v_cache, k_scale, v_scale, bt_row, num_blocks,
                                   num_q_heads, num_kv_heads, scale_log2, kvh, b0 * kBlockTokens,
                                   min(b1 * kBlockTokens, ctx), nt, ring, o, mr, lr);
        if (col < G) {
#pragma unroll
            for (int m = 0; m < Geo::MT; ++m)
                *reinterpret_cast<float4 *>(res + col * D + 16 * m + 4 * grp) =
                    make_float4(o[m][0], o[m][1], o[m][2], o[m][3]);
            if (grp == 0) {
                res[G * D + col] = mr;
                res[G * D + G + col] = lr;
            }
        }
    } else if (lane < G) {  // no blocks for this wave: it contributes nothing
        res[G * D + lane] = -INFINITY;
        res[G * D + G + lane] = 0.f;
    }
    __syncthreads();

    // merge: thread t produces output elements t, t + 64W, ... of the G x D tile
    constexpr int kStride = Geo::WAVE_BYTES / 4;  // floats between two waves' results
    const float *all = reinterpret_cast<const float *>(smem);
    for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
        const int g = e / D, d = e % D;
        float M = -INFINITY;
        for (int u = 0; u < W; ++u) M = fmaxf(M, all[u * kStride + G * D + g]);
        float num = 0.f, den = 0.f;
        for (int u = 0; u < W; ++u) {
            const float mu = all[u * kStride + G * D + g];
            if (mu == -INFINITY) continue;  // an idle wave (its acc is unwritten)
            const float f = fast_exp2(mu - M);
            num = fmaf(f, all[u * kStride + g * D + d], num);
            den = fmaf(f, all[u * kStride + G * D + G + g], den);
        }
        out[((size_t)kvh * G + g) * D + d] = (uint16_t)f32_to_bf16_rne(num / den);
    }
}

}  // namespace pkv
