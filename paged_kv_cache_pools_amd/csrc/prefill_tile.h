// prefill_tile.h -- one query tile of chunked causal prefill attention over
// the paged cache on the gfx950 matrix cores, shared by the prefill kernel
// (prefill.hip) and the mixed prefill + decode kernel (mixed.hip).
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
// softmax state and the rescale of O^T are lane-local, and the exponentiated
// scores become the B operand of the P V product without any cross-lane
// shuffle (the order of the contraction index inside an MFMA is free, so both
// operands use the same key permutation sigma below).
//
// Work split: a workgroup (NW = 4 or 8 wavefronts) owns one (prompt, KV head,
// block of query tokens); each wave owns 32 query columns = 32/G tokens x the G query
// heads that share the KV head, so every K/V fragment read from LDS feeds 2
// MFMAs.  32 columns keep a wave's O^T, Q^T, scores and staging within 256
// registers, so two workgroups share a CU and one's softmax overlaps the
// other's MFMAs.  Keys stream in chunks of 64 (4 cache blocks) gathered through the
// block table: while a chunk is computed from one LDS buffer, the next one is
// loaded into registers and written to the other buffer afterwards, so global
// latency hides behind the MFMAs and one barrier per chunk suffices.  K is
// stored row-major (one row per key, its 16-byte chunks XOR-swizzled), V
// transposed (one padded row per head_dim element) so the A operand of P V is
// two 8-byte LDS reads.
//
// Softmax: scores stay fp32; the scale (log2 e folded in) is applied in the
// FMA that feeds exp2.  The running maximum is raised only when a chunk's
// maximum exceeds it by more than 2^8 (the decision is taken for the whole
// wave), so O^T is rescaled on a few chunks instead of every one; weights are
// then at most 2^8, far from fp32 or bf16 overflow, and the final division by
// the weight sum, accumulated with the same stale maximum, is exact algebra.
// The weights enter the P V product rounded to bf16 (nearest even), and the
// weight sum is taken from those same rounded weights by one more MFMA whose
// A operand is all ones, so the normalisation is consistent with what was
// multiplied into V: out is a convex combination of V rows whose weights are
// off by at most 2^-9 relative, and a row dominated by one key returns that
// key's V with no weight error at all.  Waves whose rows see few keys
// (kPreciseKeys) split each weight into bf16 hi + lo parts and run P V on
// both: such rows can average a handful of V values into an output near 2,
// where half a bf16 ulp already takes most of a 1e-2 absolute budget.
//
// Keys at or past the context end are zero in LDS (V) or masked by select (S),
// so NaN bits in unused slots never reach the output.
//
// FP8 cache: K and V arrive as OCP E4M3 codes
// with one fp32 scale per (token, KV head).  Every E4M3 value is exactly a
// bf16 value, so the codes are converted once per workgroup while staged
// (global -> registers -> LDS, K like V) and the matrix products run on them
// unchanged; the scales enter the scalar work instead.  A key's K scale
// multiplies its scores before the mask and the maximum; its V scale
// multiplies its weights before their rounding to bf16, so P V sums weight
// times code times scale, and the weight sum adds each rounded weight times
// the reciprocal of the V scale, so the normalisation again matches what
// multiplied V (the FP8 decode path's rule).  That sum is the bf16 path's
// weight-sum MFMA with the reciprocal V scales, split into bf16 hi and lo
// parts (p = hi + lo to about 2^-16), in place of the all-ones A operand.
// Keys past the context end get scales 0 in LDS, so their NaN scales never
// reach the output.
#pragma once

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4 &a, const uint4 &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// two fp32 -> packed bf16 (hardware convert, round to nearest even)
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// bf16 ones in both halves of a dword: the A operand that turns the P V MFMA
// into the column sums of P
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;

// A wave whose last query sits below this position (so that every row it
// holds sees at most this many keys) carries the weights in two bf16 parts.
constexpr int kPreciseKeys = 128;

// Split two finite fp32 weights into bf16 hi and lo parts with p == hi + lo
// to about 2^-16 relative: hi is p truncated to bf16 (its upper half), lo the
// remainder p - hi (exact in fp32) rounded to bf16.
__device__ __forceinline__ void split2_bf16(float p0, float p1, uint32_t &hi, uint32_t &lo) {
    const uint32_t b0 = __float_as_uint(p0), b1 = __float_as_uint(p1);
    hi = __builtin_amdgcn_perm(b1, b0, 0x07060302u);  // (b0 >> 16) | (b1 & 0xffff0000)
    lo = cvt_pk_bf16(p0 - __uint_as_float(b0 & 0xffff0000u), p1 - __uint_as_float(b1 & 0xffff0000u));
}

// Reductions across the four 16-lane rows of a wave, in VALU: the gfx950 lane
// swaps hand each lane the value of the same lane in the partner row (16 or
// 32 lanes away), replacing an LDS-crossbar shuffle.
__device__ __forceinline__ float max_xor16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// Eight OCP E4M3 codes (bytes of u, in order) to eight bf16 values, packed in
// pairs: the gfx950 conversion at scale 1 is exact (E4M3 is a subset of bf16).
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
    return make_uint4(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true)));
}

// The running maximum is raised only when it grows by more than this (log2
// units), which bounds every softmax weight by 2^8.
constexpr float kRescaleLog2 = 8.0f;

// s_waitcnt immediate: vector-memory count 0, export and LDS counts left at
// their maxima (no wait on them).
constexpr int kWaitVmcnt0 = 0x0F70;

template <int D, int G, int NW = 4, bool FP8 = false>
struct PrefillGeom {
    static constexpr int WAVES = NW;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int COLS = 32;              // query columns per wave
    static constexpr int NT = COLS / 16;         // 16-column MFMA tiles per wave
    static constexpr int TW = COLS / G;          // query tokens per wave
    static constexpr int TWG = WAVES * TW;       // query tokens per workgroup
    static constexpr int KC = 64;                // keys per chunk (4 cache blocks)
    static constexpr int KSTEPS = D / 32;        // MFMA k-steps over head_dim
    static constexpr int MT = D / 16;            // head_dim tiles of O^T
    static constexpr int KROW = D * 2;           // bytes per K row in LDS (swizzled, unpadded)
    static constexpr int CPR = D / 8;            // 16-byte slots per K row
    static constexpr int RPS = 64 / CPR;         // K rows per 1 KiB direct-load segment
    static constexpr int VROW = KC * 2 + 8;      // bytes per V^T row in LDS (34 dwords)
    static constexpr int KBYTES = KC * KROW;
    static constexpr int VBYTES = D * VROW;
    // FP8: per key of the chunk its K scale and V scale (fp32), and its
    // reciprocal V scale as bf16 hi and lo parts
    static constexpr int SBYTES = FP8 ? 2 * KC * 4 + 2 * KC * 2 : 0;
    static constexpr int BUF = KBYTES + VBYTES + SBYTES;  // one LDS buffer
    static constexpr int CPB = kBlockTokens * D / 8;   // 16-byte chunks per block tile
    static constexpr int KLOADS = KC * D / 8 / THREADS;  // K direct loads per thread
    static constexpr int VITEMS = (KC / 2) * (D / 8) / THREADS;  // V key-pair items per thread
    static constexpr int KITEMS = KC * (D / 16) / THREADS;       // FP8: 16-code K items per thread
    static_assert(D == 64 || D == 128, "head_dim");
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
    static_assert(CPB % 64 == 0 && D % 64 == 0, "a wave's staging stays inside one block");
    static_assert(kBlockTokens % RPS == 0, "a K segment stays inside one block");
    // K slot of 16-byte chunk dc of chunk row r: an XOR swizzle that makes the
    // 16 lanes of an MFMA operand read (16 rows, one chunk) hit 16 distinct
    // bank groups; for D = 64 two rows share a 256-byte bank line, so the
    // swizzle uses the row pair.
    static __device__ __forceinline__ int kslot(int r, int dc) {
        return D == 128 ? (dc ^ (r & 15)) : (dc ^ ((r >> 1) & 7));
    }
};

// One segment's partial result of a split unit: for each wave and each of
// its columns, the unnormalised O (D values), the running maximum m and the
// weight sum l, padded to D + 4 floats so every column starts 16-byte aligned.
constexpr int prefill_partial_col_floats(int D) { return D + 4; }
template <int D, int G>
constexpr int prefill_partial_floats() {
    return PrefillGeom<D, G>::WAVES * PrefillGeom<D, G>::NT * 16 * prefill_partial_col_floats(D);
}

// A split unit gives each segment at least this many key chunks.
constexpr int kMinSegmentChunks = 8;

// Where a split unit keeps its partial results: `slots` segments' partials
// (prefill_partial_floats each), or -- when ws_out is set -- one row per
// (query row, head) of a split-KV workspace, slot slot0 + seg of ws_slots:
// unnormalised O in ws_out [rows][heads][ws_slots][D], (m, l) in ws_ml
// [rows][heads][ws_slots][2], written even when the unit does not split.
struct SplitSlot {
    float *partials = nullptr;
    int seg = 0;    // this workgroup's segment
    int slots = 1;  // most segments the unit may use
    int min_chunks = kMinSegmentChunks;  // fewest key chunks of a segment
    float *ws_out = nullptr, *ws_ml = nullptr;
    int ws_slots = 0, slot0 = 0;
};

// Cross attention over a prefix that several sequences share: n query tokens
// at q rows row0 .. row0 + n - 1 attend to every key in [0, keys) of the
// block-table row bt, with no causal mask (the prefix precedes all of them).
struct CrossGeom {
    int row0 = 0, n = 0, keys = 0;
    const int32_t *bt = nullptr;
};

// Segments a split unit of nchunks key chunks uses (0 .. slots).
__device__ __forceinline__ int prefill_segments(int nchunks, int slots,
                                                int min_chunks = kMinSegmentChunks) {
    return max(1, min(slots, nchunks / min_chunks));
}

// One work unit of chunked prefill -- prompt p, KV head kvh, query block qb
// (tokens qb * TWG .. +TWG of the prompt's new ones) -- run by the calling
// workgroup of NW waves (every thread must call).  `lds` holds 2 * BUF bytes.
// Eight waves share each staged key chunk between twice the query columns of
// four, halving the staging work per matrix operation; the split and shared
// prefix launches, whose partial results are laid out per 4-wave unit, use 4.
//
// SPLIT: the unit's key chunks are divided among up to split.slots
// workgroups (segments of at least split.min_chunks chunks, evenly; a
// workgroup whose segment is empty returns at once).  When the unit has more
// than one segment, each writes its unnormalised (O, m, l) to its slot and
// prefill_merge, run by a later launch, combines them; a unit of one segment
// writes its output directly.
//
// CROSS: the unit's queries and keys come from `cross` instead of prompt p
// (p, cu_new_lens and context_lens are not read).
//
// FP8: k_cache / v_cache hold E4M3 codes (one byte per element, the same
// [block][KV head][16][D] layout) and k_scale / v_scale their fp32 scales
// [block][KV head][16]; `lds` holds 2 * PrefillGeom<D, G, NW, true>::BUF bytes.
template <int D, int G, bool SPLIT = false, bool CROSS = false, int NW = 4, bool FP8 = false>
__device__ __forceinline__ void prefill_unit(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ cu_new_lens, const int32_t *__restrict__ context_lens,
    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_blocks, int32_t num_q_heads,
    int32_t num_kv_heads, float scale_log2, uint16_t *__restrict__ out, int p, int qb, int kvh,
    unsigned char *lds, const SplitSlot &split = SplitSlot{}, const CrossGeom &cross = CrossGeom{},
    const float *__restrict__ k_scale = nullptr, const float *__restrict__ v_scale = nullptr) {
    using Geo = PrefillGeom<D, G, NW, FP8>;
    static_assert(!SPLIT || NW == 4, "split units use the 4-wave partial layout");
    constexpr int TW = Geo::TW, TWG = Geo::TWG, KC = Geo::KC, KSTEPS = Geo::KSTEPS, NT = Geo::NT;
    constexpr int MT = Geo::MT, KROW = Geo::KROW, VROW = Geo::VROW, CPR = Geo::CPR;
    constexpr int KLOADS = Geo::KLOADS, VITEMS = Geo::VITEMS, KITEMS = Geo::KITEMS;
    const uint8_t *const k_codes = reinterpret_cast<const uint8_t *>(k_cache);
    const uint8_t *const v_codes = reinterpret_cast<const uint8_t *>(v_cache);
    const float kNegInf = -INFINITY;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = wave_id_uniform();
    const int a = lane >> 4;    // 16-lane group
    const int col = lane & 15;  // column within an N-tile

    int row0, ctx, n, c;
    const int32_t *bt;
    if constexpr (CROSS) {
        row0 = cross.row0;
        n = cross.n;
        ctx = cross.keys;
        c = 0;
        bt = cross.bt;
        if (ctx <= 0) return;  // uniform: no prefix
    } else {
        row0 = cu_new_lens[p];
        ctx = clamp_context(context_lens[p], max_context_len, max_blocks_per_seq,
                            kvh == 0 && qb == 0 && tid == 0 && (!SPLIT || split.seg == 0), p);
        n = min(cu_new_lens[p + 1] - row0, ctx);
        c = ctx - n;
        bt = block_tables + (size_t)p * max_blocks_per_seq;
    }
    const int T0 = qb * TWG;
    if (n <= 0 || T0 >= n) return;  // uniform over the workgroup
    // keys [0, kend) are visible to some query here
    const int kend = CROSS ? ctx : c + min(T0 + TWG, n);
    const int nchunks = (kend + KC - 1) / KC;
    int j_begin = 0, j_end = nchunks, nseg = 1;
    if constexpr (SPLIT) {
        nseg = prefill_segments(nchunks, split.slots, split.min_chunks);
        if (split.seg >= nseg) return;  // uniform: no segment for this workgroup
        j_begin = split.seg * nchunks / nseg;
        j_end = (split.seg + 1) * nchunks / nseg;
    }

    // a negative scale is applied by flipping the sign of q (exact in bf16),
    // so the softmax below can take the maximum of the raw scores
    const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
    const float sl = fabsf(scale_log2);

    // ---- Q^T fragments (B operand): column j = nt*16 + col of this wave is
    // token  T0 + w*TW + j / G,  query head  kvh*G + j % G
    uint4 qf[NT][KSTEPS];
    int pos[NT];  // absolute position of each N-tile's column for this lane
    bool live[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int j = nt * 16 + col;
        const int tok = T0 + w * TW + j / G;
        const int h = kvh * G + j % G;
        live[nt] = tok < n;
        pos[nt] = CROSS ? INT32_MAX : c + tok;  // cross attention: every key is before the query
        const uint4 *src = reinterpret_cast<const uint4 *>(
            q + ((size_t)(row0 + min(tok, n - 1)) * num_q_heads + h) * D);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            uint4 u = src[ks * 4 + a];
            u = make_uint4(u.x ^ qsign, u.y ^ qsign, u.z ^ qsign, u.w ^ qsign);
            if (!live[nt]) u = make_uint4(0u, 0u, 0u, 0u);
            qf[nt][ks] = u;
        }
    }

    f32x4_t o[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // running max (log2 domain, shared by the column's lanes) and the column's
    // weight sum, which arrives in all 4 rows of ol[nt] (every lane holds it)
    float m[NT];
    f32x4_t ol[NT];
    const uint4 ones = make_uint4(kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m[nt] = kNegInf;
        ol[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // positions of this wave's first and last live token: chunks wholly below
    // the first need no causal mask, chunks wholly above the last are skipped
    const int wave_min_pos = CROSS ? INT32_MAX : c + T0 + w * TW;
    const int wave_max_pos = CROSS ? ctx - 1 : c + min(T0 + (w + 1) * TW, n) - 1;
    const bool wave_live = T0 + w * TW < n;
    const bool precise = wave_max_pos < kPreciseKeys;  // wave-uniform

    const size_t tile = (size_t)kBlockTokens * D;

    // ---- staging of one key chunk.  K goes global -> LDS directly (16-byte
    // loads whose LDS destination is the wave's 1 KiB segment, lane-linear):
    // each lane fetches the global chunk that belongs at its LDS slot, so no
    // register holds K.  V goes global -> registers -> LDS, transposed: thread
    // t moves key pairs (2 keys x 8 elements).  Each wave's share of an
    // instruction lies in one cache block, so the block id is a scalar.  K rows
    // past the context end read some valid block (their scores are masked); V
    // keys past it are zero.
    auto block_id = [&](int lb) {
        int pb = 0;
        if (lb * kBlockTokens < ctx) {
            pb = bt[lb];
            PKV_DEBUG_CHECK((unsigned)pb >= (unsigned)num_blocks && lane == 0, kDbgBlockId, pb, lb);
            pb = ((unsigned)pb < (unsigned)num_blocks) ? pb : 0;
        }
        return pb;
    };
    auto stage_k = [&](unsigned char *buf, int k0) {
        if constexpr (FP8) return;  // FP8 K is staged through registers (stage_load)
#pragma unroll
        for (int it = 0; it < KLOADS; ++it) {
            const int g = it * Geo::WAVES + w;            // 1 KiB segment of the K buffer
            const int r = g * Geo::RPS + lane / CPR;      // key row within the chunk
            const int dc = Geo::kslot(r, lane % CPR);     // chunk this slot holds
            const int pb = block_id(k0 / kBlockTokens + (g * Geo::RPS) / kBlockTokens);
            const uint16_t *src =
                k_cache + (((size_t)pb * num_kv_heads + kvh) * kBlockTokens + r % kBlockTokens) * D +
                dc * 8;
            __builtin_amdgcn_global_load_lds(
                src, (__attribute__((address_space(3))) void *)(buf + g * 1024), 16, 0, 0);
        }
    };
    uint4 vreg[VITEMS][2];
    int keys[VITEMS];  // first key of each V item being staged
    // FP8: the chunk's K codes (16 per item: key row id / (D / 16), codes
    // 16 (id % (D / 16)) ..), V codes (8 per key of each V item), and the K and
    // V scales of key `lane` (wave 0), between their load and their LDS write
    uint4 kcode[FP8 ? KITEMS : 1];
    uint2 vcode[FP8 ? VITEMS : 1][2];
    float ksc = 0.f, vsc = 0.f;
    int staged_k0 = 0;
    auto stage_load_fp8 = [&](int k0) {
        staged_k0 = k0;
#pragma unroll
        for (int it = 0; it < KITEMS; ++it) {
            const int id = it * Geo::THREADS + tid;
            const int r = id / (D / 16), jj = id % (D / 16);
            // a wave's items lie in one cache block (8 or 16 rows)
            const int lb = __builtin_amdgcn_readfirstlane(k0 / kBlockTokens + r / kBlockTokens);
            const uint8_t *src = k_codes +
                                 (((size_t)block_id(lb) * num_kv_heads + kvh) * kBlockTokens + r % kBlockTokens) * D +
                                 jj * 16;
            kcode[it] = *reinterpret_cast<const uint4 *>(src);
        }
#pragma unroll
        for (int it = 0; it < VITEMS; ++it) {
            const int id = it * Geo::THREADS + tid;
            const int blk = __builtin_amdgcn_readfirstlane(id / D);  // D items per block
            const int within = id % D;
            const int pair = within % 8, dc = within / 8;
            const int lb = k0 / kBlockTokens + blk;
            const uint2 *base = reinterpret_cast<const uint2 *>(
                v_codes + ((size_t)block_id(lb) * num_kv_heads + kvh) * kBlockTokens * D);
            vcode[it][0] = base[(2 * pair) * (D / 8) + dc];
            vcode[it][1] = base[(2 * pair + 1) * (D / 8) + dc];
            keys[it] = lb * kBlockTokens + 2 * pair;
        }
        if (w == 0) {  // uniform: one scale pair per key of the chunk
            const int key = k0 + lane;
            const size_t row = ((size_t)block_id(key / kBlockTokens) * num_kv_heads + kvh) * kBlockTokens +
                               key % kBlockTokens;
            ksc = key < ctx ? k_scale[row] : 0.f;
            vsc = key < ctx ? v_scale[row] : 0.f;
        }
    };
    auto stage_load = [&](int k0) {
        if constexpr (FP8) {
            stage_load_fp8(k0);
            return;
        }
#pragma unroll
        for (int it = 0; it < VITEMS; ++it) {
            const int id = it * Geo::THREADS + tid;
            const int blk = __builtin_amdgcn_readfirstlane(id / D);  // D items per block
            const int within = id % D;
            const int pair = within % 8, dc = within / 8;
            const int lb = k0 / kBlockTokens + blk;
            const int key = lb * kBlockTokens + 2 * pair;
            // a key past the context end contributes exactly nothing: its V is
            // zero (the block id is clamped to a valid block before the read)
            const uint4 *base = reinterpret_cast<const uint4 *>(
                v_cache + ((size_t)block_id(lb) * num_kv_heads + kvh) * tile);
            vreg[it][0] = base[(2 * pair) * (D / 8) + dc];
            vreg[it][1] = base[(2 * pair + 1) * (D / 8) + dc];
            keys[it] = key;
        }
        // only the chunk holding the context end has keys past it (uniform)
        if (k0 + KC > ctx) {
#pragma unroll
            for (int it = 0; it < VITEMS; ++it) {
                const uint32_t k0m = keys[it] < ctx ? 0xffffffffu : 0u;
                const uint32_t k1m = keys[it] + 1 < ctx ? 0xffffffffu : 0u;
                uint4 &x0 = vreg[it][0], &x1 = vreg[it][1];
                x0 = make_uint4(x0.x & k0m, x0.y & k0m, x0.z & k0m, x0.w & k0m);
                x1 = make_uint4(x1.x & k1m, x1.y & k1m, x1.z & k1m, x1.w & k1m);
            }
        }
    };
    auto stage_store = [&](unsigned char *buf) {
        unsigned char *lv = buf + Geo::KBYTES;
        if constexpr (FP8) {
            // K: each item's 16 codes as two swizzled 16-byte slots of bf16
#pragma unroll
            for (int it = 0; it < KITEMS; ++it) {
                const int id = it * Geo::THREADS + tid;
                const int r = id / (D / 16), jj = id % (D / 16);
                unsigned char *row = buf + r * KROW;
                *reinterpret_cast<uint4 *>(row + Geo::kslot(r, 2 * jj) * 16) =
                    e4m3x8_to_bf16(kcode[it].x, kcode[it].y);
                *reinterpret_cast<uint4 *>(row + Geo::kslot(r, 2 * jj + 1) * 16) =
                    e4m3x8_to_bf16(kcode[it].z, kcode[it].w);
            }
            if (w == 0) {
                float *sb = reinterpret_cast<float *>(buf + Geo::KBYTES + Geo::VBYTES);
                sb[lane] = ksc;
                sb[KC + lane] = vsc;
                // 1 / V scale as bf16 hi (truncated) + lo (the rest, rounded)
                const float rv = vsc != 0.f ? __builtin_amdgcn_rcpf(vsc) : 0.f;
                const uint32_t rb = __float_as_uint(rv);
                uint16_t *rh = reinterpret_cast<uint16_t *>(sb + 2 * KC);
                rh[lane] = (uint16_t)(rb >> 16);
                rh[KC + lane] = (uint16_t)(cvt_pk_bf16(rv - __uint_as_float(rb & 0xffff0000u), 0.f) & 0xffffu);
            }
            // V: the codes as bf16, zero past the context end (as below)
#pragma unroll
            for (int it = 0; it < VITEMS; ++it) {
                vreg[it][0] = e4m3x8_to_bf16(vcode[it][0].x, vcode[it][0].y);
                vreg[it][1] = e4m3x8_to_bf16(vcode[it][1].x, vcode[it][1].y);
            }
            if (staged_k0 + KC > ctx) {
#pragma unroll
                for (int it = 0; it < VITEMS; ++it) {
                    const uint32_t k0m = keys[it] < ctx ? 0xffffffffu : 0u;
                    const uint32_t k1m = keys[it] + 1 < ctx ? 0xffffffffu : 0u;
                    uint4 &x0 = vreg[it][0], &x1 = vreg[it][1];
                    x0 = make_uint4(x0.x & k0m, x0.y & k0m, x0.z & k0m, x0.w & k0m);
                    x1 = make_uint4(x1.x & k1m, x1.y & k1m, x1.z & k1m, x1.w & k1m);
                }
            }
        }
#pragma unroll
        for (int it = 0; it < VITEMS; ++it) {
            const int id = it * Geo::THREADS + tid;
            const int blk = id / D, within = id % D;
            const int pair = within % 8, dc = within / 8;
            const int kcol = blk * kBlockTokens + 2 * pair;  // key column within the chunk
            const uint32_t w0[4] = {vreg[it][0].x, vreg[it][0].y, vreg[it][0].z, vreg[it][0].w};
            const uint32_t w1[4] = {vreg[it][1].x, vreg[it][1].y, vreg[it][1].z, vreg[it][1].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = __builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u);
                const uint32_t hi = __builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u);
                *reinterpret_cast<uint32_t *>(lv + (dc * 8 + 2 * e) * VROW + kcol * 2) = lo;
                *reinterpret_cast<uint32_t *>(lv + (dc * 8 + 2 * e + 1) * VROW + kcol * 2) = hi;
            }
        }
    };

    // ---- one chunk's attention for this wave, from LDS buffer `buf`, in two
    // halves of 32 keys (Q K^T, softmax, P V each), which keeps the scores of
    // only half a chunk in registers at a time
    auto compute = [&](const unsigned char *buf, int k0) {
        const bool need_mask = (k0 + KC - 1 > wave_min_pos) || (k0 + KC > ctx);
        const unsigned char *lk = buf;
        const unsigned char *lv = buf + Geo::KBYTES;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            // S^T = K Q^T over key tiles 2 hf and 2 hf + 1
            f32x4_t s[2][NT];
            // (both key tiles per k-step: 4 independent accumulators)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) s[t][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            // the half's K fragments, all read before its first MFMA
            uint4 kfr[KSTEPS][2];
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int r = (2 * hf + t) * 16 + col;
                    kfr[ks][t] = *reinterpret_cast<const uint4 *>(lk + r * KROW + Geo::kslot(r, ks * 4 + a) * 16);
                }
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) s[t][nt] = mfma16x16x32(kfr[ks][t], qf[nt][ks], s[t][nt]);
                }
            }
            // FP8: this lane's keys' scales (s[t][nt][r] is key 32 hf + 16 t + 4 a + r)
            float4 fks[2], fvs[2];
            uint4 rvh, rvl;  // A operands of the weight sum: 1 / V scale of the k-slot's key
            if constexpr (FP8) {
                const float *sb = reinterpret_cast<const float *>(buf + Geo::KBYTES + Geo::VBYTES);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int k = hf * 32 + t * 16 + a * 4;
                    fks[t] = *reinterpret_cast<const float4 *>(sb + k);
                    fvs[t] = *reinterpret_cast<const float4 *>(sb + KC + k);
                }
                // k-slots (a, 0..3) and (a, 4..7) hold keys 4a .. and 16 + 4a .. of the half
                const uint16_t *rh = reinterpret_cast<const uint16_t *>(sb + 2 * KC);
                const uint2 h0 = *reinterpret_cast<const uint2 *>(rh + hf * 32 + a * 4);
                const uint2 h1 = *reinterpret_cast<const uint2 *>(rh + hf * 32 + 16 + a * 4);
                const uint2 l0 = *reinterpret_cast<const uint2 *>(rh + KC + hf * 32 + a * 4);
                const uint2 l1 = *reinterpret_cast<const uint2 *>(rh + KC + hf * 32 + 16 + a * 4);
                rvh = make_uint4(h0.x, h0.y, h1.x, h1.y);
                rvl = make_uint4(l0.x, l0.y, l1.x, l1.y);
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        s[t][nt][0] *= fks[t].x;
                        s[t][nt][1] *= fks[t].y;
                        s[t][nt][2] *= fks[t].z;
                        s[t][nt][3] *= fks[t].w;
                    }
            }

            // V^T fragments of the half, read now so the softmax hides their latency
            uint4 vfr[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const unsigned char *vrow = lv + (mt * 16 + col) * VROW;
                const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + (hf * 32 + a * 4) * 2);
                const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + (hf * 32 + 16 + a * 4) * 2);
                vfr[mt] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }

            // the causal and context-end mask, for the chunks that cross either
            // (s[t][nt][r] is key k0 + 32 hf + 16 t + 4 a + r): one uniform
            // branch around all of it; bit (t NT + nt) 4 + r of `dead` marks a
            // removed score, whose weight is set to 0 below
            uint32_t dead = 0;
            if (need_mask) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int key = k0 + hf * 32 + t * 16 + a * 4 + r;
                            const bool keep = key < ctx && key <= pos[nt];
                            s[t][nt][r] = keep ? s[t][nt][r] : kNegInf;
                            dead |= (keep ? 0u : 1u) << ((t * NT + nt) * 4 + r);
                        }
            }
            // per column: is some raw score more than 2^8 above the running
            // maximum?  Each lane tests its own scores; only when some lane
            // finds one (rare after the first chunks) are the column maxima
            // taken across lanes and the maxima raised (and O rescaled), a
            // wave-wide decision, so the branch is uniform
            float lmax[NT];
            bool grow = false;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                float bm = kNegInf;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) bm = fmaxf(bm, s[t][nt][r]);
                lmax[nt] = bm;
                grow |= (bm != kNegInf) && (bm * sl > m[nt] + kRescaleLog2);
            }
            if (__any(grow)) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const float bm = max_xor32(max_xor16(lmax[nt]));
                    const float bms = (bm == kNegInf) ? kNegInf : bm * sl;
                    const float mc = fmaxf(m[nt], bms);
                    const float alpha = (mc == kNegInf) ? 1.f : exp2f(m[nt] - mc);
                    m[nt] = mc;
                    ol[nt] *= alpha;
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) o[mt][nt] *= alpha;
                }
            }

            // weights and P^T as the B operand (bf16).  Key permutation sigma:
            // MFMA k-slot (a, 0..3) <- keys 4a..4a+3 of the half's first 16,
            // k-slot (a, 4..7) <- keys 16+4a..16+4a+3
            uint4 ph[NT], pl[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float mu = (m[nt] == kNegInf) ? 0.f : m[nt];
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        s[t][nt][r] = __builtin_amdgcn_exp2f(fmaf(s[t][nt][r], sl, -mu));
            }
            // a removed score is weight 0 (exp2 gives 0 for it except when sl is
            // 0, where -inf * 0 is NaN): again only for the chunks that masked
            if (need_mask) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            s[t][nt][r] = (dead >> ((t * NT + nt) * 4 + r)) & 1u ? 0.f : s[t][nt][r];
            }
            if constexpr (FP8) {  // weight times V scale (0 past the context end)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        s[t][nt][0] *= fvs[t].x;
                        s[t][nt][1] *= fvs[t].y;
                        s[t][nt][2] *= fvs[t].z;
                        s[t][nt][3] *= fvs[t].w;
                    }
            }
            if (precise) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    split2_bf16(s[0][nt][0], s[0][nt][1], ph[nt].x, pl[nt].x);
                    split2_bf16(s[0][nt][2], s[0][nt][3], ph[nt].y, pl[nt].y);
                    split2_bf16(s[1][nt][0], s[1][nt][1], ph[nt].z, pl[nt].z);
                    split2_bf16(s[1][nt][2], s[1][nt][3], ph[nt].w, pl[nt].w);
                }
            } else {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    ph[nt].x = cvt_pk_bf16(s[0][nt][0], s[0][nt][1]);
                    ph[nt].y = cvt_pk_bf16(s[0][nt][2], s[0][nt][3]);
                    ph[nt].z = cvt_pk_bf16(s[1][nt][0], s[1][nt][1]);
                    ph[nt].w = cvt_pk_bf16(s[1][nt][2], s[1][nt][3]);
                }
            }

            // O^T += V^T P^T over the half's 32 keys, two head_dim tiles at a
            // time so that 4 independent accumulators separate each MFMA from
            // the one that reads its result
#pragma unroll
            for (int mt = 0; mt < MT; mt += 2) {
                const uint4 vf[2] = {vfr[mt], vfr[mt + 1]};
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        o[mt + u][nt] = mfma16x16x32(vf[u], ph[nt], o[mt + u][nt]);
            }
            // the weight sums of the half, from the same bf16 weights (FP8:
            // each over its key's V scale)
            auto fp8_sum = [&](const uint4 (&p)[NT]) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    ol[nt] = mfma16x16x32(rvh, p[nt], ol[nt]);
                    ol[nt] = mfma16x16x32(rvl, p[nt], ol[nt]);
                }
            };
            if constexpr (FP8) {
                fp8_sum(ph);
            } else {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) ol[nt] = mfma16x16x32(ones, ph[nt], ol[nt]);
            }
            if (precise) {  // the lo parts, into O and the sums alike
#pragma unroll
                for (int mt = 0; mt < MT; mt += 2) {
                    const uint4 vf[2] = {vfr[mt], vfr[mt + 1]};
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
                            o[mt + u][nt] = mfma16x16x32(vf[u], pl[nt], o[mt + u][nt]);
                }
                if constexpr (FP8) {
                    fp8_sum(pl);
                } else {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) ol[nt] = mfma16x16x32(ones, pl[nt], ol[nt]);
                }
            }
        }
    };

    // ---- the chunk pipeline: compute chunk j from buffer j % 2 while chunk
    // j + 1 travels global -> registers; the registers go to the other buffer
    // after the compute.  That buffer was last read in chunk j - 1, which every
    // wave finished before the previous barrier.
    // The direct K loads complete asynchronously: every wave waits for its own
    // (vmcnt 0) before the barrier that publishes the buffer.
    stage_k(lds, j_begin * KC);
    stage_load(j_begin * KC);
    stage_store(lds);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    for (int j = j_begin; j < j_end; ++j) {
        const int k0 = j * KC;
        const bool more = j + 1 < j_end;
        if (more) {
            stage_k(lds + ((j + 1 - j_begin) & 1) * Geo::BUF, k0 + KC);
            stage_load(k0 + KC);
        }
        if (wave_live && k0 <= wave_max_pos) compute(lds + ((j - j_begin) & 1) * Geo::BUF, k0);
        if (more) stage_store(lds + ((j + 1 - j_begin) & 1) * Geo::BUF);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
    }

    // ---- the column sums of the weights (each lane holds its column's)
    float lt[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) lt[nt] = ol[nt][0];

    if constexpr (SPLIT) {
        if (split.ws_out != nullptr) {  // uniform: rows of a split-KV workspace
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if (!live[nt]) continue;
                const int j = nt * 16 + col;
                const int tok = T0 + w * TW + j / G;
                const size_t r = ((size_t)(row0 + tok) * num_q_heads + kvh * G + j % G) * split.ws_slots +
                                 split.slot0 + split.seg;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    *reinterpret_cast<f32x4_t *>(split.ws_out + r * D + mt * 16 + a * 4) = o[mt][nt];
                if (a == 0) {
                    split.ws_ml[r * 2] = m[nt];
                    split.ws_ml[r * 2 + 1] = lt[nt];
                }
            }
            return;
        }
        if (nseg > 1) {
            // publish this segment: o[mt][nt][r] is O^T[d = 16 mt + 4 a + r][column]
            constexpr int COLF = prefill_partial_col_floats(D);
            float *mine = split.partials + (size_t)split.seg * prefill_partial_floats<D, G>() +
                          (size_t)w * NT * 16 * COLF;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                float *colp = mine + (nt * 16 + col) * COLF;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    *reinterpret_cast<f32x4_t *>(colp + mt * 16 + a * 4) = o[mt][nt];
                if (a == 0) {
                    colp[D] = m[nt];
                    colp[D + 1] = lt[nt];
                }
            }
            return;
        }
    }

    // ---- normalise and write: o[mt][nt][r] is O^T[d = 16 mt + 4 a + r][column]
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if (!live[nt]) continue;
        const float inv = 1.f / lt[nt];
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


// Workgroups (of 256 threads) that merge one split unit: a thread takes one
// column and 8 consecutive head_dim elements of it.
template <int D, int G>
constexpr int prefill_merge_parts() {
    return PrefillGeom<D, G>::WAVES * PrefillGeom<D, G>::NT * 16 * (D / 8) / 256;
}

// Combine the segments of one split prefill unit (prompt p, query block qb,
// KV head kvh) written by prefill_unit<SPLIT>: for each of the unit's columns
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over its segments in
// order, M = max_s m_s.  A unit that did not split returns at once (its
// output is written).  Workgroup `part` of the unit's prefill_merge_parts
// calls with all 256 threads; thread t takes column part * 256 / (D / 8) +
// t / (D / 8) and elements 8 (t % (D / 8)) .. +8.  Every segment's loads are
// issued before the first is used.
template <int D, int G>
__device__ __forceinline__ void prefill_merge(
    const int32_t *__restrict__ cu_new_lens, const int32_t *__restrict__ context_lens,
    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_q_heads,
    uint16_t *__restrict__ out, int p, int qb, int kvh, const float *__restrict__ partials,
    int slots, int part) {
    using Geo = PrefillGeom<D, G>;
    constexpr int TW = Geo::TW, TWG = Geo::TWG, KC = Geo::KC, NT = Geo::NT;
    constexpr int COLF = prefill_partial_col_floats(D), SLOT = prefill_partial_floats<D, G>();
    constexpr int SLICES = D / 8, COLS_PER_WG = 256 / SLICES;
    const int row0 = cu_new_lens[p];
    const int ctx = clamp_context(context_lens[p], max_context_len, max_blocks_per_seq, false, p);
    const int n = min(cu_new_lens[p + 1] - row0, ctx);
    const int c = ctx - n;
    const int T0 = qb * TWG;
    if (n <= 0 || T0 >= n) return;
    const int kend = c + min(T0 + TWG, n);
    const int nseg = prefill_segments((kend + KC - 1) / KC, slots);
    if (nseg <= 1) return;  // uniform: written by its only segment

    const int cidx = part * COLS_PER_WG + threadIdx.x / SLICES;  // column = w * 32 + j
    const int d0 = (threadIdx.x % SLICES) * 8;
    const int w = cidx / (NT * 16), j = cidx % (NT * 16);
    const int tok = T0 + w * TW + j / G;
    if (tok >= n) return;  // a column past the prompt's new tokens
    const float *col0 = partials + (size_t)cidx * COLF;
    float ms[kMaxSegments], ls[kMaxSegments];
    f32x4_t a0[kMaxSegments], a1[kMaxSegments];
#pragma unroll
    for (int sg = 0; sg < kMaxSegments; ++sg) {
        if (sg < nseg) {
            const float *colp = col0 + (size_t)sg * SLOT;
            ms[sg] = colp[D];
            ls[sg] = colp[D + 1];
            a0[sg] = *reinterpret_cast<const f32x4_t *>(colp + d0);
            a1[sg] = *reinterpret_cast<const f32x4_t *>(colp + d0 + 4);
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int sg = 0; sg < kMaxSegments; ++sg)
        if (sg < nseg) M = fmaxf(M, ms[sg]);
    f32x4_t o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0;
    float L = 0.f;
#pragma unroll
    for (int sg = 0; sg < kMaxSegments; ++sg) {
        if (sg < nseg) {
            const float f = (ms[sg] == -INFINITY) ? 0.f : exp2f(ms[sg] - M);
            L = fmaf(f, ls[sg], L);
            o0 += f * a0[sg];
            o1 += f * a1[sg];
        }
    }
    const float inv = 1.f / L;
    uint4 pk;
    pk.x = pack_bf16x2(o0[0] * inv, o0[1] * inv);
    pk.y = pack_bf16x2(o0[2] * inv, o0[3] * inv);
    pk.z = pack_bf16x2(o1[0] * inv, o1[1] * inv);
    pk.w = pack_bf16x2(o1[2] * inv, o1[3] * inv);
    *reinterpret_cast<uint4 *>(out + ((size_t)(row0 + tok) * num_q_heads + kvh * G + j % G) * D + d0) = pk;
}

}  // namespace pkv
