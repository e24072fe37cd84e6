// pkv_device.h -- small device helpers shared by the gfx950 kernels of libpkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlockTokens = 16;  // tokens per physical block

// bf16 is the upper half of an IEEE binary32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Eight bf16 (one 16-byte load) to fp32.
__device__ __forceinline__ void unpack8(const uint4 &u, float (&f)[8]) {
    f[0] = bf16_lo(u.x);
    f[1] = bf16_hi(u.x);
    f[2] = bf16_lo(u.y);
    f[3] = bf16_hi(u.y);
    f[4] = bf16_lo(u.z);
    f[5] = bf16_hi(u.z);
    f[6] = bf16_lo(u.w);
    f[7] = bf16_hi(u.w);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
    uint4 u;
    u.x = pack_bf16x2(f[0], f[1]);
    u.y = pack_bf16x2(f[2], f[3]);
    u.z = pack_bf16x2(f[4], f[5]);
    u.w = pack_bf16x2(f[6], f[7]);
    return u;
}

// ---- FP8 cache: OCP E4M3 codes with one fp32 scale per (token, KV head) ----
//
// The LLM primer (part 4, §17.6) counts an FP8 KV cache at one byte per
// element.  Each (token, KV head) row of head_dim values is quantized on its
// own: scale = amax / 448 (448 = the largest finite E4M3 magnitude; 1 when
// the row is all zero) and code = E4M3(x / scale), rounded to nearest even,
// with x / scale clamped to [-448, 448] first so the conversion never
// saturates.  Both divisions are correctly rounded fp32.  A group of D/8
// lanes owns a row (8 values per lane, one 16-byte load); the row's amax is
// an all-reduce over the group.

__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
    uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
}

// Quantize this lane's 8 values of a row whose group is LPR lanes wide; every
// lane of the wave must call it (it shuffles across the group).
template <int LPR>
__device__ __forceinline__ uint2 quantize8(const uint4 &u, float &scale) {
    float f[8];
    unpack8(u, f);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    scale = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(__fdiv_rn(f[i], scale), -448.f), 448.f);
    return make_uint2(fp8x4(y[0], y[1], y[2], y[3]), fp8x4(y[4], y[5], y[6], y[7]));
}

__device__ __forceinline__ int wave_id_uniform() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// ---- debug-bounds builds (compiled with PKV_DEBUG_BOUNDS) ----
//
// Device-resident indices (block ids, slots, context lengths, copy pairs) are
// caller preconditions.  Every kernel clamps a broken one so that no access
// leaves the pools; a debug-bounds build also records the first one a kernel
// of this translation unit meets, in the unit's own status word:
//   [0] what broke (kDbg*), [1] the offending value, [2] where it was met (a
//   sequence, token, block-table position or copy pair), [3] how many reports
//   were made in all.
// The first report takes word 0 with a compare-and-swap; the others only
// count.  Ordinary vector-memory atomics on global memory.  The host reads and
// clears the words through pkv_debug_status (pkv_api.cpp).
constexpr uint32_t kDbgBlockId = 1;  // a block id outside [0, num_blocks)
constexpr uint32_t kDbgSlot = 2;     // a slot past the pool
constexpr uint32_t kDbgContext = 3;  // a context length < 0 or past the table / host bound
constexpr uint32_t kDbgCopy = 4;     // a copy pair with an id outside the pool

#ifdef PKV_DEBUG_BOUNDS
static __device__ uint32_t g_debug_word[4];

__device__ __noinline__ void debug_report(uint32_t kind, int32_t value, int32_t where) {
    if (atomicCAS(&g_debug_word[0], 0u, kind) == 0u) {
        g_debug_word[1] = (uint32_t)value;
        g_debug_word[2] = (uint32_t)where;
    }
    atomicAdd(&g_debug_word[3], 1u);
}
#define PKV_DEBUG_CHECK(bad, kind, value, where)             \
    do {                                                     \
        if (bad) ::pkv::debug_report((kind), (value), (where)); \
    } while (0)
// Host access to this translation unit's word: copy it out, optionally clear.
#define PKV_DEBUG_WORD_ACCESS(name)                                                          \
    hipError_t debug_word_##name(uint32_t *out, bool clear) {                                \
        hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_debug_word), 4 * sizeof(uint32_t), \
                                           0, hipMemcpyDeviceToHost);                        \
        if (e == hipSuccess && clear) {                                                      \
            const uint32_t zero[4] = {0u, 0u, 0u, 0u};                                       \
            e = hipMemcpyToSymbol(HIP_SYMBOL(g_debug_word), zero, sizeof zero, 0,            \
                                  hipMemcpyHostToDevice);                                    \
        }                                                                                    \
        return e;                                                                            \
    }
#else
#define PKV_DEBUG_CHECK(bad, kind, value, where) \
    do {                                         \
    } while (0)
#define PKV_DEBUG_WORD_ACCESS(name)                           \
    hipError_t debug_word_##name(uint32_t *out, bool) {       \
        out[0] = out[1] = out[2] = out[3] = 0u;               \
        return hipSuccess;                                    \
    }
#endif

// A context length clamped to the block table and the host-side bound (a
// length past either is a caller error; a negative one reads as empty).
// `reporter`: the one thread that reports a clamp in debug-bounds builds.
__device__ __forceinline__ int clamp_context(int ctx, int32_t max_context_len,
                                             int32_t max_blocks_per_seq, bool reporter,
                                             int where) {
    const int cap = min(max_context_len, max_blocks_per_seq * kBlockTokens);
    PKV_DEBUG_CHECK(reporter && (ctx < 0 || ctx > cap), kDbgContext, ctx, where);
    return min(ctx, cap);
}

}  // namespace pkv
