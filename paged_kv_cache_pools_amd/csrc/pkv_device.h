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

}  // namespace pkv
