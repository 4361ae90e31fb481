// common.hpp — device helpers shared by the libds4attn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds4a {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).
// Lane layout (wave64): A: lane l holds A[l%16][8*(l/16) + 0..7];
// B: lane l holds B[8*(l/16) + 0..7][l%16]; D: lane l holds D[4*(l/16) + 0..3][l%16].
// Any permutation of the k index that A and B share gives the same sum.
__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) {
    return __builtin_bit_cast(bf16x8, v);
}

// Round-to-nearest-even fp32 -> bf16 bit pattern (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi): 16 significant bits of x.
__device__ __forceinline__ void split_hi_lo(float x, uint32_t &hi, uint32_t &lo) {
    hi = f32_to_bf16_bits(x);
    lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}

// Pack 8 floats into bf16x8 hi and lo halves.
__device__ __forceinline__ void pack_hi_lo8(const float (&v)[8], bf16x8 &hi, bf16x8 &lo) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t h0, l0, h1, l1;
        split_hi_lo(v[2 * i], h0, l0);
        split_hi_lo(v[2 * i + 1], h1, l1);
        h[i] = h0 | (h1 << 16);
        l[i] = l0 | (l1 << 16);
    }
    hi = as_bf16x8(h);
    lo = as_bf16x8(l);
}

// f16 bit pattern -> float (exact).
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
    return (float)v;
}

// Order-preserving map of a float to uint32: a > b  <=>  key(a) > key(b);
// -0 is folded onto +0 so that equal floats give equal keys.
__device__ __forceinline__ uint32_t float_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_xor_sum(float v, int mask) {
    return v + __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float wave_xor_max(float v, int mask) {
    return fmaxf(v, __shfl_xor(v, mask, kWave));
}

// Fully clamped read of a per-query visible-row count.
__device__ __forceinline__ int64_t clamp_nvis(const int32_t *n_vis, int64_t q, int64_t N) {
    if (!n_vis) return N;
    int64_t v = n_vis[q];
    return v < 0 ? 0 : (v > N ? N : v);
}

}  // namespace ds4a
