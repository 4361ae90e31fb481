// common.hpp — device helpers shared by the libds4attn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds4a {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).
// Lane layout (wave64): A: lane l holds A[l%16][8*(l/16) + 0..7];
// B: lane l holds B[8*(l/16) + 0..7][l%16]; D: lane l holds D[4*(l/16) + 0..3][l%16].
// Any permutation of the k index that A and B share gives the same sum.
__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Same shape with f16 operands (v_mfma_f32_16x16x32_f16).
__device__ __forceinline__ f32x4 mfma16h(const f16x8 &a, const f16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) {
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f16x8 as_f16x8(const u32x4 &v) {
    return __builtin_bit_cast(f16x8, v);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, source lane j supplies 4 consecutive
// 16-bit values of block row j/4 (columns 4*(j%4)..+3) of a 4 x 16 block; lane i receives
// column i (rows 0..3).  p must point into LDS and be 8-byte aligned.
__device__ __forceinline__ s16x4 lds_read_tr16(const unsigned char *p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
}

// Round-to-nearest-even fp32 -> bf16 bit pattern (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// 8 OCP E4M3FN codes (byte k = element k) -> the same 8 values as bf16 (exact: every E4M3
// value is a bf16 value); v_cvt_scalef32_pk_bf16_fp8 with scale 1 converts two at a time.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(u32x2 v) {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true))};
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi): 16 significant bits of x.
__device__ __forceinline__ void split_hi_lo(float x, uint32_t &hi, uint32_t &lo) {
    hi = f32_to_bf16_bits(x);
    lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}

// 8 floats -> bf16 hi = rne(v) and lo = rne(v - hi) (v_cvt_pk_bf16_f32, round-to-nearest-even).
__device__ __forceinline__ void pack_hi_lo8(const float (&v)[8], bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2 x = {v[2 * i], v[2 * i + 1]};
        const bf16x2 h = __builtin_convertvector(x, bf16x2);
        const f32x2 hf = __builtin_convertvector(h, f32x2);
        const bf16x2 l = __builtin_convertvector(x - hf, bf16x2);
        hi[2 * i] = h[0];
        hi[2 * i + 1] = h[1];
        lo[2 * i] = l[0];
        lo[2 * i + 1] = l[1];
    }
}

// 8 floats -> f16 hi = rne(v) and lo = rne(v - hi).
__device__ __forceinline__ void pack_hi_lo8_f16(const float (&v)[8], f16x8 &hi, f16x8 &lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hi[i] = (_Float16)v[i];
        lo[i] = (_Float16)(v[i] - (float)hi[i]);
    }
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
    u = u == 0x80000000u ? 0u : u;                 // -0 ties with +0
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);   // negative: all bits flip; else the sign bit
}

// ---- DPP (data-parallel primitives on VALU lanes, no LDS round trip)
// dpp_ctrl codes: row_shr:n = 0x110 + n, row_ror:n = 0x120 + n, row_bcast:15 = 0x142, row_bcast:31 = 0x143.
// Lanes whose DPP source does not exist read 0 (old = 0, bound_ctrl off).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t x) {
    x += dpp_u32<0x111>(x);          // row_shr:1
    x += dpp_u32<0x112>(x);          // row_shr:2
    x += dpp_u32<0x114>(x);          // row_shr:4
    x += dpp_u32<0x118>(x);          // row_shr:8   -> prefix within each row of 16
    x += dpp_u32<0x142, 0xA>(x);     // row_bcast:15 into rows 1 and 3
    x += dpp_u32<0x143, 0xC>(x);     // row_bcast:31 into rows 2 and 3
    return x;
}

// Sum over the 16 lanes of each row; every lane of the row receives it.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f32<0x128>(x);          // row_ror:8
    x += dpp_f32<0x124>(x);          // row_ror:4
    x += dpp_f32<0x122>(x);          // row_ror:2
    x += dpp_f32<0x121>(x);          // row_ror:1
    return x;
}

// Min and max over the 64 lanes of a wave (uniform result).
__device__ __forceinline__ void wave_minmax_u32(uint32_t &mn, uint32_t &mx) {
#define DS4A_ROW_ROR(n)                                                         \
    {                                                                           \
        const uint32_t a = (uint32_t)__builtin_amdgcn_update_dpp((int)mn, (int)mn, 0x120 + (n), 0xF, 0xF, false); \
        const uint32_t b = (uint32_t)__builtin_amdgcn_update_dpp((int)mx, (int)mx, 0x120 + (n), 0xF, 0xF, false); \
        mn = a < mn ? a : mn;                                                   \
        mx = b > mx ? b : mx;                                                   \
    }
    DS4A_ROW_ROR(8) DS4A_ROW_ROR(4) DS4A_ROW_ROR(2) DS4A_ROW_ROR(1)
#undef DS4A_ROW_ROR
    uint32_t m0 = __builtin_amdgcn_readlane(mn, 0), m1 = __builtin_amdgcn_readlane(mn, 16);
    uint32_t m2 = __builtin_amdgcn_readlane(mn, 32), m3 = __builtin_amdgcn_readlane(mn, 48);
    uint32_t x0 = __builtin_amdgcn_readlane(mx, 0), x1 = __builtin_amdgcn_readlane(mx, 16);
    uint32_t x2 = __builtin_amdgcn_readlane(mx, 32), x3 = __builtin_amdgcn_readlane(mx, 48);
    m0 = m0 < m1 ? m0 : m1;
    m2 = m2 < m3 ? m2 : m3;
    mn = m0 < m2 ? m0 : m2;
    x0 = x0 > x1 ? x0 : x1;
    x2 = x2 > x3 ? x2 : x3;
    mx = x0 > x2 ? x0 : x2;
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
