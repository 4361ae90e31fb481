// cache.hip — cache upkeep after a token: the raw window push and the compressor's frontier.
//
// "Reading the architecture of DwarfStar (ds4.c), part 1/8" (Qiita):
//  * section 3-1: the last cap (128) tokens' KV rows stay in a raw window, every value
//    rounded to f16 when it enters; a full window slides down by one row per new token;
//  * section 3-2: each token's compressor KV row, and its score row with the positional bias
//    of its place in the group (pos mod ratio) added, go into frontier row pos mod ratio.
//
// push_raw_kernel: one workgroup per unit.  Pushing T rows equals T single pushes: rows that
// still fit are appended; otherwise the last cap - min(T, cap) old rows move to the front (the
// slide, in passes of kMoveRows rows whose loads all complete before any store of the pass)
// and the last min(T, cap) new rows fill the rest.
#include <hip/hip_fp16.h>

#include "common.hpp"
#include "launch.hpp"

namespace ds4a {

namespace {

constexpr int kPThreads = 1024;
constexpr int kMoveChunks = 8;                                  // 16-byte chunks per thread per pass

// f16 bit patterns of 4 floats, round to nearest even (v_cvt_f16_f32), packed.
__device__ __forceinline__ u32x2 f16x4_bits(f32x4 v) {
    const uint32_t a = __half_as_ushort(__float2half_rn(v[0])), b = __half_as_ushort(__float2half_rn(v[1]));
    const uint32_t c = __half_as_ushort(__float2half_rn(v[2])), d = __half_as_ushort(__float2half_rn(v[3]));
    return u32x2{a | (b << 16), c | (d << 16)};
}

__global__ __launch_bounds__(kPThreads) void push_raw_kernel(int T, int D, int cap, const float *__restrict__ kv,
                                                            uint16_t *__restrict__ raw, int32_t *__restrict__ n_raw)
{
    const int64_t u = blockIdx.x;
    int n = n_raw[u];
    n = n < 0 ? 0 : (n > cap ? cap : n);
    const int m = T < cap ? T : cap;                            // new rows that stay
    const bool fits = (int64_t)n + T <= cap;
    const int keep = fits ? n : cap - m;                        // old rows that stay, at the front
    const int shift = n - keep;                                 // rows each kept row moves down
    const int cpr = D / 8;                                      // 16-byte chunks per f16 row
    u32x4 *w = reinterpret_cast<u32x4 *>(raw + u * (int64_t)cap * D);

    if (shift > 0) {
        const int total = keep * cpr;
        for (int p0 = 0; p0 < total; p0 += kMoveChunks * kPThreads) {
            u32x4 v[kMoveChunks];
#pragma unroll
            for (int k = 0; k < kMoveChunks; ++k) {
                const int i = p0 + k * kPThreads + threadIdx.x;
                v[k] = i < total ? w[i + shift * cpr] : u32x4{0u, 0u, 0u, 0u};
            }
            // every load of the pass has returned before any wave stores: a destination chunk
            // may be another thread's source
#pragma unroll
            for (int k = 0; k < kMoveChunks; ++k) asm volatile("" : : "v"(v[k]));
            __syncthreads();
#pragma unroll
            for (int k = 0; k < kMoveChunks; ++k) {
                const int i = p0 + k * kPThreads + threadIdx.x;
                if (i < total) w[i] = v[k];
            }
            __syncthreads();
        }
    }
    // new rows T - m .. T - 1 into rows keep .. keep + m - 1, 4 values (8 bytes) per step
    const f32x4 *src = reinterpret_cast<const f32x4 *>(kv + (u * T + (T - m)) * (int64_t)D);
    u32x2 *dst = reinterpret_cast<u32x2 *>(raw + (u * (int64_t)cap + keep) * D);
    const int64_t quads = (int64_t)m * (D / 4);
    for (int64_t i = threadIdx.x; i < quads; i += kPThreads) dst[i] = f16x4_bits(src[i]);
    __syncthreads();                                            // every thread has read n_raw[u]
    if (threadIdx.x == 0) n_raw[u] = keep + m;
}

// One workgroup per unit: frontier row pos mod ratio takes the token's KV row and its score
// row plus the bias row of that place (an f32 add).
__global__ __launch_bounds__(256) void frontier_push_kernel(int width, int ratio, const float *__restrict__ kv,
                                                           const float *__restrict__ score,
                                                           const float *__restrict__ ape,
                                                           const int64_t *__restrict__ pos,
                                                           float *__restrict__ state_kv,
                                                           float *__restrict__ state_score)
{
    const int64_t u = blockIdx.x;
    int64_t row = pos[u] % ratio;
    if (row < 0) row += ratio;
    const int nq = width / 4;
    const f32x4 *k = reinterpret_cast<const f32x4 *>(kv + u * (int64_t)width);
    const f32x4 *s = reinterpret_cast<const f32x4 *>(score + u * (int64_t)width);
    const f32x4 *a = reinterpret_cast<const f32x4 *>(ape + row * width);
    f32x4 *dk = reinterpret_cast<f32x4 *>(state_kv + (u * ratio + row) * (int64_t)width);
    f32x4 *ds = reinterpret_cast<f32x4 *>(state_score + (u * ratio + row) * (int64_t)width);
    for (int i = threadIdx.x; i < nq; i += 256) {
        dk[i] = k[i];
        ds[i] = s[i] + a[i];
    }
}

}  // namespace

hipError_t launch_push_raw(int U, int T, int D, int cap, const float *kv, uint16_t *raw, int32_t *n_raw,
                           hipStream_t stream)
{
    hipLaunchKernelGGL(push_raw_kernel, dim3((unsigned)U), dim3(kPThreads), 0, stream, T, D, cap, kv, raw, n_raw);
    return hipGetLastError();
}

hipError_t launch_frontier_push(int U, int width, int ratio, const float *kv, const float *score, const float *ape,
                                const int64_t *pos, float *state_kv, float *state_score, hipStream_t stream)
{
    hipLaunchKernelGGL(frontier_push_kernel, dim3((unsigned)U), dim3(256), 0, stream, width, ratio, kv, score, ape,
                       pos, state_kv, state_score);
    return hipGetLastError();
}

}  // namespace ds4a
