// rope_q.hip — A3 alone: the query's tail RoPE, written out as f32 for inspection.
//
// "Reading the architecture of DwarfStar (ds4.c), part 1/8" (Qiita), sections 2 and 3-2: RoPE
// acts on the last 64 of the 512 dims of each query head (adjacent pairs); stored rows are
// already rotated.  The angle and the rotation are the attention kernels' own (rope.hpp: fp64,
// rounded once to f32), so this shows exactly the query the attention uses.
#include "common.hpp"
#include "launch.hpp"
#include "rope.hpp"

#include <math.h>

namespace ds4a {

namespace {

constexpr int kQD = 512;
constexpr int kQRot = 64;

// One thread per 8 dims of one head of one query.
__global__ __launch_bounds__(256) void rope_q_kernel(int H, const void *q, int q_bf16, const int64_t *q_pos,
                                                     double log2_theta, int64_t total8, float *__restrict__ q_out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total8) return;
    const int d = (int)(i % (kQD / 8)) * 8;
    const int64_t qh = i / (kQD / 8);
    const int64_t qi = qh / H;
    float v[8];
    if (q_bf16) {
        const u32x4 x = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(q) + qh * kQD + d);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = bf16_bits_to_f32(x[k] & 0xFFFFu);
            v[2 * k + 1] = bf16_bits_to_f32(x[k] >> 16);
        }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(q) + qh * kQD + d);
        const float4 x0 = p[0], x1 = p[1];
        v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
        v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
    }
    if (d >= kQD - kQRot) {
        const int64_t pos = q_pos[qi];
#pragma unroll
        for (int e = 0; e < 8; e += 2) rope_pair(log2_theta, (d + e - (kQD - kQRot)) >> 1, pos, v[e], v[e + 1]);
    }
    float4 *dst = reinterpret_cast<float4 *>(q_out + qh * kQD + d);
    dst[0] = make_float4(v[0], v[1], v[2], v[3]);
    dst[1] = make_float4(v[4], v[5], v[6], v[7]);
}

}  // namespace

hipError_t launch_rope(int U, int T, int H, const void *q, int q_bf16, const int64_t *q_pos,
                       double theta, float *q_out, hipStream_t stream)
{
    const int64_t total8 = (int64_t)U * T * H * (kQD / 8);
    hipLaunchKernelGGL(rope_q_kernel, dim3((unsigned)((total8 + 255) / 256)), dim3(256), 0, stream, H, q, q_bf16,
                       q_pos, log2(theta), total8, q_out);
    return hipGetLastError();
}

}  // namespace ds4a
