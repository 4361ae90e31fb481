// ceiling.hip — measured ceilings of the two units the hot path is bound by, so that a kernel's
// roofline fraction can be read against what this GPU delivers as well as against its
// published peak: a plain HBM read stream and a plain bf16 matrix-core loop.  Neither is a
// step of the method.
#include "common.hpp"

#include "../../include/ds4ceil.h"

namespace ds4a {

namespace {

// HBM read stream: every thread reads 16 bytes per iteration, grid-stride, four loads in flight;
// the loads are non-temporal so that the stream does not settle in the caches.  One XOR per
// thread is written so that nothing is optimised away.
__global__ __launch_bounds__(256) void ceiling_read_kernel(const u32x4 *__restrict__ p, int64_t n16,
                                                            uint32_t *__restrict__ sink)
{
    u32x4 acc = {0u, 0u, 0u, 0u};
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i), b = __builtin_nontemporal_load(p + i + stride);
        const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride), d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// bf16 matrix cores: v_mfma_f32_16x16x32_bf16 in 8 independent chains per wave (operands in
// registers, no memory traffic in the loop).
constexpr int kChains = 8;
__global__ __launch_bounds__(256) void ceiling_mfma_kernel(int64_t iters, float *__restrict__ sink)
{
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)threadIdx.x + (float)i);
        b[i] = (__bf16)(0.5f * (float)i);
    }
    f32x4 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = mfma16(a, b, acc[c]);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

}  // namespace ds4a

extern "C" {

int ds4a_ceiling_read(const void *src, int64_t bytes, int grid, uint32_t *sink, void *stream) {
    if (!src || !sink || bytes < 16 || (bytes & 15) || grid < 1 || grid > (1 << 20)) return DS4A_CEIL_EINVAL;
    if ((reinterpret_cast<uintptr_t>(src) & 15) != 0) return DS4A_CEIL_EINVAL;
    hipLaunchKernelGGL(ds4a::ceiling_read_kernel, dim3((unsigned)grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const ds4a::u32x4 *>(src), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : DS4A_CEIL_ELAUNCH;
}

int ds4a_ceiling_mfma(int64_t iters, int grid, float *sink, double *flops, void *stream) {
    if (!sink || iters < 1 || grid < 1 || grid > (1 << 20)) return DS4A_CEIL_EINVAL;
    hipLaunchKernelGGL(ds4a::ceiling_mfma_kernel, dim3((unsigned)grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), iters, sink);
    if (flops) *flops = (double)grid * (256 / 64) * (double)iters * ds4a::kChains * (16.0 * 16.0 * 32.0 * 2.0);
    return hipGetLastError() == hipSuccess ? 0 : DS4A_CEIL_ELAUNCH;
}

}  // extern "C"
