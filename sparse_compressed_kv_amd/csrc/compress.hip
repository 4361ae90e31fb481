// compress.hip — compressor row emission: the step that makes the compressed rows the
// indexer and the attention read.
//
// "Reading the architecture of DwarfStar (ds4.c), part 1/8" (Qiita), section 3-2: tokens
// older than the raw window are not dropped but folded, `ratio` at a time (4 or 128 by
// layer), into one row.  Each token's KV and score rows (scores with a positional bias
// added) go into a frontier of `ratio` rows; at the ratio boundary the frontier is pooled
// channel by channel with the scores as softmax logits, and the pooled row is normalised
// (RMS), its tail rotated (RoPE) and round-tripped through FP8.  The indexer keeps its
// own, narrower compressor of the same form.
//
// One workgroup of 1024 threads per emitted row (one unit: a layer or a session).  The
// pooling reads the frontier once in 16-byte lane-consecutive loads, several rows in flight
// per thread, as an online softmax per row group whose partials merge in LDS; the RMS and
// the FP8 scale are block reductions; the rotation reuses the query's fp64 angle code
// (rope.hpp).  Readings of what
// the page leaves open (the norm's epsilon and gain, the rotation's position, the FP8
// format and scale) are stated at ds4a_compress_rows in the header.
#include "common.hpp"
#include "launch.hpp"
#include "rope.hpp"

namespace ds4a {

namespace {

constexpr int kCThreads = 1024;
constexpr int kCMaxWidth = 1024;
constexpr int kCUnroll = 8;                   // frontier rows in flight per thread (long frontiers)

// max and sum over the workgroup (kCThreads threads); every thread gets the result.
__device__ float block_sum(float v, float *red) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    v = wave_xor_sum(v, 1); v = wave_xor_sum(v, 2); v = wave_xor_sum(v, 4);
    v = wave_xor_sum(v, 8); v = wave_xor_sum(v, 16); v = wave_xor_sum(v, 32);
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float s = 0.f;
    for (int i = 0; i < kCThreads / kWave; ++i) s += red[i];   // the same order in every thread
    __syncthreads();
    return s;
}

__device__ float block_max(float v, float *red) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    v = wave_xor_max(v, 1); v = wave_xor_max(v, 2); v = wave_xor_max(v, 4);
    v = wave_xor_max(v, 8); v = wave_xor_max(v, 16); v = wave_xor_max(v, 32);
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float m = 0.f;
    for (int i = 0; i < kCThreads / kWave; ++i) m = fmaxf(m, red[i]);
    __syncthreads();
    return m;
}

// Nearest OCP E4M3FN value of x (ties to even), clipped to +-448; x finite.  The quantum of
// x's binade is a power of two, so x / quantum is exact and rintf rounds it to even.
__device__ __forceinline__ float round_e4m3(float x) {
    const float a = fabsf(x);
    if (a >= 448.f) return copysignf(448.f, x);
    int e = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;   // binade of a (-127 for 0 / subnormal)
    if (e < -6) e = -6;                                          // E4M3 subnormals: quantum 2^-9
    const float r = ldexpf(rintf(ldexpf(a, 3 - e)), e - 3);
    return copysignf(r, x);
}

// Power-of-two scale s, the smallest with amax / s <= 448 = 0.875 * 2^9 (amax > 0).
__device__ __forceinline__ float e4m3_scale(float amax) {
    int e;
    const float f = frexpf(amax, &e);                            // amax = f * 2^e, f in [0.5, 1)
    return ldexpf(1.f, f <= 0.875f ? e - 9 : e - 8);
}

// OCP E4M3FN code of an E4M3FN value r (|r| <= 448): sign, then the biased exponent and the
// top 3 fraction bits of r's f32 pattern, or for |r| < 2^-6 the subnormal count |r| / 2^-9.
__device__ __forceinline__ uint32_t e4m3_code(float r) {
    const uint32_t b = __float_as_uint(r);
    const uint32_t sign = (b >> 24) & 0x80u;
    const float a = fabsf(r);
    const uint32_t mag = a < 0.015625f ? (uint32_t)(a * 512.f)
                                       : ((((b >> 23) & 0xffu) - 120u) << 3) | ((b >> 20) & 7u);
    return sign | mag;
}

// Online softmax-weighted sum: fold (score s, value v) into (reference m, sum of weights den,
// weighted sum num), weights relative to m.
__device__ __forceinline__ void fold(float s, float v, float &m, float &den, float &num) {
    const float mn = fmaxf(m, s);
    const float a = __expf(m - mn), b = __expf(s - mn);          // a = 0 for the first row (m = -inf)
    den = den * a + b;
    num = num * a + b * v;
    m = mn;
}

// One workgroup per unit.  Pooling: thread t takes 4 consecutive channels (column t % ncol,
// one 16-byte load per frontier row and array) and every G-th frontier row from row t / ncol,
// UNROLL rows' loads in flight (1 when a thread has a single row, kCUnroll otherwise); the G
// partial (reference, weight sum, weighted sum) of a
// channel are merged through LDS.  `dst` says where the row goes (see RowDest in launch.hpp):
// appends emit only for units whose token closes a group and write row n_rows[u] of the
// unit's cache (when it is below cap), then count it.
template <int UNROLL>
__global__ __launch_bounds__(kCThreads) void compress_rows_kernel(
    int width, int ratio, const float *__restrict__ state_kv, const float *__restrict__ state_score,
    const float *__restrict__ gain, float eps, int n_rot, const int64_t *__restrict__ row_pos, double log2_theta,
    RowDest dst)
{
    __shared__ float s_y[kCMaxWidth];
    __shared__ f32x4 s_part[3][kCThreads];                       // (m, den, num) per thread, 4 channels each
    __shared__ float s_red[kCThreads / kWave];
    const int64_t u = blockIdx.x;
    if (dst.emit_pos) {                                          // uniform across the workgroup
        int64_t ph = dst.emit_pos[u] % ratio;
        if (ph < 0) ph += ratio;
        if (ph != ratio - 1) return;
    }
    const int32_t row = dst.n_rows ? dst.n_rows[u] : 0;
    const int ncol = width / 4;
    const int G = min(kCThreads / ncol, ratio);                  // row groups
    const int col = threadIdx.x % ncol, grp = threadIdx.x / ncol;
    const f32x4 *kv = reinterpret_cast<const f32x4 *>(state_kv + u * (int64_t)ratio * width) + col;
    const f32x4 *sc = reinterpret_cast<const f32x4 *>(state_score + u * (int64_t)ratio * width) + col;

    if (grp < G) {
        float m[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}, den[4] = {0.f, 0.f, 0.f, 0.f};
        float num[4] = {0.f, 0.f, 0.f, 0.f};
        for (int r0 = grp; r0 < ratio; r0 += UNROLL * G) {
            f32x4 a[UNROLL], b[UNROLL];
#pragma unroll
            for (int k = 0; k < UNROLL; ++k) {
                const int r = r0 + k * G < ratio ? r0 + k * G : r0;   // past the end: repeat r0, masked below
                a[k] = kv[(int64_t)r * ncol];
                b[k] = sc[(int64_t)r * ncol];
            }
            // Rows past the end fold as score -inf, an exact no-op (weight 0, the others times 1;
            // row r0 is always real, so the reference is finite by then).  No branch: one would
            // let the compiler issue each row's loads only when the row is folded.
#pragma unroll
            for (int k = 0; k < UNROLL; ++k) {
                const bool ok = r0 + k * G < ratio;
#pragma unroll
                for (int e = 0; e < 4; ++e) fold(ok ? b[k][e] : -INFINITY, ok ? a[k][e] : 0.f, m[e], den[e], num[e]);
            }
        }
        s_part[0][threadIdx.x] = f32x4{m[0], m[1], m[2], m[3]};
        s_part[1][threadIdx.x] = f32x4{den[0], den[1], den[2], den[3]};
        s_part[2][threadIdx.x] = f32x4{num[0], num[1], num[2], num[3]};
    }
    __syncthreads();
    // merge the row groups of each channel, then the sum of squares of the pooled row
    float ss = 0.f;
    for (int j = threadIdx.x; j < width; j += kCThreads) {
        const int c = j / 4, e = j % 4;
        float mm = -INFINITY;
        for (int g = 0; g < G; ++g) mm = fmaxf(mm, s_part[0][g * ncol + c][e]);
        float d = 0.f, n = 0.f;
        for (int g = 0; g < G; ++g) {
            const float w = __expf(s_part[0][g * ncol + c][e] - mm);
            d += s_part[1][g * ncol + c][e] * w;
            n += s_part[2][g * ncol + c][e] * w;
        }
        const float p = n / d;                                   // d >= 1 (the max row's weight)
        s_y[j] = p;
        ss += p * p;
    }
    ss = block_sum(ss, s_red);
    const float inv = 1.f / sqrtf(ss / (float)width + eps);
    for (int j = threadIdx.x; j < width; j += kCThreads) s_y[j] = s_y[j] * inv * gain[u * width + j];
    __syncthreads();

    // tail RoPE: thread i < n_rot/2 rotates the pair (width - n_rot + 2i, +1)
    if (threadIdx.x < n_rot / 2) {
        const int i = threadIdx.x, j0 = width - n_rot + 2 * i;
        double cs, sn;
        rope_angle(log2_theta, i, row_pos[u], cs, sn, n_rot);
        rope_rotate(cs, sn, s_y[j0], s_y[j0 + 1]);
    }
    __syncthreads();

    const bool fp8 = dst.format != DS4A_ROW_BF16;
    float s = 1.f;
    if (fp8) {
        float amax = 0.f;
        for (int j = threadIdx.x; j < width; j += kCThreads) amax = fmaxf(amax, fabsf(s_y[j]));
        amax = block_max(amax, s_red);
        if (amax > 0.f) s = e4m3_scale(amax);
    }
    if (row >= 0 && row < dst.cap) {                             // uniform
        const int64_t e0 = u * dst.unit_stride + (int64_t)row * width;
        if (dst.format == DS4A_ROW_E4M3) {
            uint8_t *o = static_cast<uint8_t *>(dst.out) + e0;
            for (int j = threadIdx.x; j < width; j += kCThreads) o[j] = (uint8_t)e4m3_code(round_e4m3(s_y[j] / s));
            if (threadIdx.x == 0) dst.scale[u * dst.cap + row] = s;
        } else {
            uint16_t *o = static_cast<uint16_t *>(dst.out) + e0;
            for (int j = threadIdx.x; j < width; j += kCThreads) {
                const float y = fp8 ? round_e4m3(s_y[j] / s) * s : s_y[j];   // s a power of two: exact
                o[j] = (uint16_t)f32_to_bf16_bits(y);
            }
        }
    }
    if (dst.n_rows) {
        __syncthreads();                                         // every thread has read n_rows[u]
        if (threadIdx.x == 0) dst.n_rows[u] = row + 1;
    }
}

}  // namespace

hipError_t launch_compress(int U, int width, int ratio, const float *state_kv, const float *state_score,
                           const float *gain, float eps, int n_rot, const int64_t *row_pos, double theta,
                           const RowDest &dst, hipStream_t stream)
{
    const int G = kCThreads / (width / 4) < ratio ? kCThreads / (width / 4) : ratio;
    const auto kernel = ratio <= G ? compress_rows_kernel<1> : compress_rows_kernel<kCUnroll>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)U), dim3(kCThreads), 0, stream, width, ratio, state_kv, state_score,
                       gain, eps, n_rot, row_pos, log2(theta), dst);
    return hipGetLastError();
}

}  // namespace ds4a
