// indexer.hip — A1: indexer scores of every compressed row.
//
// "Reading the architecture of DwarfStar (ds4.c), part 1/8" (Qiita), section
// 3-3: ratio-4 layers carry a thin indexer (64 heads x 128 dims, section 2)
// whose query scores every compressed row; its scores decide which rows the
// main attention reads.  Score (reading: ReLU between the per-head dot product
// and the weighted head sum):
//     s[j] = sum_h w[h] * max(0, <qI[h], kI[j]>)
//
// Design (decode and prefill alike): one query per workgroup and 1024-row
// chunk; the query's 64x128 bf16 block sits in VGPRs as the MFMA A operand
// (64 VGPRs), key rows stream from HBM straight into B-operand registers.
// Each wave takes 32 consecutive rows (8 KiB) per iteration: two 16-row
// blocks, each row read as 4 x 64-byte contiguous segments.  Per 16-row block:
// 4 head tiles x 4 k-steps = 16 v_mfma_f32_16x16x32_bf16 with the keys as the
// A operand, so D holds 4 rows x 1 head per lane; the fp32 ReLU + weighted head
// sum is 16 in-lane FMAs plus a 4-step DPP butterfly across the 16 lanes of a
// row.  Scores collect in LDS and are stored once per workgroup.  The op is
// HBM-bound (64 flop/byte).
#include "common.hpp"
#include "launch.hpp"

namespace ds4a {

namespace {

constexpr int kHeads = 64;
constexpr int kDim = 128;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kBlocksPerIter = 2;                              // 16-row blocks per wave iteration
constexpr int kRowsPerIter = 16 * kBlocksPerIter * kWaves;     // 128 rows per workgroup iteration
constexpr int64_t kRowsPerWg = 1024;                          // rows per workgroup (256 KiB of keys)
constexpr int kChunksPerRow = kDim * 2 / 16;                   // 16-byte chunks per key row (16)

__global__ __launch_bounds__(kThreads) void indexer_score_kernel(
    int T, int64_t N, int64_t rows_per_wg, int64_t wg_per_query,
    const uint16_t *__restrict__ qI, const float *__restrict__ w, const uint16_t *__restrict__ kI,
    const int32_t *__restrict__ n_vis, float *__restrict__ scores)
{
    const int64_t q = (int64_t)blockIdx.x / wg_per_query;          // flattened (u, t)
    const int64_t part = (int64_t)blockIdx.x % wg_per_query;
    const int64_t u = q / T;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int g = lane >> 4;       // k-group (A/B) and row-group (D) of this lane
    const int c = lane & 15;       // row of A / column of B and D

    const int64_t nv = clamp_nvis(n_vis, q, N);
    const int64_t r0 = part * rows_per_wg;
    const int64_t r1 = r0 + rows_per_wg < N ? r0 + rows_per_wg : N;
    float *srow = scores + q * N;

    // Invisible rows of this chunk.
    for (int64_t j = (r0 > nv ? r0 : nv) + threadIdx.x; j < r1; j += kThreads) srow[j] = -INFINITY;
    const int64_t rv1 = r1 < nv ? r1 : nv;   // visible rows [r0, rv1)
    if (r0 >= rv1) return;

    // Indexer query -> LDS, 16-byte chunk k of head h stored at h*16 + (k ^ (h & 15)) so that the
    // 16 lanes reading 16 heads at one k hit distinct banks; then A fragments
    // aq[ht][s] = qI[16ht + c][32s + 8g .. +7].
    __shared__ u32x4 sq[kHeads * kDim / 8];
    __shared__ __align__(16) float s_sc[kRowsPerWg];   // this chunk's scores, stored at the end
    const u32x4 *gq = reinterpret_cast<const u32x4 *>(qI + q * (int64_t)(kHeads * kDim));
    for (int i = threadIdx.x; i < kHeads * kDim / 8; i += kThreads) {
        const int h = i / kChunksPerRow, k = i % kChunksPerRow;
        sq[h * kChunksPerRow + (k ^ (h & 15))] = gq[i];
    }
    __syncthreads();
    bf16x8 aq[4][4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int s = 0; s < 4; ++s) aq[ht][s] = as_bf16x8(sq[(16 * ht + c) * kChunksPerRow + ((4 * s + g) ^ c)]);

    // Head weight of the D column this lane holds in head tile ht: head 16ht + c.
    float wh[4];
    const float *wq = w + q * kHeads;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) wh[ht] = wq[16 * ht + c];

    const u32x4 *gk = reinterpret_cast<const u32x4 *>(kI + u * N * kDim);
    const bool row_aligned = ((q * N) & 3) == 0;      // scores of this query start 16-byte aligned

    for (int64_t base = r0 + 16 * kBlocksPerIter * wave; base < rv1; base += kRowsPerIter) {
        // Issue all loads of this iteration first: B fragment (k-step s) of row base+16bi+c
        // is the 16-byte chunk 4s+g of that row (16 rows x 64 contiguous bytes per instruction).
        u32x4 kb[kBlocksPerIter][4];
#pragma unroll
        for (int bi = 0; bi < kBlocksPerIter; ++bi) {
            const int64_t row = base + 16 * bi + c;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                kb[bi][s] = row < rv1 ? gk[row * kChunksPerRow + 4 * s + g] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int bi = 0; bi < kBlocksPerIter; ++bi) {
            const int64_t blk = base + 16 * bi;
            if (blk >= rv1) break;                    // uniform across the wave
            // D[row 4g + r][head 16ht + c] = <key row, query head> (A = keys, B = query).
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) {
                f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) d = mfma16(as_bf16x8(kb[bi][s]), aq[ht][s], d);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] += wh[ht] * fmaxf(d[r], 0.f);
            }
            // Sum over the 16 heads of each row: the 16 lanes of a DPP row.
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = row16_sum(acc[r]);
            if (c == 0) *reinterpret_cast<f32x4 *>(s_sc + (blk - r0) + 4 * g) = acc;
        }
    }

    // Scores leave in one coalesced burst at the end: a global store inside the loop would make
    // every later wait for key loads also wait for that store (one in-order counter).
    __syncthreads();
    const int n_out = (int)(rv1 - r0);
    if (row_aligned) {
        for (int i = threadIdx.x; i < n_out / 4; i += kThreads)
            reinterpret_cast<f32x4 *>(srow + r0)[i] = reinterpret_cast<const f32x4 *>(s_sc)[i];
        for (int i = (n_out & ~3) + threadIdx.x; i < n_out; i += kThreads) srow[r0 + i] = s_sc[i];
    } else {
        for (int i = threadIdx.x; i < n_out; i += kThreads) srow[r0 + i] = s_sc[i];
    }
}

}  // namespace

hipError_t launch_indexer(int U, int T, int64_t N, const uint16_t *idx_q, const float *idx_w,
                          const uint16_t *idx_k, const int32_t *n_vis, float *scores,
                          hipStream_t stream)
{
    const int64_t Q = (int64_t)U * T;
    // 1024-row chunks (256 KiB of keys per workgroup): fastest on MI355X among 256..8192-row chunks,
    // and faster than persistent or prefetch-ring variants of the same loop.
    const int64_t rows = kRowsPerWg;
    const int64_t per_q = (N + rows - 1) / rows;
    const int64_t blocks = per_q * Q;
    hipLaunchKernelGGL(indexer_score_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       T, N, rows, per_q, idx_q, idx_w, idx_k, n_vis, scores);
    return hipGetLastError();
}

}  // namespace ds4a
