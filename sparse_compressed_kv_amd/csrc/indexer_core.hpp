// indexer_core.hpp — the per-row indexer score loop shared by the score kernel and the
// fused score + select kernel, so both produce bit-identical scores.
//
// Score (reading: ReLU between the per-head dot product and the weighted head sum):
//     s[j] = sum_h w[h] * max(0, <qI[h], kI[j]>)
// The query's 64x128 bf16 block sits in VGPRs as MFMA B fragments; key rows stream from
// HBM straight into A-operand registers.  Each wave takes 16*BPI consecutive rows per
// iteration: BPI 16-row blocks, all loads issued before any is used, each row read as
// 4 x 64-byte contiguous segments.  Per 16-row block: 4 head tiles x 4 k-steps = 16
// v_mfma_f32_16x16x32_bf16 with the keys as A, so D holds 4 rows x 1 head per lane; the fp32
// ReLU + weighted head sum is 16 in-lane FMAs plus a 4-step DPP butterfly across the 16
// lanes of a row.
#pragma once

#include "common.hpp"

namespace ds4a {

namespace {

constexpr int kHeads = 64;
constexpr int kDim = 128;
constexpr int kChunksPerRow = kDim * 2 / 16;                   // 16-byte chunks per key row (16)

// max(x, 0) as one integer max on the bit pattern (negative floats, -0 included, have
// negative int bits): no NaN-quieting pass, which fmaxf needs in IEEE mode.  MFMA outputs
// of finite inputs are finite.
__device__ __forceinline__ float relu(float x) {
    const int b = __float_as_int(x);
    return __int_as_float(b > 0 ? b : 0);
}

// Query block of query q as B fragments aq[ht][s] = qI[16ht + c][32s + 8g .. +7], through an
// LDS copy whose 16-byte chunk k of head h sits at h*16 + (k ^ (h & 15)), so the 16 lanes
// reading 16 heads at one k hit distinct banks.  Every thread of the workgroup calls it.
template <int THREADS>
__device__ __forceinline__ void indexer_query_frags(const uint16_t *__restrict__ qI, int64_t q, u32x4 *sq, int g,
                                                    int c, bf16x8 (&aq)[4][4]) {
    const u32x4 *gq = reinterpret_cast<const u32x4 *>(qI + q * (int64_t)(kHeads * kDim));
    for (int i = threadIdx.x; i < kHeads * kDim / 8; i += THREADS) {
        const int h = i / kChunksPerRow, k = i % kChunksPerRow;
        sq[h * kChunksPerRow + (k ^ (h & 15))] = gq[i];
    }
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int s = 0; s < 4; ++s) aq[ht][s] = as_bf16x8(sq[(16 * ht + c) * kChunksPerRow + ((4 * s + g) ^ c)]);
}

// Keys of the 16*BPI rows from `base` as MFMA A fragments: lane (g, c) takes the 16-byte
// chunks 4s + g of row base + 16bi + c; rows at or past rv1 read as zero (no load).
template <int BPI>
__device__ __forceinline__ void indexer_load_keys(const u32x4 *__restrict__ gk, int64_t base, int64_t rv1, int g,
                                                  int c, u32x4 (&kb)[BPI][4]) {
#pragma unroll
    for (int bi = 0; bi < BPI; ++bi) {
        const int64_t row = base + 16 * bi + c;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            kb[bi][s] = row < rv1 ? gk[row * kChunksPerRow + 4 * s + g] : u32x4{0u, 0u, 0u, 0u};
    }
}

// First row of a wave's first iteration in indexer_score_rows.
template <int BPI>
__device__ __forceinline__ int64_t indexer_first_row(int64_t r0, int wave) { return r0 + 16 * BPI * wave; }

// Scores of the visible rows [r0, rv1) of one query into s_out[row - r0] (LDS), by the
// WAVES waves of the workgroup, BPI 16-row blocks per wave iteration; wh[ht] is the weight
// of head 16ht + c.  kb holds the wave's first iteration of keys (indexer_load_keys at
// indexer_first_row), so a caller can issue those loads before it sets up the query; the
// next iteration's loads are issued as soon as the current blocks are used.  A row's score
// does not depend on WAVES or BPI.
template <int WAVES, int BPI>
__device__ __forceinline__ void indexer_score_rows(const bf16x8 (&aq)[4][4], const float (&wh)[4],
                                                   const u32x4 *__restrict__ gk, int64_t r0, int64_t rv1,
                                                   int wave, int g, int c, float *s_out, u32x4 (&kb)[BPI][4]) {
    constexpr int kRowsPerIter = 16 * BPI * WAVES;
    for (int64_t base = indexer_first_row<BPI>(r0, wave); base < rv1; base += kRowsPerIter) {
#pragma unroll
        for (int bi = 0; bi < BPI; ++bi) {
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
                for (int r = 0; r < 4; ++r) acc[r] += wh[ht] * relu(d[r]);
            }
            // Sum over the 16 heads of each row: the 16 lanes of a DPP row.
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = row16_sum(acc[r]);
            if (c == 0) *reinterpret_cast<f32x4 *>(s_out + (blk - r0) + 4 * g) = acc;
        }
        indexer_load_keys<BPI>(gk, base + kRowsPerIter, rv1, g, c, kb);
    }
}

}  // namespace

}  // namespace ds4a
