// indexer_core.hpp — the per-row indexer score loop shared by the score kernel and the
// fused score + select kernel, so both produce bit-identical scores.
//
// Score (reading: ReLU between the per-head dot product and the weighted head sum):
//     s[j] = sum_h w[h] * max(0, <qI[h], kI[j]>)
// The query's 64x128 bf16 block sits in VGPRs as MFMA B fragments; key rows stream from
// HBM straight into A-operand registers.  Each wave takes 16*BPI consecutive rows per
// iteration: BPI 16-row blocks in flight, the dims of a row in the k-step order of kdim.  Per 16-row block: 4 head tiles x 4 k-steps = 16
// v_mfma_f32_16x16x32_bf16 with the keys as A, so D holds 4 rows x 1 head per lane; the fp32
// ReLU + weighted head sum is 16 in-lane FMAs plus a 4-step DPP butterfly across the 16
// lanes of a row.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

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

// The 128 dims of a key or query row, in the order the MFMA k-steps take them: k-step s of
// lane group g holds dims kdim(s, g) .. +7, kdim(s, g) = 64(s >> 1) + 16g + 8(s & 1).  So a
// lane's k-steps 0 and 1 (and 2 and 3) are 16 adjacent dims: one 16-byte load of E4M3 codes,
// with the 4 lane groups of a row reading 64 adjacent bytes (a bf16 row is read as 16-byte
// chunks, 2 per 32 adjacent bytes).  Any fixed order gives the same sum up to fp32 rounding;
// using one order for both key formats keeps them bit-identical.
__device__ __forceinline__ constexpr int kdim(int s, int g) { return 64 * (s >> 1) + 16 * g + 8 * (s & 1); }

// Query block of query q as B fragments aq[ht][s] = qI[16ht + c][kdim(s, g) .. +7], through an
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
        for (int s = 0; s < 4; ++s) aq[ht][s] = as_bf16x8(sq[(16 * ht + c) * kChunksPerRow + ((kdim(s, g) / 8) ^ c)]);
}

// Per-lane key registers of one 16-row block: 4 k-steps of 8 values, as bf16 (16 bytes each)
// or as E4M3 codes (8 bytes each, converted to bf16 just before the MFMAs) plus the scale of
// row 4g + (c & 3) of the block, the row whose score the lane stores.
template <bool FP8>
struct KeyBlock {
    u32x4 v[4];
};
template <>
struct KeyBlock<true> {
    u32x2 v[4];
    float sc;
};

// The visible key rows [r0, r0 + n) of one unit as buffer resources: 32-bit offsets relative
// to row r0 (n * row bytes < 2^32 for the chunk sizes used here), and reads past the last
// visible row return zero without touching memory, so no row needs a bounds branch.
template <bool FP8>
struct KeyStream {
    __amdgpu_buffer_rsrc_t k;
    __amdgpu_buffer_rsrc_t sc;
};

template <bool FP8>
constexpr int kKeyRowBytes = FP8 ? kDim : 2 * kDim;

// ks: the unit's rows (row 0 at ks.k, scale 0 at ks.scale).
template <bool FP8>
__device__ __forceinline__ KeyStream<FP8> key_stream(const KeyRows &ks, int64_t r0, int n) {
    constexpr int kRaw = 0x00020000;              // word 3 of a raw (stride 0) buffer resource
    KeyStream<FP8> st;
    const char *k = static_cast<const char *>(ks.k) + r0 * kKeyRowBytes<FP8>;
    st.k = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(k), (short)0, n * kKeyRowBytes<FP8>, kRaw);
    if constexpr (FP8)
        st.sc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(ks.scale + r0), (short)0, n * 4, kRaw);
    return st;
}

// Keys of the 16-row block at local row `blk`: lane (g, c) takes dims kdim(s, g) .. +7 of row
// blk + c for k-step s, so both formats feed the same dims to the same MFMA slots: two 16-byte
// loads of 16 codes (k-steps 0-1 and 2-3) for E4M3 rows, four of 8 bf16 values for bf16 rows.
// Rows past the stream read as zero.
template <bool FP8>
__device__ __forceinline__ void indexer_load_block(const KeyStream<FP8> &st, int blk, int g, int c,
                                                   KeyBlock<FP8> &kb) {
    const int off = (blk + c) * kKeyRowBytes<FP8>;
    if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(st.k, off + kdim(2 * j, g), 0, 0);
            kb.v[2 * j] = u32x2{v[0], v[1]};
            kb.v[2 * j + 1] = u32x2{v[2], v[3]};
        }
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(st.k, off + 2 * kdim(s, g), 0, 0);
            kb.v[s] = u32x4{v[0], v[1], v[2], v[3]};
        }
    }
}

template <bool FP8>
__device__ __forceinline__ float indexer_load_scale(const KeyStream<FP8> &st, int blk, int g, int c) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(st.sc, (blk + 4 * g + (c & 3)) * 4, 0, 0));
}

// The BPI blocks of a wave's first iteration in indexer_score_rows.
template <int BPI, bool FP8>
__device__ __forceinline__ void indexer_first_keys(const KeyStream<FP8> &st, int wave, int g, int c,
                                                   KeyBlock<FP8> (&kb)[BPI]) {
#pragma unroll
    for (int bi = 0; bi < BPI; ++bi) {
        const int blk = 16 * (BPI * wave + bi);
        indexer_load_block<FP8>(st, blk, g, c, kb[bi]);
        if constexpr (FP8) kb[bi].sc = indexer_load_scale<FP8>(st, blk, g, c);
    }
}

// Scores of the n visible rows of a key stream into s_out[0 .. n) (LDS; the slots up to the next
// multiple of 16 are written too), by the WAVES waves of the workgroup, BPI 16-row blocks per
// wave iteration; wh[ht] is the weight of head 16ht + c.  kb holds the wave's first iteration
// of keys (indexer_first_keys), so a caller can issue those loads before it sets up the
// query.  A block's registers are refilled with the same block of the next iteration as soon
// as its MFMAs are issued (its scale once the score is stored), so BPI blocks stay in flight
// while the epilogues run; loads complete in issue order, the order the blocks are used in.
// A row's score does not depend on WAVES, BPI or which wave computes it.  E4M3 keys: the
// products use the code values and the row's score is multiplied by its scale at the end
// (scale > 0 commutes with the ReLU); with power-of-two scales the score is bit-identical to
// that of the bf16 keys code * scale.
// KEYS: s_out receives float_key of each score (as uint32), and 0 for the rows of the last
// 16-row block past n, the form the workgroup select takes.
// Wave w starts with rows 16*BPI*w ..; its next 16*BPI rows are WAVES*16*BPI further on, or,
// with a claim counter (LDS, set to WAVES before any wave reaches the loop), the next unclaimed
// group of 16*BPI rows: waves that the hardware serves first take more of them, so the waves
// of a workgroup finish together and all of them keep streaming until the end.
template <int WAVES, int BPI, bool FP8, bool KEYS = false>
__device__ __forceinline__ void indexer_score_rows(const bf16x8 (&aq)[4][4], const float (&wh)[4],
                                                   const KeyStream<FP8> &st, int n, int wave, int g, int c,
                                                   float *s_out, KeyBlock<FP8> (&kb)[BPI],
                                                   uint32_t *claim = nullptr) {
    constexpr int kWaveRows = 16 * BPI;
    constexpr int kRowsPerIter = kWaveRows * WAVES;
    // The head weights arrive before the loop: a wait for them inside it would also wait for
    // every key load issued after them.
    asm volatile("" : : "v"(wh[0]), "v"(wh[1]), "v"(wh[2]), "v"(wh[3]));
    for (int base = kWaveRows * wave, next; base < n; base = next) {
        if (claim) {                                  // the result is first needed after 16 MFMAs
            uint32_t v = 0;
            if ((threadIdx.x & (kWave - 1)) == 0) v = atomicAdd(claim, 1u);
            next = kWaveRows * (int)__builtin_amdgcn_readfirstlane(v);
        } else {
            next = base + kRowsPerIter;
        }
#pragma unroll
        for (int bi = 0; bi < BPI; ++bi) {
            // Every block is computed, also past n (its keys read as zero): a branch here would
            // make the loop's waits cover the next block's loads as well.
            const int blk = base + 16 * bi;
            const bool live = blk < n;
            u32x4 a[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if constexpr (FP8) a[s] = e4m3x8_to_bf16x8(kb[bi].v[s]);
                else a[s] = kb[bi].v[s];
            }
            // D[row 4g + r][head 16ht + c] = <key row, query head> (A = keys, B = query).
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) {
                f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) d = mfma16(as_bf16x8(a[s]), aq[ht][s], d);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] += wh[ht] * relu(d[r]);
            }
            indexer_load_block<FP8>(st, next + 16 * bi, g, c, kb[bi]);
            // Sum over the 16 heads of each row: the 16 lanes of a DPP row.
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = row16_sum(acc[r]);
            if constexpr (FP8) {
                // lanes c < 4 of group g store row 4g + c, scaled
                const int r = c & 3;
                float v = acc[0];
                v = r == 1 ? acc[1] : v;
                v = r == 2 ? acc[2] : v;
                v = r == 3 ? acc[3] : v;
                v *= kb[bi].sc;
                if constexpr (KEYS) {
                    const uint32_t kv = blk + 4 * g + r < n ? float_key(v) : 0u;
                    if (live && c < 4) reinterpret_cast<uint32_t *>(s_out)[blk + 4 * g + r] = kv;
                } else {
                    if (live && c < 4) s_out[blk + 4 * g + r] = v;
                }
                kb[bi].sc = indexer_load_scale<FP8>(st, next + 16 * bi, g, c);
            } else {
                if constexpr (KEYS) {
                    u32x4 kv;
#pragma unroll
                    for (int r = 0; r < 4; ++r) kv[r] = blk + 4 * g + r < n ? float_key(acc[r]) : 0u;
                    if (live && c == 0) *reinterpret_cast<u32x4 *>(s_out + blk + 4 * g) = kv;
                } else {
                    if (live && c == 0) *reinterpret_cast<f32x4 *>(s_out + blk + 4 * g) = acc;
                }
            }
        }
    }
}

}  // namespace

}  // namespace ds4a
