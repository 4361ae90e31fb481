// indexer.hip — A1: indexer scores of every compressed row.
//
// "Reading the architecture of DwarfStar (ds4.c), part 1/8" (Qiita), section
// 3-3: ratio-4 layers carry a thin indexer (64 heads x 128 dims, section 2)
// whose query scores every compressed row; its scores decide which rows the
// main attention reads.  Score (reading: ReLU between the per-head dot product
// and the weighted head sum):
//     s[j] = sum_h w[h] * max(0, <qI[h], kI[j]>)
//
// Decode shape (few queries per unit): one query per workgroup and 1024-row chunk; the
// row loop is indexer_score_rows (indexer_core.hpp).  Scores collect in LDS and leave in
// one coalesced burst at the end of the workgroup.  The op is HBM-bound (64 flop/byte).
#include "common.hpp"
#include "indexer_core.hpp"
#include "launch.hpp"

namespace ds4a {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int64_t kRowsPerWg = 1024;                          // rows per workgroup (256 KiB of keys)
// 16-row blocks in flight per wave, for both key formats (3 or 4 blocks of E4M3 rows measured
// no faster on MI355X: their loads are limited by request rate, not by bytes in flight).
constexpr int kBpi = 2;

template <bool FP8>
__global__ __launch_bounds__(kThreads) void indexer_score_kernel(
    int T, int64_t N, int64_t rows_per_wg, int64_t wg_per_query,
    const uint16_t *__restrict__ qI, const float *__restrict__ w, KeyRows keys,
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

    __shared__ u32x4 sq[kHeads * kDim / 8];
    __shared__ __align__(16) float s_sc[kRowsPerWg];
    const KeyRows unit = {static_cast<const char *>(keys.k) + u * N * kKeyRowBytes<FP8>,
                          FP8 ? keys.scale + u * N : nullptr};
    const KeyStream<FP8> st = key_stream<FP8>(unit, r0, (int)(rv1 - r0));
    KeyBlock<FP8> kb[kBpi];
    indexer_first_keys<kBpi, FP8>(st, wave, g, c, kb);   // in flight during the query set-up
    bf16x8 aq[4][4];
    indexer_query_frags<kThreads>(qI, q, sq, g, c, aq);
    float wh[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) wh[ht] = w[q * kHeads + 16 * ht + c];
    indexer_score_rows<kWaves, kBpi, FP8>(aq, wh, st, (int)(rv1 - r0), wave, g, c, s_sc, kb);

    __syncthreads();
    const bool row_aligned = ((q * N) & 3) == 0;      // scores of this query start 16-byte aligned
    const int n_out = (int)(rv1 - r0);
    if (row_aligned) {
        for (int i = threadIdx.x; i < n_out / 4; i += kThreads)
            reinterpret_cast<f32x4 *>(srow + r0)[i] = reinterpret_cast<const f32x4 *>(s_sc)[i];
        for (int i = (n_out & ~3) + threadIdx.x; i < n_out; i += kThreads) srow[r0 + i] = s_sc[i];
    } else {
        for (int i = threadIdx.x; i < n_out; i += kThreads) srow[r0 + i] = s_sc[i];
    }
}

// ---------------------------------------------------------------- many queries per unit

// Prefill shape (T >= 4 queries of one unit share the same keys).  A workgroup of 4 waves
// owns 4 consecutive queries and a contiguous range of 64-row key tiles; each key tile is
// read once into LDS and used by all 4 waves (one query each), so keys are read T/4 times
// instead of T times (the repeats hit L2).  Small workgroups let three share a CU, so one
// waiting at its barrier leaves the MFMA pipes to the others.  Per wave and tile: 4 row
// blocks x 4 head tiles x 4 k-steps = 64 v_mfma_f32_16x16x32_bf16 with the query as A (VGPRs) and the keys as B (LDS), so a
// lane's D values are 4 heads of one row: ReLU and weighting are in-lane FMAs and only the
// 4 lane groups need a cross-lane sum, once per tile.  LDS rows are 256 B with 16-byte chunks XOR-swizzled
// by the row's low 4 bits, so the 16 rows one A-fragment read touches hit distinct banks.
constexpr int kPQ = 4;                         // queries per workgroup (one per wave)
constexpr int kPThreads = kPQ * kWave;
constexpr int kPTile = 64;                     // key rows per tile (4 threads stage a row)
constexpr int kPTileBytes = kPTile * kDim * 2; // 16 KiB
constexpr int kPRB = kPTile / 16;              // 16-row blocks per tile
static_assert(kPThreads == 4 * kPTile && kPRB % 4 == 0, "staging and score-store mappings");
static_assert(kPQ == kIndexerManyQueries, "the prefill kernel's query count per workgroup");

template <bool FP8>
__global__ __launch_bounds__(kPThreads) void indexer_prefill_kernel(
    int T, int64_t N, int n_qb, int n_split,
    const uint16_t *__restrict__ qI, const float *__restrict__ w, KeyRows keys,
    const int32_t *__restrict__ n_vis, float *__restrict__ scores)
{
    __shared__ __align__(16) unsigned char s_k[2 * kPTileBytes];
    __shared__ __align__(16) float s_sc[kPQ][kPTile];

    const int sp = (int)(blockIdx.x % n_split);
    const int64_t rest = blockIdx.x / n_split;
    const int qb = (int)(rest % n_qb);
    const int64_t u = rest / n_qb;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int g = lane >> 4, c = lane & 15;
    const int t = qb * kPQ + wave;
    const bool active = t < T;
    const int64_t q = u * T + (active ? t : T - 1);
    const int64_t nv = active ? clamp_nvis(n_vis, q, N) : 0;
    float *srow = scores + q * N;

    // Rows any query of the workgroup sees, and this split's share of their tiles.
    int64_t nv_max = 0;
    for (int i = 0; i < kPQ; ++i) {
        const int ti = qb * kPQ + i;
        if (ti < T) {
            const int64_t v = clamp_nvis(n_vis, u * T + ti, N);
            nv_max = v > nv_max ? v : nv_max;
        }
    }
    const int64_t n_tiles = (nv_max + kPTile - 1) / kPTile;
    const int64_t per = (n_tiles + n_split - 1) / n_split;
    const int64_t tile0 = sp * per;
    const int64_t tile1 = tile0 + per < n_tiles ? tile0 + per : n_tiles;

    // Rows past every processed tile are invisible to all 8 queries: the last split writes them.
    if (sp == n_split - 1 && active) {
        for (int64_t j = n_tiles * kPTile + lane; j < N; j += kWave) srow[j] = -INFINITY;
    }
    if (tile0 >= tile1) return;                  // uniform across the workgroup

    // Query block of this wave as B fragments: qf[ht][s] = qI[q][16ht + c][32s + 8g .. +7].
    const u32x4 *gq = reinterpret_cast<const u32x4 *>(qI + q * (int64_t)(kHeads * kDim));
    u32x4 qf[4][4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[ht][s] = gq[(16 * ht + c) * kChunksPerRow + 4 * s + g];
    // Head weights of the D rows this lane holds: head 16ht + 4g + r.
    float wh[4][4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int r = 0; r < 4; ++r) wh[ht][r] = w[q * kHeads + 16 * ht + 4 * g + r];

    // Tile staging: thread tid moves dims 32(tid%4) .. +31 of tile row tid/4, i.e. 16-byte
    // chunks 4(tid%4) .. +3 of the bf16 row in LDS; E4M3 rows arrive as four 8-byte pieces and
    // are widened to bf16 (exactly) on the way into LDS, their scale applied to the scores.
    using Piece = typename std::conditional<FP8, u32x2, u32x4>::type;
    const Piece *gk = static_cast<const Piece *>(keys.k) + u * N * kChunksPerRow;
    const float *gsc = FP8 ? keys.scale + u * N : nullptr;
    const int sr = tid >> 2, sc0 = (tid & 3) * 4;
    Piece st[4];
    auto load_tile = [&](int64_t tile) __attribute__((always_inline)) {
        const int64_t row = tile * kPTile + sr;
#pragma unroll
        for (int k = 0; k < 4; ++k) st[k] = row < N ? gk[row * kChunksPerRow + sc0 + k] : Piece{};
    };
    auto store_tile = [&](int buf) __attribute__((always_inline)) {
        unsigned char *base = s_k + buf * kPTileBytes + sr * 256;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            u32x4 v;
            if constexpr (FP8) v = e4m3x8_to_bf16x8(st[k]);
            else v = st[k];
            *reinterpret_cast<u32x4 *>(base + (((sc0 + k) ^ (sr & 15)) << 4)) = v;
        }
    };
    // A-fragment read offsets: row 16rb + c, chunk (4s + g) ^ c (the row's low 4 bits are c).
    int a_off[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) a_off[s] = c * 256 + (((4 * s + g) ^ c) << 4);
    const bool row_aligned = ((q * N) & 3) == 0;

    load_tile(tile0);
    store_tile(0);
    __syncthreads();
    for (int64_t tile = tile0; tile < tile1; ++tile) {
        const int buf = (int)((tile - tile0) & 1);
        const int64_t trow0 = tile * kPTile;
        // scales of the rows this lane stores (row 16rb + c of blocks rb = (kPRB/4) g + k)
        float rsc[kPRB / 4];
        if constexpr (FP8) {
#pragma unroll
            for (int k = 0; k < kPRB / 4; ++k) {
                const int64_t row = trow0 + ((kPRB / 4) * g + k) * 16 + c;
                rsc[k] = gsc[row < N ? row : N - 1];
            }
        }
        if (tile + 1 < tile1) load_tile(tile + 1);
        if (active) {
            const unsigned char *tb = s_k + buf * kPTileBytes;
            // D[head 16ht + 4g + r][row 16rb + c] (A = query, B = keys): the head sum is mostly
            // in-lane; the 4 lane groups g are added once per tile.
            float part[kPRB];
#pragma unroll
            for (int rb = 0; rb < kPRB; ++rb) {
                u32x4 b[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) b[s] = *reinterpret_cast<const u32x4 *>(tb + a_off[s] + rb * 16 * 256);
                // four independent accumulation chains (one per head tile), k-step outermost
                f32x4 d[4];
#pragma unroll
                for (int ht = 0; ht < 4; ++ht) d[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int ht = 0; ht < 4; ++ht) d[ht] = mfma16(as_bf16x8(qf[ht][s]), as_bf16x8(b[s]), d[ht]);
                __builtin_amdgcn_sched_barrier(0);   // keep the 4 chains interleaved as written
                float acc[4];
#pragma unroll
                for (int ht = 0; ht < 4; ++ht) {
                    acc[ht] = wh[ht][0] * relu(d[ht][0]);
#pragma unroll
                    for (int r = 1; r < 4; ++r) acc[ht] += wh[ht][r] * relu(d[ht][r]);
                }
                part[rb] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            }
#pragma unroll
            for (int rb = 0; rb < kPRB; ++rb) {
                part[rb] = wave_xor_sum(part[rb], 16);
                part[rb] = wave_xor_sum(part[rb], 32);
            }
            // lane (g, c) stores row 16rb + c of blocks rb = (kPRB/4) g + k
#pragma unroll
            for (int k = 0; k < kPRB / 4; ++k) {
                const int rb = (kPRB / 4) * g + k;
                float v = part[0];
#pragma unroll
                for (int i = 1; i < kPRB; ++i) v = rb == i ? part[i] : v;
                if constexpr (FP8) v *= rsc[k];
                if (trow0 + rb * 16 + c >= nv) v = -INFINITY;
                s_sc[wave][rb * 16 + c] = v;
            }
        }
        if (tile + 1 < tile1) store_tile(buf ^ 1);
        // This tile's 128 scores of the wave's query (the LDS writes above are the same wave's).
        if (active) {
            const int64_t j = trow0 + 4 * lane;
            if (lane < kPTile / 4) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(&s_sc[wave][4 * lane]);
                if (row_aligned && j + 3 < N) {
                    *reinterpret_cast<f32x4 *>(srow + j) = v;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (j + r < N) srow[j + r] = v[r];
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_indexer(int U, int T, int64_t N, const uint16_t *idx_q, const float *idx_w,
                          KeyRows keys, const int32_t *n_vis, float *scores, hipStream_t stream)
{
    const bool fp8 = keys.scale != nullptr;
    const int64_t Q = (int64_t)U * T;
    if (T >= kIndexerManyQueries) {
        const int n_qb = (T + kPQ - 1) / kPQ;
        const int64_t wgs = (int64_t)U * n_qb;
        // Three workgroups fit on a CU (163 VGPRs); split the key range so that about two full
        // rounds of them run (a sweep over 512..6,144 workgroups at 2,048 queries: 1,536 is
        // fastest, 152 us against 163 us for 1,024), never a split shorter than 4 tiles.
        int n_split = (int)((1536 + wgs - 1) / wgs);
        const int64_t max_split = (N + 4 * kPTile - 1) / (4 * kPTile);
        if (n_split > max_split) n_split = (int)max_split;
        if (n_split < 1) n_split = 1;
        const auto kernel = fp8 ? indexer_prefill_kernel<true> : indexer_prefill_kernel<false>;
        hipLaunchKernelGGL(kernel, dim3((unsigned)(wgs * n_split)), dim3(kPThreads), 0, stream,
                           T, N, n_qb, n_split, idx_q, idx_w, keys, n_vis, scores);
        return hipGetLastError();
    }
    // 1024-row chunks (256 KiB of keys per workgroup): fastest on MI355X among 256..8192-row chunks,
    // and faster than persistent or prefetch-ring variants of the same loop.
    const int64_t rows = kRowsPerWg;
    const int64_t per_q = (N + rows - 1) / rows;
    const int64_t blocks = per_q * Q;
    const auto kernel = fp8 ? indexer_score_kernel<true> : indexer_score_kernel<false>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, T, N, rows, per_q, idx_q, idx_w, keys,
                       n_vis, scores);
    return hipGetLastError();
}

}  // namespace ds4a
