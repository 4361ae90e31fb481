// fused.hip — A1 + A2 in one pass over the keys.
//
// "Reading the architecture of DwarfStar (ds4.c), part 1/8" (Qiita), section
// 3-3: the indexer's scores exist only to pick the top-k rows that reach the
// main attention.  So in decode shapes the scores need not leave the chip: a
// workgroup scores a chunk of one query's rows into LDS (the same row loop,
// hence the same bits, as the score kernel) and selects the chunk's top-K there;
// only K (key, row) candidates per chunk go to memory, and the candidate lists
// are merged as in the chunked top-k.  A chunk's own top-K contains every global
// top-K row of that chunk (one total order: score, then lower row), so the
// result is exactly the top-k of the full score vector.
// Many queries per unit (prefill shapes), and calls too small to fill the GPU
// with chunk workgroups, go through the score kernel into the workspace and the
// top-k on it.
#include "common.hpp"
#include "indexer_core.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace ds4a {

namespace {

constexpr int kFWaves = kNT / kWave;
// 16-row blocks in flight per wave, for both key formats (3 or 4 blocks of E4M3 rows measured
// no faster on MI355X: their loads are limited by request rate, not by bytes in flight).
constexpr int kFBpi = 2;
// Device figures behind the chunk rule (MI355X, measured with bf16 keys): a chunk workgroup
// alone on a CU streams its keys at ~23 GB/s (its loads in flight set the rate), two on one CU
// at ~26 GB/s together, and all of them at most at the device's read rate, ~6.1 TB/s; 256 CUs
// hold two chunk workgroups each (the row loop keeps the query in VGPRs, 125 per lane: 4 waves
// per SIMD).  Fixed, so that workspace sizes do not depend on the device a call runs on.
constexpr int64_t kFCUs = 256;
constexpr int64_t kFSlots = 2 * kFCUs;
constexpr double kFRate1 = 23.0;              // bytes per ns: one chunk workgroup on a CU
constexpr double kFRate2 = 26.0;              // two on a CU, together
constexpr double kFRateAll = 6100.0;          // the device

// A chunk of up to EPT * 512 rows (`rows` per chunk): each thread selects over EPT keys.  Two
// workgroups share a CU (4 waves per SIMD: at most 128 VGPRs).
template <int EPT, bool FP8>
__global__ __launch_bounds__(kNT, 4) void indexer_select_kernel(
    int T, int64_t N, int K, int rows, int64_t chunks,
    const uint16_t *__restrict__ qI, const float *__restrict__ w, KeyRows keys,
    const int32_t *__restrict__ n_vis, int32_t *__restrict__ out, uint32_t *__restrict__ out_keys)
{
    __shared__ u32x4 sq[kHeads * kDim / 8];
    constexpr int kRows = EPT * kNT;
    static_assert(EPT % 4 == 0, "scores are read from LDS four at a time");
    __shared__ __align__(16) float s_sc[kRows];    // keys of the chunk's rows (float_key of the scores)
    __shared__ SelectShared sm;                   // one copy: eight measured slower here (LDS, scan reads)
    __shared__ uint32_t s_claim;                  // next unclaimed group of rows

    const int64_t q = blockIdx.x / chunks;
    const int64_t ch = blockIdx.x % chunks;
    const int64_t u = q / T;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int g = lane >> 4, c = lane & 15;
    const int64_t nv = clamp_nvis(n_vis, q, N);
    const int64_t c0 = ch * rows;
    const int64_t rem = nv - c0;
    const int n = rem <= 0 ? 0 : (rem < rows ? (int)rem : rows);     // visible rows of this chunk

    // Positions past the last 16-row block of scores hold 0, the absent key.
    for (int j = (n + 15) / 16 * 16 + (int)threadIdx.x; j < kRows; j += kNT) reinterpret_cast<uint32_t *>(s_sc)[j] = 0u;
    if (n > 0) {                                  // uniform across the workgroup
        const KeyRows unit = {static_cast<const char *>(keys.k) + u * N * kKeyRowBytes<FP8>,
                              FP8 ? keys.scale + u * N : nullptr};
        const KeyStream<FP8> st = key_stream<FP8>(unit, c0, n);
        KeyBlock<FP8> kb[kFBpi];
        indexer_first_keys<kFBpi, FP8>(st, wave, g, c, kb);   // in flight during the query set-up
        bf16x8 aq[4][4];
        if (threadIdx.x == 0) s_claim = kFWaves;  // published by the query set-up's barrier
        indexer_query_frags<kNT>(qI, q, sq, g, c, aq);
        float wh[4];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) wh[ht] = w[q * kHeads + 16 * ht + c];
        indexer_score_rows<kFWaves, kFBpi, FP8, true>(aq, wh, st, n, wave, g, c, s_sc, kb, &s_claim);
    }
    __syncthreads();

    const int j0 = threadIdx.x * EPT;
    uint32_t key[EPT];
    int32_t id[EPT];
#pragma unroll
    for (int i = 0; i < EPT; i += 4) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(s_sc + j0 + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            key[i + e] = v[e];
            id[i + e] = 0;
        }
    }
    const int need = K < n ? K : n;
    const int64_t slot = (q * chunks + ch) * K;
    if (2 * K > kRows) {                          // uniform; chunks of fewer than 2K key slots
        block_select<EPT, false>(key, id, c0, n, need, K, out + slot, out_keys ? out_keys + slot : nullptr, sm);
        return;
    }
    // The selection is gathered in LDS (the scores' buffer, K ids then K keys) and leaves in one
    // coalesced pass instead of the collection's scattered stores.
    __syncthreads();                              // every thread holds its keys: s_sc is free
    int32_t *g_id = reinterpret_cast<int32_t *>(s_sc);
    uint32_t *g_key = reinterpret_cast<uint32_t *>(s_sc) + K;
    block_select<EPT, false>(key, id, c0, n, need, K, g_id, out_keys ? g_key : nullptr, sm);
    __syncthreads();
    for (int i = (int)threadIdx.x; i < K; i += kNT) {
        out[slot + i] = g_id[i];
        if (out_keys) out_keys[slot + i] = g_key[i];
    }
}

struct FusedShape {
    int ept;                                  // keys per thread: chunk capacity ept * 512 rows
    int rows;                                 // rows per chunk
    int64_t chunks;                           // chunks per query
};

// Chunk rule: the chunk count with the least modelled time, in ns.  A call streams for as long
// as its busiest CU needs (one or two chunk workgroups per CU per resident round, at the rates
// above) and at least as long as the device needs for all the keys; each resident round ends
// with a select (~3 us + 0.15 us per key per thread); a merge (more than one chunk) costs ~3 us
// + 0.6 ns per candidate, plus ~8 us per extra level, and a final list longer than the attention
// kernel merges itself costs the one-call step that extra level too.  Chunks hold at most 8192 rows (16 keys per thread)
// and at least 2 rows per candidate.
FusedShape fused_shape(int64_t Q, int64_t N, int K) {
    const int64_t cmin = (N + 8191) / 8192 > 0 ? (N + 8191) / 8192 : 1;
    int64_t cmax = N / (2 * (int64_t)K);
    if (cmax > cmin + 64) cmax = cmin + 64;
    if (cmax < cmin) cmax = cmin;
    FusedShape best = {16, 8192, cmin};
    double best_cost = -1.0;
    for (int64_t c = cmin; c <= cmax; ++c) {
        const int64_t rows = ((N + c - 1) / c + 15) / 16 * 16;
        const int ept = (int)((rows + 2047) / 2048 * 4);
        const int64_t wgs = Q * c;
        const int64_t rounds = (wgs + kFSlots - 1) / kFSlots;
        const int64_t last = wgs - (rounds - 1) * kFSlots;          // workgroups of the last round
        const double chunk_bytes = (double)rows * 256.0;
        double cu_ns = (double)(rounds - 1) * 2.0 * chunk_bytes / kFRate2;
        cu_ns += last <= kFCUs ? chunk_bytes / kFRate1 : 2.0 * chunk_bytes / kFRate2;
        const double all_ns = (double)Q * (double)N * 256.0 / kFRateAll;
        int64_t levels = 0;
        int64_t stride = c * K;
        for (; stride > kMergeMax; stride = (stride + kLevelChunk - 1) / kLevelChunk * K) ++levels;
        if (stride > kAttnMergeMax) ++levels;
        const double merge_ns = c > 1 ? 3000.0 + 0.6 * (double)stride + 8000.0 * (double)levels : 0.0;
        const double cost = (cu_ns > all_ns ? cu_ns : all_ns) + (double)rounds * (3000.0 + 150.0 * ept) + merge_ns;
        if (best_cost < 0.0 || cost < best_cost) {
            best_cost = cost;
            best = {ept, (int)rows, c};
        }
    }
    return best;
}

// The fused kernel needs enough chunk workgroups to stream the keys at full rate while its
// chunks keep at least 4 rows per candidate; with fewer (a handful of units) the score kernel's
// smaller 1024-row chunks plus the separate top-k are faster, and so are many queries per unit
// (prefill shapes).
bool use_fused(int T, int64_t Q, int64_t N, int K) {
    if (T >= kIndexerManyQueries) return false;
    const int64_t cmin = (N + 8191) / 8192 > 0 ? (N + 8191) / 8192 : 1;
    int64_t c4 = N / (4 * (int64_t)K);
    if (c4 > cmin + 32) c4 = cmin + 32;
    if (c4 < cmin) c4 = cmin;
    return Q * c4 >= 128;
}

template <int EPT>
void launch_select(int64_t grid, int T, int64_t N, int K, int rows, int64_t chunks, const uint16_t *idx_q,
                   const float *idx_w, KeyRows idx_k, const int32_t *n_vis, int32_t *ids, uint32_t *keys,
                   hipStream_t stream)
{
    const auto kernel = idx_k.scale ? indexer_select_kernel<EPT, true> : indexer_select_kernel<EPT, false>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kNT), 0, stream, T, N, K, rows, chunks, idx_q, idx_w, idx_k,
                       n_vis, ids, keys);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t indexer_topk_workspace_bytes(int U, int T, int64_t N, int K) {
    const int64_t Q = (int64_t)U * T;
    if (!use_fused(T, Q, N, K)) return align256((size_t)Q * (size_t)N * 4) + topk_workspace_bytes(Q, N, K);
    const int64_t chunks = fused_shape(Q, N, K).chunks;
    return chunks > 1 ? topk_cand_workspace_bytes(Q, chunks, K) : 0;
}

hipError_t launch_indexer_topk(int U, int T, int64_t N, int K, const uint16_t *idx_q, const float *idx_w,
                               KeyRows idx_k, const int32_t *n_vis, int32_t *idx, void *workspace,
                               hipStream_t stream)
{
    const int64_t Q = (int64_t)U * T;
    if (!use_fused(T, Q, N, K)) {
        float *scores = static_cast<float *>(workspace);
        void *ws2 = static_cast<char *>(workspace) + align256((size_t)Q * (size_t)N * 4);
        hipError_t e = launch_indexer(U, T, N, idx_q, idx_w, idx_k, n_vis, scores, stream);
        if (e != hipSuccess) return e;
        return launch_topk(Q, N, K, scores, n_vis, idx, ws2, stream);
    }
    const FusedShape fs = fused_shape(Q, N, K);
    uint32_t *keys = nullptr;
    int32_t *ids = idx;                       // one chunk: its selection is the result
    if (fs.chunks > 1) topk_level1_buffers(workspace, Q, fs.chunks, K, &keys, &ids);
    const int64_t grid = Q * fs.chunks;
    switch (fs.ept) {
    case 4: launch_select<4>(grid, T, N, K, fs.rows, fs.chunks, idx_q, idx_w, idx_k, n_vis, ids, keys, stream); break;
    case 8: launch_select<8>(grid, T, N, K, fs.rows, fs.chunks, idx_q, idx_w, idx_k, n_vis, ids, keys, stream); break;
    case 12: launch_select<12>(grid, T, N, K, fs.rows, fs.chunks, idx_q, idx_w, idx_k, n_vis, ids, keys, stream); break;
    default: launch_select<16>(grid, T, N, K, fs.rows, fs.chunks, idx_q, idx_w, idx_k, n_vis, ids, keys, stream); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || fs.chunks == 1) return e;
    return launch_topk_merge(Q, N, K, fs.rows, fs.chunks, n_vis, idx, workspace, stream);
}

bool indexer_candidates_apply(int U, int T, int64_t N, int K) {
    const int64_t Q = (int64_t)U * T;
    return use_fused(T, Q, N, K) && fused_shape(Q, N, K).chunks > 1;
}

hipError_t launch_indexer_candidates(int U, int T, int64_t N, int K, const uint16_t *idx_q, const float *idx_w,
                                     KeyRows idx_k, const int32_t *n_vis, void *workspace, int64_t max_last,
                                     CandList *list, hipStream_t stream)
{
    const int64_t Q = (int64_t)U * T;
    const FusedShape fs = fused_shape(Q, N, K);
    uint32_t *keys = nullptr;
    int32_t *ids = nullptr;
    topk_level1_buffers(workspace, Q, fs.chunks, K, &keys, &ids);
    const int64_t grid = Q * fs.chunks;
    switch (fs.ept) {
    case 4: launch_select<4>(grid, T, N, K, fs.rows, fs.chunks, idx_q, idx_w, idx_k, n_vis, ids, keys, stream); break;
    case 8: launch_select<8>(grid, T, N, K, fs.rows, fs.chunks, idx_q, idx_w, idx_k, n_vis, ids, keys, stream); break;
    case 12: launch_select<12>(grid, T, N, K, fs.rows, fs.chunks, idx_q, idx_w, idx_k, n_vis, ids, keys, stream); break;
    default: launch_select<16>(grid, T, N, K, fs.rows, fs.chunks, idx_q, idx_w, idx_k, n_vis, ids, keys, stream); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_topk_merge_levels(Q, N, K, fs.rows, fs.chunks, n_vis, workspace, max_last, list, stream);
}

}  // namespace ds4a
