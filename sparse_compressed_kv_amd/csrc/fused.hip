// fused.hip — A1 + A2 in one pass over the keys.
//
// "Reading the architecture of DwarfStar (ds4.c), part 1/8" (Qiita), section
// 3-3: the indexer's scores exist only to pick the top-k rows that reach the
// main attention.  So in decode shapes the scores need not leave the chip: a
// workgroup scores a 4096-row chunk of one query into LDS (the same row loop,
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

constexpr int kFRows = 4096;                  // rows per workgroup = 8 keys x 512 threads
constexpr int kFEpt = kFRows / kNT;
constexpr int kFWaves = kNT / kWave;
constexpr int kFBpi = 2;                      // 16-row blocks in flight per wave

__global__ __launch_bounds__(kNT) void indexer_select_kernel(
    int T, int64_t N, int K, int64_t chunks,
    const uint16_t *__restrict__ qI, const float *__restrict__ w, const uint16_t *__restrict__ kI,
    const int32_t *__restrict__ n_vis, int32_t *__restrict__ out, uint32_t *__restrict__ out_keys)
{
    __shared__ u32x4 sq[kHeads * kDim / 8];
    __shared__ __align__(16) float s_sc[kFRows];
    __shared__ SelectShared sm;

    const int64_t q = blockIdx.x / chunks;
    const int64_t ch = blockIdx.x % chunks;
    const int64_t u = q / T;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int g = lane >> 4, c = lane & 15;
    const int64_t nv = clamp_nvis(n_vis, q, N);
    const int64_t c0 = ch * kFRows;
    const int64_t rem = nv - c0;
    const int n = rem <= 0 ? 0 : (rem < kFRows ? (int)rem : kFRows);   // visible rows of this chunk

    if (n > 0) {                                  // uniform across the workgroup
        bf16x8 aq[4][4];
        indexer_query_frags<kNT>(qI, q, sq, g, c, aq);
        float wh[4];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) wh[ht] = w[q * kHeads + 16 * ht + c];
        const u32x4 *gk = reinterpret_cast<const u32x4 *>(kI + u * N * kDim);
        indexer_score_rows<kFWaves, kFBpi>(aq, wh, gk, c0, c0 + n, wave, g, c, s_sc);
    }
    __syncthreads();

    const int j0 = threadIdx.x * kFEpt;
    uint32_t key[kFEpt];
    int32_t id[kFEpt];
#pragma unroll
    for (int i = 0; i < kFEpt; i += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(s_sc + j0 + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            key[i + e] = j0 + i + e < n ? float_key(v[e]) : 0u;
            id[i + e] = 0;
        }
    }
    const int need = K < n ? K : n;
    const int64_t slot = (q * chunks + ch) * K;
    block_select<kFEpt, false>(key, id, c0, n, need, K, out + slot, out_keys ? out_keys + slot : nullptr, sm);
}

int64_t fused_chunks(int64_t N) { return (N + kFRows - 1) / kFRows; }

// The fused kernel needs enough chunk workgroups to stream the keys at full rate; with fewer
// (a handful of units) the score kernel's smaller 1024-row chunks plus the separate top-k
// are faster, and so are many queries per unit (prefill shapes).
bool use_fused(int T, int64_t Q, int64_t N) { return T < kIndexerManyQueries && Q * fused_chunks(N) >= 128; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t indexer_topk_workspace_bytes(int U, int T, int64_t N, int K) {
    const int64_t Q = (int64_t)U * T;
    if (!use_fused(T, Q, N)) return align256((size_t)Q * (size_t)N * 4) + topk_workspace_bytes(Q, N, K);
    const int64_t chunks = fused_chunks(N);
    return chunks > 1 ? topk_cand_workspace_bytes(Q, chunks, K) : 0;
}

hipError_t launch_indexer_topk(int U, int T, int64_t N, int K, const uint16_t *idx_q, const float *idx_w,
                               const uint16_t *idx_k, const int32_t *n_vis, int32_t *idx, void *workspace,
                               hipStream_t stream)
{
    const int64_t Q = (int64_t)U * T;
    if (!use_fused(T, Q, N)) {
        float *scores = static_cast<float *>(workspace);
        void *ws2 = static_cast<char *>(workspace) + align256((size_t)Q * (size_t)N * 4);
        hipError_t e = launch_indexer(U, T, N, idx_q, idx_w, idx_k, n_vis, scores, stream);
        if (e != hipSuccess) return e;
        return launch_topk(Q, N, K, scores, n_vis, idx, ws2, stream);
    }
    const int64_t chunks = fused_chunks(N);
    if (chunks == 1) {
        hipLaunchKernelGGL(indexer_select_kernel, dim3((unsigned)Q), dim3(kNT), 0, stream, T, N, K, chunks, idx_q,
                           idx_w, idx_k, n_vis, idx, (uint32_t *)nullptr);
        return hipGetLastError();
    }
    uint32_t *keys;
    int32_t *ids;
    topk_level1_buffers(workspace, Q, chunks, K, &keys, &ids);
    hipLaunchKernelGGL(indexer_select_kernel, dim3((unsigned)(Q * chunks)), dim3(kNT), 0, stream, T, N, K, chunks,
                       idx_q, idx_w, idx_k, n_vis, ids, keys);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_topk_merge(Q, N, K, kFRows, chunks, n_vis, idx, workspace, stream);
}

}  // namespace ds4a
