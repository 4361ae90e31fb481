// topk.hip — A2: exact top-k of the indexer scores, ties to the lower row index.
//
// "Reading the architecture of DwarfStar (ds4.c), part 1/8" (Qiita), section
// 3-3: only the n_indexer_top_k best-scoring compressed rows (512; 1024 for
// Pro, section 2) reach the main attention.  Selection is exact on the fp32
// scores, compared through an order-preserving uint32 key; equal scores go to
// the lower row index; the chosen rows are returned in ascending order.
//
// Core: block_select, one workgroup radix-selecting `need` of n keys held in
// registers (each thread a contiguous run of up to 32 keys, all loaded before
// first use); LDS holds only 256-bin histograms and scan scratch:
//   1. min/max of the keys; the bits above their highest differing bit are
//      common to all keys and are skipped;
//   2. 8-bit digit passes: each wave histograms its keys that match the prefix
//      so far, then every wave sums the per-wave histograms and scans the 256
//      bins (descending, DPP wavefront scan) for the bin holding the need-th
//      key, one barrier per pass; stop early once a whole bin is taken;
//   3. the result is a threshold key T plus a number of ties (keys == T) to
//      take in row order; one block scan of packed (above, tie) counts gives
//      every thread its output offset, so the set is written in ascending row
//      order with no sort.
// Shapes:
//   * direct: one workgroup per query (N <= 8192, or N <= 16384 with many queries);
//   * chunked: workgroups select the top-k of 8192- or 16384-row chunks and
//     write (key, row) candidates; candidate lists are reduced the same way
//     until one workgroup per query selects the final set.
// A chunk's own top-k contains every global top-k row of that chunk (the tie
// rule is one total order everywhere), so the result is exact.
#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

#include <type_traits>

namespace ds4a {

namespace {

// ---------------------------------------------------------------- kernels

// One workgroup per (query, chunk of `chunk` <= EPT*kNT rows).  Direct path: chunks == 1,
// out = idx.  Chunked path: out/out_keys = the chunk's K candidate slots.
template <int EPT>
__global__ __launch_bounds__(kNT) void topk_rows_kernel(int64_t N, int K, int chunk, int64_t chunks,
                                                        const float *__restrict__ scores,
                                                        const int32_t *__restrict__ n_vis,
                                                        int32_t *__restrict__ out, uint32_t *__restrict__ out_keys)
{
    __shared__ SelectSharedT<kSelCopies> sm;       // copies: later passes crowd into the boundary bin
    const int64_t q = blockIdx.x / chunks;
    const int64_t c = blockIdx.x % chunks;
    const int64_t nv = clamp_nvis(n_vis, q, N);
    const int64_t c0 = c * chunk;
    const int64_t rem = nv - c0;
    const int n = rem <= 0 ? 0 : (rem < chunk ? (int)rem : chunk);
    const float *s = scores + q * N + c0;
    const int j0 = threadIdx.x * EPT;
    // All loads of the thread's contiguous run are issued before any is used (scores of one
    // query are contiguous, so the run is a few full cache lines per thread).
    float v[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) v[i] = j0 + i < n ? s[j0 + i] : 0.f;
    uint32_t key[EPT];
    int32_t id[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        key[i] = j0 + i < n ? float_key(v[i]) : 0u;   // absent positions hold 0
        id[i] = 0;
    }
    const int need = K < n ? K : n;
    const int64_t slot = (q * chunks + c) * K;
    block_select<EPT, false, kNT, kSelCopies>(key, id, c0, n, need, K, out + slot, out_keys ? out_keys + slot : nullptr, sm);
}

// One workgroup per (query, chunk of `chunk` <= EPT*kNT candidates).  The candidates of query q
// are the first cand_count(nv, K, lv) entries of in_keys/in_ids[q * in_stride ...].
template <int EPT>
__global__ __launch_bounds__(kNT) void topk_cand_kernel(int64_t N, int K, Levels lv, int64_t in_stride, int chunk,
                                                        int64_t chunks, const uint32_t *__restrict__ in_keys,
                                                        const int32_t *__restrict__ in_ids,
                                                        const int32_t *__restrict__ n_vis,
                                                        int32_t *__restrict__ out, uint32_t *__restrict__ out_keys)
{
    __shared__ SelectShared sm;
    const int64_t q = blockIdx.x / chunks;
    const int64_t c = blockIdx.x % chunks;
    int64_t count = cand_count(clamp_nvis(n_vis, q, N), K, lv);
    if (count > in_stride) count = in_stride;
    const int64_t c0 = c * chunk;
    const int64_t rem = count - c0;
    const int n = rem <= 0 ? 0 : (rem < chunk ? (int)rem : chunk);
    const uint32_t *ik = in_keys + q * in_stride + c0;
    const int32_t *ii = in_ids + q * in_stride + c0;
    // Thread t's contiguous run of candidates straight into registers, 16 bytes per load when
    // both lists start 16-byte aligned (K a multiple of 4), else 4; the buffers end at the list's
    // n entries, so positions past it read as zeros.
    static_assert(EPT % 4 == 0, "candidates are loaded four at a time");
    const __amdgpu_buffer_rsrc_t rk = list_rsrc(ik, (uint32_t)n * 4u), ri = list_rsrc(ii, (uint32_t)n * 4u);
    const int j0 = threadIdx.x * EPT;
    uint32_t key[EPT];
    int32_t id[EPT];
    if (((reinterpret_cast<uintptr_t>(ik) | reinterpret_cast<uintptr_t>(ii)) & 15u) == 0) {
#pragma unroll
        for (int v = 0; v < EPT / 4; ++v) {
            const uint32_t off = (uint32_t)(j0 + 4 * v) * 4u;
            const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
            const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ri, off, 0, 0));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                key[4 * v + e] = a[e];
                id[4 * v + e] = (int32_t)b[e];
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            key[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, (uint32_t)(j0 + i) * 4u, 0, 0);
            id[i] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ri, (uint32_t)(j0 + i) * 4u, 0, 0);
        }
    }
    const int need = K < n ? K : n;
    const int64_t slot = (q * chunks + c) * K;
    block_select<EPT, true>(key, id, 0, n, need, K, out + slot, out_keys ? out_keys + slot : nullptr, sm);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool direct_path(int64_t Q, int64_t N) { return N <= 8192 || (N <= kDirectMax && Q >= 256); }

int first_chunk(int64_t N, int K) {
    const int64_t c8 = (N + 8191) / 8192;
    return c8 * K <= kMergeMax ? 8192 : kDirectMax;
}

}  // namespace

size_t topk_cand_workspace_bytes(int64_t Q, int64_t chunks, int K) {
    const size_t per = (size_t)Q * (size_t)chunks * (size_t)K;      // candidate slots of level 1
    return 4 * align256(per * 4);                                     // two (keys, ids) sets
}

void topk_level1_buffers(void *workspace, int64_t Q, int64_t chunks, int K, uint32_t **keys, int32_t **ids) {
    const size_t per = (size_t)Q * (size_t)chunks * (size_t)K;
    char *p = static_cast<char *>(workspace);
    *keys = reinterpret_cast<uint32_t *>(p);
    *ids = reinterpret_cast<int32_t *>(p + align256(per * 4));
}

size_t topk_workspace_bytes(int64_t Q, int64_t N, int K) {
    if (direct_path(Q, N)) return 0;
    const int ch = first_chunk(N, K);
    return topk_cand_workspace_bytes(Q, (N + ch - 1) / ch, K);
}

hipError_t launch_topk_merge_levels(int64_t Q, int64_t N, int K, int chunk, int64_t chunks, const int32_t *n_vis,
                                    void *workspace, int64_t max_last, CandList *list, hipStream_t stream)
{
    static_assert(kMaxLevels <= CandList::kMaxLevels, "level chunk sizes fit the host list");
    const size_t per = (size_t)Q * (size_t)chunks * (size_t)K;
    char *p = static_cast<char *>(workspace);
    uint32_t *keys_a = reinterpret_cast<uint32_t *>(p);
    int32_t *ids_a = reinterpret_cast<int32_t *>(p + align256(per * 4));
    uint32_t *keys_b = reinterpret_cast<uint32_t *>(p + 2 * align256(per * 4));
    int32_t *ids_b = reinterpret_cast<int32_t *>(p + 3 * align256(per * 4));
    Levels lv = {};
    lv.n = 1;
    lv.ch[0] = chunk;
    int64_t stride = chunks * K;                 // candidate slots per query in the current list
    while (stride > max_last && lv.n < kMaxLevels) {
        const int64_t chunks2 = (stride + kLevelChunk - 1) / kLevelChunk;
        hipLaunchKernelGGL(topk_cand_kernel<16>, dim3((unsigned)(Q * chunks2)), dim3(kNT), 0, stream, N, K, lv,
                           stride, kLevelChunk, chunks2, keys_a, ids_a, n_vis, ids_b, keys_b);
        lv.ch[lv.n++] = kLevelChunk;
        stride = chunks2 * K;
        uint32_t *tk = keys_a; keys_a = keys_b; keys_b = tk;
        int32_t *ti = ids_a; ids_a = ids_b; ids_b = ti;
    }
    if (stride > max_last) return hipErrorInvalidValue;
    list->keys = keys_a;
    list->ids = ids_a;
    list->stride = stride;
    list->n_levels = lv.n;
    for (int l = 0; l < lv.n; ++l) list->level_rows[l] = lv.ch[l];
    return hipGetLastError();
}

hipError_t launch_topk_merge(int64_t Q, int64_t N, int K, int chunk, int64_t chunks, const int32_t *n_vis,
                             int32_t *idx, void *workspace, hipStream_t stream)
{
    CandList cl;
    if (hipError_t e = launch_topk_merge_levels(Q, N, K, chunk, chunks, n_vis, workspace, kMergeMax, &cl, stream);
        e != hipSuccess)
        return e;
    const uint32_t *keys_a = cl.keys;
    const int32_t *ids_a = cl.ids;
    const int64_t stride = cl.stride;
    Levels lv = {};
    lv.n = cl.n_levels;
    for (int l = 0; l < lv.n; ++l) lv.ch[l] = cl.level_rows[l];
    // The last level: one workgroup per query, with as few candidates per thread as the list
    // needs (each select pass walks every thread's EPT keys).
    const auto last = [&](auto ept_tag) {
        constexpr int kEpt = decltype(ept_tag)::value;
        hipLaunchKernelGGL(topk_cand_kernel<kEpt>, dim3((unsigned)Q), dim3(kNT), 0, stream, N, K, lv, stride,
                           kEpt * kNT, (int64_t)1, keys_a, ids_a, n_vis, idx, (uint32_t *)nullptr);
    };
    if (stride <= 4 * kNT)
        last(std::integral_constant<int, 4>{});
    else if (stride <= 8 * kNT)
        last(std::integral_constant<int, 8>{});
    else if (stride <= 12 * kNT)
        last(std::integral_constant<int, 12>{});
    else if (stride <= kLevelChunk)
        last(std::integral_constant<int, 16>{});
    else
        hipLaunchKernelGGL(topk_cand_kernel<24>, dim3((unsigned)Q), dim3(kNT), 0, stream, N, K, lv, stride, kMergeMax,
                           (int64_t)1, keys_a, ids_a, n_vis, idx, (uint32_t *)nullptr);
    return hipGetLastError();
}

hipError_t launch_topk(int64_t Q, int64_t N, int K, const float *scores, const int32_t *n_vis,
                       int32_t *idx, void *workspace, hipStream_t stream)
{
    if (direct_path(Q, N)) {
        if (N <= 8192)
            hipLaunchKernelGGL(topk_rows_kernel<16>, dim3((unsigned)Q), dim3(kNT), 0, stream, N, K, (int)N,
                               (int64_t)1, scores, n_vis, idx, (uint32_t *)nullptr);
        else
            hipLaunchKernelGGL(topk_rows_kernel<32>, dim3((unsigned)Q), dim3(kNT), 0, stream, N, K, (int)N,
                               (int64_t)1, scores, n_vis, idx, (uint32_t *)nullptr);
        return hipGetLastError();
    }
    const int ch = first_chunk(N, K);
    const int64_t chunks = (N + ch - 1) / ch;
    uint32_t *keys_a;
    int32_t *ids_a;
    topk_level1_buffers(workspace, Q, chunks, K, &keys_a, &ids_a);
    if (ch == 8192)
        hipLaunchKernelGGL(topk_rows_kernel<16>, dim3((unsigned)(Q * chunks)), dim3(kNT), 0, stream, N, K, ch, chunks,
                           scores, n_vis, ids_a, keys_a);
    else
        hipLaunchKernelGGL(topk_rows_kernel<32>, dim3((unsigned)(Q * chunks)), dim3(kNT), 0, stream, N, K, ch, chunks,
                           scores, n_vis, ids_a, keys_a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_topk_merge(Q, N, K, ch, chunks, n_vis, idx, workspace, stream);
}

}  // namespace ds4a
