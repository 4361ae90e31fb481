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
// first use); LDS holds only the 256-bin histogram and scan scratch:
//   1. min/max of the keys; the bits above their highest differing bit are
//      common to all keys and are skipped;
//   2. 8-bit digit passes: LDS histogram of the keys that match the prefix so
//      far, then wave 0 scans the 256 bins (descending, DPP wavefront scan)
//      for the bin holding the need-th key; stop early once a whole bin is
//      taken;
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

namespace ds4a {

namespace {

constexpr int kNT = 512;                      // threads per selecting workgroup
constexpr int kNW = kNT / kWave;
constexpr int kDirectMax = 16384;             // keys per workgroup (implicit rows)
constexpr int kMergeMax = 12288;              // candidates per workgroup (explicit rows)
constexpr int kLevelChunk = 8192;             // candidates per workgroup in intermediate levels
constexpr int kBins = 256;
constexpr int kMaxLevels = 12;              // each level shrinks a list by >= 4x

constexpr int kMaxK = 2048;

struct SelectShared {
    uint32_t hist[kBins];
    uint32_t wave_a[kNW];
    uint32_t wave_b[kNW];
    uint32_t res[4];
    int32_t sel_id[kMaxK];      // the selected set, in row order, before the coalesced copy-out
    uint32_t sel_key[kMaxK];
};

// Chunk sizes of the levels that produced a candidate list, first level on rows.
struct Levels {
    int n;
    int ch[kMaxLevels];
};

// Valid candidates of a query with nv visible rows after the given levels: each chunk of
// a level keeps min(K, its size), and the kept ones are stored contiguously.
__device__ __forceinline__ int64_t cand_count(int64_t nv, int K, const Levels &lv) {
    int64_t c = nv;
    for (int l = 0; l < lv.n; ++l) {
        const int64_t m = c % lv.ch[l];
        c = (c / lv.ch[l]) * K + (m < K ? m : K);
    }
    return c;
}

// Exclusive prefix sum over the workgroup.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t *wave_sums) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const uint32_t incl = wave_incl_scan_dpp(v);
    if (lane == kWave - 1) wave_sums[wave] = incl;
    __syncthreads();
    uint32_t off = 0;
    for (int i = 0; i < wave; ++i) off += wave_sums[i];
    __syncthreads();
    return off + incl - v;
}

__device__ void block_minmax(uint32_t &kmin, uint32_t &kmax, SelectShared &sm) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    wave_minmax_u32(kmin, kmax);
    if (lane == 0) {
        sm.wave_a[wave] = kmin;
        sm.wave_b[wave] = kmax;
    }
    __syncthreads();
    kmin = 0xFFFFFFFFu;
    kmax = 0u;
    for (int i = 0; i < kNW; ++i) {
        kmin = sm.wave_a[i] < kmin ? sm.wave_a[i] : kmin;
        kmax = sm.wave_b[i] > kmax ? sm.wave_b[i] : kmax;
    }
    __syncthreads();
}

// Selects the `need` largest of the n keys held in registers (thread t holds positions
// t*EPT .. t*EPT+EPT-1; ties go to the lower position) and writes their rows (id[i] if IDS, else
// row0 + position) in ascending position order to out[0..need), then -1 up to K.  If out_keys,
// the selected keys go there too.  Every thread of the workgroup calls it.
template <int EPT, bool IDS>
__device__ void block_select(const uint32_t (&key)[EPT], const int32_t (&id)[EPT], int64_t row0, int n, int need,
                             int K, int32_t *out, uint32_t *out_keys, SelectShared &sm)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int j0 = threadIdx.x * EPT;
    uint32_t T = 0, ties = 0xFFFFFFFFu;       // take key > T, and the first `ties` keys == T
    if (need > 0 && need < n) {
        uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            if (j0 + i < n) {
                kmin = key[i] < kmin ? key[i] : kmin;
                kmax = key[i] > kmax ? key[i] : kmax;
            }
        }
        block_minmax(kmin, kmax, sm);
        int bit = kmin == kmax ? 0 : 32 - __clz(kmin ^ kmax);
        uint32_t pmask = bit >= 32 ? 0u : ~((1u << bit) - 1u);
        uint32_t prefix = kmin & pmask;
        uint32_t remaining = (uint32_t)need;
        bool whole_bin = false;
        while (bit > 0) {
            const int width = bit < 8 ? bit : 8;
            const int shift = bit - width;
            const uint32_t dmask = (1u << width) - 1u;
            for (int b = threadIdx.x; b < kBins; b += kNT) sm.hist[b] = 0;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < EPT; ++i)
                if (j0 + i < n && (key[i] & pmask) == prefix) atomicAdd(&sm.hist[(key[i] >> shift) & dmask], 1u);
            __syncthreads();
            if (threadIdx.x < kWave) {
                // lane l owns bins 255-4l .. 252-4l, highest first
                uint32_t v[4], s = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[i] = sm.hist[kBins - 1 - (4 * lane + i)];
                    s += v[i];
                }
                uint32_t cum = wave_incl_scan_dpp(s) - s;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (cum < remaining && remaining <= cum + v[i]) {
                        sm.res[0] = (uint32_t)(kBins - 1 - (4 * lane + i));
                        sm.res[1] = cum;
                        sm.res[2] = v[i];
                    }
                    cum += v[i];
                }
            }
            __syncthreads();
            remaining -= sm.res[1];
            prefix |= sm.res[0] << shift;
            pmask |= dmask << shift;
            bit = shift;
            whole_bin = sm.res[2] == remaining;   // the whole boundary bin is taken
            __syncthreads();
            if (whole_bin) break;
        }
        T = prefix;
        ties = whole_bin ? 0xFFFFFFFFu : remaining;
    }

    // Index-ordered collection over each thread's contiguous positions.
    uint32_t gt = 0, eq = 0;
    if (need > 0) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            if (j0 + i < n) {
                gt += key[i] > T;
                eq += key[i] == T;
            }
        }
    }
    // gt and eq totals stay below 2^16 (n <= 16384), so one scan carries both.
    const uint32_t packed = block_excl_scan((gt << 16) | eq, sm.wave_a);
    uint32_t tie_rank = packed & 0xFFFFu;
    uint32_t pos = (packed >> 16) + (tie_rank < ties ? tie_rank : ties);
    if (need > 0) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            if (j0 + i < n) {
                bool take = key[i] > T;
                if (key[i] == T) {
                    take = tie_rank < ties;
                    ++tie_rank;
                }
                if (take && pos < (uint32_t)K) {
                    sm.sel_id[pos] = IDS ? id[i] : (int32_t)(row0 + j0 + i);
                    sm.sel_key[pos] = key[i];
                    ++pos;
                }
            }
        }
    }
    (void)lane;
    __syncthreads();
    const int taken = need > 0 ? need : 0;
    for (int i = threadIdx.x; i < K; i += kNT) {
        out[i] = i < taken ? sm.sel_id[i] : -1;
        if (out_keys) out_keys[i] = i < taken ? sm.sel_key[i] : 0u;
    }
}

// ---------------------------------------------------------------- kernels

// One workgroup per (query, chunk of `chunk` <= EPT*kNT rows).  Direct path: chunks == 1,
// out = idx.  Chunked path: out/out_keys = the chunk's K candidate slots.
template <int EPT>
__global__ __launch_bounds__(kNT) void topk_rows_kernel(int64_t N, int K, int chunk, int64_t chunks,
                                                        const float *__restrict__ scores,
                                                        const int32_t *__restrict__ n_vis,
                                                        int32_t *__restrict__ out, uint32_t *__restrict__ out_keys)
{
    __shared__ SelectShared sm;
    const int64_t q = blockIdx.x / chunks;
    const int64_t c = blockIdx.x % chunks;
    const int64_t nv = clamp_nvis(n_vis, q, N);
    const int64_t c0 = c * chunk;
    const int64_t rem = nv - c0;
    const int n = rem <= 0 ? 0 : (rem < chunk ? (int)rem : chunk);
    const float *s = scores + q * N + c0;
    const int j0 = threadIdx.x * EPT;
    // All loads of the thread's contiguous run are issued before any is used.
    float v[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) v[i] = j0 + i < n ? s[j0 + i] : 0.f;
    uint32_t key[EPT];
    int32_t id[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        key[i] = float_key(v[i]);
        id[i] = 0;
    }
    const int need = K < n ? K : n;
    const int64_t slot = (q * chunks + c) * K;
    block_select<EPT, false>(key, id, c0, n, need, K, out + slot, out_keys ? out_keys + slot : nullptr, sm);
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
    const int j0 = threadIdx.x * EPT;
    uint32_t key[EPT];
    int32_t id[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const bool in = j0 + i < n;
        key[i] = in ? ik[j0 + i] : 0u;
        id[i] = in ? ii[j0 + i] : -1;
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

size_t topk_workspace_bytes(int64_t Q, int64_t N, int K) {
    if (direct_path(Q, N)) return 0;
    const int ch = first_chunk(N, K);
    const int64_t chunks = (N + ch - 1) / ch;
    const size_t per = (size_t)Q * (size_t)chunks * (size_t)K;      // candidate slots of level 1
    return 4 * align256(per * 4);                                     // two (keys, ids) sets
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
    const size_t per = (size_t)Q * (size_t)chunks * (size_t)K;
    char *p = static_cast<char *>(workspace);
    uint32_t *keys_a = reinterpret_cast<uint32_t *>(p);
    int32_t *ids_a = reinterpret_cast<int32_t *>(p + align256(per * 4));
    uint32_t *keys_b = reinterpret_cast<uint32_t *>(p + 2 * align256(per * 4));
    int32_t *ids_b = reinterpret_cast<int32_t *>(p + 3 * align256(per * 4));

    if (ch == 8192)
        hipLaunchKernelGGL(topk_rows_kernel<16>, dim3((unsigned)(Q * chunks)), dim3(kNT), 0, stream, N, K, ch, chunks,
                           scores, n_vis, ids_a, keys_a);
    else
        hipLaunchKernelGGL(topk_rows_kernel<32>, dim3((unsigned)(Q * chunks)), dim3(kNT), 0, stream, N, K, ch, chunks,
                           scores, n_vis, ids_a, keys_a);
    Levels lv = {};
    lv.n = 1;
    lv.ch[0] = ch;
    int64_t stride = chunks * K;                 // candidate slots per query in the current list
    while (stride > kMergeMax && lv.n < kMaxLevels) {
        const int64_t chunks2 = (stride + kLevelChunk - 1) / kLevelChunk;
        hipLaunchKernelGGL(topk_cand_kernel<16>, dim3((unsigned)(Q * chunks2)), dim3(kNT), 0, stream, N, K, lv,
                           stride, kLevelChunk, chunks2, keys_a, ids_a, n_vis, ids_b, keys_b);
        lv.ch[lv.n++] = kLevelChunk;
        stride = chunks2 * K;
        uint32_t *tk = keys_a; keys_a = keys_b; keys_b = tk;
        int32_t *ti = ids_a; ids_a = ids_b; ids_b = ti;
    }
    if (stride > kMergeMax) return hipErrorInvalidValue;
    hipLaunchKernelGGL(topk_cand_kernel<24>, dim3((unsigned)Q), dim3(kNT), 0, stream, N, K, lv, stride, kMergeMax,
                       (int64_t)1, keys_a, ids_a, n_vis, idx, (uint32_t *)nullptr);
    return hipGetLastError();
}

}  // namespace ds4a
