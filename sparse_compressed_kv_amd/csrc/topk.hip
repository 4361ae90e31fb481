// topk.hip — A2: exact top-k of the indexer scores, ties to the lower row index.
//
// "Reading the architecture of DwarfStar (ds4.c), part 1/8" (Qiita), section
// 3-3: only the n_indexer_top_k best-scoring compressed rows (512; 1024 for
// Pro, section 2) reach the main attention.  Selection here is exact on the
// fp32 scores, compared through an order-preserving uint32 key; equal scores
// go to the lower row index; the chosen rows are returned in ascending order.
//
// Two shapes of the same radix select:
//  * N <= kLdsMaxN: one 1024-thread workgroup per query holds all keys in LDS.
//    It first reduces min/max, skips the key bits all keys share, then runs
//    11-bit digit passes (LDS histogram, block scan for the bin holding the
//    k-th key) until the k-th key is exact; the ties it needs are then taken
//    in index order by a block-wide ordered scan.
//  * larger N: (1) a fill kernel clears the per-query histograms; (2) many
//    workgroups per query histogram the top 12 key bits, and the last one to
//    finish finds the boundary bin; (3) the same workgroups write every row
//    above that bin straight to the output and compact the boundary bin's rows
//    as 64-bit (key, ~index) composites (all distinct, so no tie rule is left);
//    (4) one workgroup per query radix-selects the remainder from those
//    composites and sorts the final set.
// Wave-level ballots aggregate the output/candidate counters, and all scans are
// LDS-staged wave scans.
#include "common.hpp"
#include "launch.hpp"

namespace ds4a {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kLdsMaxN = 16384;
constexpr int kMaxK = 2048;
constexpr int kBins = 2048;                 // 11-bit digits in the LDS passes
constexpr int kTopBins = 4096;              // 12-bit first digit of the multi-workgroup path
constexpr int kCtr = 8;                     // per-query counters after the histogram
constexpr int kChunk = 16384;               // scores per workgroup in the multi-workgroup path
constexpr int kPassThreads = 256;

// ------------------------------------------------------------ block helpers

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        uint32_t t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
}

// Exclusive prefix sum over the block; also returns the block total.  s_wave: NT/64 words.
template <int NT>
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t *s_wave, uint32_t &total) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const uint32_t incl = wave_incl_scan(v, lane);
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        uint32_t x = lane < NT / kWave ? s_wave[lane] : 0u;
        x = wave_incl_scan(x, lane);
        if (lane < NT / kWave) s_wave[lane] = x;
    }
    __syncthreads();
    const uint32_t off = wave ? s_wave[wave - 1] : 0u;
    total = s_wave[NT / kWave - 1];
    __syncthreads();
    return off + incl - v;
}

// Largest bin b with sum_{b' >= b} hist[b'] >= need (need >= 1, total >= need).
// Writes b and the count strictly above it to out[0], out[1].
template <int NT, int NB>
__device__ void find_boundary(const uint32_t *hist, uint32_t need, uint32_t *s_wave, uint32_t *out) {
    constexpr int BPT = NB / NT;
    const int t = threadIdx.x;
    uint32_t v[BPT], local = 0;
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
        v[k] = hist[NB - 1 - (t * BPT + k)];      // descending bin order
        local += v[k];
    }
    uint32_t total;
    uint32_t cum = block_excl_scan<NT>(local, s_wave, total);
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
        if (cum < need && need <= cum + v[k]) {
            out[0] = (uint32_t)(NB - 1 - (t * BPT + k));
            out[1] = cum;
        }
        cum += v[k];
    }
    __syncthreads();
}

// Ascending bitonic sort of sel[0..n) (n <= kMaxK), then idx_out[0..K) = sorted set, -1 padded.
__device__ void sort_and_write(int32_t *sel, int n, int K, int32_t *idx_out) {
    int P = 1;
    while (P < n) P <<= 1;
    for (int i = n + threadIdx.x; i < P; i += blockDim.x) sel[i] = 0x7FFFFFFF;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < P; i += blockDim.x) {
                const int p = i ^ j;
                if (p > i) {
                    const int32_t a = sel[i], b = sel[p];
                    const bool up = (i & k) == 0;
                    if ((a > b) == up) {
                        sel[i] = b;
                        sel[p] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = threadIdx.x; i < K; i += blockDim.x) idx_out[i] = i < n ? sel[i] : -1;
}

// Wave-aggregated atomic slot reservation: returns this lane's slot if pred.
__device__ __forceinline__ uint32_t wave_reserve(uint32_t *ctr, bool pred) {
    const int lane = threadIdx.x & (kWave - 1);
    const unsigned long long mask = __ballot(pred);
    if (!mask) return 0;
    const int leader = __ffsll((long long)mask) - 1;
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(ctr, (uint32_t)__popcll(mask));
    base = __shfl(base, leader, kWave);
    return base + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
}

// ------------------------------------------------------------- LDS path

__global__ __launch_bounds__(kSelThreads) void topk_lds_kernel(
    int64_t N, int K, const float *__restrict__ scores, const int32_t *__restrict__ n_vis,
    int32_t *__restrict__ idx)
{
    extern __shared__ uint32_t keys[];                 // nv keys
    __shared__ uint32_t hist[kBins];
    __shared__ int32_t sel[kMaxK];
    __shared__ uint32_t s_wave[kSelThreads / kWave];
    __shared__ uint32_t s_res[4];
    __shared__ uint32_t s_n;

    const int64_t q = blockIdx.x;
    const int nv = (int)clamp_nvis(n_vis, q, N);
    const float *s = scores + q * N;
    int32_t *out = idx + q * (int64_t)K;
    const int need = K < nv ? K : nv;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;

    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for (int j = threadIdx.x; j < nv; j += kSelThreads) {
        const uint32_t k = float_key(s[j]);
        keys[j] = k;
        kmin = k < kmin ? k : kmin;
        kmax = k > kmax ? k : kmax;
    }
    if (threadIdx.x == 0) s_n = 0;
    // min / max over the block
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const uint32_t a = __shfl_xor(kmin, o, kWave), b = __shfl_xor(kmax, o, kWave);
        kmin = a < kmin ? a : kmin;
        kmax = b > kmax ? b : kmax;
    }
    __shared__ uint32_t s_min[kSelThreads / kWave], s_max[kSelThreads / kWave];
    if (lane == 0) {
        s_min[wave] = kmin;
        s_max[wave] = kmax;
    }
    __syncthreads();
    kmin = 0xFFFFFFFFu;
    kmax = 0u;
    for (int i = 0; i < kSelThreads / kWave; ++i) {
        kmin = s_min[i] < kmin ? s_min[i] : kmin;
        kmax = s_max[i] > kmax ? s_max[i] : kmax;
    }

    if (need == 0) {
        for (int i = threadIdx.x; i < K; i += kSelThreads) out[i] = -1;
        return;
    }

    uint32_t kth;
    uint32_t ties_needed;
    if (need == nv) {
        kth = kmin;                       // everything is taken
        ties_needed = 0xFFFFFFFFu;
    } else {
        // Bits above `bit` are common to every key.
        int bit = (kmin == kmax) ? 0 : 32 - __clz(kmin ^ kmax);
        uint32_t pmask = bit >= 32 ? 0u : ~((1u << bit) - 1u);
        uint32_t prefix = kmin & pmask;
        uint32_t remaining = (uint32_t)need;
        while (bit > 0) {
            const int width = bit < 11 ? bit : 11;
            const int shift = bit - width;
            const uint32_t dmask = (1u << width) - 1u;
            for (int b = threadIdx.x; b < kBins; b += kSelThreads) hist[b] = 0;
            __syncthreads();
            for (int j = threadIdx.x; j < nv; j += kSelThreads) {
                const uint32_t k = keys[j];
                if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
            }
            __syncthreads();
            find_boundary<kSelThreads, kBins>(hist, remaining, s_wave, s_res);
            remaining -= s_res[1];
            prefix |= s_res[0] << shift;
            pmask |= dmask << shift;
            bit = shift;
            __syncthreads();
        }
        kth = prefix;
        ties_needed = remaining;          // >= 1 rows equal to kth, taken in index order
    }

    // Collect: every key > kth, and the first ties_needed keys == kth in row order.
    const int per = (nv + kSelThreads - 1) / kSelThreads;
    const int j0 = threadIdx.x * per;
    const int j1 = j0 + per < nv ? j0 + per : nv;
    uint32_t my_ties = 0;
    for (int j = j0; j < j1; ++j) my_ties += keys[j] == kth;
    uint32_t total;
    uint32_t rank = block_excl_scan<kSelThreads>(my_ties, s_wave, total);
    for (int j = j0; j < j1; ++j) {
        const uint32_t k = keys[j];
        bool take = k > kth;
        if (k == kth) {
            take = rank < ties_needed;
            ++rank;
        }
        if (take) {
            const uint32_t slot = atomicAdd(&s_n, 1u);
            if (slot < (uint32_t)kMaxK) sel[slot] = j;
        }
    }
    __syncthreads();
    sort_and_write(sel, need, K, out);
}

// -------------------------------------------------- multi-workgroup path

struct TopkWs {
    uint32_t *hist;      // [Q][kTopBins]
    uint32_t *ctr;       // [Q][kCtr]: 0 done, 1 n_definite, 2 n_cand, 3 boundary bin, 4 above
    uint64_t *cand;      // [Q][N]
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline TopkWs carve(void *ws, int64_t Q, int64_t N) {
    char *p = static_cast<char *>(ws);
    TopkWs w;
    w.hist = reinterpret_cast<uint32_t *>(p);
    p += align256(sizeof(uint32_t) * (size_t)Q * kTopBins);
    w.ctr = reinterpret_cast<uint32_t *>(p);
    p += align256(sizeof(uint32_t) * (size_t)Q * kCtr);
    w.cand = reinterpret_cast<uint64_t *>(p);
    return w;
}

__global__ void topk_clear_kernel(uint32_t *p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

__global__ __launch_bounds__(kPassThreads) void topk_hist_kernel(
    int64_t N, int K, int64_t chunks, const float *__restrict__ scores,
    const int32_t *__restrict__ n_vis, TopkWs ws)
{
    __shared__ uint32_t h[kTopBins];
    __shared__ uint32_t s_wave[kPassThreads / kWave];
    __shared__ uint32_t s_res[2];
    __shared__ bool s_last;
    const int64_t q = blockIdx.x / chunks;
    const int64_t part = blockIdx.x % chunks;
    const int64_t nv = clamp_nvis(n_vis, q, N);
    const int64_t j0 = part * kChunk;
    const int64_t j1 = j0 + kChunk < nv ? j0 + kChunk : nv;
    const float *s = scores + q * N;
    uint32_t *gh = ws.hist + q * kTopBins;
    uint32_t *ctr = ws.ctr + q * kCtr;

    for (int b = threadIdx.x; b < kTopBins; b += kPassThreads) h[b] = 0;
    __syncthreads();
    for (int64_t j = j0 + threadIdx.x; j < j1; j += kPassThreads) atomicAdd(&h[float_key(s[j]) >> 20], 1u);
    __syncthreads();
    for (int b = threadIdx.x; b < kTopBins; b += kPassThreads)
        if (h[b]) atomicAdd(&gh[b], h[b]);
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(&ctr[0], 1u) == (uint32_t)(chunks - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const int64_t need = K < nv ? K : nv;
    if (need == 0) {
        if (threadIdx.x == 0) {
            ctr[3] = 0xFFFFFFFFu;
            ctr[4] = 0;
        }
        return;
    }
    for (int b = threadIdx.x; b < kTopBins; b += kPassThreads) h[b] = __hip_atomic_load(&gh[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    find_boundary<kPassThreads, kTopBins>(h, (uint32_t)need, s_wave, s_res);
    if (threadIdx.x == 0) {
        ctr[3] = s_res[0];
        ctr[4] = s_res[1];
    }
}

__global__ __launch_bounds__(kPassThreads) void topk_filter_kernel(
    int64_t N, int K, int64_t chunks, const float *__restrict__ scores,
    const int32_t *__restrict__ n_vis, int32_t *__restrict__ idx, TopkWs ws)
{
    const int64_t q = blockIdx.x / chunks;
    const int64_t part = blockIdx.x % chunks;
    const int64_t nv = clamp_nvis(n_vis, q, N);
    uint32_t *ctr = ws.ctr + q * kCtr;
    const uint32_t b1 = ctr[3];
    if (b1 == 0xFFFFFFFFu) return;
    const int64_t j0 = part * kChunk;
    const int64_t j1 = j0 + kChunk < nv ? j0 + kChunk : nv;
    const float *s = scores + q * N;
    int32_t *out = idx + q * (int64_t)K;
    uint64_t *cand = ws.cand + q * N;
    // Uniform trip count across the wave so the ballots see every lane.
    for (int64_t jb = j0; jb < j1; jb += kPassThreads) {
        const int64_t j = jb + threadIdx.x;
        const bool in = j < j1;
        const uint32_t k = in ? float_key(s[j]) : 0u;
        const uint32_t bin = k >> 20;
        const bool def = in && bin > b1;
        const bool cnd = in && bin == b1;
        const uint32_t pd = wave_reserve(&ctr[1], def);
        const uint32_t pc = wave_reserve(&ctr[2], cnd);
        if (def && pd < (uint32_t)K) out[pd] = (int32_t)j;
        if (cnd && (int64_t)pc < N) cand[pc] = ((uint64_t)k << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
    }
}

__global__ __launch_bounds__(kSelThreads) void topk_resolve_kernel(
    int64_t N, int K, const int32_t *__restrict__ n_vis, int32_t *__restrict__ idx, TopkWs ws)
{
    __shared__ uint32_t hist[kBins];
    __shared__ int32_t sel[kMaxK];
    __shared__ uint32_t s_wave[kSelThreads / kWave];
    __shared__ uint32_t s_res[2];
    __shared__ uint32_t s_n;
    const int64_t q = blockIdx.x;
    const int64_t nv = clamp_nvis(n_vis, q, N);
    const int need = (int)(K < nv ? K : nv);
    int32_t *out = idx + q * (int64_t)K;
    const uint32_t *ctr = ws.ctr + q * kCtr;
    if (need == 0) {
        for (int i = threadIdx.x; i < K; i += kSelThreads) out[i] = -1;
        return;
    }
    const uint32_t above = ctr[4] < (uint32_t)need ? ctr[4] : (uint32_t)need;
    const uint32_t ncand = (int64_t)ctr[2] < N ? ctr[2] : (uint32_t)N;
    const uint64_t *cand = ws.cand + q * N;
    uint32_t remaining = (uint32_t)need - above;

    // Definite rows written by the filter pass.
    for (uint32_t i = threadIdx.x; i < above; i += kSelThreads) sel[i] = out[i];
    if (threadIdx.x == 0) s_n = above;
    __syncthreads();

    uint64_t prefix = (uint64_t)ctr[3] << 52;
    uint64_t pmask = 0xFFFull << 52;
    if (remaining < ncand) {
        int bit = 52;
        while (bit > 0) {
            const int width = bit < 11 ? bit : 11;
            const int shift = bit - width;
            const uint64_t dmask = (1ull << width) - 1ull;
            for (int b = threadIdx.x; b < kBins; b += kSelThreads) hist[b] = 0;
            __syncthreads();
            for (uint32_t i = threadIdx.x; i < ncand; i += kSelThreads) {
                const uint64_t v = cand[i];
                if ((v & pmask) == prefix) atomicAdd(&hist[(v >> shift) & dmask], 1u);
            }
            __syncthreads();
            find_boundary<kSelThreads, kBins>(hist, remaining, s_wave, s_res);
            remaining -= s_res[1];
            prefix |= (uint64_t)s_res[0] << shift;
            pmask |= dmask << shift;
            bit = shift;
            __syncthreads();
        }
    } else {
        prefix = 0;    // every candidate is taken
    }
    for (uint32_t i = threadIdx.x; i < ncand; i += kSelThreads) {
        const uint64_t v = cand[i];
        if (v >= prefix) {
            const uint32_t slot = atomicAdd(&s_n, 1u);
            if (slot < (uint32_t)kMaxK) sel[slot] = (int32_t)(0xFFFFFFFFu - (uint32_t)(v & 0xFFFFFFFFull));
        }
    }
    __syncthreads();
    sort_and_write(sel, need, K, out);
}

}  // namespace

size_t topk_workspace_bytes(int64_t Q, int64_t N, int K) {
    (void)K;
    if (N <= kLdsMaxN) return 0;
    return align256(sizeof(uint32_t) * (size_t)Q * kTopBins) + align256(sizeof(uint32_t) * (size_t)Q * kCtr) +
           align256(sizeof(uint64_t) * (size_t)Q * (size_t)N);
}

hipError_t launch_topk(int64_t Q, int64_t N, int K, const float *scores, const int32_t *n_vis,
                       int32_t *idx, void *workspace, hipStream_t stream)
{
    if (N <= kLdsMaxN) {
        static bool attr_set = false;
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(topk_lds_kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)(sizeof(uint32_t) * kLdsMaxN));
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        const size_t lds = sizeof(uint32_t) * (size_t)N;
        hipLaunchKernelGGL(topk_lds_kernel, dim3((unsigned)Q), dim3(kSelThreads), lds, stream,
                           N, K, scores, n_vis, idx);
        return hipGetLastError();
    }
    TopkWs ws = carve(workspace, Q, N);
    const int64_t clear_words = (int64_t)((reinterpret_cast<char *>(ws.cand) - static_cast<char *>(workspace)) / 4);
    hipLaunchKernelGGL(topk_clear_kernel, dim3(256), dim3(256), 0, stream, static_cast<uint32_t *>(workspace),
                       clear_words);
    const int64_t chunks = (N + kChunk - 1) / kChunk;
    hipLaunchKernelGGL(topk_hist_kernel, dim3((unsigned)(chunks * Q)), dim3(kPassThreads), 0, stream,
                       N, K, chunks, scores, n_vis, ws);
    hipLaunchKernelGGL(topk_filter_kernel, dim3((unsigned)(chunks * Q)), dim3(kPassThreads), 0, stream,
                       N, K, chunks, scores, n_vis, idx, ws);
    hipLaunchKernelGGL(topk_resolve_kernel, dim3((unsigned)Q), dim3(kSelThreads), 0, stream,
                       N, K, n_vis, idx, ws);
    return hipGetLastError();
}

}  // namespace ds4a
