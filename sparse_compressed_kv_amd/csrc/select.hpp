// select.hpp — workgroup radix select of the K largest keys (device code shared by the
// top-k kernels and the fused indexer + select kernel).  Keys are order-preserving uint32
// images of fp32 scores; ties go to the lower position, so one total order holds everywhere.
#pragma once

#include "common.hpp"

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

// Thread t receives src_a/src_b[t*EPT .. t*EPT + EPT - 1] (0 past n, n <= EPT*kNT, n uniform
// across the workgroup) through LDS stages of EPT*kNT words each: the global loads of both
// arrays are lane-consecutive (one 256-byte run per wave instruction) and all issued before
// any is used; indices past n are clamped to n - 1, so no load is conditional.  Every thread
// of the workgroup calls it.
template <int EPT>
__device__ __forceinline__ void load_blocked2(const uint32_t *__restrict__ src_a, const uint32_t *__restrict__ src_b,
                                              int n, uint32_t (&va)[EPT], uint32_t (&vb)[EPT], uint32_t *stage_a,
                                              uint32_t *stage_b) {
    if (n > 0) {
        uint32_t xa[EPT], xb[EPT];
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int j = (int)threadIdx.x + i * kNT;
            xa[i] = src_a[j < n ? j : n - 1];
            xb[i] = src_b[j < n ? j : n - 1];
        }
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            stage_a[(int)threadIdx.x + i * kNT] = xa[i];
            stage_b[(int)threadIdx.x + i * kNT] = xb[i];
        }
    }
    __syncthreads();
    const int j0 = (int)threadIdx.x * EPT;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        va[i] = j0 + i < n ? stage_a[j0 + i] : 0u;
        vb[i] = j0 + i < n ? stage_b[j0 + i] : 0u;
    }
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

template <int NT>
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
    for (int i = 0; i < NT / kWave; ++i) {
        kmin = sm.wave_a[i] < kmin ? sm.wave_a[i] : kmin;
        kmax = sm.wave_b[i] > kmax ? sm.wave_b[i] : kmax;
    }
    __syncthreads();
}

// Selects the `need` largest of the n keys held in registers (thread t holds positions
// t*EPT .. t*EPT+EPT-1; ties go to the lower position) and writes their rows (id[i] if IDS, else
// row0 + position) in ascending position order to out[0..need), then -1 up to K.  If out_keys,
// the selected keys go there too.  Every thread of the NT-thread workgroup calls it.
template <int EPT, bool IDS, int NT = kNT>
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
        static_assert(NT % kWave == 0 && NT <= kNT && NT >= kWave * 2, "workgroup size");
        block_minmax<NT>(kmin, kmax, sm);
        int bit = kmin == kmax ? 0 : 32 - __clz(kmin ^ kmax);
        uint32_t pmask = bit >= 32 ? 0u : ~((1u << bit) - 1u);
        uint32_t prefix = kmin & pmask;
        uint32_t remaining = (uint32_t)need;
        bool whole_bin = false;
        while (bit > 0) {
            const int width = bit < 8 ? bit : 8;
            const int shift = bit - width;
            const uint32_t dmask = (1u << width) - 1u;
            for (int b = threadIdx.x; b < kBins; b += NT) sm.hist[b] = 0;
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
    for (int i = threadIdx.x; i < K; i += NT) {
        out[i] = i < taken ? sm.sel_id[i] : -1;
        if (out_keys) out_keys[i] = i < taken ? sm.sel_key[i] : 0u;
    }
}

}  // namespace

}  // namespace ds4a
