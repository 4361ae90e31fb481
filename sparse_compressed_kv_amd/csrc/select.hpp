// select.hpp — workgroup radix select of the K largest keys (device code shared by the
// top-k kernels and the fused indexer + select kernel).  Keys are order-preserving uint32
// images of fp32 scores; ties go to the lower position, so one total order holds everywhere.
#pragma once

#include "common.hpp"

#include <type_traits>

namespace ds4a {

namespace {

constexpr int kNT = 512;                      // threads per selecting workgroup
constexpr int kNW = kNT / kWave;
constexpr int kDirectMax = 16384;             // keys per workgroup (implicit rows)
constexpr int kMergeMax = 12288;              // candidates per workgroup (explicit rows)
constexpr int kLevelChunk = 8192;             // candidates per workgroup in intermediate levels
constexpr int kBins = 256;
constexpr int kMaxLevels = 12;              // each level shrinks a list by >= 4x
constexpr int kSelCopies = 8;               // histogram copies (SelectSharedT) where keys crowd into few bins


// Histogram scratch of the select.  CP > 1 splits every histogram into CP copies, lane l
// counting into copy l % CP: a wave's lanes whose keys fall into one bin then add to CP
// addresses instead of one (an LDS atomic serialises lanes on one address), which matters when
// the keys crowd into a few bins, as merge candidates do.  Copy c's row starts 4c banks after
// copy c - 1's (rows of kBins + 4 words), so lanes of different copies never meet in a bank on
// one bin.
template <int CP>
struct SelectSharedT {
    static constexpr int kRow = CP > 1 ? kBins + 4 : kBins;
    alignas(16) uint32_t hist[3][CP][kRow];  // digit histograms, used by turns (pass p counts into p % 3)
    alignas(16) uint32_t wave_a[kNW];
    alignas(16) uint32_t wave_mn[kNW];       // per wave: min over present keys of (key - 1), max of keys
    alignas(16) uint32_t wave_mx[kNW];
};
using SelectShared = SelectSharedT<1>;

// Chunk sizes of the levels that produced a candidate list, first level on rows.
struct Levels {
    int n;
    int ch[kMaxLevels];
};

// Valid candidates of a query with nv visible rows after the given levels: each chunk of
// a level keeps min(K, its size), and the kept ones are stored contiguously.  In 32 bits: nv
// < 2^31, and a merged level's chunks hold at least 4K rows, so every count stays below 2^30.
__device__ __forceinline__ int64_t cand_count(int64_t nv, int K, const Levels &lv) {
    uint32_t c = (uint32_t)nv;
#pragma unroll
    for (int l = 0; l < kMaxLevels; ++l) {    // constant indices: the levels stay in registers
        if (l < lv.n) {
            const uint32_t ch = (uint32_t)lv.ch[l];
            const uint32_t m = c % ch;
            c = (c / ch) * (uint32_t)K + (m < (uint32_t)K ? m : (uint32_t)K);
        }
    }
    return (int64_t)c;
}

// A buffer resource over `bytes` bytes at p (wave-uniform): loads past its end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t list_rsrc(const void *p, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uintptr_t>(p);
    const uint64_t au = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(au), (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Exclusive prefix sum over the workgroup (kNW waves: the totals are read at once, not one
// dependent read per earlier wave).  Once per workgroup: wave_sums is not reused.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t *wave_sums) {
    static_assert(kNW == 8, "two 16-byte reads cover the wave totals");
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const uint32_t incl = wave_incl_scan_dpp(v);
    if (lane == kWave - 1) wave_sums[wave] = incl;
    __syncthreads();
    const u32x4 s0 = *reinterpret_cast<const u32x4 *>(wave_sums);
    const u32x4 s1 = *reinterpret_cast<const u32x4 *>(wave_sums + 4);
    uint32_t off = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        off += i < wave ? s0[i] : 0u;
        off += i + 4 < wave ? s1[i] : 0u;
    }
    return off + incl - v;           // wave_sums is not written again: no barrier after the reads
}

// Min over present keys and max over the workgroup, from each thread's min of (key - 1) and max
// of key.  Its slots are used once per select, so no barrier follows the reads.
template <int NT, int CP>
__device__ void block_minmax(uint32_t kmin1, uint32_t kmax1, uint32_t &kmin, uint32_t &kmax, SelectSharedT<CP> &sm) {
    wave_minmax_u32(kmin1, kmax1);
    if ((threadIdx.x & (kWave - 1)) == 0) {
        sm.wave_mn[threadIdx.x / kWave] = kmin1;
        sm.wave_mx[threadIdx.x / kWave] = kmax1;
    }
    __syncthreads();
    kmin = 0xFFFFFFFFu;
    kmax = 0u;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) {
        kmin = sm.wave_mn[i] < kmin ? sm.wave_mn[i] : kmin;
        kmax = sm.wave_mx[i] > kmax ? sm.wave_mx[i] : kmax;
    }
    kmin += 1u;
}

// Selects the `need` largest of the n keys held in registers (thread t holds positions
// t*EPT .. t*EPT+EPT-1; ties go to the lower position) and writes their rows (id[i] if IDS, else
// row0 + position) in ascending position order to out[0..need), then -1 up to K.  If out_keys,
// the selected keys go there too.  Every thread of the NT-thread workgroup calls it.
// Positions 0 .. n-1 hold present keys, which are never 0 (float_key maps no float to 0), and
// every later position holds 0; need = min(K, n).  A key of 0 is thus absent, and no step tests
// positions against n: absent keys stay below every threshold, and the one histogram bin they can
// reach (bin 0) is corrected by their number.
// The selection goes from registers straight to out / out_keys: a taken key's slot is its rank.
// CP: copies of each histogram (SelectSharedT).
template <int EPT, bool IDS, int NT = kNT, int CP = 1>
__device__ __forceinline__ void block_select(const uint32_t (&key)[EPT], const int32_t (&id)[EPT], int64_t row0, int n, int need,
                             int K, int32_t *out, uint32_t *out_keys, SelectSharedT<CP> &sm)
{
    static_assert(CP >= 1 && CP <= 8 && (CP & (CP - 1)) == 0, "histogram copies");
    constexpr int kRow = SelectSharedT<CP>::kRow;
    constexpr int kHistV4 = CP * kRow / 4;    // one histogram (all copies) as 16-byte words
    static_assert(NT % kWave == 0 && NT <= kNT && NT >= 2 * kWave && kBins == 4 * kWave, "workgroup size");
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int j0 = threadIdx.x * EPT;
    uint32_t T = 1u, ties = 0xFFFFFFFFu;      // take keys > T and the first `ties` keys == T (T = 1: all present)
    if (need < n) {                           // uniform; implies n > 0 and need > 0
        // min over present keys: key - 1 takes absent keys (0) to the top of the range
        uint32_t kmin1 = 0xFFFFFFFFu, kmax1 = 0u;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const uint32_t k1 = key[i] - 1u;
            kmin1 = k1 < kmin1 ? k1 : kmin1;
            kmax1 = key[i] > kmax1 ? key[i] : kmax1;
        }
        // the first two histograms, cleared before the barrier of the min/max
        for (int i = (int)threadIdx.x; i < 2 * kHistV4; i += NT)
            reinterpret_cast<u32x4 *>(&sm.hist[0][0][0])[i] = u32x4{0u, 0u, 0u, 0u};
        uint32_t kmin, kmax;
        block_minmax<NT, CP>(kmin1, kmax1, kmin, kmax, sm);
        int bit = kmin == kmax ? 0 : 32 - __clz(kmin ^ kmax);
        uint32_t pmask = bit >= 32 ? 0u : ~((1u << bit) - 1u);
        uint32_t prefix = kmin & pmask;
        uint32_t remaining = (uint32_t)need;
        const uint32_t absent = (uint32_t)(NT * EPT - n);
        bool whole_bin = false;
        // One histogram per pass, three in turn: after pass p's barrier every wave reads
        // hist[p % 3] and finds the boundary bin itself (no second barrier), and wave 0 clears
        // hist[(p + 2) % 3], last read before that barrier and next counted into after the next.
        int h = 0;
        bool first = true;
        while (bit > 0) {
            const int width = bit < 8 ? bit : 8;
            const int shift = bit - width;
            const uint32_t dmask = (1u << width) - 1u;
            uint32_t *hist = sm.hist[h][CP > 1 ? (lane & (CP - 1)) : 0];   // this lane's copy
            // Absent keys reach bin 0 when they match the prefix: in the first pass, which tests no
            // prefix (every present key shares it), or when the prefix is 0.
            const bool absent_in_0 = first || prefix == 0u;
            if (first) {
#pragma unroll
                for (int i = 0; i < EPT; ++i) atomicAdd(&hist[(key[i] >> shift) & dmask], 1u);
            } else {
                // Few keys still match: a wave with none branches over the atomic (an LDS atomic
                // costs the same with or without active lanes).
#pragma unroll
                for (int i = 0; i < EPT; ++i) {
                    const bool m = (key[i] & pmask) == prefix;
                    if (__builtin_amdgcn_ballot_w64(m) != 0) {
                        asm volatile("" ::: "memory");     // keeps the uniform branch a branch
                        if (m) atomicAdd(&hist[(key[i] >> shift) & dmask], 1u);
                    }
                }
            }
            __syncthreads();
            const int hc = h == 0 ? 2 : h - 1;            // (h + 2) % 3
            if (CP == 1) {
                if (wave == 0) reinterpret_cast<u32x4 *>(&sm.hist[hc][0][0])[lane] = u32x4{0u, 0u, 0u, 0u};
            } else {
                for (int i = (int)threadIdx.x; i < kHistV4; i += NT)
                    reinterpret_cast<u32x4 *>(&sm.hist[hc][0][0])[i] = u32x4{0u, 0u, 0u, 0u};
            }
            // lane l owns bins 255-4l .. 252-4l, highest first (summed over the copies)
            u32x4 hv = reinterpret_cast<const u32x4 *>(sm.hist[h][0])[kWave - 1 - lane];
#pragma unroll
            for (int cp = 1; cp < CP; ++cp) hv += reinterpret_cast<const u32x4 *>(sm.hist[h][cp])[kWave - 1 - lane];
            uint32_t v[4] = {hv[3], hv[2], hv[1], hv[0]};
            if (absent_in_0 && lane == kWave - 1) v[3] -= absent;
            const uint32_t s = v[0] + v[1] + v[2] + v[3];
            uint32_t cum = wave_incl_scan_dpp(s) - s;
            uint32_t f_bin = 0, f_cum = 0, f_cnt = 0;
            bool found = false;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (cum < remaining && remaining <= cum + v[i]) {
                    found = true;
                    f_bin = (uint32_t)(kBins - 1 - (4 * lane + i));
                    f_cum = cum;
                    f_cnt = v[i];
                }
                cum += v[i];
            }
            const uint64_t fb = __builtin_amdgcn_ballot_w64(found);   // exactly one lane
            const int src = (int)__builtin_ctzll(fb);
            const uint32_t bin = __builtin_amdgcn_readlane(f_bin, src);
            remaining -= __builtin_amdgcn_readlane(f_cum, src);
            prefix |= bin << shift;
            pmask |= dmask << shift;
            bit = shift;
            whole_bin = __builtin_amdgcn_readlane(f_cnt, src) == remaining;   // the whole boundary bin is taken
            h = h == 2 ? 0 : h + 1;
            first = false;
            if (whole_bin) break;
        }
        T = prefix;
        ties = whole_bin ? 0xFFFFFFFFu : remaining;
    }

    // Index-ordered collection over each thread's contiguous positions.  When every key equal
    // to T is taken (the boundary bin was taken whole, as with distinct keys), a key is taken iff
    // it is >= T and the ties need no ranks.
    const bool all_ties = ties == 0xFFFFFFFFu;        // uniform
    uint32_t gt = 0, eq = 0;
    if (all_ties) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) gt += key[i] >= T ? 1u : 0u;
    } else {
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            gt += key[i] > T ? 1u : 0u;
            eq += key[i] == T ? 1u : 0u;
        }
    }
    // gt and eq totals stay below 2^16 (n <= 16384), so one scan carries both.
    const uint32_t packed = block_excl_scan((gt << 16) | eq, sm.wave_a);
    uint32_t tie_rank = packed & 0xFFFFu;
    uint32_t pos = (packed >> 16) + (tie_rank < ties ? tie_rank : ties);
    // A taken key's slot is its rank; waves with no taken key at a position branch over the store.
    auto collect = [&](auto keys_tag, auto all_tag) __attribute__((always_inline)) {
        constexpr bool KEYS = decltype(keys_tag)::value;
        constexpr bool ALL = decltype(all_tag)::value;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            bool take;
            if (ALL) {
                take = key[i] >= T;
            } else {
                const bool eqk = key[i] == T;
                take = key[i] > T || (eqk && tie_rank < ties);
                tie_rank += eqk ? 1u : 0u;
            }
            if (__builtin_amdgcn_ballot_w64(take) != 0) {
                asm volatile("" ::: "memory");         // keeps the uniform branch a branch
                if (take) {
                    out[pos] = IDS ? id[i] : (int32_t)(row0 + j0 + i);
                    if (KEYS) out_keys[pos] = key[i];
                }
            }
            pos += take ? 1u : 0u;
        }
    };
    if (all_ties) {
        if (out_keys) collect(std::true_type{}, std::true_type{});
        else collect(std::false_type{}, std::true_type{});
    } else {
        if (out_keys) collect(std::true_type{}, std::false_type{});
        else collect(std::false_type{}, std::false_type{});
    }
    for (int i = need + (int)threadIdx.x; i < K; i += NT) {
        out[i] = -1;
        if (out_keys) out_keys[i] = 0u;
    }
}

}  // namespace

}  // namespace ds4a
