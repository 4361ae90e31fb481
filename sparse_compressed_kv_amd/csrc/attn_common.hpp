// attn_common.hpp — pieces shared by the two attention kernels (attn.hip: workgroups of
// 64 heads for many queries; attn_dq.hip: workgroups of 16 heads with the dims split over the
// waves, for few queries): the step geometry in LDS, the argument block, the loads that write
// LDS directly, cross-lane reductions and the hi/lo operand split.
#pragma once

#include "common.hpp"

#include <type_traits>

namespace ds4a {

namespace {

constexpr int kAT = 256;                      // threads per workgroup
constexpr int kAW = kAT / kWave;              // waves (4)
constexpr int kWH = 16;                       // heads per MFMA tile (per wave or per workgroup)
constexpr int kD = 512;
constexpr int kRot = 64;
constexpr int kKs = kD / 32;                  // k-steps of QK (16)
constexpr int kDB = kD / 16;                  // 16-dim blocks of PV (32)
constexpr int kSR = 32;                       // rows per step
constexpr int kHR = 16;                       // rows per half step
constexpr int kRW = kSR / kAW;                // rows each wave loads per step (8)
constexpr int kRowStride = 1056;              // LDS bytes per row (1024 + 32)
constexpr int kHalfBuf = kHR * kRowStride;    // 16,896 B
constexpr int kBuf = kSR * kRowStride;        // one ring slot: 33,792 B
constexpr int kCodeRow = 512;                 // E4M3 row as codes
constexpr int kScaleWave = 256;               // E4M3 row scales: bytes per slot and wave (one dword per lane)
constexpr int kCodeBatch = kRW / 2 + 1;       // E4M3 step: DMA instructions per wave (codes, scales)
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
    int T, H, W, K, n_hg, n_chunks, steps_per_chunk, n_steps, n_items;   // n_hg: head groups per query
    int64_t N;
    const void *q;
    const int64_t *pos;
    const uint16_t *raw;
    const void *comp;                        // bf16 [U][N][512], or E4M3 codes [U][N][512]
    const float *comp_scale;                 // E4M3 rows: f32 [U][N]
    const int32_t *idx;                      // sparse: [U][T][K]
    const int32_t *n_vis;                    // dense: visible compressed rows per query, or NULL
    const int32_t *raw_vis;                  // raw rows of each query's window that take part, or NULL
    float scale;
    float *out;
    uint32_t *count;                         // split unions: arrivals per (query, 16-head group)
    float *part;                             // split unions: records
    double log2_theta;
    // Last top-k merge level inside the 16-head kernel (unsplit unions): each query's final
    // candidate list, selected by the workgroup itself into its row table.
    const uint32_t *cand_keys;
    const int32_t *cand_ids;
    int64_t cand_stride;
    const int32_t *cand_nvis;                // the indexer's visible rows per query, or NULL
    int32_t *idx_out;                        // the selected rows [U][T][K], or NULL
    int lv_n;                                // levels that produced the list, and their chunk rows
    int lv_ch[12];
};

// Wait until at most N vector-memory operations of this wave are in flight.  The row loads
// that write LDS directly are issued from inline assembly, so the compiler neither tracks them
// nor adds conservative waits for them; the kernel places these waits itself, and the memory
// clobber keeps every memory access on its side.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

// Loads straight into LDS: buffer_load_dword{x4} ... lds, lane l's 16 (4) bytes at byte offset
// voff of the buffer landing at LDS address lds + 16 l (4 l).  The buffer resource bounds every
// read: a lane whose offset lies past the buffer's last byte reads zeros, which is how rows that
// take no part (offset from row -1, or a raw row at or past raw_vis) become rows of zeros with
// no branch and no other row to read.  M0 takes the LDS address; the s_nop is the one wait
// state an LDS load needs after M0 is written.
// The LDS address is made wave-uniform explicitly (it is, but without optimisation the
// compiler may keep it in a VGPR, which an SGPR operand cannot take).
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, __amdgpu_buffer_rsrc_t rs) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 : : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rs) : "memory", "m0");
}

__device__ __forceinline__ void dma4(uint32_t lds, uint32_t voff, __amdgpu_buffer_rsrc_t rs) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 : : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rs) : "memory", "m0");
}

constexpr int kRawRsrc = 0x00020000;          // word 3 of a raw (stride 0) buffer resource

// A buffer resource over `bytes` bytes at p (bytes < 2^32), from wave-uniform values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uintptr_t>(p);
    const uint64_t au = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(au), (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes), kRawRsrc);
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    typedef __attribute__((address_space(3))) const unsigned char lds_byte;
    return (uint32_t)reinterpret_cast<uintptr_t>((lds_byte *)p);
}

// Lane l and lane l ^ 16 (l ^ 32) combined, with the gfx950 row swaps: after the swap one of
// the two results is the lane's own value and the other its partner's.
__device__ __forceinline__ f32x2 swap16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ f32x2 swap32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float max_g(float v) {       // over the 4 lane groups (lanes c + 16 g)
    f32x2 s = swap16(v);
    v = fmaxf(s[0], s[1]);
    s = swap32(v);
    return fmaxf(s[0], s[1]);
}
__device__ __forceinline__ float sum_g(float v) {
    f32x2 s = swap16(v);
    v = s[0] + s[1];
    s = swap32(v);
    return s[0] + s[1];
}

// 8 floats -> hi/lo pairs of the MFMA operand type as a u32x4 each.
template <bool F16>
__device__ __forceinline__ void split8(const float (&x)[8], u32x4 &hi, u32x4 &lo) {
    if (F16) {
        f16x8 h, l;
        pack_hi_lo8_f16(x, h, l);
        hi = __builtin_bit_cast(u32x4, h);
        lo = __builtin_bit_cast(u32x4, l);
    } else {
        bf16x8 h, l;
        pack_hi_lo8(x, h, l);
        hi = __builtin_bit_cast(u32x4, h);
        lo = __builtin_bit_cast(u32x4, l);
    }
}

template <bool F16>
__device__ __forceinline__ f32x4 mma(const u32x4 &a, const u32x4 &b, f32x4 c) {
    if (F16) return mfma16h(as_f16x8(a), as_f16x8(b), c);
    return mfma16(as_bf16x8(a), as_bf16x8(b), c);
}

using F16T = std::true_type;
using BF16T = std::false_type;


// Row loads of the union's 32-row steps into an LDS ring of NB slots (step j in slot j % NB).
// Raw step: this wave's 8 rows of the query's raw window, 1 KiB each, one instruction per row;
// rows at or past raw_vis lie past the window resource and read as zeros.  Compressed step:
// bf16 rows likewise from their entries (row index, or -1: past the resource, zeros); E4M3 rows
// as codes, two rows per instruction, packed at the start of the slot, plus the rows' scales
// (one dword per lane, lane l holding row l % 8).  The chunk's compressed steps come after its
// raw ones; steps past the chunk are compressed steps of -1 entries.  Row data within a slot:
// row r at r * kRowStride, its 16-byte chunk k at position k ^ ((r >> 2) & 1).
template <bool DENSE, bool E8, int NB>
struct StepLoader {
    unsigned char *ring;
    unsigned char *s_scale;                  // E4M3: [slot][wave][64] f32
    const int32_t *s_row;                    // sparse: compressed row of each union row of the chunk
    __amdgpu_buffer_rsrc_t raw_rs, comp_rs, scale_rs;
    int step0, n, n_raw, rho0, W, wave, lane;
    int64_t j_lim;                           // dense: visible compressed rows

    __device__ __forceinline__ void issue_raw(int j) const {
        const int R0 = (step0 + j) * kSR + wave * kRW;
        const uint32_t dst = lds_addr(ring + (j % NB) * kBuf + wave * kRW * kRowStride);
#pragma unroll
        for (int e = 0; e < kRW; ++e) {
            const int r = wave * kRW + e;
            dma16(dst + e * kRowStride, ((uint32_t)(R0 + e) << 10) + ((uint32_t)(lane ^ ((r >> 2) & 1)) << 4), raw_rs);
        }
    }
    __device__ __forceinline__ void issue_comp(int j, const i32x4 &e0, const i32x4 &e1) const {
        const int slot = j % NB;
        if (!E8) {
            const uint32_t dst = lds_addr(ring + slot * kBuf + wave * kRW * kRowStride);
#pragma unroll
            for (int e = 0; e < kRW; ++e) {
                const int r = wave * kRW + e;
                const int32_t ent = e < 4 ? e0[e] : e1[e - 4];
                dma16(dst + e * kRowStride, ((uint32_t)ent << 10) + ((uint32_t)(lane ^ ((r >> 2) & 1)) << 4), comp_rs);
            }
        } else {
            const uint32_t dst = lds_addr(ring + slot * kBuf + wave * kRW * kCodeRow);
#pragma unroll
            for (int i = 0; i < kRW / 2; ++i) {
                const int32_t ea = i < 2 ? e0[2 * i] : e1[2 * i - 4];
                const int32_t eb = i < 2 ? e0[2 * i + 1] : e1[2 * i - 3];
                const int32_t ent = lane < 32 ? ea : eb;
                dma16(dst + i * 2 * kCodeRow, ((uint32_t)ent << 9) + ((uint32_t)(lane & 31) << 4), comp_rs);
            }
            const int l8 = lane & 7;
            const int32_t es = l8 < 4 ? e0[l8 & 3] : e1[l8 & 3];
            dma4(lds_addr(s_scale + (slot * kAW + wave) * kScaleWave), (uint32_t)es << 2, scale_rs);
        }
    }
    // This wave's 8 row entries of local step j: from the row table (sparse) or the position
    // (dense); raw steps and steps past the chunk have none.
    __device__ __forceinline__ void entries(int j, i32x4 &e0, i32x4 &e1) const {
        e0 = i32x4{-1, -1, -1, -1};
        e1 = e0;
        if (j >= n || j < n_raw) return;
        const int rho = (step0 + j) * kSR + wave * kRW;
        if (!DENSE) {
            e0 = *reinterpret_cast<const i32x4 *>(s_row + (rho - rho0));   // same address in every lane
            e1 = *reinterpret_cast<const i32x4 *>(s_row + (rho - rho0) + 4);
            return;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            e0[r] = (int64_t)(rho + r - W) < j_lim ? rho + r - W : -1;
            e1[r] = (int64_t)(rho + 4 + r - W) < j_lim ? rho + 4 + r - W : -1;
        }
    }
    __device__ __forceinline__ void issue(int j, const i32x4 &e0, const i32x4 &e1) const {
        if (j < n_raw) issue_raw(j);
        else issue_comp(j, e0, e1);
    }
    // DMA instructions this wave issued for step j.
    __device__ __forceinline__ int batch(int j) const { return (E8 && j >= n_raw) ? kCodeBatch : kRW; }
    // E4M3 compressed step j, in place: each wave reads its 8 code rows, then (after a barrier,
    // as the bf16 rows overlap other waves' codes) writes them as bf16 rows.  Every wave of the
    // workgroup must call it.
    __device__ __forceinline__ void widen(int j) const {
        unsigned char *sb = ring + (j % NB) * kBuf;
        u32x2 x[kRW];
#pragma unroll
        for (int e = 0; e < kRW; ++e)
            x[e] = *reinterpret_cast<const u32x2 *>(sb + (wave * kRW + e) * kCodeRow + 8 * lane);
        wait_lds();
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kRW; ++e) {
            const int r = wave * kRW + e;
            *reinterpret_cast<u32x4 *>(sb + r * kRowStride + ((lane ^ ((r >> 2) & 1)) << 4)) = e4m3x8_to_bf16x8(x[e]);
        }
        wait_lds();
    }
};

// LDS addresses within a half step: QK operand of lane (g, c) for k-step s at qk_base + 64 s
// (row c, chunk 4s + g, swizzle bit (c >> 2) & 1 flips g's low bit); the transposed V read of
// dim block b at pv_base + 32 b (lane (g, c) points at row 4g + c/4, dims 16b + 4(c%4): chunk
// 2b + ((c >> 1) & 1), whose swizzle bit is g & 1).
__device__ __forceinline__ int qk_base_of(int g, int c) { return c * kRowStride + ((g ^ ((c >> 2) & 1)) << 4); }
__device__ __forceinline__ int pv_base_of(int g, int c) {
    return (4 * g + (c >> 2)) * kRowStride + ((((c >> 1) & 1) ^ (g & 1)) << 4) + (c & 1) * 8;
}

// V^T fragment of dim block b of the step at tb (+ pv_base): .xy rows 4g..4g+3 of the first
// half, .zw the same rows of the second.
__device__ __forceinline__ u32x4 tr_frag(const unsigned char *tb, int b) {
    const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(tb + 32 * b));
    const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr16(tb + kHalfBuf + 32 * b));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

}  // namespace

}  // namespace ds4a
