// mqa.hip — A3..A6: query-tail RoPE and multi-query attention over the raw
// window plus the selected compressed rows, one softmax over the union.
//
// "Reading the architecture of DwarfStar (ds4.c), part 1/8" (Qiita):
//  * section 2: 64 query heads (Pro 128) share ONE KV head of 512 dims;
//    RoPE covers only the last n_rot = 64 dims;
//  * section 3: recent tokens stay exact in a raw sliding window (128 rows,
//    f16-rounded, section 3-1), older ones live as compressed rows of which
//    the indexer's top-k reach the attention;
//  * section 3-2: compressed rows are rotated ("tail RoPE") when emitted, so
//    stored rows are already rotated and only the query is rotated here.
// Readings: each stored row is both key and value; the union is raw rows then
// selected rows, not de-duplicated; RoPE pairs are adjacent dims.
//
// Design.  A workgroup (8 waves) owns one query, 64 heads and a contiguous
// chunk of 32-row union tiles, so every row is brought into LDS once for all
// 64 heads.  Wave (ht, dh) owns heads 16ht..16ht+15 and dims 256dh..256dh+255:
//   QK  : partial L^T[32 rows x 16 heads] over its 256 dims with 16x16x32
//         MFMA tiles (A = rows from LDS, B = rotated query held in VGPRs);
//         the two halves are added through LDS in a fixed order;
//   softmax: online (running max / sum per head), fp32;
//   PV  : O^T[256 dims x 16 heads] += V^T * P^T; P^T is already in the
//         B-operand layout of the QK result, V^T fragments come from the same
//         LDS tile through ds_read_b64_tr_b16.
// Each row format gets the MFMA of its own type, so rows are never converted:
// compressed rows are bf16 (v_mfma_f32_16x16x32_bf16), raw-window rows are f16
// (v_mfma_f32_16x16x32_f16).  Operands not already in that type are carried
// as hi + lo pairs: the query (only its rotated tail when it is bf16) and the
// probabilities.  The raw tiles come first in the union, so the query is held
// as an f16 pair for them and re-split as a bf16 pair for the compressed tiles.
// LDS rows are 1056 bytes apart and their 16-byte chunks are XOR-swizzled by
// row bit 2, which keeps both the row reads of QK and the transposed reads of
// PV free of bank conflicts.  Loads run three tiles ahead: two register stages
// (one row per wave instruction) feed three LDS tile buffers, so one barrier per
// tile (after the exchange of logit halves) also covers the buffer turnover.
// When the union is split over several workgroups each writes (max, sum,
// unnormalised O) and a merge kernel combines them by log-sum-exp.
// Compressed rows stored as FP8 (E4M3 codes, 512 bytes, plus one f32 scale per row; the
// compressor's output format) are widened to bf16 while they are staged, exactly, and their
// scale is kept in the row's LDS padding: it multiplies the row's logit and, for the PV
// product, its probability.  With power-of-two scales the output is bit-identical to that of
// the bf16 rows code * scale.
#include "common.hpp"
#include "launch.hpp"
#include "rope.hpp"

#include <math.h>
#include <mutex>
#include <type_traits>

namespace ds4a {

namespace {

constexpr int kThreads = 512;                 // 8 waves: 4 head tiles x 2 halves of the dims
constexpr int kWaves = kThreads / kWave;
constexpr int kHW = 16;                       // heads per wave
constexpr int kHG = 64;                       // heads per workgroup
constexpr int kD = 512;
constexpr int kDH = kD / 2;                   // dims per wave
constexpr int kRot = 64;
constexpr int kKs = kDH / 32;                 // k-steps of QK per wave (8)
constexpr int kDB = kDH / 16;                 // 16-dim blocks of PV per wave (16)
constexpr int kTile = 32;                     // union rows per tile
constexpr int kRowStride = 1056;              // LDS bytes per row (1024 + 32)
constexpr int kTileBytes = kTile * kRowStride;
constexpr int kXchBytes = kWaves * 2 * kWave * 16;           // partial logits of every wave (one of two)
constexpr int kStage = kTile / kWaves;        // rows each wave stages per tile (4)
constexpr int kQtBytes = kHG * kRot * 4;                     // rotated query tails of the 64 heads (f32)
constexpr int kTileBufs = 3;                 // tile buffers in LDS: one barrier per tile
constexpr int kLdsBytes = kTileBufs * kTileBytes + 2 * kXchBytes + kQtBytes;   // + 4 bytes per union row (row table)
constexpr int kPadTiles = 3;                 // row-table padding for the look-ahead loads past a chunk's end
constexpr int kMaxTilesPerChunk = 96;         // LDS: kLdsBytes + 128 B per tile of row table <= 160 KiB
constexpr int kMaxLdsBytes = kLdsBytes + 4 * kTile * (kMaxTilesPerChunk + kPadTiles);
static_assert(kMaxLdsBytes <= 160 * 1024, "the largest chunk's LDS fits a CU");
constexpr int kRowRegs = 2;            // row-table entries per thread loaded ahead of the first gathers
constexpr int kRec = 2 * kHG + kHG * kD;      // partial record: m[64], l[64], O[64][512]
constexpr float kRescale = 8.f;               // softmax reference moves when a logit exceeds it by this

// The row that a union entry taking no part is read from: 1 KiB of zeros (a bf16 or f16 row,
// or an E4M3 row of codes 0).
__device__ __align__(16) const unsigned char g_zero_row[2 * kD] = {};

// Byte offset of 16-byte chunk c (0..63) of tile row r, XOR-swizzled by row bit 2.
__device__ __forceinline__ int chunk_off(int r, int c) {
    return r * kRowStride + ((c ^ ((r >> 2) & 1)) << 4);
}

struct MqaArgs {
    int T, H, W, K, n_hg, n_tiles, tiles_per_chunk, n_chunks;
    int64_t N, n_items;
    const void *q;
    int q_bf16;
    const int64_t *pos;
    const uint16_t *raw;
    const void *comp;                        // bf16 rows [U][N][512], or E4M3 codes [U][N][512]
    const float *comp_scale;                 // E4M3 rows: f32 [U][N]
    const int32_t *idx;                      // sparse: [U][T][K]; dense: unused
    const int32_t *n_vis;                    // dense: visible compressed rows per query, or NULL (all N)
    const int32_t *raw_vis;                  // raw rows of each query's window that take part, or NULL (all W)
    float scale;
    float *out;
    float *part;
    double log2_theta;                       // log2(rope_theta), computed on the host in fp64
};

// Query dims [d, d+8) of head h of query q as f32, as stored (no rotation).
__device__ __forceinline__ void load_q8_plain(const MqaArgs &a, int64_t q, int h, int d, float (&v)[8]) {
    const int64_t off = (q * a.H + h) * (int64_t)kD + d;
    if (a.q_bf16) {
        const u32x4 x = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.q) + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_bits_to_f32(x[i] & 0xFFFFu);
            v[2 * i + 1] = bf16_bits_to_f32(x[i] >> 16);
        }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(a.q) + off);
        const float4 x0 = p[0], x1 = p[1];
        v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
        v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
    }
}

// Query dims [d, d+8) of head h of query q as f32, rotated where they fall in the tail.
__device__ __forceinline__ void load_q8(const MqaArgs &a, int64_t q, int h, int d, float (&v)[8]) {
    load_q8_plain(a, q, h, d, v);
    if (d >= kD - kRot) {
        const int64_t pos = a.pos[q];
#pragma unroll
        for (int e = 0; e < 8; e += 2) rope_pair(a.log2_theta, (d + e - (kD - kRot)) >> 1, pos, v[e], v[e + 1]);
    }
}

// The query as MFMA B fragments, k-step s <-> dims d0 + 32s + 8g + (0..7) of head h:
// hi/lo pairs of one operand type (bf16 or f16).  load_q_plain issues every global load
// (the stored values as f32); pack_q_frags takes the rotated tail (dims 448..511, the k-steps
// with d0 + 32s >= 448, a wave-uniform test) from `tail`, this head's 64 floats in LDS.
template <bool QF32>
__device__ __forceinline__ void load_q_plain(const MqaArgs &a, int64_t q, int h, int d0, int g,
                                             float (&v)[kKs][8]) {
    const int64_t off = (q * a.H + h) * (int64_t)kD + d0 + 8 * g;
#pragma unroll
    for (int s = 0; s < kKs; ++s) {
        if (QF32) {
            const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(a.q) + off + 32 * s);
            const float4 x0 = p[0], x1 = p[1];
            v[s][0] = x0.x; v[s][1] = x0.y; v[s][2] = x0.z; v[s][3] = x0.w;
            v[s][4] = x1.x; v[s][5] = x1.y; v[s][6] = x1.z; v[s][7] = x1.w;
        } else {
            const u32x4 x = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.q) + off + 32 * s);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[s][2 * i] = bf16_bits_to_f32(x[i] & 0xFFFFu);
                v[s][2 * i + 1] = bf16_bits_to_f32(x[i] >> 16);
            }
        }
    }
}

template <bool F16>
__device__ __forceinline__ void pack_q_frags(const float (&v)[kKs][8], const float *tail, int d0, int g,
                                             u32x4 (&hi)[kKs], u32x4 (&lo)[kKs]) {
#pragma unroll
    for (int s = 0; s < kKs; ++s) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            x[e] = d0 + 32 * s >= kD - kRot ? tail[d0 + 32 * s + 8 * g - (kD - kRot) + e] : v[s][e];
        if (F16) {
            f16x8 h8, l8;
            pack_hi_lo8_f16(x, h8, l8);
            hi[s] = __builtin_bit_cast(u32x4, h8);
            lo[s] = __builtin_bit_cast(u32x4, l8);
        } else {
            bf16x8 h8, l8;
            pack_hi_lo8(x, h8, l8);
            hi[s] = __builtin_bit_cast(u32x4, h8);
            lo[s] = __builtin_bit_cast(u32x4, l8);
        }
    }
}

// LO_ALL: the query is f32, so every k-step carries a lo half; otherwise (bf16 query)
// only the rotated tail does.  DENSE: the union is the raw window plus compressed rows
// 0 .. n_vis-1 in order (a.K = N; no index list), else the raw window plus idx's rows.
// E8: compressed rows are E4M3 codes with row scales (N >= 1), else bf16.
template <bool LO_ALL, bool DENSE, bool E8>
__global__ __launch_bounds__(kThreads) void sparse_mqa_kernel(MqaArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *tiles = smem;
    f32x4 *xch = reinterpret_cast<f32x4 *>(smem + kTileBufs * kTileBytes);   // two exchange buffers
    float *s_qt = reinterpret_cast<float *>(smem + kTileBufs * kTileBytes + 2 * kXchBytes);   // [64 heads][64]
    int32_t *s_row = reinterpret_cast<int32_t *>(smem + kLdsBytes);   // per union row: comp row, -2 raw, -1 none

    // Workgroup -> (query, chunk, head group), in 32-bit arithmetic: the grid is below 2^31
    // workgroups (U*T <= 2^24, and the union is split only when there are fewer than 256
    // queries), and 64-bit divisions by runtime values cost hundreds of scalar instructions
    // ahead of the first load.
    const uint32_t lin = blockIdx.x;
    const int hg = a.n_hg == 1 ? 0 : (int)(lin % (uint32_t)a.n_hg);
    const uint32_t item = a.n_hg == 1 ? lin : lin / (uint32_t)a.n_hg;
    const uint32_t q32 = item / (uint32_t)a.n_chunks;
    const int chunk = (int)(item - q32 * (uint32_t)a.n_chunks);
    const uint32_t u32 = q32 / (uint32_t)a.T;
    const int64_t q = q32, u = u32, t = q32 - u32 * (uint32_t)a.T;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int g = lane >> 4, c = lane & 15;
    const int ht = wave >> 1, dh = wave & 1;               // head tile, half of the dims
    const int h0 = hg * kHG + kHW * ht;                   // this wave's first head
    const int d0 = kDH * dh;                              // this wave's first dim
    const bool active = h0 < a.H;                          // H is a multiple of 16
    const int tile0 = chunk * a.tiles_per_chunk;
    const int tile1 = tile0 + a.tiles_per_chunk < a.n_tiles ? tile0 + a.tiles_per_chunk : a.n_tiles;
    const int tile_raw = a.W / kTile;                      // tiles [0, tile_raw) are raw rows

    const uint16_t *raw_q = a.raw + (u * (int64_t)(a.T + a.W - 1) + t) * kD;
    constexpr int kCompRowBytes = E8 ? kD : 2 * kD;
    const unsigned char *comp_u = static_cast<const unsigned char *>(a.comp) + u * a.N * kCompRowBytes;
    const float *cscale_u = E8 ? a.comp_scale + u * a.N : nullptr;
    const int32_t *idx_q = a.idx + q * (int64_t)a.K;

    // Union row rho of this chunk: a compressed row, -2 for a raw row, -1 for none (past the
    // chunk's end, a -1 or out-of-range index, past K).  idx is always read, at a clamped
    // position (idx_at), so a run of these loads issues back to back with no branch.
    const int64_t j_lim = DENSE ? clamp_nvis(a.n_vis, q, a.N) : a.N;   // compressed rows that may enter
    auto idx_at = [&](int rho) __attribute__((always_inline)) -> int32_t {
        const int k = rho - a.W;
        if (DENSE) return k;
        return idx_q[k < 0 ? 0 : (k < a.K ? k : a.K - 1)];
    };
    // raw rows r < raw_lim of the window take part (a window that is not yet full)
    const int raw_lim = a.raw_vis ? (int)clamp_nvis(a.raw_vis, q, a.W) : a.W;
    auto union_row = [&](int rho, int32_t j) __attribute__((always_inline)) -> int32_t {
        const int k = rho - a.W;
        const int32_t comp = (k < a.K && j >= 0 && (int64_t)j < j_lim) ? j : -1;
        return rho >= tile1 * kTile ? -1 : (k < 0 ? (rho < raw_lim ? -2 : -1) : comp);
    };
    // A row that takes no part (-1) is read from a row of zeros in device memory (a pointer
    // select, so no branch guards the load): its logit is masked to -inf, its probability is 0
    // and its values are 0, so nothing the caller's buffers hold outside the union (an
    // unwritten raw row past raw_vis, compressed row 0 before the first one is emitted) can
    // reach the output, not even a NaN or an infinity through 0 * x.
    const unsigned char *raw_b = reinterpret_cast<const unsigned char *>(raw_q);
    auto union_ptr = [&](int rho, int32_t v, bool) __attribute__((always_inline)) -> const unsigned char * {
        return v == -2 ? raw_b + (int64_t)rho * (2 * kD)
                       : (v >= 0 ? comp_u + (int64_t)v * kCompRowBytes : g_zero_row);
    };
    // One staged row: lane = 16-byte chunk of a bf16 / f16 row; an E4M3 row arrives as 8 bytes
    // per lane (x, y), widened at the store.
    auto load_row = [&](int rho, int32_t v, bool raw_tile) __attribute__((always_inline)) -> u32x4 {
        const unsigned char *p = union_ptr(rho, v, raw_tile);
        if (E8 && !raw_tile) {
            const u32x2 x = reinterpret_cast<const u32x2 *>(p)[lane];
            return u32x4{x[0], x[1], 0u, 0u};
        }
        return reinterpret_cast<const u32x4 *>(p)[lane];
    };
    // E4M3 rows: the scales of a wave's kStage rows of a tile in one load, lane l holding that of
    // row l % kStage (in z of the first staged row); v = the rows' union entries.
    static_assert(kStage == 4, "one scale per lane group of four");
    auto load_scales = [&](const int32_t (&v)[kStage], bool raw_tile, u32x4 (&st)[kStage])
        __attribute__((always_inline)) {
        if (E8 && !raw_tile) {
            const int k = lane & (kStage - 1);
            const int32_t vl = k == 0 ? v[0] : (k == 1 ? v[1] : (k == 2 ? v[2] : v[3]));
            st[0][2] = vl >= 0 ? __float_as_uint(cscale_u[vl]) : 0x3F800000u;   // none rows: scale 1
        }
    };
    // Set-up loads first, then the first two tiles' row gathers, then the set-up's use of its
    // loads: vector loads complete in issue order, so a gather issued before the set-up's own
    // loads would hold the set-up up until the rows arrive.
    //  - row table of this chunk's union rows from idx, plus kPadTiles tiles of padding for
    //    the look-ahead loads past the chunk's end (the first kRowRegs entries per thread are
    //    loaded into registers here, any further ones after the gathers);
    const int64_t pos = a.pos[q];
    const int rho0 = tile0 * kTile;
    const int n_rows = (tile1 - tile0 + kPadTiles) * kTile;
    int32_t rv[kRowRegs];
#pragma unroll
    for (int k = 0; k < kRowRegs; ++k) {
        const int r = tid + k * kThreads < n_rows ? tid + k * kThreads : n_rows - 1;
        rv[k] = idx_at(rho0 + r);
    }
    //  - the query tail of this workgroup's heads, four adjacent pairs per thread (heads past H
    //    read head H-1 and store nothing);
    constexpr int kPairs = kHG * (kRot / 2) / kThreads;
    float qx[kPairs], qy[kPairs];
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
        const int i = tid + k * kThreads;
        const int hl = i / (kRot / 2), pr = i % (kRot / 2);
        const int h = hg * kHG + hl < a.H ? hg * kHG + hl : a.H - 1;
        const int64_t off = (q * a.H + h) * (int64_t)kD + (kD - kRot) + 2 * pr;
        if (!LO_ALL) {                                    // bf16 query
            const uint32_t w = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(a.q) + off);
            qx[k] = bf16_bits_to_f32(w & 0xFFFFu);
            qy[k] = bf16_bits_to_f32(w >> 16);
        } else {
            const float2 w = *reinterpret_cast<const float2 *>(static_cast<const float *>(a.q) + off);
            qx[k] = w.x;
            qy[k] = w.y;
        }
    }
    //  - this wave's query values (packed into MFMA fragments once the tail is rotated; a
    //    wave past H reads head H-1 and never uses it);
    float qv[kKs][8];
    load_q_plain<LO_ALL>(a, q, active ? h0 + c : a.H - 1, d0, g, qv);
    //  - wave w stages rows w + 8i (i = 0..3) of a tile, lane = 16-byte chunk of the row; the
    //    first two tiles' rows come straight from idx (wave-uniform reads).
    u32x4 st0[kStage], st1[kStage];
    {
        const int wave_u = __builtin_amdgcn_readfirstlane(wave);
        int32_t j0[kStage], j1[kStage];
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            j0[i] = idx_at(tile0 * kTile + wave_u + kWaves * i);
            j1[i] = idx_at((tile0 + 1) * kTile + wave_u + kWaves * i);
        }
        // The position arrives with these reads, not after the gathers (the compiler would
        // otherwise issue its load at its first use, behind them).
        asm volatile("" : : "s"(pos));
        int32_t v0[kStage], v1[kStage];
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int r0 = tile0 * kTile + wave_u + kWaves * i, r1 = r0 + kTile;
            v0[i] = union_row(r0, j0[i]);
            v1[i] = union_row(r1, j1[i]);
            st0[i] = load_row(r0, v0[i], tile0 < tile_raw);
            st1[i] = load_row(r1, v1[i], tile0 + 1 < tile_raw);
        }
        load_scales(v0, tile0 < tile_raw, st0);
        load_scales(v1, tile0 + 1 < tile_raw, st1);
    }
    // (stored at the same clamped position, with no branch, so that the compiler does not move
    // the load down here, behind the gathers)
#pragma unroll
    for (int k = 0; k < kRowRegs; ++k) {
        const int r = tid + k * kThreads < n_rows ? tid + k * kThreads : n_rows - 1;
        s_row[r] = union_row(rho0 + r, rv[k]);
    }
    for (int r = tid + kRowRegs * kThreads; r < n_rows; r += kThreads) s_row[r] = union_row(rho0 + r, idx_at(rho0 + r));
    // Rotated query tails into LDS.  A thread's pairs are all pair tid % 32 of their heads
    // (kThreads is a multiple of 32), so one angle serves them all.
    {
        static_assert(kThreads % (kRot / 2) == 0, "one pair index per thread");
        double cs, sn;
        rope_angle(a.log2_theta, tid % (kRot / 2), pos, cs, sn);
#pragma unroll
        for (int k = 0; k < kPairs; ++k) {
            const int i = tid + k * kThreads;
            const int hl = i / (kRot / 2), pr = i % (kRot / 2);
            rope_rotate(cs, sn, qx[k], qy[k]);
            s_qt[hl * kRot + 2 * pr] = qx[k];
            s_qt[hl * kRot + 2 * pr + 1] = qy[k];
        }
    }
    __syncthreads();

    auto load_tile = [&](int tt, u32x4 (&st)[kStage], bool raw_tile) __attribute__((always_inline)) {
        int32_t v[kStage];
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int rho = tt * kTile + wave + kWaves * i;
            v[i] = s_row[rho - rho0];
            st[i] = load_row(rho, v[i], raw_tile);
        }
        load_scales(v, raw_tile, st);
    };
    // Every LDS address below is a per-lane base plus a compile-time offset: the swizzle bit
    // of the rows a lane touches does not depend on the unrolled index.
    //   staging: row wave + 8i has swizzle bit (wave >> 2) & 1;
    //   QK:      row 16rt + c, chunk d0/8 + 4s + g  -> bit (c >> 2) & 1 flips g's low bit;
    //   PV:      rows 4g + c/4 (+16), dims d0 + 16b + 4(c%4) -> bit g & 1 flips chunk bit (c >> 1) & 1.
    const int st_base = chunk_off(wave, lane);
    const int qk_base = c * kRowStride + (((kDH * dh) >> 3) + (g ^ ((c >> 2) & 1))) * 16;
    const int pv_base = (4 * g + (c >> 2)) * kRowStride + (((kDH * dh) >> 3) + (((c >> 1) & 1) ^ (g & 1))) * 16 +
                        (c & 1) * 8;
    // E4M3 rows: the widened row, and the scale at byte kD * 2 of the LDS row (its padding).
    auto store_tile = [&](int buf, const u32x4 (&st)[kStage], bool raw_tile) __attribute__((always_inline)) {
        unsigned char *base = tiles + buf * kTileBytes + st_base;
        if (E8 && !raw_tile) {
#pragma unroll
            for (int i = 0; i < kStage; ++i)
                *reinterpret_cast<u32x4 *>(base + i * kWaves * kRowStride) = e4m3x8_to_bf16x8(u32x2{st[i][0], st[i][1]});
            if (lane < kStage)                     // lane l: the scale of row wave + 8l
                *reinterpret_cast<uint32_t *>(tiles + buf * kTileBytes + (wave + kWaves * lane) * kRowStride + 2 * kD) =
                    st[0][2];
        } else {
#pragma unroll
            for (int i = 0; i < kStage; ++i)
                *reinterpret_cast<u32x4 *>(base + i * kWaves * kRowStride) = st[i];
        }
    };
    const float *tail = s_qt + (kHW * ht + c) * kRot;
    u32x4 qhi[kKs], qlo[kKs];
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[kDB];
#pragma unroll
    for (int b = 0; b < kDB; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Fragments for the first row format.
    const int tmid = tile1 < tile_raw ? tile1 : (tile0 > tile_raw ? tile0 : tile_raw);
    if (active) {
        if (tile0 < tmid) pack_q_frags<true>(qv, tail, d0, g, qhi, qlo);
        else pack_q_frags<false>(qv, tail, d0, g, qhi, qlo);
    }
    store_tile(0, st0, tile0 < tile_raw);
    load_tile(tile0 + 2, st0, tile0 + 2 < tile_raw);
    // Waves w and w + 4 share a SIMD.  Between two barriers both would otherwise run the
    // same phases in lock-step (softmax on the VALU while the matrix core idles, then both
    // queue their MFMAs); a higher issue priority for waves 0-3 lets them run ahead, so one
    // wave's softmax and LDS work overlap the other's MFMAs.
    if (wave < kWaves / 2) __builtin_amdgcn_s_setprio(1);
    __syncthreads();

    // One tile, one barrier.  Tile i (counted from tile0) sits in LDS buffer i % 3 and is
    // staged through registers two steps ahead.  On entry `sv` holds tile tt+1: it goes into
    // buffer `bnext` (whose last tile, tt-2, every wave finished before the barrier of step
    // tt-1), and `sv` then takes tile tt+3.  The barrier after the logit exchange publishes
    // both the partial logits (exchange buffer `xb`, alternating by step) and tile tt+1.
    // F16: raw rows (f16 MFMA), else compressed rows (bf16 MFMA).
    auto step = [&](auto f16_tag, auto xb_tag, int tt, int bcur, int bnext, u32x4 (&sv)[kStage])
        __attribute__((always_inline)) {
        constexpr bool F16 = decltype(f16_tag)::value;
        constexpr int kXb = decltype(xb_tag)::value;
        // Raw tiles come first in the union: after a compressed tile every tile is compressed,
        // so in compressed steps the format of the tiles staged ahead is known at compile time.
        store_tile(bnext, sv, F16 && tt + 1 < tile_raw);
        load_tile(tt + 3, sv, F16 && tt + 3 < tile_raw);
        const unsigned char *tb = tiles + bcur * kTileBytes;
        f32x4 *xc = xch + kXb * (kXchBytes / 16);

        // ---- QK: partial logits of 32 rows x this wave's 16 heads over its 256 dims;
        // hi and lo products go to separate accumulators (two short chains, not one long).
        f32x4 acc[2], acl[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            acl[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (active) {
#pragma unroll
            for (int s = 0; s < kKs; ++s) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const u32x4 x = *reinterpret_cast<const u32x4 *>(tb + qk_base + rt * 16 * kRowStride + s * 64);
                    if (F16) {
                        acc[rt] = mfma16h(as_f16x8(x), as_f16x8(qhi[s]), acc[rt]);
                        if (LO_ALL || s >= kKs - 2) acl[rt] = mfma16h(as_f16x8(x), as_f16x8(qlo[s]), acl[rt]);
                    } else {
                        acc[rt] = mfma16(as_bf16x8(x), as_bf16x8(qhi[s]), acc[rt]);
                        if (LO_ALL || s >= kKs - 2) acl[rt] = mfma16(as_bf16x8(x), as_bf16x8(qlo[s]), acl[rt]);
                    }
                }
            }
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) xc[(wave * 2 + rt) * kWave + lane] = acc[rt] + acl[rt];
        __syncthreads();

        if (active) {
            // full logits: lower half + upper half, the same order in both waves of the pair
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                acc[rt] = xc[((2 * ht) * 2 + rt) * kWave + lane] + xc[((2 * ht + 1) * 2 + rt) * kWave + lane];

            // ---- mask, online softmax (head c; rows 16rt + 4g + r)
            float p[2][4], rsc[2][4] = {{1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}};
            float tmax = -INFINITY;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rho = tt * kTile + 16 * rt + 4 * g + r;
                    float l = a.scale * acc[rt][r];
                    if (E8 && !F16) {                   // E4M3 rows: the row's scale (LDS padding)
                        rsc[rt][r] = *reinterpret_cast<const float *>(tb + (16 * rt + 4 * g + r) * kRowStride + 2 * kD);
                        l *= rsc[rt][r];
                    }
                    p[rt][r] = s_row[rho - rho0] != -1 ? l : -INFINITY;
                    tmax = fmaxf(tmax, p[rt][r]);
                }
            tmax = wave_xor_max(tmax, 16);
            tmax = wave_xor_max(tmax, 32);
            // m_run is a reference, not always the running maximum: it moves (and O and the
            // sum are rescaled) only when some head of the wave sees a logit more than
            // kRescale above it, so every exponent stays below e^kRescale.  The result does
            // not depend on the reference; both waves of a head tile take the same decision
            // from the same logits.
            const float m_new = fmaxf(m_run, tmax);
            if (__builtin_amdgcn_ballot_w64(m_new > m_run + kRescale)) {   // also the first visible row
                const float alpha = __expf(m_run - m_new);          // 0 while nothing was visible
                l_run *= alpha;
#pragma unroll
                for (int b = 0; b < kDB; ++b) o[b] *= alpha;
                m_run = m_new;
            }
            const float m_use = m_run == -INFINITY ? 0.f : m_run;  // nothing visible yet: all p = 0
            float psum = 0.f;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    p[rt][r] = __expf(p[rt][r] - m_use);
                    psum += p[rt][r];
                }
            l_run += psum;

            // ---- PV: P^T fragment, element e <-> row e<4 ? 4g+e : 16+4g+(e-4); V^T fragment by two
            // transposed reads: source lane (g, c) points at row 4g + c/4 (+16), dims d0 + 4(c%4).
            const float pv[8] = {p[0][0], p[0][1], p[0][2], p[0][3], p[1][0], p[1][1], p[1][2], p[1][3]};
            if (F16) {
                f16x8 phi, plo;
                pack_hi_lo8_f16(pv, phi, plo);
#pragma unroll
                for (int b = 0; b < kDB; ++b) {
                    const s16x4 v1 = lds_read_tr16(tb + pv_base + 32 * b);
                    const s16x4 v2 = lds_read_tr16(tb + pv_base + 16 * kRowStride + 32 * b);
                    const f16x8 av = __builtin_bit_cast(f16x8, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
                    o[b] = mfma16h(av, phi, o[b]);
                    o[b] = mfma16h(av, plo, o[b]);
                }
            } else {
                bf16x8 phi, plo;
                if (E8) {                               // value rows carry their scale too
                    const float pvs[8] = {p[0][0] * rsc[0][0], p[0][1] * rsc[0][1], p[0][2] * rsc[0][2],
                                          p[0][3] * rsc[0][3], p[1][0] * rsc[1][0], p[1][1] * rsc[1][1],
                                          p[1][2] * rsc[1][2], p[1][3] * rsc[1][3]};
                    pack_hi_lo8(pvs, phi, plo);
                } else {
                    pack_hi_lo8(pv, phi, plo);
                }
#pragma unroll
                for (int b = 0; b < kDB; ++b) {
                    const s16x4 v1 = lds_read_tr16(tb + pv_base + 32 * b);
                    const s16x4 v2 = lds_read_tr16(tb + pv_base + 16 * kRowStride + 32 * b);
                    const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
                    o[b] = mfma16(av, phi, o[b]);
                    o[b] = mfma16(av, plo, o[b]);
                }
            }
        }
    };
    // Tiles [ta, tb) of one row format; unrolled by two so that the register stages and the
    // exchange buffers stay statically named (tile i: stage st1 if i is even, st0 if odd;
    // exchange buffer i & 1); the LDS buffer i % 3 rotates at run time.  Both continue across
    // calls.
    using X0 = std::integral_constant<int, 0>;
    using X1 = std::integral_constant<int, 1>;
    int bcur = 0;
    auto next3 = [](int b) __attribute__((always_inline)) { return b == 2 ? 0 : b + 1; };
    auto run = [&](auto f16_tag, int ta, int tb) __attribute__((always_inline)) {
        int tt = ta;
        if (tt < tb && ((tt - tile0) & 1)) {
            step(f16_tag, X1{}, tt, bcur, next3(bcur), st0);
            bcur = next3(bcur);
            ++tt;
        }
        for (; tt + 1 < tb; tt += 2) {
            step(f16_tag, X0{}, tt, bcur, next3(bcur), st1);
            bcur = next3(bcur);
            step(f16_tag, X1{}, tt + 1, bcur, next3(bcur), st0);
            bcur = next3(bcur);
        }
        if (tt < tb) {
            step(f16_tag, X0{}, tt, bcur, next3(bcur), st1);
            bcur = next3(bcur);
        }
    };
    if (tile0 < tmid) run(std::true_type{}, tile0, tmid);
    if (tmid < tile1) {
        if (active && tile0 < tmid) {
            float qv2[kKs][8];
            load_q_plain<LO_ALL>(a, q, h0 + c, d0, g, qv2);
            pack_q_frags<false>(qv2, tail, d0, g, qhi, qlo);
        }
        run(std::false_type{}, tmid, tile1);
    }

    if (!active) return;
    // ---- epilogue: per-head sum over the four row groups
    l_run = wave_xor_sum(l_run, 16);
    l_run = wave_xor_sum(l_run, 32);
    const int hl = kHW * ht + c;                          // head within the workgroup
    if (a.n_chunks == 1) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float *orow = a.out + (q * a.H + h0 + c) * (int64_t)kD + d0 + 4 * g;
#pragma unroll
        for (int b = 0; b < kDB; ++b) *reinterpret_cast<f32x4 *>(orow + 16 * b) = o[b] * inv;
    } else {
        float *rec = a.part + ((q * a.n_hg + hg) * (int64_t)a.n_chunks + chunk) * kRec;
        if (g == 0 && dh == 0) {
            rec[hl] = m_run;
            rec[kHG + hl] = l_run;
        }
        float *orow = rec + 2 * kHG + hl * kD + d0 + 4 * g;
#pragma unroll
        for (int b = 0; b < kDB; ++b) *reinterpret_cast<f32x4 *>(orow + 16 * b) = o[b];
    }
}

// Combines the per-chunk (reference, sum, O) records of one (query, head group of 64).
// One thread per (head, 8 dims): 64 heads x 64 = 4096 threads over 16 workgroups of 256.
// Chunks are taken 8 at a time with every load of a batch issued before any is used
// (indices past the last chunk are clamped and weighted 0), so a batch costs one round
// trip to memory.
constexpr int kMergeBatch = 8;
constexpr int kMergeWgs = 16;

__global__ __launch_bounds__(256) void mqa_merge_kernel(int H, int n_hg, int n_chunks,
                                                        const float *__restrict__ part, float *__restrict__ out)
{
    const int64_t qh = blockIdx.x / kMergeWgs;             // (query, head group)
    const int64_t q = qh / n_hg;
    const int hg = (int)(qh % n_hg);
    const int hl = (int)(blockIdx.x % kMergeWgs) * 4 + (threadIdx.x >> 6);
    if (hg * kHG + hl >= H) return;
    const float *base = part + qh * n_chunks * (int64_t)kRec;
    const int d0 = (threadIdx.x & 63) * 8;
    float M = -INFINITY, L = 0.f;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < n_chunks; c0 += kMergeBatch) {
        float m[kMergeBatch], l[kMergeBatch];
        f32x4 x0[kMergeBatch], x1[kMergeBatch];
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i) {
            const int ch = c0 + i < n_chunks ? c0 + i : n_chunks - 1;
            const float *rec = base + ch * (int64_t)kRec;
            m[i] = rec[hl];
            l[i] = rec[kHG + hl];
            const f32x4 *src = reinterpret_cast<const f32x4 *>(rec + 2 * kHG + hl * kD + d0);
            x0[i] = src[0];
            x1[i] = src[1];
        }
        float mb = M;
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i) mb = c0 + i < n_chunks ? fmaxf(mb, m[i]) : mb;
        const float sc = M == -INFINITY ? 0.f : __expf(M - mb);   // nothing accumulated yet: all zero
        L *= sc;
        acc0 *= sc;
        acc1 *= sc;
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i) {
            // a chunk past the end, or one with no visible row, weighs 0
            const float w = (c0 + i < n_chunks && m[i] != -INFINITY) ? __expf(m[i] - mb) : 0.f;
            L += w * l[i];
            acc0 += w * x0[i];
            acc1 += w * x1[i];
        }
        M = mb;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    f32x4 *dst = reinterpret_cast<f32x4 *>(out + (q * H + hg * kHG + hl) * (int64_t)kD + d0);
    dst[0] = acc0 * inv;
    dst[1] = acc1 * inv;
}

// A3 alone: one thread per 8 dims of one head.
__global__ __launch_bounds__(256) void rope_q_kernel(MqaArgs a, int64_t total8, float *__restrict__ q_out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total8) return;
    const int d = (int)(i % (kD / 8)) * 8;
    const int64_t qh = i / (kD / 8);
    const int h = (int)(qh % a.H);
    const int64_t q = qh / a.H;
    float v[8];
    load_q8(a, q, h, d, v);
    float4 *dst = reinterpret_cast<float4 *>(q_out + qh * kD + d);
    dst[0] = make_float4(v[0], v[1], v[2], v[3]);
    dst[1] = make_float4(v[4], v[5], v[6], v[7]);
}



}  // namespace

MqaPlan plan_mqa(int U, int T, int H, int W, int K) {
    MqaPlan p;
    p.n_hg = (H + kHG - 1) / kHG;
    p.n_tiles = (W + K + kTile - 1) / kTile;
    const int64_t items = (int64_t)U * T * p.n_hg;
    // Split the union over workgroups only when there are too few (query, head group) items
    // to give every CU a workgroup; aim for ~256 workgroups (one per CU at this register use).
    int64_t want = (256 + items - 1) / items;
    if (want < 1) want = 1;
    if (want > p.n_tiles) want = p.n_tiles;
    p.tiles_per_chunk = (int)((p.n_tiles + want - 1) / want);
    if (p.tiles_per_chunk > kMaxTilesPerChunk) p.tiles_per_chunk = kMaxTilesPerChunk;   // row table fits in LDS
    p.n_chunks = (p.n_tiles + p.tiles_per_chunk - 1) / p.tiles_per_chunk;
    p.workspace_bytes = p.n_chunks > 1 ? sizeof(float) * (size_t)items * (size_t)p.n_chunks * kRec : 0;
    return p;
}

hipError_t launch_mqa(int U, int T, int H, int W, int64_t N, int K, const void *q, int q_bf16,
                      const int64_t *q_pos, double theta, const uint16_t *raw, const void *comp,
                      const float *comp_scale, const int32_t *idx, const int32_t *n_vis, const int32_t *raw_vis,
                      float scale, float *out, void *workspace, hipStream_t stream)
{
    const bool dense = idx == nullptr;       // dense: K = N, rows 0 .. n_vis-1 follow the raw window
    // E4M3 rows need at least one compressed row (the none rows of compressed tiles read row
    // 0); with N = 0 there is no compressed row to read, so the format does not matter.
    const bool e8 = comp_scale != nullptr && N > 0;
    const MqaPlan p = plan_mqa(U, T, H, W, K);
    const int lds = kLdsBytes + 4 * kTile * (p.tiles_per_chunk + kPadTiles);
    using Fn = void (*)(MqaArgs);
    const int variant = (q_bf16 ? 1 : 0) + (dense ? 2 : 0) + (e8 ? 4 : 0);
    static const Fn kernels[8] = {sparse_mqa_kernel<true, false, false>, sparse_mqa_kernel<false, false, false>,
                                  sparse_mqa_kernel<true, true, false>,  sparse_mqa_kernel<false, true, false>,
                                  sparse_mqa_kernel<true, false, true>,  sparse_mqa_kernel<false, false, true>,
                                  sparse_mqa_kernel<true, true, true>,   sparse_mqa_kernel<false, true, true>};
    // Each variant's dynamic LDS limit is raised once, to the largest size any plan asks
    // for, so concurrent calls from several host threads never race on it.
    static std::once_flag attr_once[8];
    static hipError_t attr_err[8];
    const Fn fn = kernels[variant];
    std::call_once(attr_once[variant], [&] {
        attr_err[variant] = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsBytes);
    });
    if (attr_err[variant] != hipSuccess) return attr_err[variant];
    MqaArgs a = {};
    a.T = T; a.H = H; a.W = W; a.K = K; a.n_hg = p.n_hg; a.n_tiles = p.n_tiles;
    a.tiles_per_chunk = p.tiles_per_chunk; a.n_chunks = p.n_chunks;
    a.N = N;
    a.n_items = (int64_t)U * T * p.n_chunks;
    a.q = q; a.q_bf16 = q_bf16; a.pos = q_pos; a.raw = raw; a.comp = comp; a.idx = idx; a.n_vis = n_vis;
    a.comp_scale = e8 ? comp_scale : nullptr;
    a.raw_vis = W > 0 ? raw_vis : nullptr;
    a.scale = scale; a.out = out; a.part = static_cast<float *>(workspace);
    a.log2_theta = log2(theta);
    const int64_t blocks = a.n_items * p.n_hg;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kThreads), lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_chunks == 1) return e;
    hipLaunchKernelGGL(mqa_merge_kernel, dim3((unsigned)((int64_t)U * T * p.n_hg * kMergeWgs)), dim3(256), 0, stream,
                       H, p.n_hg, p.n_chunks, static_cast<const float *>(workspace), out);
    return hipGetLastError();
}

hipError_t launch_rope(int U, int T, int H, const void *q, int q_bf16, const int64_t *q_pos,
                       double theta, float *q_out, hipStream_t stream)
{
    MqaArgs a = {};
    a.T = T; a.H = H; a.q = q; a.q_bf16 = q_bf16; a.pos = q_pos;
    a.log2_theta = log2(theta);
    const int64_t total8 = (int64_t)U * T * H * (kD / 8);
    hipLaunchKernelGGL(rope_q_kernel, dim3((unsigned)((total8 + 255) / 256)), dim3(256), 0, stream, a, total8, q_out);
    return hipGetLastError();
}

}  // namespace ds4a
