// attn_dq.hip — A3..A6 for few queries (decode): query-tail RoPE and multi-query attention
// over the raw window plus the selected compressed rows, one softmax over the union.
//
// "Reading the architecture of DwarfStar (ds4.c), part 1/8" (Qiita), sections 2 and 3: the
// query heads share one KV head of 512 dims, RoPE on the last 64 dims of the query only (rows
// are stored rotated, section 3-2), one softmax over the raw window (section 3-1) and the
// selected compressed rows (section 3-3).  Same readings as the many-query kernel (attn.hip).
//
// Design.  With few queries, workgroups of 64 heads are too few to fill the chip unless each
// query's union is split over many of them, and a split costs an f32 record per head and chunk
// (as large as the rows read) plus the query re-read by every chunk.  Here a workgroup owns
// one query and 16 heads (one MFMA tile), so a decode step of 43 queries x 64 heads already
// gives 172 workgroups; the four head groups of a query run on one XCD and share its rows
// through that XCD's L2.  The four waves split the 512 dims: wave w holds dims
// 128w..128w+127 of the query (its hi + lo pair) and of O.  Per 32-row step a wave
//   - QK: partial logits of the 32 rows x 16 heads over its 128 dims, 4 k-steps x 2 halves of
//     v_mfma_f32_16x16x32, hi and lo;
//   - exchanges partial logits through LDS (8 floats per lane; double-buffered by step parity)
//     and adds the four in a fixed order, so every wave holds the same logits and runs the same
//     online softmax;
//   - PV: O^T[128 dims x 16 heads] += V^T P^T, 8 dim blocks x (hi, lo) of P, with the V^T
//     fragments (two ds_read_b64_tr_b16 per block) read one step ahead into registers.
// The rows go through an LDS ring of the same geometry as in attn.hip (buffer_load ... lds
// straight from memory, zeros for rows that take no part), 4 slots, loads issued 3 steps ahead:
// a step's slot is free once its QK and V^T reads are done, one step before its PV.  Two more
// waves issue those loads (16 rows of each step each) and widen E4M3 rows to bf16 in place:
// a load into LDS holds its wave at issue until the CU's address unit takes it (64 bytes per
// clock, so 512 clocks for a step's 32 KiB), which the four computing waves then never wait
// for.  Waves meet at one barrier per step; the producers wait for a step's loads before it.
// Per step, in one
// stretch of code, the softmax of step j (VALU) runs beside QK of step j+1 (matrix core), then
// PV of step j, reading step j+1's V^T fragments as step j's are consumed; the partial logits
// of j+1 are published and one barrier ends the step.
// When even 16-head workgroups are too few (Pro decode: 4 queries x 128 heads), the union is
// split in chunks; each workgroup writes one record (m, l and O of its 16 heads, O in the
// lanes' register order so that every access is a whole 1 KiB), and the last workgroup of a
// (query, head group), counted with a device-scope atomic, merges the records by log-sum-exp.
//
// Precision as in attn.hip: rows in their stored type (f16 raw, bf16 compressed, E4M3 widened
// exactly to bf16), query and P as hi + lo pairs of that type, fp32 accumulation, softmax in
// log2 units with the exact running maximum.
#include "attn_common.hpp"
#include "launch.hpp"
#include "rope.hpp"

#include <math.h>
#include <mutex>

namespace ds4a {

namespace {

constexpr int kDqP = 2;                       // producer waves
constexpr int kDqT = kAT + kDqP * kWave;      // threads per workgroup: 4 computing + 2 producer waves
constexpr int kPR = kSR / kDqP;               // rows each producer loads per step (16): half step p
constexpr int kDqCodeOff = kHalfBuf - kPR * kCodeRow;   // E4M3 codes of a half step: its last 8 KiB
constexpr int kPCodeBatch = kPR / 2 + 2;      // E4M3 step: loads per producer (codes, 2 x scales)
constexpr int kQKs = kKs / kAW;               // QK k-steps per wave (4)
constexpr int kQDB = kDB / kAW;               // PV dim blocks per wave (8)
constexpr int kDqNB = 4;                      // ring slots
constexpr int kXchOff = kDqNB * kBuf;         // partial logits: [parity][half][wave][lane][4] f32
constexpr int kXchBuf = kAW * kWave * 8 * 4;  // 8 KiB per parity
constexpr int kXchPlane = kAW * kWave * 4;     // floats of one half step's plane
constexpr int kDqScaleOff = kXchOff + 2 * kXchBuf;
template <bool E8> constexpr int kDqAngOff = kDqScaleOff + (E8 ? kDqNB * kAW * kScaleWave : 0);  // [32] (cos, sin) fp64
template <bool E8> constexpr int kDqMaskOff = kDqAngOff<E8> + 32 * 16;      // sparse: row validity per step
constexpr int kDqMaxChunkSteps = 48;          // longer unions are split
template <bool E8> constexpr int kDqRowTabOff = kDqMaskOff<E8> + 4 * kDqMaxChunkSteps;
template <bool E8> constexpr int kDqMaxLds = kDqRowTabOff<E8> + 4 * kSR * kDqMaxChunkSteps;
static_assert(kDqMaxLds<false> <= 160 * 1024 && kDqMaxLds<true> <= 160 * 1024, "LDS of one workgroup");
static_assert(kDqMaxChunkSteps * kSR % kAT == 0, "row table fill");
constexpr int kDqRec = 2 * kWH + kWH * kD;    // record: m[16], l[16], O[wave][block][lane][4]

// Row loads of the union's 32-row steps for producer wave p: rows 16p..16p+15 of each step
// (half step p), step j in ring slot j % kDqNB.  Raw steps: rows of the query's window, 1 KiB
// each, one instruction per row; rows at or past raw_vis lie past the window resource and read
// as zeros.  Compressed steps: bf16 rows from their entries (row index, or -1: past the
// resource, zeros); E4M3 rows as codes, two rows per instruction, into the last 8 KiB of the
// half step, plus the rows' scales as the computing waves read them (per 8-row quarter, lane l
// holding row l % 8).  Steps past the chunk are compressed steps of -1 entries.  Row data:
// row r of the step at r * kRowStride, its 16-byte chunk k at position k ^ ((r >> 2) & 1).
template <bool DENSE, bool E8>
struct DqProducer {
    unsigned char *ring;
    uint32_t ring_a, scale_a;                // LDS addresses of the ring and of the E4M3 row scales
    const int32_t *s_row;                    // sparse: compressed row of each union row of the chunk
    __amdgpu_buffer_rsrc_t raw_rs, comp_rs, scale_rs;
    int step0, n, n_raw, rho0, W, p, lane;
    int64_t j_lim;                           // dense: visible compressed rows

    __device__ __forceinline__ void entries(int j, i32x4 (&e)[4]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = i32x4{-1, -1, -1, -1};
        if (j >= n || j < n_raw) return;
        const int rho = (step0 + j) * kSR + p * kPR;
        if (!DENSE) {
#pragma unroll
            for (int i = 0; i < 4; ++i)       // same address in every lane
                e[i] = *reinterpret_cast<const i32x4 *>(s_row + (rho - rho0) + 4 * i);
            return;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t x = (int64_t)rho + 4 * i + r - W;
                e[i][r] = x < j_lim ? (int32_t)x : -1;
            }
    }
    __device__ __forceinline__ void issue(int j, const i32x4 (&e)[4]) const {
        const int slot = j % kDqNB;
        const uint32_t hb = ring_a + (uint32_t)(slot * kBuf + p * kHalfBuf);
        if (j < n_raw) {
            const int R0 = (step0 + j) * kSR + p * kPR;
            const uint32_t dst = hb;
#pragma unroll
            for (int r = 0; r < kPR; ++r)
                dma16(dst + r * kRowStride, ((uint32_t)(R0 + r) << 10) + ((uint32_t)(lane ^ ((r >> 2) & 1)) << 4), raw_rs);
        } else if (!E8) {
            const uint32_t dst = hb;
#pragma unroll
            for (int r = 0; r < kPR; ++r)
                dma16(dst + r * kRowStride, ((uint32_t)e[r >> 2][r & 3] << 10) + ((uint32_t)(lane ^ ((r >> 2) & 1)) << 4),
                      comp_rs);
        } else {
            const uint32_t dst = hb + kDqCodeOff;
#pragma unroll
            for (int i = 0; i < kPR / 2; ++i) {
                const int32_t ent = lane < 32 ? e[i >> 1][2 * (i & 1)] : e[i >> 1][2 * (i & 1) + 1];
                dma16(dst + i * 2 * kCodeRow, ((uint32_t)ent << 9) + ((uint32_t)(lane & 31) << 4), comp_rs);
            }
            const int l8 = lane & 7;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int32_t es = l8 < 4 ? e[2 * h][l8 & 3] : e[2 * h + 1][l8 & 3];
                dma4(scale_a + (uint32_t)((slot * kAW + 2 * p + h) * kScaleWave), (uint32_t)es << 2, scale_rs);
            }
        }
    }
    // E4M3 compressed step j, in place: this wave's 16 code rows, then the same rows as bf16.
    // The codes lie in the half step's last 8 KiB, so the bf16 rows overwrite only codes this
    // wave has already read.
    __device__ __forceinline__ void widen(int j) const {
        unsigned char *hb = ring + (j % kDqNB) * kBuf + p * kHalfBuf;
        u32x2 x[kPR];
#pragma unroll
        for (int r = 0; r < kPR; ++r) x[r] = *reinterpret_cast<const u32x2 *>(hb + kDqCodeOff + r * kCodeRow + 8 * lane);
        wait_lds();
#pragma unroll
        for (int r = 0; r < kPR; ++r)
            *reinterpret_cast<u32x4 *>(hb + r * kRowStride + ((lane ^ ((r >> 2) & 1)) << 4)) = e4m3x8_to_bf16x8(x[r]);
        wait_lds();
    }
};

template <bool QF32, bool DENSE, bool E8>
__global__ __launch_bounds__(kDqT, 1) void attn_dq_kernel(AttnArgs a)
{
    constexpr int NB = kDqNB;
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *ring = smem;
    float *s_xch = reinterpret_cast<float *>(smem + kXchOff);
    unsigned char *s_scale = smem + kDqScaleOff;
    double *s_ang = reinterpret_cast<double *>(smem + kDqAngOff<E8>);
    uint32_t *s_mask = reinterpret_cast<uint32_t *>(smem + kDqMaskOff<E8>);
    int32_t *s_row = reinterpret_cast<int32_t *>(smem + kDqRowTabOff<E8>);

    // Workgroup -> item = ((query, 16-head group), chunk); consecutive items (the head groups
    // and chunks of a query) are dealt to one XCD (lin mod 8).
    const uint32_t lin = blockIdx.x;
    const uint32_t xcd = lin & 7u, r8 = lin >> 3;
    const uint32_t per_xcd = ((uint32_t)a.n_items + 7u) >> 3;
    const uint32_t item = xcd * per_xcd + r8;
    if (r8 >= per_xcd || item >= (uint32_t)a.n_items) return;    // grid padding
    const uint32_t qg = item / (uint32_t)a.n_chunks;
    const int chunk = (int)(item - qg * (uint32_t)a.n_chunks);
    const uint32_t q32 = qg / (uint32_t)a.n_hg;                   // n_hg = H / 16 here
    const int hg = (int)(qg - q32 * (uint32_t)a.n_hg);
    const uint32_t u32 = q32 / (uint32_t)a.T;
    const int64_t q = q32, u = u32, t = q32 - u32 * (uint32_t)a.T;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // dim quarter, or producer kAW + p
    const int g = lane >> 4, c = lane & 15;
    const int h0 = hg * kWH;

    const int step0 = chunk * a.steps_per_chunk;
    const int step1 = step0 + a.steps_per_chunk < a.n_steps ? step0 + a.steps_per_chunk : a.n_steps;
    const int n = step1 - step0;
    const int rho0 = step0 * kSR;
    const int raw_steps = a.W / kSR;
    const int n_raw = step0 < raw_steps ? min(raw_steps - step0, n) : 0;

    const uint16_t *raw_q = a.raw + (u * (int64_t)(a.T + a.W - 1) + t) * kD;
    constexpr int kCompRowBytes = E8 ? kCodeRow : 2 * kD;
    const unsigned char *comp_u = static_cast<const unsigned char *>(a.comp) + u * a.N * kCompRowBytes;
    const float *cscale_u = E8 ? a.comp_scale + u * a.N : nullptr;
    const int raw_lim = a.raw_vis ? (int)clamp_nvis(a.raw_vis, q, a.W) : a.W;
    const int64_t j_lim = DENSE ? clamp_nvis(a.n_vis, q, a.N) : a.N;

    if (wave >= kAW) {
        // ---- producer wave: raw steps' loads at once (they need no index), the first
        // compressed steps' after the row table, then per step: wait for step k+2's loads
        // (widen it if E4M3), the barrier, and step k+5's loads into the slot of step k+1.
        DqProducer<DENSE, E8> ld;
        ld.ring = ring;
        ld.ring_a = lds_addr(ring);
        ld.scale_a = lds_addr(s_scale);
        ld.s_row = s_row;
        ld.raw_rs = rsrc(raw_q, (uint32_t)raw_lim * (2 * kD));
        ld.comp_rs = rsrc(comp_u, (uint32_t)((uint64_t)a.N * kCompRowBytes));
        ld.scale_rs = rsrc(cscale_u, E8 ? (uint32_t)a.N * 4u : 0u);
        ld.step0 = step0; ld.n = n; ld.n_raw = n_raw; ld.rho0 = rho0; ld.W = a.W;
        ld.p = wave - kAW; ld.lane = lane; ld.j_lim = j_lim;
        // Only step 0 goes out before the row table's barrier: the loads of a cold start are
        // slow to issue, and the computing waves would wait for them at that barrier.
        i32x4 ent[4];
        ld.entries(-1, ent);                  // no entries (raw steps)
        if (n_raw > 0) ld.issue(0, ent);
        __syncthreads();                      // row table
#pragma unroll
        for (int j = 0; j < NB - 1; ++j)
            if (j > 0 || n_raw == 0) {
                ld.entries(j, ent);
                ld.issue(j, ent);
            }
        ld.entries(NB - 1, ent);
        for (int k = -2; k <= n - 2; ++k) {
            // loads issued after step k+2's: steps k+3 and k+4
            if (!E8) {
                wait_vm<2 * kPR>();
            } else {
                const int later_raw = min(max(n_raw - (k + 3), 0), 2);
                if (later_raw == 0) wait_vm<2 * kPCodeBatch>();
                else if (later_raw == 1) wait_vm<kPCodeBatch + kPR>();
                else wait_vm<2 * kPR>();
                if (k + 2 >= n_raw && k + 2 < n) ld.widen(k + 2);
            }
            __syncthreads();
            ld.issue(k + NB + 1, ent);
            ld.entries(k + NB + 2, ent);
        }
        wait_vm<0>();                         // no load may land in LDS after the workgroup ends
        if (a.n_chunks > 1) {                 // the barriers of the record exchange
            __syncthreads();
            __syncthreads();
        }
        return;
    }

    // ---- computing waves: set-up (index entries, query, row table), then the steps.
    const int64_t pos = a.pos[q];             // first: the rotation angles need only it
    constexpr int kPer = kDqMaxChunkSteps * kSR / kAT;        // index entries per thread (6)
    int32_t v_idx[kPer];
    if (!DENSE) {
        const int32_t *idx_q = a.idx + q * (int64_t)a.K;
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int i = tid + r * kAT, k = rho0 + i - a.W;
            v_idx[r] = (i < n * kSR && k >= 0 && k < a.K) ? idx_q[k] : -1;
        }
    }
    // This wave's quarter of the query: k-steps 4w + s (s < 4), dims 32(4w + s) + 8g + e.
    float qv[kQKs][8];
    const int64_t q_off = (q * a.H + h0 + c) * (int64_t)kD + 8 * g + 32 * kQKs * wave;
#pragma unroll
    for (int s = 0; s < kQKs; ++s) {
        if (QF32) {
            const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(a.q) + q_off + 32 * s);
            const float4 x0 = p[0], x1 = p[1];
            qv[s][0] = x0.x; qv[s][1] = x0.y; qv[s][2] = x0.z; qv[s][3] = x0.w;
            qv[s][4] = x1.x; qv[s][5] = x1.y; qv[s][6] = x1.z; qv[s][7] = x1.w;
        } else {
            const u32x4 x = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.q) + q_off + 32 * s);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qv[s][2 * i] = bf16_bits_to_f32(x[i] & 0xFFFFu);
                qv[s][2 * i + 1] = bf16_bits_to_f32(x[i] >> 16);
            }
        }
    }
    if (!DENSE) {
        // row table (local union row -> compressed row or -1) and per-step validity masks
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int i = tid + r * kAT;
            const int32_t e = (v_idx[r] >= 0 && (int64_t)v_idx[r] < a.N) ? v_idx[r] : -1;
            if (i < n * kSR) s_row[i] = e;
            const int rho = rho0 + i;
            const bool ok = i < n * kSR && (rho < a.W ? rho < raw_lim : e >= 0);
            const uint64_t bits = __builtin_amdgcn_ballot_w64(ok);
            if (lane == 0 && (r * kAT + wave * kWave) < n * kSR) {
                s_mask[(r * kAT + wave * kWave) / kSR] = (uint32_t)bits;
                s_mask[(r * kAT + wave * kWave) / kSR + 1] = (uint32_t)(bits >> 32);
            }
        }
    }
    // The rotated tail (dims 448..511) is wave 3's k-steps 2 and 3: pair 16(s-2) + 4g + e/2,
    // rotated in fp64 and rounded once to f32 (rope.hpp, as the compressor rotates its rows).
    // Before the barrier, so that it overlaps the producers' first loads.
    if (wave == kAW - 1) {
        if (lane < kRot / 2) {
            double cs, sn;
            rope_angle(a.log2_theta, lane, pos, cs, sn);
            s_ang[2 * lane] = cs;
            s_ang[2 * lane + 1] = sn;
        }
#pragma unroll
        for (int s = kQKs - 2; s < kQKs; ++s)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const int pr = 16 * (s - (kQKs - 2)) + 4 * g + e / 2;
                rope_rotate(s_ang[2 * pr], s_ang[2 * pr + 1], qv[s][e], qv[s][e + 1]);
            }
    }
    __syncthreads();                          // row table

    // Query fragments: f16 pair while the steps are raw, bf16 pair after (a bf16 query's
    // unrotated dims have lo = 0).
    u32x4 qh[kQKs], ql[kQKs];
#pragma unroll
    for (int s = 0; s < kQKs; ++s) {
        if (n_raw > 0) split8<true>(qv[s], qh[s], ql[s]);
        else split8<false>(qv[s], qh[s], ql[s]);
    }
    // At the switch to compressed steps: the f16 pair holds q to ~22 bits, so the bf16 pair
    // made from hi + lo is as good as one made from q (about 16 bits).
    auto to_bf16_pair = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < kQKs; ++s) {
            const f16x8 h = as_f16x8(qh[s]), l = as_f16x8(ql[s]);
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = (float)h[e] + (float)l[e];
            split8<false>(x, qh[s], ql[s]);
        }
    };

    const float scale2 = a.scale * kLog2e;
    const int qk_base = qk_base_of(g, c), pv_base = pv_base_of(g, c);
    const int sg0 = wave * kQKs, b0 = wave * kQDB;          // this wave's first k-step, dim block
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[kQDB];
#pragma unroll
    for (int b = 0; b < kQDB; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 va[kQDB];                           // V^T fragments of the step whose PV is next
    f32x4 acc[2][2];                          // partial logits [half][k-step parity]
    float rs_cur[8], rs_next[8];              // E4M3 row scales of the current and the next step

    auto step_mask = [&](int j) __attribute__((always_inline)) -> uint32_t {
        if (!DENSE) return s_mask[j];
        const int rho = (step0 + j) * kSR;
        const int64_t lim = j < n_raw ? (int64_t)raw_lim : j_lim + a.W;
        const int64_t cnt = lim - rho;
        return cnt >= kSR ? 0xFFFFFFFFu : (cnt <= 0 ? 0u : (1u << (uint32_t)cnt) - 1u);
    };
    // Row scales of step j (rows 4g+e, 16+4g+e) into rs_next, read while its slot holds them.
    auto read_scales = [&](auto f16_tag, int j) __attribute__((always_inline)) {
        constexpr bool F16 = decltype(f16_tag)::value;
#pragma unroll
        for (int e = 0; e < 8; ++e) rs_next[e] = 1.f;
        if (E8 && !F16) {
            const unsigned char *sb = s_scale + (j % NB) * kAW * kScaleWave + 16 * (g & 1);
            const f32x4 s0 = *reinterpret_cast<const f32x4 *>(sb + (g >> 1) * kScaleWave);
            const f32x4 s1 = *reinterpret_cast<const f32x4 *>(sb + (2 + (g >> 1)) * kScaleWave);
#pragma unroll
            for (int e = 0; e < 4; ++e) { rs_next[e] = s0[e]; rs_next[4 + e] = s1[e]; }
        }
    };
    // Partial logits of step j (this wave's dims) to the exchange buffer of j's parity.
    auto publish = [&](int j) __attribute__((always_inline)) {
        f32x4 p0, p1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p0[i] = acc[0][0][i] + acc[0][1][i];
            p1[i] = acc[1][0][i] + acc[1][1][i];
        }
        // one plane per half step, 16 contiguous bytes per lane (no bank conflicts)
        float *dst = s_xch + (j & 1) * (kXchBuf / 4) + (wave * kWave + lane) * 4;
        *reinterpret_cast<f32x4 *>(dst) = p0;
        *reinterpret_cast<f32x4 *>(dst + kXchPlane) = p1;
    };
    // One step: the softmax of step j from the four waves' partial logits (added in the same
    // order in every wave), interleaved with QK of step jq (when QK), then PV of step j with, as
    // each V^T fragment is consumed, step jq's fragment read in its place.  P^T is a hi + lo
    // pair, k = 8g + e (e < 4: rows 4g + e of the first half; e >= 4: of the second).
    auto step = [&](auto fp, auto fq, auto has_qk, int j, int jq) __attribute__((always_inline)) {
        constexpr bool FP = decltype(fp)::value, FQ = decltype(fq)::value;
        constexpr bool QK = decltype(has_qk)::value;
        const unsigned char *tn = ring + (jq % NB) * kBuf;
        // loads first: QK operands of step jq, the partial logits of step j
        u32x4 x[kQKs][2];
        if (QK) {
#pragma unroll
            for (int s = 0; s < kQKs; ++s) {
                x[s][0] = *reinterpret_cast<const u32x4 *>(tn + qk_base + 64 * (sg0 + s));
                x[s][1] = *reinterpret_cast<const u32x4 *>(tn + kHalfBuf + qk_base + 64 * (sg0 + s));
            }
        }
        const uint32_t mask = step_mask(j);
        const float *src = s_xch + (j & 1) * (kXchBuf / 4) + lane * 4;
        f32x4 s0 = *reinterpret_cast<const f32x4 *>(src);
        f32x4 s1 = *reinterpret_cast<const f32x4 *>(src + kXchPlane);
#pragma unroll
        for (int w = 1; w < kAW; ++w) {
            s0 += *reinterpret_cast<const f32x4 *>(src + w * kWave * 4);
            s1 += *reinterpret_cast<const f32x4 *>(src + w * kWave * 4 + kXchPlane);
        }
        // QK of step jq (independent of the softmax)
        if (QK) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int p = 0; p < 2; ++p) acc[h][p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < kQKs; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    acc[h][s & 1] = mma<FQ>(x[s][h], qh[s], acc[h][s & 1]);
                    acc[h][s & 1] = mma<FQ>(x[s][h], ql[s], acc[h][s & 1]);
                }
        }
        // softmax of step j
        float lg[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float l = (e < 4 ? s0[e] : s1[e - 4]) * scale2 * rs_cur[e];
            lg[e] = (mask >> (16 * (e >> 2) + 4 * g + (e & 3))) & 1u ? l : -INFINITY;
            tmax = fmaxf(tmax, lg[e]);
        }
        tmax = max_g(tmax);
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);   // 0 from -inf
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < kQDB; ++b) o[b] *= alpha;
        m_run = m_new;
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(lg[e] - m_use);
            l_run += p;
            pv[e] = p * rs_cur[e];
        }
        u32x4 ph, pl;
        split8<FP>(pv, ph, pl);
        // PV of step j; V^T of step jq in place
#pragma unroll
        for (int i = 0; i < kQDB; ++i) {
            o[i] = mma<FP>(va[i], ph, o[i]);
            o[i] = mma<FP>(va[i], pl, o[i]);
            if (QK) va[i] = tr_frag(tn + pv_base, b0 + i);
        }
    };
    // QK and V^T of step 0 alone.
    auto first = [&](auto fq) __attribute__((always_inline)) {
        constexpr bool FQ = decltype(fq)::value;
        const unsigned char *tn = ring;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int p = 0; p < 2; ++p) acc[h][p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kQKs; ++s)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4 x = *reinterpret_cast<const u32x4 *>(tn + h * kHalfBuf + qk_base + 64 * (sg0 + s));
                acc[h][s & 1] = mma<FQ>(x, qh[s], acc[h][s & 1]);
                acc[h][s & 1] = mma<FQ>(x, ql[s], acc[h][s & 1]);
            }
#pragma unroll
        for (int i = 0; i < kQDB; ++i) va[i] = tr_frag(tn + pv_base, b0 + i);
    };
    // Barrier k: step k+2 may be used (the producers have waited for its loads, and widened it
    // if E4M3), the partial logits written before it are published, and this wave's QK and V^T
    // reads of step k+1 are done, so the producers refill its slot with step k + NB + 1.
    auto advance = [&](int k) __attribute__((always_inline)) {
        (void)k;
        wait_lds();
        __syncthreads();
    };

    // ---- the pipeline.  Barrier -2: step 0's rows.  Then QK and V^T of step 0, its partial
    // logits, barrier -1.  Step j: softmax(j) with QK(j+1), PV(j) with V^T(j+1), the partial
    // logits of j+1, barrier j.
    advance(-2);
    if (n_raw > 0) { first(F16T{}); read_scales(F16T{}, 0); }
    else { first(BF16T{}); read_scales(BF16T{}, 0); }
    publish(0);
    advance(-1);

    auto body = [&](auto fj, auto fn, int j) __attribute__((always_inline)) {
        constexpr bool FJ = decltype(fj)::value, FN = decltype(fn)::value;
        if (FJ && !FN) to_bf16_pair();
#pragma unroll
        for (int e = 0; e < 8; ++e) rs_cur[e] = rs_next[e];
        step(fj, fn, std::true_type{}, j, j + 1);
        read_scales(fn, j + 1);
        publish(j + 1);
        advance(j);
    };
    int j = 0;
    for (; j + 1 < n_raw; ++j) body(F16T{}, F16T{}, j);
    if (j + 1 == n_raw && j + 1 < n) {
        body(F16T{}, BF16T{}, j);
        ++j;
    }
    for (; j + 1 < n; ++j) body(BF16T{}, BF16T{}, j);
#pragma unroll
    for (int e = 0; e < 8; ++e) rs_cur[e] = rs_next[e];
    if (j < n_raw) step(F16T{}, F16T{}, std::false_type{}, j, j);
    else step(BF16T{}, BF16T{}, std::false_type{}, j, j);

    l_run = sum_g(l_run);                     // the same in every wave
    if (a.n_chunks == 1) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float *orow = a.out + (q * a.H + h0 + c) * (int64_t)kD + 16 * b0 + 4 * g;
#pragma unroll
        for (int b = 0; b < kQDB; ++b) *reinterpret_cast<f32x4 *>(orow + 16 * b) = o[b] * inv;
        return;
    }
    // ---- split union: the workgroup's record, then the last workgroup of the (query, head
    // group) merges.  Records and the counter are accessed with agent-scope coherence on every
    // access (sc1), and the record stores have completed before the count is added.
    constexpr int kSc1 = 16;
    const int nc = a.n_chunks;
    const int64_t grp = q * a.n_hg + hg;
    const __amdgpu_buffer_rsrc_t rec_rs = rsrc(a.part + grp * nc * (int64_t)kDqRec, (uint32_t)(nc * kDqRec * 4));
    const uint32_t rec0 = (uint32_t)(chunk * kDqRec * 4);
    const uint32_t o_off = 4 * (2 * kWH + (wave * kQDB * kWave + lane) * 4);   // + b * 1 KiB
    if (wave == 0 && g == 0) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_run), rec_rs, rec0 + 4 * c, 0, kSc1);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_run), rec_rs, rec0 + 4 * (kWH + c), 0, kSc1);
    }
#pragma unroll
    for (int b = 0; b < kQDB; ++b)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[b]), rec_rs, rec0 + o_off + b * 1024, 0, kSc1);
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");   // this wave's record stores are done
    __syncthreads();                                      // ... and every wave's
    uint32_t *s_flag = reinterpret_cast<uint32_t *>(s_xch);
    if (tid == 0)
        s_flag[0] = __hip_atomic_fetch_add(a.count + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_flag[0] != (uint32_t)nc - 1) return;
    // Merge: this wave's quarter of O, online over the chunks, 4 records per pass.
    float M = -INFINITY, L = 0.f;
    f32x4 sum[kQDB];
#pragma unroll
    for (int b = 0; b < kQDB; ++b) sum[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nc; c0 += 4) {
        float mv[4], lv[4];
        f32x4 xv[4][kQDB];
#pragma unroll
        for (int k = 0; k < 4; ++k) {         // records past the last read as zeros
            const uint32_t r = (uint32_t)((c0 + k) * kDqRec * 4);
            mv[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rec_rs, r + 4 * c, 0, kSc1));
            lv[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rec_rs, r + 4 * (kWH + c), 0, kSc1));
#pragma unroll
            for (int b = 0; b < kQDB; ++b)
                xv[k][b] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rec_rs, r + o_off + b * 1024, 0, kSc1));
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (c0 + k >= nc || mv[k] == -INFINITY) continue;   // no visible row in that chunk
            const float M2 = fmaxf(M, mv[k]);
            const float wa = __builtin_amdgcn_exp2f(M - M2), wb = __builtin_amdgcn_exp2f(mv[k] - M2);   // M = -inf: 0
            L = L * wa + lv[k] * wb;
#pragma unroll
            for (int b = 0; b < kQDB; ++b) sum[b] = sum[b] * wa + xv[k][b] * wb;
            M = M2;
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float *orow = a.out + (q * a.H + h0 + c) * (int64_t)kD + 16 * b0 + 4 * g;
#pragma unroll
    for (int b = 0; b < kQDB; ++b) *reinterpret_cast<f32x4 *>(orow + 16 * b) = sum[b] * inv;
    if (tid == 0) __hip_atomic_store(a.count + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // ready for the next call
}

}  // namespace

AttnPlan plan_attn_dq(int U, int T, int H, int W, int K) {
    AttnPlan p;
    p.dq = true;
    p.n_hg = H / kWH;
    p.n_steps = (W + K + kSR - 1) / kSR;
    const int64_t Q = (int64_t)U * T;
    const int64_t items = Q * p.n_hg;
    // One workgroup per CU (LDS): split the union only when (query, head group) pairs leave
    // most CUs idle, keeping at least 2 steps per chunk; unions longer than the row table are
    // split too.
    int64_t want = items >= 192 ? 1 : 256 / items;
    const int64_t max_split = p.n_steps / 2 > 1 ? p.n_steps / 2 : 1;
    if (want > max_split) want = max_split;
    const int64_t need = (p.n_steps + kDqMaxChunkSteps - 1) / kDqMaxChunkSteps;
    if (want < need) want = need;
    if (want < 1) want = 1;
    p.steps_per_chunk = (int)((p.n_steps + want - 1) / want);
    p.n_chunks = (p.n_steps + p.steps_per_chunk - 1) / p.steps_per_chunk;
    p.count_bytes = p.n_chunks > 1 ? (((size_t)Q * (size_t)p.n_hg * 4 + 255) & ~(size_t)255) : 0;
    p.workspace_bytes =
        p.n_chunks > 1 ? p.count_bytes + sizeof(float) * (size_t)Q * (size_t)p.n_hg * (size_t)p.n_chunks * kDqRec : 0;
    p.blocks = ((Q * p.n_hg * p.n_chunks + 7) / 8) * 8;
    return p;
}

hipError_t launch_attn_dq(const AttnPlan &p, int U, int T, int H, int W, int64_t N, int K, const void *q, int q_bf16,
                          const int64_t *q_pos, double theta, const uint16_t *raw, const void *comp,
                          const float *comp_scale, const int32_t *idx, const int32_t *n_vis, const int32_t *raw_vis,
                          float scale, float *out, uint32_t *count, float *part, hipStream_t stream)
{
    const bool dense = idx == nullptr;
    const bool e8 = comp_scale != nullptr && N > 0;
    using Fn = void (*)(AttnArgs);
    const int variant = (q_bf16 ? 1 : 0) + (dense ? 2 : 0) + (e8 ? 4 : 0);
    static const Fn kernels[8] = {attn_dq_kernel<true, false, false>, attn_dq_kernel<false, false, false>,
                                  attn_dq_kernel<true, true, false>,  attn_dq_kernel<false, true, false>,
                                  attn_dq_kernel<true, false, true>,  attn_dq_kernel<false, false, true>,
                                  attn_dq_kernel<true, true, true>,   attn_dq_kernel<false, true, true>};
    static std::once_flag attr_once[8];
    static hipError_t attr_err[8];
    const Fn fn = kernels[variant];
    std::call_once(attr_once[variant], [&] {
        attr_err[variant] = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                                e8 ? kDqMaxLds<true> : kDqMaxLds<false>);
    });
    if (attr_err[variant] != hipSuccess) return attr_err[variant];
    const int lds = (e8 ? kDqRowTabOff<true> : kDqRowTabOff<false>) + (dense ? 0 : 4 * kSR * p.steps_per_chunk);
    AttnArgs a = {};
    a.T = T; a.H = H; a.W = W; a.K = K; a.n_hg = p.n_hg; a.n_chunks = p.n_chunks;
    a.steps_per_chunk = p.steps_per_chunk; a.n_steps = p.n_steps;
    a.n_items = (int)((int64_t)U * T * p.n_hg * p.n_chunks);
    a.N = N;
    a.q = q; a.pos = q_pos; a.raw = raw; a.comp = comp; a.idx = idx; a.n_vis = n_vis;
    a.comp_scale = e8 ? comp_scale : nullptr;
    a.raw_vis = W > 0 ? raw_vis : nullptr;
    a.scale = scale; a.out = out;
    a.count = count;
    a.part = part;
    a.log2_theta = log2(theta);
    hipLaunchKernelGGL(fn, dim3((unsigned)p.blocks), dim3(kDqT), lds, stream, a);
    return hipGetLastError();
}

}  // namespace ds4a
