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
#include "select.hpp"

#include <math.h>
#include <mutex>

namespace ds4a {

namespace {

constexpr int kDqP = 2;                       // producer waves
constexpr int kDqT = kAT + kDqP * kWave;      // threads per workgroup: 4 computing + 2 producer waves
constexpr int kPR = kSR / kDqP;               // rows each producer loads per step (16): half step p
constexpr int kDqCodeOff = kHalfBuf - kPR * kCodeRow;   // E4M3 codes of a half step: its last 8 KiB
constexpr int kPCodeBatch = kPR / 2 + 2;      // E4M3 step: loads per producer (codes, 2 x scales)
constexpr int kHKs = kKs / 2;                 // QK k-steps per wave: its half of the dims (8)
constexpr int kQKs = kKs / kAW;               // k-steps of a quarter of the dims (4)
constexpr int kHDB = kDB / 2;                 // PV dim blocks per wave (16)
constexpr int kQDB = kDB / kAW;               // dim blocks each wave keeps after the merge (8)
constexpr int kDqNB = 4;                      // ring slots
constexpr int kXchOff = kDqNB * kBuf;         // partial logits: [parity][wave][lane][4] f32
constexpr int kXchBuf = kAW * kWave * 4 * 4;  // 4 KiB per parity
constexpr int kDqScaleOff = kXchOff + 2 * kXchBuf;
template <bool E8> constexpr int kDqAngOff = kDqScaleOff + (E8 ? kDqNB * kAW * kScaleWave : 0);  // [32] (cos, sin) fp64
template <bool E8> constexpr int kDqMlOff = kDqAngOff<E8> + 32 * 16;        // merge: m[wave][16], l[wave][16]
template <bool E8> constexpr int kDqMaskOff = kDqMlOff<E8> + 2 * kAW * kWH * 4;   // sparse: row validity per step
constexpr int kDqMaxChunkSteps = 48;          // longer unions are split
template <bool E8> constexpr int kDqRowTabOff = kDqMaskOff<E8> + 4 * kDqMaxChunkSteps;
template <bool E8> constexpr int kDqMaxLds = kDqRowTabOff<E8> + 4 * kSR * kDqMaxChunkSteps;
static_assert(kDqMaxLds<false> <= 160 * 1024 && kDqMaxLds<true> <= 160 * 1024, "LDS of one workgroup");
static_assert(kDqMaxChunkSteps * kSR % kAT == 0, "row table fill");
constexpr int kDqRec = 2 * kWH + kWH * kD;    // record: m[16], l[16], O[quarter][block][lane][4]
constexpr int kMEpt = 16;                     // last merge level in the kernel: candidates per thread
constexpr int kDqMergeMax = kMEpt * kDqT;     // ... and per query (6,144)
static_assert(sizeof(SelectSharedT<kSelCopies>) <= kBuf, "the selection's scratch fits in one ring slot");
static_assert(kDqMergeMax == kAttnMergeMax, "the host's bound on the in-kernel merge");
static_assert(kAW * kQDB * kWave * 16 <= kDqNB * kBuf, "row-half merge fits in the ring");
static_assert(kAW * kQKs * 2 * kWave * 16 <= kBuf, "query quarters fit in one ring slot");
constexpr float kLazy = 8.f;                  // reference slack (log2 units): P stays below 2^8

// 4 floats -> hi + lo pair of the MFMA operand type, as the B operand of a folded PV step:
// k = 8g + e takes hi of value e (e < 4) and lo of value e - 4 (e >= 4).
template <bool F16>
__device__ __forceinline__ u32x4 split4_fold(const float (&x)[4]) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const f32x2 v = {x[2 * i], x[2 * i + 1]};
        if (F16) {
            const f16x2 h = __builtin_convertvector(v, f16x2);
            const f16x2 l = __builtin_convertvector(v - __builtin_convertvector(h, f32x2), f16x2);
            r[i] = __builtin_bit_cast(uint32_t, h);
            r[2 + i] = __builtin_bit_cast(uint32_t, l);
        } else {
            const bf16x2 h = __builtin_convertvector(v, bf16x2);
            const bf16x2 l = __builtin_convertvector(v - __builtin_convertvector(h, f32x2), bf16x2);
            r[i] = __builtin_bit_cast(uint32_t, h);
            r[2 + i] = __builtin_bit_cast(uint32_t, l);
        }
    }
    return r;
}

// Row loads of the union's 32-row steps for producer wave p: rows 16p..16p+15 of each step
// (half step p), step j in ring slot j % kDqNB.  Raw steps: rows of the query's window, 1 KiB
// each, one instruction per row; rows at or past raw_vis lie past the window resource and read
// as zeros.  Compressed steps: bf16 rows from their entries (row index, or -1: past the
// resource, zeros); E4M3 rows as codes, two rows per instruction, into the last 8 KiB of the
// half step, plus the rows' scales as the computing waves read them (per 8-row quarter, lane l
// holding row l % 8).  Row data:
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

// MERGE (sparse, unsplit unions): the workgroup selects the query's K rows from the last
// candidate list of the chunked top-k itself (every wave: kMEpt candidates per thread, the same
// workgroup radix select as the top-k kernels, so the set is the same), straight into its row
// table; the workgroup of head group 0 also writes them out.
template <bool QF32, bool DENSE, bool E8, bool MERGE = false>
__global__ __launch_bounds__(kDqT, 1) void attn_dq_kernel(AttnArgs a)
{
    static_assert(!(MERGE && DENSE), "the merge feeds the sparse union");
    constexpr int NB = kDqNB;
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *ring = smem;
    float *s_xch = reinterpret_cast<float *>(smem + kXchOff);
    unsigned char *s_scale = smem + kDqScaleOff;
    double *s_ang_all = reinterpret_cast<double *>(smem + kDqAngOff<E8>);
    float *s_m = reinterpret_cast<float *>(smem + kDqMlOff<E8>);
    float *s_l = s_m + kAW * kWH;
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
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // (row half, dim half), or producer kAW + p
    const int rh = wave >> 1, dh = wave & 1;  // computing wave: rows 16 rh.. of each step, dims 256 dh..
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

    // The last merge level (every thread of the workgroup): the selection lands in s_row[W ..
    // W + K) in ascending row order, -1 past the selected.  Its candidates are loaded first of
    // all (cand_load), so their latency overlaps the query set-up and the first raw rows' loads;
    // ring slot 2 holds the select's scratch (slots 0 and 1 take raw rows meanwhile, slot 3 the
    // query quarters), free again after the barrier that follows the select.
    uint32_t ckey[kMEpt];
    int32_t cid[kMEpt];
    int cand_n = 0;
    auto cand_load = [&]() __attribute__((always_inline)) {
        Levels lv = {};
        lv.n = a.lv_n;
#pragma unroll
        for (int l = 0; l < kMaxLevels; ++l) lv.ch[l] = a.lv_ch[l];
        int64_t count = cand_count(clamp_nvis(a.cand_nvis, q, a.N), a.K, lv);
        if (count > a.cand_stride) count = a.cand_stride;
        cand_n = (int)count;
        const uint32_t *ik = a.cand_keys + q * a.cand_stride;
        const int32_t *ii = a.cand_ids + q * a.cand_stride;
        const __amdgpu_buffer_rsrc_t rk = list_rsrc(ik, (uint32_t)cand_n * 4u), ri = list_rsrc(ii, (uint32_t)cand_n * 4u);
        const int j0 = tid * kMEpt;
        if (((reinterpret_cast<uintptr_t>(ik) | reinterpret_cast<uintptr_t>(ii)) & 15u) == 0) {
#pragma unroll
            for (int v = 0; v < kMEpt / 4; ++v) {
                const uint32_t off = (uint32_t)(j0 + 4 * v) * 4u;
                const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
                const u32x4 y = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ri, off, 0, 0));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ckey[4 * v + e] = x[e];
                    cid[4 * v + e] = (int32_t)y[e];
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kMEpt; ++i) {
                ckey[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, (uint32_t)(j0 + i) * 4u, 0, 0);
                cid[i] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ri, (uint32_t)(j0 + i) * 4u, 0, 0);
            }
        }
    };
    // The candidates are waited for here, while nothing else is in flight: the rows' and the
    // query's loads go out after them, during the select's passes, and do not delay them.
    auto cand_wait = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kMEpt; ++i) asm volatile("" : : "v"(ckey[i]), "v"(cid[i]));
    };
    auto cand_select = [&]() __attribute__((always_inline)) {
        SelectSharedT<kSelCopies> &sm = *reinterpret_cast<SelectSharedT<kSelCopies> *>(ring + (NB - 2) * kBuf);
        block_select<kMEpt, true, kDqT, kSelCopies>(ckey, cid, 0, cand_n, a.K < cand_n ? a.K : cand_n, a.K,
                                                    s_row + a.W, nullptr, sm);
    };
    // Raw steps whose loads go out before the row table: with the merge, as many as the slots
    // the select leaves free (its own slot and the query quarters' stay untouched); without it,
    // step 0 only (a cold start's loads are slow to issue, and the computing waves would wait
    // for them at the row table's barrier).
    const int n_pre = MERGE ? min(n_raw, NB - 2) : min(n_raw, 1);

    if (wave >= kAW) {
        // ---- producer wave: raw steps' loads at once (they need no index), the first
        // compressed steps' after the row table, then per step: wait for step k+2's loads
        // (widen it if E4M3), the barrier, and step k+5's loads into the slot of step k+1.
        DqProducer<DENSE, E8> ld;
        ld.ring = ring;
        ld.ring_a = lds_addr(ring);
        ld.scale_a = lds_addr(s_scale);
        ld.s_row = MERGE ? s_row + rho0 : s_row;   // merge: the row table covers the whole union
        ld.raw_rs = rsrc(raw_q, (uint32_t)raw_lim * (2 * kD));
        ld.comp_rs = rsrc(comp_u, (uint32_t)((uint64_t)a.N * kCompRowBytes));
        ld.scale_rs = rsrc(cscale_u, E8 ? (uint32_t)a.N * 4u : 0u);
        ld.step0 = step0; ld.n = n; ld.n_raw = n_raw; ld.rho0 = rho0; ld.W = a.W;
        ld.p = wave - kAW; ld.lane = lane; ld.j_lim = j_lim;
        if (MERGE) {
            cand_load();
            cand_wait();
        }
        i32x4 ent[4];
        ld.entries(-1, ent);                  // no entries (raw steps)
        for (int j = 0; j < n_pre; ++j) ld.issue(j, ent);
        if (MERGE) {
            cand_select();
            __syncthreads();                  // the selection is in the row table
        }
        __syncthreads();                      // row table
#pragma unroll
        for (int j = 0; j < NB - 1; ++j)
            if (j >= n_pre && j < n) {
                ld.entries(j, ent);
                ld.issue(j, ent);
            }
        ld.entries(NB - 1, ent);
        // loads of step j: none past the chunk
        auto batch = [&](int j) __attribute__((always_inline)) -> int {
            return j >= n ? 0 : (E8 && j >= n_raw ? kPCodeBatch : kPR);
        };
        for (int k = -2; k <= n - 2; ++k) {
            // wait for step k+2's loads: only steps k+3's and k+4's may still be in flight
            const int later = batch(k + 3) + batch(k + 4);
            if (later >= 2 * kPR) wait_vm<2 * kPR>();
            else if (E8 && later >= kPR + kPCodeBatch) wait_vm<kPR + kPCodeBatch>();
            else if (E8 && later >= 2 * kPCodeBatch) wait_vm<2 * kPCodeBatch>();
            else if (later >= kPR) wait_vm<kPR>();
            else if (E8 && later >= kPCodeBatch) wait_vm<kPCodeBatch>();
            else wait_vm<0>();
            if (E8 && k + 2 >= n_raw && k + 2 < n) ld.widen(k + 2);
            __syncthreads();
            if (k + NB + 1 < n) ld.issue(k + NB + 1, ent);
            ld.entries(k + NB + 2, ent);
        }
        wait_vm<0>();                         // every load has landed before the ring is reused
        __syncthreads();                      // the barriers of the row-half merge
        __syncthreads();
        if (a.n_chunks > 1) {                 // ... and of the record exchange
            __syncthreads();
            __syncthreads();
        }
        return;
    }

    // ---- computing waves: set-up (index entries, query, row table), then the steps.
    const int64_t pos = a.pos[q];             // first: the rotation angles need only it
    if (MERGE) {
        cand_load();
        cand_wait();
    }
    constexpr int kPer = kDqMaxChunkSteps * kSR / kAT;        // index entries per thread (6)
    int32_t v_idx[kPer];
    if (!DENSE && !MERGE) {
        const int32_t *idx_q = a.idx + q * (int64_t)a.K;
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int i = tid + r * kAT, k = rho0 + i - a.W;
            v_idx[r] = (i < n * kSR && k >= 0 && k < a.K) ? idx_q[k] : -1;
        }
    }
    // This wave loads a quarter of the query, qq = 2 dh + rh: k-steps 4 qq + i (i < 4), dims
    // 32(4 qq + i) + 8g + e; the wave of the other row half brings the rest of its dim half.
    const int qq = 2 * dh + rh;
    float qv[kQKs][8];
    const int64_t q_off = (q * a.H + h0 + c) * (int64_t)kD + 8 * g + 32 * kQKs * qq;
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
    // The rotated tail (dims 448..511) is quarter 3's k-steps 2 and 3: pair 16(s - 2) + 4g + e/2,
    // rotated in fp64 and rounded once to f32 (rope.hpp, as the compressor rotates its rows).
    // The angles need only the position, so they are formed while the loads are in flight.
    if (qq == kAW - 1 && lane < kRot / 2) {
        double cs, sn;
        rope_angle(a.log2_theta, lane, pos, cs, sn);
        s_ang_all[2 * lane] = cs;
        s_ang_all[2 * lane + 1] = sn;
    }
    if (MERGE) {
        cand_select();                        // waits for the candidates only (loaded before the query)
        __syncthreads();                      // the selection is in the row table
        if (a.idx_out && hg == 0 && chunk == 0) {
            int32_t *dst = a.idx_out + q * (int64_t)a.K;
            for (int k = tid; k < a.K; k += kAT) dst[k] = s_row[a.W + k];
        }
    }
    if (qq == kAW - 1) {
        wait_lds();                           // this wave's angles
#pragma unroll
        for (int s = kQKs - 2; s < kQKs; ++s)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const int pr = 16 * (s - (kQKs - 2)) + 4 * g + e / 2;
                rope_rotate(s_ang_all[2 * pr], s_ang_all[2 * pr + 1], qv[s][e], qv[s][e + 1]);
            }
    }
    // Query fragments: f16 pair while the steps are raw, bf16 pair after (a bf16 query's
    // unrotated dims have lo = 0).  Each wave publishes its quarter's pairs in ring slot 3, which
    // takes rows only after the barrier of step -2, and reads its partner's after the row
    // table's barrier.  Without the merge all of this comes before the row table, whose index
    // entries it waits for.
    u32x4 qh_m[kQKs], ql_m[kQKs];
#pragma unroll
    for (int s = 0; s < kQKs; ++s) {
        if (n_raw > 0) split8<true>(qv[s], qh_m[s], ql_m[s]);
        else split8<false>(qv[s], qh_m[s], ql_m[s]);
    }
    u32x4 *xq = reinterpret_cast<u32x4 *>(ring + (NB - 1) * kBuf);      // [wave][k-step][hi, lo][lane]
#pragma unroll
    for (int s = 0; s < kQKs; ++s) {
        xq[((wave * kQKs + s) * 2) * kWave + lane] = qh_m[s];
        xq[((wave * kQKs + s) * 2 + 1) * kWave + lane] = ql_m[s];
    }
    if (!DENSE) {
        // row table (local union row -> compressed row or -1) and per-step validity masks
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int i = tid + r * kAT;
            int32_t e;
            if (MERGE) {
                // the selection's entries, -1 outside them (raw rows, the last step's tail); the
                // table is indexed by union row, so this chunk's rows start at rho0
                const int k = rho0 + i - a.W;
                e = (i < n * kSR && k >= 0 && k < a.K) ? s_row[rho0 + i] : -1;
                e = (e >= 0 && (int64_t)e < a.N) ? e : -1;
                if (i < n * kSR && (k < 0 || k >= a.K)) s_row[rho0 + i] = e;
            } else {
                e = (v_idx[r] >= 0 && (int64_t)v_idx[r] < a.N) ? v_idx[r] : -1;
                if (i < n * kSR) s_row[i] = e;
            }
            const int rho = rho0 + i;
            const bool ok = i < n * kSR && (rho < a.W ? rho < raw_lim : e >= 0);
            const uint64_t bits = __builtin_amdgcn_ballot_w64(ok);
            if (lane == 0 && (r * kAT + wave * kWave) < n * kSR) {
                s_mask[(r * kAT + wave * kWave) / kSR] = (uint32_t)bits;
                s_mask[(r * kAT + wave * kWave) / kSR + 1] = (uint32_t)(bits >> 32);
            }
        }
    }
    __syncthreads();                          // row table, query quarters
    u32x4 qh[kHKs], ql[kHKs];
    auto assemble = [&](auto half) __attribute__((always_inline)) {
        constexpr int R = decltype(half)::value;          // this wave's row half
        const int partner = wave ^ 2;
#pragma unroll
        for (int s = 0; s < kQKs; ++s) {
            qh[R * kQKs + s] = qh_m[s];
            ql[R * kQKs + s] = ql_m[s];
            qh[(1 - R) * kQKs + s] = xq[((partner * kQKs + s) * 2) * kWave + lane];
            ql[(1 - R) * kQKs + s] = xq[((partner * kQKs + s) * 2 + 1) * kWave + lane];
        }
    };
    if (rh == 0) assemble(std::integral_constant<int, 0>{});
    else assemble(std::integral_constant<int, 1>{});
    // At the switch to compressed steps: the f16 pair holds q to ~22 bits, so the bf16 pair
    // made from hi + lo is as good as one made from q (about 16 bits).
    auto to_bf16_pair = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < kHKs; ++s) {
            const f16x8 h = as_f16x8(qh[s]), l = as_f16x8(ql[s]);
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = (float)h[e] + (float)l[e];
            split8<false>(x, qh[s], ql[s]);
        }
    };

    const float scale2 = a.scale * kLog2e;
    // this wave's row half of a step, and its first k-step and dim block
    const int qk_base = qk_base_of(g, c) + rh * kHalfBuf, pv_base = pv_base_of(g, c) + rh * kHalfBuf;
    const int sg0 = dh * kHKs, bd0 = dh * kHDB;
    float m_ref = -INFINITY, l_run = 0.f;     // lazy reference and sum of head c over this row half
    f32x4 o[kHDB];                            // O^T of dims 256 dh + 16 i + 4g + (0..3), head c
#pragma unroll
    for (int b = 0; b < kHDB; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x2 va[kHDB];                           // V^T fragments of the step whose PV is next
    f32x4 acc[2];                             // partial logits [k-step parity]
    float rs_cur[4], rs_next[4];              // E4M3 row scales of the current and the next step

    auto step_mask = [&](int j) __attribute__((always_inline)) -> uint32_t {
        if (!DENSE) return s_mask[j];
        const int rho = (step0 + j) * kSR;
        const int64_t lim = j < n_raw ? (int64_t)raw_lim : j_lim + a.W;
        const int64_t cnt = lim - rho;
        return cnt >= kSR ? 0xFFFFFFFFu : (cnt <= 0 ? 0u : (1u << (uint32_t)cnt) - 1u);
    };
    // Row scales of step j (rows 16 rh + 4g + e) into rs_next, read while its slot holds them.
    auto read_scales = [&](auto f16_tag, int j) __attribute__((always_inline)) {
        constexpr bool F16 = decltype(f16_tag)::value;
#pragma unroll
        for (int e = 0; e < 4; ++e) rs_next[e] = 1.f;
        if (E8 && !F16) {
            const f32x4 s0 = *reinterpret_cast<const f32x4 *>(s_scale + ((j % NB) * kAW + 2 * rh + (g >> 1)) * kScaleWave +
                                                              16 * (g & 1));
#pragma unroll
            for (int e = 0; e < 4; ++e) rs_next[e] = s0[e];
        }
    };
    // Partial logits of step j (this wave's dims) to the exchange buffer of j's parity.
    auto publish = [&](int j) __attribute__((always_inline)) {
        *reinterpret_cast<f32x4 *>(s_xch + (j & 1) * (kXchBuf / 4) + (wave * kWave + lane) * 4) = acc[0] + acc[1];
    };
    // One step: the softmax of step j over this wave's row half, from the two dim halves'
    // partial logits (added in dim order, so both waves of the row half hold the same logits and
    // take the same decisions), interleaved with QK of step jq (when QK), then PV of step j with,
    // as each V^T fragment is consumed, step jq's fragment read in its place.  P^T is a hi + lo
    // pair folded into k = 8g + e: hi of row 4g + e for e < 4, lo of the same row for e >= 4.
    auto step = [&](auto fp, auto fq, auto has_qk, int j, int jq) __attribute__((always_inline)) {
        constexpr bool FP = decltype(fp)::value, FQ = decltype(fq)::value;
        constexpr bool QK = decltype(has_qk)::value;
        const unsigned char *tn = ring + (jq % NB) * kBuf;
        // loads first: QK operands of step jq, the partial logits of step j
        u32x4 x[kHKs];
        if (QK) {
#pragma unroll
            for (int s = 0; s < kHKs; ++s) x[s] = *reinterpret_cast<const u32x4 *>(tn + qk_base + 64 * (sg0 + s));
        }
        const uint32_t mask = step_mask(j) >> (16 * rh);
        const float *src = s_xch + (j & 1) * (kXchBuf / 4) + ((2 * rh) * kWave + lane) * 4;
        const f32x4 sl = *reinterpret_cast<const f32x4 *>(src) + *reinterpret_cast<const f32x4 *>(src + kWave * 4);
        // QK of step jq: independent of the softmax of step j.  Without E4M3 rows it comes after
        // the softmax's logits, the row half's maximum and the rare rescale, so that the rest of
        // the softmax (exponentials, the sum, the hi + lo split) is issued between its MFMAs;
        // with them it comes first (the other order leaves their row scales no registers).
        auto qk_mfmas = [&]() __attribute__((always_inline)) {
            if (QK) {
                acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
                acc[1] = acc[0];
#pragma unroll
                for (int s = 0; s < kHKs; ++s) {
                    acc[s & 1] = mma<FQ>(x[s], qh[s], acc[s & 1]);
                    acc[s & 1] = mma<FQ>(x[s], ql[s], acc[s & 1]);
                }
            }
        };
        if (E8) qk_mfmas();
        float lg[4];
        float tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float l = sl[e] * scale2 * rs_cur[e];
            lg[e] = (mask >> (4 * g + e)) & 1u ? l : -INFINITY;
            tmax = fmaxf(tmax, lg[e]);
        }
        tmax = max_g(tmax);                   // head c over the row half's 16 rows
        if (__builtin_amdgcn_ballot_w64(tmax > m_ref + kLazy) != 0) {
            const float m_new = fmaxf(m_ref, tmax);
            const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);   // 0 from -inf
            l_run *= alpha;
#pragma unroll
            for (int b = 0; b < kHDB; ++b) o[b] *= alpha;
            m_ref = m_new;
        }
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
        if (!E8) qk_mfmas();
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p = __builtin_amdgcn_exp2f(lg[e] - m_use);
            l_run += p;
            pv[e] = p * rs_cur[e];
        }
        const u32x4 pp = split4_fold<FP>(pv);
        if (QK && !E8) {
            // one QK MFMA, then two VALU instructions of the softmax, in turn
#pragma unroll
            for (int i = 0; i < 2 * kHKs; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x402, 2, 0);
            }
        }
        // PV of step j; V^T of step jq in place
#pragma unroll
        for (int i = 0; i < kHDB; ++i) {
            o[i] = mma<FP>(u32x4{va[i][0], va[i][1], va[i][0], va[i][1]}, pp, o[i]);
            if (QK) va[i] = __builtin_bit_cast(u32x2, lds_read_tr16(tn + pv_base + 32 * (bd0 + i)));
        }
    };
    // QK and V^T of step 0 alone.
    auto first = [&](auto fq) __attribute__((always_inline)) {
        constexpr bool FQ = decltype(fq)::value;
        const unsigned char *tn = ring;
        acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[1] = acc[0];
#pragma unroll
        for (int s = 0; s < kHKs; ++s) {
            const u32x4 x = *reinterpret_cast<const u32x4 *>(tn + qk_base + 64 * (sg0 + s));
            acc[s & 1] = mma<FQ>(x, qh[s], acc[s & 1]);
            acc[s & 1] = mma<FQ>(x, ql[s], acc[s & 1]);
        }
#pragma unroll
        for (int i = 0; i < kHDB; ++i) va[i] = __builtin_bit_cast(u32x2, lds_read_tr16(tn + pv_base + 32 * (bd0 + i)));
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
        for (int e = 0; e < 4; ++e) rs_cur[e] = rs_next[e];
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
    for (int e = 0; e < 4; ++e) rs_cur[e] = rs_next[e];
    if (j < n_raw) step(F16T{}, F16T{}, std::false_type{}, j, j);
    else step(BF16T{}, BF16T{}, std::false_type{}, j, j);

    // ---- the two row halves merged: wave (rh, dh) keeps dims 256 dh + 128 rh .. + 127 (quarter
    // 2 dh + rh) and takes the other row half's (m, l, O) for them through LDS.
    l_run = sum_g(l_run);                     // head c over this row half
    wait_lds();
    __syncthreads();                          // the producers' loads have landed; the ring is free
    if (g == 0) {
        s_m[wave * kWH + c] = m_ref;
        s_l[wave * kWH + c] = l_run;
    }
    float *xo = reinterpret_cast<float *>(ring);                     // [wave][block][lane][4]
    if (rh == 0) {
#pragma unroll
        for (int i = 0; i < kQDB; ++i) *reinterpret_cast<f32x4 *>(xo + ((wave * kQDB + i) * kWave + lane) * 4) = o[kQDB + i];
    } else {
#pragma unroll
        for (int i = 0; i < kQDB; ++i) *reinterpret_cast<f32x4 *>(xo + ((wave * kQDB + i) * kWave + lane) * 4) = o[i];
    }
    wait_lds();
    __syncthreads();
    const int partner = wave ^ 2;             // same dim half, other row half
    const float mo = s_m[partner * kWH + c], lo_ = s_l[partner * kWH + c];
    const float m_run = fmaxf(m_ref, mo);
    const float f_own = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_run);
    const float f_oth = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - m_run);
    const float l_tot = l_run * f_own + lo_ * f_oth;
    f32x4 om[kQDB];
    auto merge_half = [&](auto half) __attribute__((always_inline)) {
        constexpr int H0 = decltype(half)::value * kQDB;
#pragma unroll
        for (int i = 0; i < kQDB; ++i)
            om[i] = o[H0 + i] * f_own + *reinterpret_cast<const f32x4 *>(xo + ((partner * kQDB + i) * kWave + lane) * 4) * f_oth;
    };
    if (rh == 0) merge_half(std::integral_constant<int, 0>{});
    else merge_half(std::integral_constant<int, 1>{});
    const int b0 = (2 * dh + rh) * kQDB;      // this wave's quarter, as dim blocks

    if (a.n_chunks == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float *orow = a.out + (q * a.H + h0 + c) * (int64_t)kD + 16 * b0 + 4 * g;
#pragma unroll
        for (int b = 0; b < kQDB; ++b) *reinterpret_cast<f32x4 *>(orow + 16 * b) = om[b] * inv;
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
    const uint32_t o_off = 4 * (2 * kWH + (b0 * kWave + lane) * 4);   // + b * 1 KiB
    if (wave == 0 && g == 0) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_run), rec_rs, rec0 + 4 * c, 0, kSc1);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_tot), rec_rs, rec0 + 4 * (kWH + c), 0, kSc1);
    }
#pragma unroll
    for (int b = 0; b < kQDB; ++b)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, om[b]), rec_rs, rec0 + o_off + b * 1024, 0, kSc1);
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

bool attn_dq_merge_apply(const AttnPlan &p, int64_t list_stride) {
    return p.dq && p.n_steps <= kDqMaxChunkSteps && list_stride <= kDqMergeMax;
}

hipError_t launch_attn_dq_merge(const AttnPlan &p, int U, int T, int H, int W, int64_t N, int K, const void *q,
                                int q_bf16, const int64_t *q_pos, double theta, const uint16_t *raw, const void *comp,
                                const float *comp_scale, const CandList &cl, const int32_t *cand_nvis,
                                const int32_t *raw_vis, float scale, int32_t *idx_out, float *out, uint32_t *count,
                                float *part, hipStream_t stream)
{
    if (!attn_dq_merge_apply(p, cl.stride) || cl.n_levels < 1 || cl.n_levels > kMaxLevels) return hipErrorInvalidValue;
    const bool e8 = comp_scale != nullptr && N > 0;
    using Fn = void (*)(AttnArgs);
    const int variant = (q_bf16 ? 1 : 0) + (e8 ? 2 : 0);
    static const Fn kernels[4] = {attn_dq_kernel<true, false, false, true>, attn_dq_kernel<false, false, false, true>,
                                  attn_dq_kernel<true, false, true, true>, attn_dq_kernel<false, false, true, true>};
    static std::once_flag attr_once[4];
    static hipError_t attr_err[4];
    const Fn fn = kernels[variant];
    std::call_once(attr_once[variant], [&] {
        attr_err[variant] = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                                e8 ? kDqMaxLds<true> : kDqMaxLds<false>);
    });
    if (attr_err[variant] != hipSuccess) return attr_err[variant];
    const int lds = (e8 ? kDqRowTabOff<true> : kDqRowTabOff<false>) + 4 * kSR * p.n_steps;   // the whole union's rows
    AttnArgs a = {};
    a.T = T; a.H = H; a.W = W; a.K = K; a.n_hg = p.n_hg; a.n_chunks = p.n_chunks;
    a.steps_per_chunk = p.steps_per_chunk; a.n_steps = p.n_steps;
    a.n_items = (int)((int64_t)U * T * p.n_hg * p.n_chunks);
    a.N = N;
    a.q = q; a.pos = q_pos; a.raw = raw; a.comp = comp;
    a.comp_scale = e8 ? comp_scale : nullptr;
    a.raw_vis = W > 0 ? raw_vis : nullptr;
    a.scale = scale; a.out = out;
    a.log2_theta = log2(theta);
    a.cand_keys = cl.keys; a.cand_ids = cl.ids; a.cand_stride = cl.stride; a.cand_nvis = cand_nvis;
    a.idx_out = idx_out;
    a.count = count;
    a.part = part;
    a.lv_n = cl.n_levels;
    for (int l = 0; l < cl.n_levels; ++l) a.lv_ch[l] = cl.level_rows[l];
    hipLaunchKernelGGL(fn, dim3((unsigned)p.blocks), dim3(kDqT), lds, stream, a);
    return hipGetLastError();
}

}  // namespace ds4a
