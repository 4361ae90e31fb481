// attn.hip — A3..A6: query-tail RoPE and multi-query attention over the raw window plus
// the selected compressed rows, one softmax over the union.
//
// "Reading the architecture of DwarfStar (ds4.c), part 1/8" (Qiita):
//  * section 2: the query heads (64, Pro 128) share ONE KV head of 512 dims; RoPE covers
//    only the last n_rot = 64 dims;
//  * section 3: recent tokens stay exact in a raw sliding window (128 rows, f16-rounded,
//    section 3-1); older ones live as compressed rows, of which the indexer's top-k reach
//    the attention (section 3-3);
//  * section 3-2: compressed rows are rotated ("tail RoPE") when emitted, so stored rows are
//    already rotated and only the query is rotated here.
// Readings: each stored row is both key and value; the union is raw rows then selected
// rows, not de-duplicated; RoPE pairs are adjacent dims.
//
// Design.  A workgroup owns one query, a group of 64 heads and a contiguous chunk of the
// union, cut into 32-row steps.  Wave w owns heads 16w..16w+15 over all 512 dims, so the QK
// of a wave needs no other wave's partial sums, and each wave keeps its own online softmax.
// The four waves share the rows: an LDS ring of kNB steps, filled straight from memory
// (buffer_load_dwordx4 ... lds, one row per instruction, no VGPRs; each wave loads 8 rows of a
// step) kNB-1 steps ahead of use, with one barrier per step.  So each row is read once for
// 64 heads.  Per step a wave
//   - QK: L^T[32 rows x 16 heads] over 512 dims, two 16-row halves of 16 k-steps of
//     v_mfma_f32_16x16x32 with the rows as A (from LDS) and the rotated query as B (held in
//     VGPRs for the whole chunk); lane (g, c) ends with rows 4g..4g+3 of each half, head c;
//   - softmax: online, fp32, in log2 units;
//   - PV: O^T[512 dims x 16 heads] += V^T P^T in 64 MFMAs.  P is carried as a hi + lo pair:
//     one MFMA takes the hi parts of the lane's 8 rows (k = 8g..8g+3: rows 4g..4g+3 of the
//     first half, k = 8g+4..8g+7: the same rows of the second half), a second one the lo
//     parts, and both read the same V^T fragment: two ds_read_b64_tr_b16 (one per half) give
//     it, and P needs no cross-lane move.
// The step loop is software-pipelined: while the matrix core runs PV of step j, the wave
// reads step j+1's rows for QK(j+1) (issued in the same stretch) and, as each V^T fragment of
// step j is consumed, reads step j+1's fragment into its registers.  The softmax of step j+1
// then overlaps the tail of those reads.
// When a query's union is split over several workgroups (few queries per call), each wave
// writes its (reference, sum, O) record; the last wave to arrive for a (query, 16-head group),
// counted with a device-scope atomic, merges the records by log-sum-exp and resets the
// counter to zero.  No second launch.
// Chunks of one query are dealt to one XCD (workgroups go to the 8 XCDs round-robin), so the
// rows two head groups share tend to stay in that XCD's L2.
//
// Precision: rows are used in their stored type, so compressed rows go through the bf16 MFMA
// and raw rows through the f16 MFMA with no conversion of row data.  Operands not already of
// that type are carried as hi + lo pairs of it: the query (all dims of an f32 query, the
// rotated tail of a bf16 one) and P.  Raw steps come first, so the query is first held as an
// f16 pair, then (once) re-split as a bf16 pair.
// Compressed rows stored as FP8 (E4M3 codes plus one f32 scale per row) arrive as codes, with
// their scales, in the step's ring slot; before the step is used each wave widens its 8 rows
// to bf16 (exact) in place.  The row scale multiplies the row's logit and, for PV, its
// probability.
#include "attn_common.hpp"
#include "launch.hpp"
#include "rope.hpp"

#include <math.h>
#include <mutex>

namespace ds4a {

namespace {

constexpr int kGH = kAW * kWH;                // heads per workgroup (64)
constexpr int kNB = 4;                        // ring slots
constexpr int kScaleOff = kNB * kBuf;
template <bool E8> constexpr int kAngOff = kScaleOff + (E8 ? kNB * kAW * kScaleWave : 0);  // [wave][32] (cos, sin) fp64
template <bool E8> constexpr int kMaskOff = kAngOff<E8> + kAW * 32 * 16;    // sparse: row validity per step
constexpr int kMaxChunkSteps = 96;            // (1024 + 2048) / 32: the largest sparse union
template <bool E8> constexpr int kRowTabOff = kMaskOff<E8> + 4 * kMaxChunkSteps;  // sparse: 4 B per union row
template <bool E8> constexpr int kMaxLds = kRowTabOff<E8> + 4 * kSR * kMaxChunkSteps;
static_assert(kMaxLds<false> <= 160 * 1024 && kMaxLds<true> <= 160 * 1024, "LDS of one workgroup");
static_assert(kMaxChunkSteps * kSR % kAT == 0, "row table fill");
constexpr int kRec = 2 * kWH + kWH * kD;      // split-union record of a wave: m[16], l[16], O[16][512]
constexpr float kRescale = 8.f;               // softmax reference moves when a logit exceeds it by this (log2 units)

// QF32: the query is f32 (every k-step carries a lo half), else bf16 (only the rotated tail,
// k-steps 14 and 15, does).  DENSE: the union is the raw window plus compressed rows
// 0 .. n_vis-1 (a.K = N), else the raw window plus idx's rows.  E8: compressed rows are E4M3
// codes with row scales (N >= 1).
template <bool QF32, bool DENSE, bool E8>
__global__ __launch_bounds__(kAT, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_kernel(AttnArgs a)
{
    constexpr int NB = kNB;
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *ring = smem;
    unsigned char *s_scale = smem + kScaleOff;
    double *s_ang = reinterpret_cast<double *>(smem + kAngOff<E8>);
    uint32_t *s_mask = reinterpret_cast<uint32_t *>(smem + kMaskOff<E8>);
    int32_t *s_row = reinterpret_cast<int32_t *>(smem + kRowTabOff<E8>);

    // Workgroup -> (item = (query, chunk), head group of 64).  Items are dealt so that the
    // chunks of a query (consecutive items) share an XCD (lin mod 8).
    const uint32_t lin = blockIdx.x;
    const uint32_t xcd = lin & 7u, r8 = lin >> 3;
    const uint32_t per_xcd = ((uint32_t)a.n_items + 7u) >> 3;          // items per XCD
    const uint32_t hg = r8 % (uint32_t)a.n_hg;
    const uint32_t item = xcd * per_xcd + r8 / (uint32_t)a.n_hg;
    if (r8 / (uint32_t)a.n_hg >= per_xcd || item >= (uint32_t)a.n_items) return;   // grid padding
    const uint32_t q32 = item / (uint32_t)a.n_chunks;
    const int chunk = (int)(item - q32 * (uint32_t)a.n_chunks);
    const uint32_t u32 = q32 / (uint32_t)a.T;
    const int64_t q = q32, u = u32, t = q32 - u32 * (uint32_t)a.T;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = lane >> 4, c = lane & 15;
    const int h0 = (int)hg * kGH + wave * kWH;                // this wave's first head
    const bool active = h0 < a.H;                             // H is a multiple of 16

    const int step0 = chunk * a.steps_per_chunk;
    const int step1 = step0 + a.steps_per_chunk < a.n_steps ? step0 + a.steps_per_chunk : a.n_steps;
    const int n = step1 - step0;                              // steps of this chunk (>= 1)
    const int rho0 = step0 * kSR;
    const int raw_steps = a.W / kSR;                          // W is a multiple of 32
    const int n_raw = step0 < raw_steps ? min(raw_steps - step0, n) : 0;   // raw steps come first

    const uint16_t *raw_q = a.raw + (u * (int64_t)(a.T + a.W - 1) + t) * kD;
    constexpr int kCompRowBytes = E8 ? kCodeRow : 2 * kD;
    const unsigned char *comp_u = static_cast<const unsigned char *>(a.comp) + u * a.N * kCompRowBytes;
    const float *cscale_u = E8 ? a.comp_scale + u * a.N : nullptr;
    const int raw_lim = a.raw_vis ? (int)clamp_nvis(a.raw_vis, q, a.W) : a.W;
    const int64_t j_lim = DENSE ? clamp_nvis(a.n_vis, q, a.N) : a.N;

    // Buffer resources over the query's raw window (its first raw_lim rows) and the unit's
    // compressed rows (and their E4M3 scales): a row that takes no part is an offset past the
    // end, which reads as zeros.
    const __amdgpu_buffer_rsrc_t raw_rs = rsrc(raw_q, (uint32_t)raw_lim * (2 * kD));
    const __amdgpu_buffer_rsrc_t comp_rs = rsrc(comp_u, (uint32_t)((uint64_t)a.N * kCompRowBytes));
    const __amdgpu_buffer_rsrc_t scale_rs = rsrc(cscale_u, E8 ? (uint32_t)a.N * 4u : 0u);

    // Loads of local step j into ring slot j % NB.  Raw step: this wave's 8 rows, 1 KiB each.
    // Compressed step: bf16 rows likewise; E4M3 rows as codes, two rows per instruction, packed
    // at the start of the slot, plus the rows' scales.  Steps past the chunk load zeros, so the
    // count of loads per step depends only on its kind.
    auto issue_raw = [&](int j) __attribute__((always_inline)) {
        const int R0 = (step0 + j) * kSR + wave * kRW;
        const uint32_t dst = lds_addr(ring + (j % NB) * kBuf + wave * kRW * kRowStride);
#pragma unroll
        for (int e = 0; e < kRW; ++e) {
            const int r = wave * kRW + e;                     // row within the step
            dma16(dst + e * kRowStride, ((uint32_t)(R0 + e) << 10) + ((uint32_t)(lane ^ ((r >> 2) & 1)) << 4), raw_rs);
        }
    };
    auto issue_comp = [&](int j, const i32x4 &e0, const i32x4 &e1) __attribute__((always_inline)) {
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
            const int l8 = lane & 7;                          // lane l: the scale of row l % 8
            const int32_t es = l8 < 4 ? e0[l8 & 3] : e1[l8 & 3];
            dma4(lds_addr(s_scale + (slot * kAW + wave) * kScaleWave), (uint32_t)es << 2, scale_rs);
        }
    };
    // This wave's 8 row entries of local step j (compressed row, or -1): from the row table
    // (sparse) or from the position (dense).  Raw steps and steps past the chunk have none.
    auto entries = [&](int j, i32x4 &e0, i32x4 &e1) __attribute__((always_inline)) {
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
            e0[r] = (int64_t)(rho + r - a.W) < j_lim ? rho + r - a.W : -1;
            e1[r] = (int64_t)(rho + 4 + r - a.W) < j_lim ? rho + 4 + r - a.W : -1;
        }
    };

    // ---- set-up.  Raw steps need no index: their loads go out first.  Then the index entries
    // and the query are loaded, the row table is built, and the first compressed steps' loads go.
#pragma unroll
    for (int j = 0; j < NB - 2; ++j)
        if (j < n_raw) issue_raw(j);

    constexpr int kPer = kMaxChunkSteps * kSR / kAT;          // index entries per thread (12)
    int32_t v_idx[kPer];
    if (!DENSE) {
        const int32_t *idx_q = a.idx + q * (int64_t)a.K;
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int i = tid + r * kAT, k = rho0 + i - a.W;
            v_idx[r] = (i < n * kSR && k >= 0 && k < a.K) ? idx_q[k] : -1;
        }
    }
    float qv[kKs][8];
    {
        const int hq = active ? h0 + c : a.H - 1;             // an idle wave reads a valid head
        const int64_t off = (q * a.H + hq) * (int64_t)kD + 8 * g;
#pragma unroll
        for (int s = 0; s < kKs; ++s) {
            if (QF32) {
                const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(a.q) + off + 32 * s);
                const float4 x0 = p[0], x1 = p[1];
                qv[s][0] = x0.x; qv[s][1] = x0.y; qv[s][2] = x0.z; qv[s][3] = x0.w;
                qv[s][4] = x1.x; qv[s][5] = x1.y; qv[s][6] = x1.z; qv[s][7] = x1.w;
            } else {
                const u32x4 x = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.q) + off + 32 * s);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    qv[s][2 * i] = bf16_bits_to_f32(x[i] & 0xFFFFu);
                    qv[s][2 * i + 1] = bf16_bits_to_f32(x[i] >> 16);
                }
            }
        }
    }
    const int64_t pos = a.pos[q];
    if (!DENSE) {
        // Row table: compressed union row (local index i = rho - rho0) -> its row j, or -1 (a -1
        // or out-of-range index, or past K).  Validity mask of each step: bit r is row r of the
        // step (raw rows: below raw_lim).  One ballot covers 64 rows, i.e. two steps.
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
    __syncthreads();                          // row table
#pragma unroll
    for (int j = 0; j < NB - 2; ++j)
        if (j >= n_raw) {
            i32x4 e0, e1;
            entries(j, e0, e1);
            issue_comp(j, e0, e1);
        }
    i32x4 ent_a, ent_b;                       // entries of the next step to issue (NB - 2)
    entries(NB - 2, ent_a, ent_b);

    double *w_ang = s_ang + wave * 64;        // this wave's copy of the 32 tail angles
    if (lane < kRot / 2) {
        double cs, sn;
        rope_angle(a.log2_theta, lane, pos, cs, sn);
        w_ang[2 * lane] = cs;
        w_ang[2 * lane + 1] = sn;
    }
    // Rotated tail: k-steps 14, 15 hold dims 448 + 32(s-14) + 8g + e, pair 16(s-14) + 4g + e/2;
    // rotation in fp64 rounded once to f32 (rope.hpp, as the compressor rotates its rows).
#pragma unroll
    for (int s = kKs - 2; s < kKs; ++s)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const int pr = 16 * (s - (kKs - 2)) + 4 * g + e / 2;
            rope_rotate(w_ang[2 * pr], w_ang[2 * pr + 1], qv[s][e], qv[s][e + 1]);
        }
    // Query fragments: f16 pair while the steps are raw, bf16 pair after.  A bf16 query needs
    // a lo part only in its rotated tail (k-steps 14, 15); elsewhere its f16 hi is exact (a bf16
    // value below the f16 normal range loses bits under 2^-24, far below the other roundings).
    u32x4 qh[kKs], ql[kKs];
#pragma unroll
    for (int s = 0; s < kKs; ++s) {
        if (!QF32 && s < kKs - 2) {
            ql[s] = u32x4{0u, 0u, 0u, 0u};    // never read
            if (n_raw > 0) {
                f16x8 h;
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = (_Float16)qv[s][e];
                qh[s] = __builtin_bit_cast(u32x4, h);
            } else {
                qh[s] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.q) +
                                                          (q * a.H + (active ? h0 + c : a.H - 1)) * (int64_t)kD + 8 * g + 32 * s);
            }
        } else if (n_raw > 0) {
            split8<true>(qv[s], qh[s], ql[s]);
        } else {
            split8<false>(qv[s], qh[s], ql[s]);
        }
    }
    // At the switch to compressed steps: the f16 pair holds q to ~22 bits, so the bf16 pair
    // made from hi + lo is as good as one made from q (about 16 bits); a bf16 query's
    // unrotated dims are its own bits again, read back from memory.
    auto to_bf16_pair = [&]() __attribute__((always_inline)) {
        const uint16_t *qrow = static_cast<const uint16_t *>(a.q) + (q * a.H + (active ? h0 + c : a.H - 1)) * (int64_t)kD + 8 * g;
#pragma unroll
        for (int s = 0; s < kKs; ++s) {
            if (!QF32 && s < kKs - 2) {
                qh[s] = *reinterpret_cast<const u32x4 *>(qrow + 32 * s);
                continue;
            }
            const f16x8 h = as_f16x8(qh[s]), l = as_f16x8(ql[s]);
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = (float)h[e] + (float)l[e];
            split8<false>(x, qh[s], ql[s]);
        }
    };

    const float scale2 = a.scale * kLog2e;    // logits in log2 units
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[kDB];
#pragma unroll
    for (int b = 0; b < kDB; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // LDS addresses within a half step: QK reads row c, chunk 4s + g (swizzle bit (c >> 2) & 1
    // flips g's low bit); PV transposed reads: lane (g, c) points at row 4g + c/4, dims
    // 16b + 4(c%4): chunk 2b + ((c >> 1) & 1), whose swizzle bit is g & 1.
    const int qk_base = c * kRowStride + ((g ^ ((c >> 2) & 1)) << 4);
    const int pv_base = (4 * g + (c >> 2)) * kRowStride + ((((c >> 1) & 1) ^ (g & 1)) << 4) + (c & 1) * 8;

    // Validity of the 32 rows of local step j (uniform): bit r is row r.
    auto step_mask = [&](int j) __attribute__((always_inline)) -> uint32_t {
        if (!DENSE) return s_mask[j];
        const int rho = (step0 + j) * kSR;
        const int64_t lim = j < n_raw ? (int64_t)raw_lim : j_lim + a.W;   // rows below lim take part
        const int64_t cnt = lim - rho;
        return cnt >= kSR ? 0xFFFFFFFFu : (cnt <= 0 ? 0u : (1u << (uint32_t)cnt) - 1u);
    };

    f32x4 acc[2][2];                          // QK accumulators [half][k-step parity]
    float lg[8], rsc[8];                      // the lane's logits and row scales (rows 4g+e, 16+4g+e)

    // V^T fragment of dims 16b..16b+15 of the step at tb: .xy rows 4g..4g+3 of the first half,
    // .zw those of the second.
    auto tr = [&](const unsigned char *tb, int b) __attribute__((always_inline)) -> u32x4 {
        const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(tb + 32 * b));
        const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr16(tb + kHalfBuf + 32 * b));
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    // Softmax of step j, first part: logits, their maximum, and the reference move (with the
    // rescale of O and the sum) if one is due.  E4M3 compressed steps read their row scales.
    auto sm1 = [&](auto f16_tag, int j, uint32_t mask) __attribute__((always_inline)) {
        constexpr bool F16 = decltype(f16_tag)::value;
#pragma unroll
        for (int e = 0; e < 8; ++e) rsc[e] = 1.f;
        if (E8 && !F16) {
            const unsigned char *sb = s_scale + (j % NB) * kAW * kScaleWave + 16 * (g & 1);
            const f32x4 s0 = *reinterpret_cast<const f32x4 *>(sb + (g >> 1) * kScaleWave);
            const f32x4 s1 = *reinterpret_cast<const f32x4 *>(sb + (2 + (g >> 1)) * kScaleWave);
#pragma unroll
            for (int e = 0; e < 4; ++e) { rsc[e] = s0[e]; rsc[4 + e] = s1[e]; }
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int h = e >> 2, i = e & 3;
            const float l = (acc[h][0][i] + acc[h][1][i]) * scale2 * rsc[e];
            lg[e] = (mask >> (16 * h + 4 * g + i)) & 1u ? l : -INFINITY;
            tmax = fmaxf(tmax, lg[e]);
        }
        tmax = max_g(tmax);
        // m_run is a reference, not always the running maximum: it moves (and O and the sum are
        // rescaled) only when some head of the wave sees a logit more than kRescale above it,
        // so every exponent stays below 2^kRescale; the result does not depend on the reference.
        const float m_new = fmaxf(m_run, tmax);
        if (__builtin_amdgcn_ballot_w64(m_new > m_run + kRescale)) {   // also the first visible row
            const float alpha = exp2f(m_run - m_new);                  // 0 while nothing was visible
            l_run *= alpha;
#pragma unroll
            for (int b = 0; b < kDB; ++b) o[b] *= alpha;
            m_run = m_new;
        }
    };
    // Second part: probabilities, the sum, and P^T as a hi + lo pair (k = 8g + e: e < 4 rows
    // 4g + e of the first half, e >= 4 rows 4g + e - 4 of the second).  Terms below 2^-126 of
    // the reference flush to zero.
    auto sm2 = [&](auto f16_tag, u32x4 &ph, u32x4 &pl) __attribute__((always_inline)) {
        constexpr bool F16 = decltype(f16_tag)::value;
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(lg[e] - m_use);
            l_run += p;
            pv[e] = p * rsc[e];
        }
        split8<F16>(pv, ph, pl);
    };
    // One pass over the matrix core: PV of step jp (its V^T fragments read from LDS as they are
    // needed) and QK of step jq, interleaved in 16 slices (QK k-step i; PV dim blocks 2i, 2i+1),
    // with each slice's LDS reads issued two slices ahead.
    auto mfma_pass = [&](auto fp, auto fq, auto has_pv, auto has_qk, int jp, int jq,
                         const u32x4 &ph, const u32x4 &pl) __attribute__((always_inline)) {
        constexpr bool FP = decltype(fp)::value, FQ = decltype(fq)::value;
        constexpr bool PV = decltype(has_pv)::value, QK = decltype(has_qk)::value;
        constexpr int kAhead = 2;
        const unsigned char *tq = ring + (jq % NB) * kBuf + qk_base;
        const unsigned char *tp = ring + (jp % NB) * kBuf + pv_base;
        if (QK) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int p = 0; p < 2; ++p) acc[h][p] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        u32x4 xq[kKs][2], xv[kKs][2];
        auto load = [&](int i) __attribute__((always_inline)) {
            if (QK) {
                xq[i][0] = *reinterpret_cast<const u32x4 *>(tq + 64 * i);
                xq[i][1] = *reinterpret_cast<const u32x4 *>(tq + kHalfBuf + 64 * i);
            }
            if (PV) {
                xv[i][0] = tr(tp, 2 * i);
                xv[i][1] = tr(tp, 2 * i + 1);
            }
        };
#pragma unroll
        for (int i = 0; i < kAhead; ++i) load(i);
#pragma unroll
        for (int i = 0; i < kKs; ++i) {
            if (i + kAhead < kKs) load(i + kAhead);
            const int p = i & 1;
            if (QK) {
                acc[0][p] = mma<FQ>(xq[i][0], qh[i], acc[0][p]);
                acc[1][p] = mma<FQ>(xq[i][1], qh[i], acc[1][p]);
            }
            if (PV) {
                o[2 * i] = mma<FP>(xv[i][0], ph, o[2 * i]);
                o[2 * i + 1] = mma<FP>(xv[i][1], ph, o[2 * i + 1]);
            }
            if (QK && (QF32 || i >= kKs - 2)) {
                acc[0][p] = mma<FQ>(xq[i][0], ql[i], acc[0][p]);
                acc[1][p] = mma<FQ>(xq[i][1], ql[i], acc[1][p]);
            }
            if (PV) {
                o[2 * i] = mma<FP>(xv[i][0], pl, o[2 * i]);
                o[2 * i + 1] = mma<FP>(xv[i][1], pl, o[2 * i + 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Step j+1 may start: this wave's loads of it have landed (E4M3 compressed steps: the
    // workgroup widens it in place), and the barrier publishes everyone's.  Every wave has
    // finished step j-1 by then, so its slot takes step j + NB - 1's loads.
    auto advance = [&](int j) __attribute__((always_inline)) {
        if (!E8) {
            wait_vm<kRW *(NB - 3)>();
        } else {                              // loads issued after step j+1's: step j+2
            if (j + 2 < n_raw) wait_vm<kRW *(NB - 3)>();
            else wait_vm<kCodeBatch *(NB - 3)>();
        }
        wait_lds();
        if (E8 && j + 1 >= n_raw && j + 1 < n) {
            // widen in place: each wave reads its 8 code rows, then (after a barrier, as the
            // bf16 rows overlap other waves' codes) writes them as bf16 rows
            unsigned char *sb = ring + ((j + 1) % NB) * kBuf;
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
        __syncthreads();
        const int jn = j + NB - 1;
        if (jn < n_raw) issue_raw(jn);
        else issue_comp(jn, ent_a, ent_b);
        entries(jn + 1, ent_a, ent_b);
    };

    // ---- the pipeline.  Step j computes from ring slot j % NB while later steps load.  Raw
    // steps come first, then compressed ones; each loop holds one instance of each phase.
    advance(-1);                              // step 0 landed (E4M3: widened), step NB-2 loading
    uint32_t mask_next = 0;
    const u32x4 z4 = u32x4{0u, 0u, 0u, 0u};
    if (active) {
        mask_next = step_mask(0);
        if (n_raw > 0) mfma_pass(F16T{}, F16T{}, std::false_type{}, std::true_type{}, 0, 0, z4, z4);
        else mfma_pass(BF16T{}, BF16T{}, std::false_type{}, std::true_type{}, 0, 0, z4, z4);
    }
    auto body = [&](auto fj, auto fn, int j) __attribute__((always_inline)) {
        constexpr bool FJ = decltype(fj)::value, FN = decltype(fn)::value;
        const uint32_t mask = mask_next;
        if (active) sm1(fj, j, mask);
        advance(j);
        if (FJ && !FN) to_bf16_pair();
        if (active) {
            mask_next = step_mask(j + 1);
            u32x4 ph, pl;
            sm2(fj, ph, pl);
            mfma_pass(fj, fn, std::true_type{}, std::true_type{}, j, j + 1, ph, pl);
        }
    };
    auto last = [&](auto fj, int j) __attribute__((always_inline)) {
        if (active) {
            sm1(fj, j, mask_next);
            u32x4 ph, pl;
            sm2(fj, ph, pl);
            mfma_pass(fj, fj, std::true_type{}, std::false_type{}, j, j, ph, pl);
        }
    };
    int j = 0;
    for (; j + 1 < n_raw; ++j) body(F16T{}, F16T{}, j);
    if (j + 1 == n_raw && j + 1 < n) {        // the last raw step, a compressed one after it
        body(F16T{}, BF16T{}, j);
        ++j;
    }
    for (; j + 1 < n; ++j) body(BF16T{}, BF16T{}, j);
    if (j < n_raw) last(F16T{}, j);
    else last(BF16T{}, j);
    wait_vm<0>();                             // no load may land in LDS after the workgroup ends

    if (!active) return;
    l_run = sum_g(l_run);
    if (a.n_chunks == 1) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float *orow = a.out + (q * a.H + h0 + c) * (int64_t)kD + 4 * g;
#pragma unroll
        for (int b = 0; b < kDB; ++b) *reinterpret_cast<f32x4 *>(orow + 16 * b) = o[b] * inv;
        return;
    }
    // ---- split union: this wave's record, then the last wave of the (query, head group) merges.
    // Records and counters are accessed with agent-scope coherence on every access (sc1, as the
    // memory model does for relaxed device-scope atomics), and each wave's record stores have
    // completed before its count is added, so no cache-wide write-back or invalidate is needed.
    const int n_h16 = a.H / kWH;
    const int64_t grp = q * n_h16 + h0 / kWH;
    constexpr int kSc1 = 16;                  // cache policy: sc1
    const int nc = a.n_chunks;
    const __amdgpu_buffer_rsrc_t rec_rs = rsrc(a.part + grp * nc * (int64_t)kRec, (uint32_t)(nc * kRec * 4));
    const uint32_t rec0 = (uint32_t)(chunk * kRec * 4);  // this chunk's record (bytes)
    if (g == 0) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_run), rec_rs, rec0 + 4 * c, 0, kSc1);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_run), rec_rs, rec0 + 4 * (kWH + c), 0, kSc1);
    }
#pragma unroll
    for (int b = 0; b < kDB; ++b)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[b]), rec_rs,
                                               rec0 + 4 * (2 * kWH + c * kD + 16 * b + 4 * g), 0, kSc1);
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");   // the record is written before it is counted
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(a.count + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != (uint32_t)nc - 1) return;
    asm volatile("" : : : "memory");          // the reads below follow the count
    // lane l: head l / 4, dims 128 (l % 4) .. +127.  Reads past the last record return zeros.
    const int hh = lane >> 2, d0 = (lane & 3) * 128;
    float M = -INFINITY;
    for (int c0 = 0; c0 < nc; c0 += 8) {
        float mv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            mv[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rec_rs, ((c0 + i) * kRec + hh) * 4, 0, kSc1));
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (c0 + i < nc) M = fmaxf(M, mv[i]);
    }
    float L = 0.f;
    f32x4 sum[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) sum[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ch = 0; ch < nc; ch += 2) {      // two records per pass, all their loads in flight
        f32x4 x0[32], x1[32];
        const uint32_t r0 = (uint32_t)(ch * kRec * 4), r1 = r0 + kRec * 4;
        const float m0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rec_rs, r0 + hh * 4, 0, kSc1));
        const float l0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rec_rs, r0 + (kWH + hh) * 4, 0, kSc1));
        const float m1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rec_rs, r1 + hh * 4, 0, kSc1));
        const float l1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rec_rs, r1 + (kWH + hh) * 4, 0, kSc1));
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            x0[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                        rec_rs, r0 + 4 * (2 * kWH + hh * kD + d0 + 4 * k), 0, kSc1));
            x1[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                        rec_rs, r1 + 4 * (2 * kWH + hh * kD + d0 + 4 * k), 0, kSc1));
        }
        // a chunk with no visible row (reference -inf), or past the last, weighs 0
        const float w0 = m0 == -INFINITY ? 0.f : exp2f(m0 - M);
        const float w1 = (ch + 1 >= nc || m1 == -INFINITY) ? 0.f : exp2f(m1 - M);
        L += w0 * l0 + w1 * l1;
#pragma unroll
        for (int k = 0; k < 32; ++k) sum[k] += w0 * x0[k] + w1 * x1[k];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    f32x4 *dst = reinterpret_cast<f32x4 *>(a.out + (q * a.H + h0 + hh) * (int64_t)kD + d0);
#pragma unroll
    for (int k = 0; k < 32; ++k) dst[k] = sum[k] * inv;
    if (lane == 0) __hip_atomic_store(a.count + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // ready for the next call
}

}  // namespace

AttnPlan plan_attn(int U, int T, int H, int W, int K) {
    // Few (query, 64-head group) items: the 16-head kernel fills the chip without splitting
    // the union (or with fewer, smaller records).
    if ((int64_t)U * T * ((H + kGH - 1) / kGH) < 192) return plan_attn_dq(U, T, H, W, K);
    return plan_attn_wide(U, T, H, W, K);
}

AttnPlan plan_attn_wide(int U, int T, int H, int W, int K) {
    AttnPlan p;
    p.n_hg = (H + kGH - 1) / kGH;
    p.n_steps = (W + K + kSR - 1) / kSR;
    const int64_t Q = (int64_t)U * T;
    const int64_t items = Q * p.n_hg;
    // One workgroup per CU (LDS).  Split the union only when (query, head group) pairs are too
    // few to give most CUs one, keeping at least 2 steps per chunk; dense unions longer than the
    // row table are split too.
    int64_t want = items >= 192 ? 1 : 256 / items;
    const int64_t max_split = p.n_steps / 2 > 1 ? p.n_steps / 2 : 1;
    if (want > max_split) want = max_split;
    const int64_t need = (p.n_steps + kMaxChunkSteps - 1) / kMaxChunkSteps;
    if (want < need) want = need;
    if (want < 1) want = 1;
    p.steps_per_chunk = (int)((p.n_steps + want - 1) / want);
    p.n_chunks = (p.n_steps + p.steps_per_chunk - 1) / p.steps_per_chunk;
    p.count_bytes = p.n_chunks > 1 ? (((size_t)Q * (size_t)(H / kWH) * 4 + 255) & ~(size_t)255) : 0;
    p.workspace_bytes =
        p.n_chunks > 1 ? p.count_bytes + sizeof(float) * (size_t)Q * (size_t)(H / kWH) * (size_t)p.n_chunks * kRec : 0;
    p.blocks = ((Q * p.n_chunks + 7) / 8) * 8 * p.n_hg;
    return p;
}

hipError_t launch_attn(int U, int T, int H, int W, int64_t N, int K, const void *q, int q_bf16,
                       const int64_t *q_pos, double theta, const uint16_t *raw, const void *comp,
                       const float *comp_scale, const int32_t *idx, const int32_t *n_vis, const int32_t *raw_vis,
                       float scale, float *out, void *workspace, hipStream_t stream)
{
    const AttnPlan p = plan_attn(U, T, H, W, K);
    uint32_t *count = static_cast<uint32_t *>(workspace);
    float *part = reinterpret_cast<float *>(static_cast<char *>(workspace) + p.count_bytes);
    if (p.dq)
        return launch_attn_dq(p, U, T, H, W, N, K, q, q_bf16, q_pos, theta, raw, comp, comp_scale, idx, n_vis,
                              raw_vis, scale, out, count, part, stream);
    return launch_attn_wide(p, U, T, H, W, N, K, q, q_bf16, q_pos, theta, raw, comp, comp_scale, idx, n_vis,
                            raw_vis, scale, out, count, part, stream);
}

hipError_t launch_attn_parts(int U, int T, int H, int W, int64_t N, int K, const void *q, int q_bf16,
                             const int64_t *q_pos, double theta, const uint16_t *raw, const void *comp,
                             const float *comp_scale, const int32_t *idx, const int32_t *n_vis, const int32_t *raw_vis,
                             float scale, float *out, uint32_t *count, float *part, hipStream_t stream)
{
    const AttnPlan p = plan_attn(U, T, H, W, K);
    if (p.dq)
        return launch_attn_dq(p, U, T, H, W, N, K, q, q_bf16, q_pos, theta, raw, comp, comp_scale, idx, n_vis,
                              raw_vis, scale, out, count, part, stream);
    return launch_attn_wide(p, U, T, H, W, N, K, q, q_bf16, q_pos, theta, raw, comp, comp_scale, idx, n_vis,
                            raw_vis, scale, out, count, part, stream);
}

hipError_t launch_attn_wide(const AttnPlan &p, int U, int T, int H, int W, int64_t N, int K, const void *q, int q_bf16,
                            const int64_t *q_pos, double theta, const uint16_t *raw, const void *comp,
                            const float *comp_scale, const int32_t *idx, const int32_t *n_vis, const int32_t *raw_vis,
                            float scale, float *out, uint32_t *count, float *part, hipStream_t stream)
{
    const bool dense = idx == nullptr;
    const bool e8 = comp_scale != nullptr && N > 0;
    using Fn = void (*)(AttnArgs);
    const int variant = (q_bf16 ? 1 : 0) + (dense ? 2 : 0) + (e8 ? 4 : 0);
    static const Fn kernels[8] = {attn_kernel<true, false, false>, attn_kernel<false, false, false>,
                                  attn_kernel<true, true, false>,  attn_kernel<false, true, false>,
                                  attn_kernel<true, false, true>,  attn_kernel<false, false, true>,
                                  attn_kernel<true, true, true>,   attn_kernel<false, true, true>};
    // Each variant's dynamic LDS limit is raised once, to the most any plan asks for, so
    // concurrent calls from several host threads never race on it.
    static std::once_flag attr_once[8];
    static hipError_t attr_err[8];
    const Fn fn = kernels[variant];
    std::call_once(attr_once[variant], [&] {
        attr_err[variant] = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                                e8 ? kMaxLds<true> : kMaxLds<false>);
    });
    if (attr_err[variant] != hipSuccess) return attr_err[variant];
    const int lds = (e8 ? kRowTabOff<true> : kRowTabOff<false>) + (dense ? 0 : 4 * kSR * p.steps_per_chunk);
    AttnArgs a = {};
    a.T = T; a.H = H; a.W = W; a.K = K; a.n_hg = p.n_hg; a.n_chunks = p.n_chunks;
    a.steps_per_chunk = p.steps_per_chunk; a.n_steps = p.n_steps;
    a.n_items = (int)((int64_t)U * T * p.n_chunks);
    a.N = N;
    a.q = q; a.pos = q_pos; a.raw = raw; a.comp = comp; a.idx = idx; a.n_vis = n_vis;
    a.comp_scale = e8 ? comp_scale : nullptr;
    a.raw_vis = W > 0 ? raw_vis : nullptr;
    a.scale = scale; a.out = out;
    a.count = count;
    a.part = part;
    a.log2_theta = log2(theta);
    hipLaunchKernelGGL(fn, dim3((unsigned)p.blocks), dim3(kAT), lds, stream, a);
    return hipGetLastError();
}

}  // namespace ds4a
