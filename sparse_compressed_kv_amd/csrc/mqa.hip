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
// Design.  A workgroup (4 waves) owns 16 heads of one query and a contiguous
// chunk of 32-row union tiles.  Wave w owns dims [128w, 128w+128):
//   QK  : partial logits L^T[32 rows x 16 heads] over its 128 dims with 16x16x32
//         MFMA tiles (A = rows from LDS, B = rotated query in VGPRs); the four
//         partials are summed through LDS in a fixed order;
//   softmax: online (running max / sum per head), fp32;
//   PV  : O^T[128 dims x 16 heads] += V^T * P^T; P^T is already in the
//         B-operand layout of the QK result; V^T fragments come from the same
//         LDS tile through ds_read_b64_tr_b16 (transposing 4 x 16 blocks).
// Each row format gets the MFMA of its own type, so rows are never converted:
// compressed rows are bf16 (v_mfma_f32_16x16x32_bf16), raw-window rows are f16
// (v_mfma_f32_16x16x32_f16).  What is not already in that type is carried as
// hi + lo pairs: the fp32 query (a bf16 query only in its rotated tail) and
// the probabilities.  LDS rows are 1056 bytes apart and their 16-byte
// chunks are XOR-swizzled by row bit 2, which keeps both the row reads of QK
// and the transposed reads of PV free of bank conflicts.  Tiles are
// double-buffered: the next tile's rows are fetched
// into VGPRs (1 KiB per wave instruction, row-contiguous) while the current
// tile computes.  When the union is split over several workgroups, each
// writes (max, sum, unnormalised O) and a merge kernel combines them by
// log-sum-exp.  Workgroup order is XCD-aware: the head groups that read the
// same rows are dispatched to the same XCD (same L2).
#include "common.hpp"
#include "launch.hpp"

#include <math.h>

namespace ds4a {

namespace {

constexpr int kThreads = 256;
constexpr int kHG = 16;                       // heads per workgroup
constexpr int kD = 512;
constexpr int kRot = 64;
constexpr int kTile = 32;                     // union rows per tile
constexpr int kRowStride = 1056;              // LDS bytes per row (1024 + 32)
constexpr int kTileBytes = kTile * kRowStride;
constexpr int kXchBytes = 4 * 2 * kWave * 16; // partial logits of 4 waves
constexpr int kLdsBytes = 2 * kTileBytes + kXchBytes;   // + 4 bytes per union row of the chunk (row table)
constexpr int kRec = 2 * kHG + kHG * kD;      // partial record: m[16], l[16], O[16][512]
constexpr int kXcd = 8;

// Byte offset of 16-byte chunk c (0..63) of tile row r, XOR-swizzled by row bit 2.
__device__ __forceinline__ int chunk_off(int r, int c) {
    return r * kRowStride + ((c ^ ((r >> 2) & 1)) << 4);
}

// Byte offset of element d (0..511) of tile row r.
__device__ __forceinline__ int elem_off(int r, int d) {
    return chunk_off(r, d >> 3) + ((d & 7) << 1);
}

struct MqaArgs {
    int T, H, W, K, n_hg, n_tiles, tiles_per_chunk, n_chunks;
    int64_t N, n_items;
    const void *q;
    int q_bf16;
    const int64_t *pos;
    const uint16_t *raw;
    const uint16_t *comp;
    const int32_t *idx;
    float scale;
    float *out;
    float *part;
    double inv_freq[kRot / 2];               // theta^(-2i/n_rot), computed on the host in fp64
};

// Rotate one adjacent pair of the query tail by pos * inv_freq (fp64), round once to f32.
// The angle (up to ~1e6 rad) is first reduced by a two-part 2*pi in fp64, so that sincos runs
// on |x| <= pi.
__device__ __forceinline__ void rope_pair(double inv_freq, int64_t pos, float &a, float &b) {
    const double ang = (double)pos * inv_freq;
    const double k = rint(ang * 0.15915494309189535);          // 1 / (2 pi)
    double red = fma(-k, 6.283185307179586, ang);              // 2 pi, high part
    red = fma(-k, 2.4492935982947064e-16, red);                // 2 pi, low part
    double sn, cs;
    sincos(red, &sn, &cs);
    const double x = (double)a, y = (double)b;
    a = (float)(x * cs - y * sn);
    b = (float)(x * sn + y * cs);
}

// Query dims [d, d+8) of head h of query q as f32, rotated where they fall in the tail.
__device__ __forceinline__ void load_q8(const MqaArgs &a, int64_t q, int h, int d, float (&v)[8]) {
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
    if (d >= kD - kRot) {
        const int64_t pos = a.pos[q];
#pragma unroll
        for (int e = 0; e < 8; e += 2) rope_pair(a.inv_freq[(d + e - (kD - kRot)) >> 1], pos, v[e], v[e + 1]);
    }
}

__global__ __launch_bounds__(kThreads) void sparse_mqa_kernel(MqaArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *tiles = smem;
    f32x4 *xch = reinterpret_cast<f32x4 *>(smem + 2 * kTileBytes);
    int32_t *s_row = reinterpret_cast<int32_t *>(smem + kLdsBytes);   // per union row: comp row, -2 raw, -1 none

    // XCD-aware block order: all head groups of one (query, chunk) share an XCD.
    const int lin = blockIdx.x;
    const int k8 = lin / kXcd;
    const int hg = k8 % a.n_hg;
    const int64_t item = (int64_t)(k8 / a.n_hg) * kXcd + (lin % kXcd);
    if (item >= a.n_items) return;
    const int64_t q = item / a.n_chunks;
    const int chunk = (int)(item % a.n_chunks);
    const int64_t u = q / a.T, t = q % a.T;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int g = lane >> 4, c = lane & 15;
    const int h0 = hg * kHG;
    const int tile0 = chunk * a.tiles_per_chunk;
    const int tile1 = tile0 + a.tiles_per_chunk < a.n_tiles ? tile0 + a.tiles_per_chunk : a.n_tiles;

    const uint16_t *raw_q = a.raw + (u * (int64_t)(a.T + a.W - 1) + t) * kD;
    const uint16_t *comp_u = a.comp + u * a.N * kD;
    const int32_t *idx_q = a.idx + q * (int64_t)a.K;

    // Row table of this chunk's union rows, read once from idx.
    const int rho0 = tile0 * kTile;
    const int n_rows = (tile1 - tile0) * kTile;
    for (int r = tid; r < n_rows; r += kThreads) {
        const int rho = rho0 + r;
        int32_t v = -1;
        if (rho < a.W) {
            v = -2;
        } else if (rho - a.W < a.K) {
            const int32_t j = idx_q[rho - a.W];
            if (j >= 0 && (int64_t)j < a.N) v = j;
        }
        s_row[r] = v;
    }
    __syncthreads();

    auto row_ptr = [&](int rho) -> const uint16_t * {
        const int32_t v = s_row[rho - rho0];
        if (v == -2) return raw_q + (int64_t)rho * kD;
        if (v < 0) return nullptr;
        return comp_u + (int64_t)v * kD;
    };

    // Wave w stages rows w + 4i (i = 0..7) of a tile; lane = 16-byte chunk of the row.
    u32x4 stage[8];
    auto load_tile = [&](int tt) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint16_t *p = row_ptr(tt * kTile + wave + 4 * i);
            stage[i] = p ? reinterpret_cast<const u32x4 *>(p)[lane] : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_tile = [&](int buf) {
        unsigned char *base = tiles + buf * kTileBytes;
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4 *>(base + chunk_off(wave + 4 * i, lane)) = stage[i];
    };
    if (tile0 < tile1) load_tile(tile0);

    // Rotated query as B fragments while the first tile is in flight: k-step s <-> dims
    // 128*wave + 32s + 8g + (0..7) of head h0 + c; bf16 pair for compressed rows, f16 pair for
    // raw rows.  The lo halves are zero (and skipped) for a bf16 query outside the rotated tail.
    bf16x8 qb_hi[4], qb_lo[4];
    f16x8 qh_hi[4], qh_lo[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        float v[8];
        load_q8(a, q, h0 + c, 128 * wave + 32 * s + 8 * g, v);
        pack_hi_lo8(v, qb_hi[s], qb_lo[s]);
        pack_hi_lo8_f16(v, qh_hi[s], qh_lo[s]);
    }
    const bool lo_tail = !a.q_bf16 || wave == 3;      // dims 448..511 belong to wave 3 (s = 2, 3)

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (tile0 < tile1) store_tile(0);
    __syncthreads();

    for (int tt = tile0; tt < tile1; ++tt) {
        const int buf = (tt - tile0) & 1;
        const bool has_next = tt + 1 < tile1;
        if (has_next) load_tile(tt + 1);
        const unsigned char *tb = tiles + buf * kTileBytes;
        const bool is_raw = tt * kTile < a.W;

        // ---- QK: partial logits over this wave's dims
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32x4 x = *reinterpret_cast<const u32x4 *>(tb + chunk_off(16 * rt + c, 16 * wave + 4 * s + g));
                const bool lo = !a.q_bf16 || (lo_tail && s >= 2);
                if (!is_raw) {
                    acc = mfma16(as_bf16x8(x), qb_hi[s], acc);
                    if (lo) acc = mfma16(as_bf16x8(x), qb_lo[s], acc);
                } else {
                    acc = mfma16h(as_f16x8(x), qh_hi[s], acc);
                    if (lo) acc = mfma16h(as_f16x8(x), qh_lo[s], acc);
                }
            }
            xch[(wave * 2 + rt) * kWave + lane] = acc;
        }
        __syncthreads();

        // ---- full logits (same fixed summation order in every wave), mask, online softmax
        float p[2][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const f32x4 s0 = xch[(0 * 2 + rt) * kWave + lane], s1 = xch[(1 * 2 + rt) * kWave + lane];
            const f32x4 s2 = xch[(2 * 2 + rt) * kWave + lane], s3 = xch[(3 * 2 + rt) * kWave + lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rho = tt * kTile + 16 * rt + 4 * g + r;
                const bool valid = s_row[rho - rho0] != -1;
                const float lg = a.scale * (((s0[r] + s1[r]) + s2[r]) + s3[r]);
                p[rt][r] = valid ? lg : -INFINITY;
                tmax = fmaxf(tmax, p[rt][r]);
            }
        }
        tmax = wave_xor_max(tmax, 16);
        tmax = wave_xor_max(tmax, 32);
        const float m_new = fmaxf(m_run, tmax);
        float alpha = 1.f, psum = 0.f;
        if (m_new == -INFINITY) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) p[rt][r] = 0.f;
        } else {
            alpha = __expf(m_run - m_new);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    p[rt][r] = __expf(p[rt][r] - m_new);
                    psum += p[rt][r];
                }
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int b = 0; b < 8; ++b) o[b] *= alpha;

        // ---- PV: P^T fragment, element e <-> row e<4 ? 4g+e : 16+4g+(e-4); V^T fragment by two
        // transposed reads: source lane (g, c) points at row 4g + c/4 (+16), dims d0 + 4(c%4).
        const float pv[8] = {p[0][0], p[0][1], p[0][2], p[0][3], p[1][0], p[1][1], p[1][2], p[1][3]};
        const int r1 = 4 * g + (c >> 2);
        if (!is_raw) {
            bf16x8 phi, plo;
            pack_hi_lo8(pv, phi, plo);
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const int d = 128 * wave + 16 * b + 4 * (c & 3);
                const s16x4 v1 = lds_read_tr16(tb + elem_off(r1, d));
                const s16x4 v2 = lds_read_tr16(tb + elem_off(r1 + 16, d));
                const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
                o[b] = mfma16(av, phi, o[b]);
                o[b] = mfma16(av, plo, o[b]);
            }
        } else {
            f16x8 phi, plo;
            pack_hi_lo8_f16(pv, phi, plo);
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const int d = 128 * wave + 16 * b + 4 * (c & 3);
                const s16x4 v1 = lds_read_tr16(tb + elem_off(r1, d));
                const s16x4 v2 = lds_read_tr16(tb + elem_off(r1 + 16, d));
                const f16x8 av = __builtin_bit_cast(f16x8, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
                o[b] = mfma16h(av, phi, o[b]);
                o[b] = mfma16h(av, plo, o[b]);
            }
        }
        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: per-head sum over the four row groups
    l_run = wave_xor_sum(l_run, 16);
    l_run = wave_xor_sum(l_run, 32);
    if (a.n_chunks == 1) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float *orow = a.out + (q * a.H + h0 + c) * (int64_t)kD + 128 * wave + 4 * g;
#pragma unroll
        for (int b = 0; b < 8; ++b) *reinterpret_cast<f32x4 *>(orow + 16 * b) = o[b] * inv;
    } else {
        float *rec = a.part + ((q * a.n_hg + hg) * (int64_t)a.n_chunks + chunk) * kRec;
        if (wave == 0 && g == 0) {
            rec[c] = m_run;
            rec[kHG + c] = l_run;
        }
        float *orow = rec + 2 * kHG + c * kD + 128 * wave + 4 * g;
#pragma unroll
        for (int b = 0; b < 8; ++b) *reinterpret_cast<f32x4 *>(orow + 16 * b) = o[b];
    }
}

// Combines the per-chunk (max, sum, O) records of one (query, head group).
__global__ __launch_bounds__(256) void mqa_merge_kernel(int H, int n_hg, int n_chunks,
                                                        const float *__restrict__ part, float *__restrict__ out)
{
    const int64_t qh = blockIdx.x;
    const int64_t q = qh / n_hg;
    const int hg = (int)(qh % n_hg);
    const float *base = part + qh * n_chunks * (int64_t)kRec;
    const int hc = threadIdx.x >> 4;
    const int d0 = (threadIdx.x & 15) * 32;
    float M = -INFINITY;
    for (int ch = 0; ch < n_chunks; ++ch) M = fmaxf(M, base[ch * (int64_t)kRec + hc]);
    float L = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
        for (int ch = 0; ch < n_chunks; ++ch) {
            const float *rec = base + ch * (int64_t)kRec;
            const float m = rec[hc];
            if (m == -INFINITY) continue;
            const float wgt = __expf(m - M);
            L += wgt * rec[kHG + hc];
            const f32x4 *src = reinterpret_cast<const f32x4 *>(rec + 2 * kHG + hc * kD + d0);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += wgt * src[i];
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    f32x4 *dst = reinterpret_cast<f32x4 *>(out + (q * H + hg * kHG + hc) * (int64_t)kD + d0);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = acc[i] * inv;
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

void fill_inv_freq(double theta, double *inv_freq) {
    for (int i = 0; i < kRot / 2; ++i) inv_freq[i] = pow(theta, -2.0 * (double)i / (double)kRot);
}

}  // namespace

MqaPlan plan_mqa(int U, int T, int H, int W, int K) {
    MqaPlan p;
    p.n_hg = H / kHG;
    p.n_tiles = (W + K + kTile - 1) / kTile;
    const int64_t items = (int64_t)U * T * p.n_hg;
    // Split the union over workgroups only when there are too few (query, head group) items
    // to give every CU work; aim for ~1024 workgroups.
    int64_t want = (1024 + items - 1) / items;
    if (want < 1) want = 1;
    if (want > p.n_tiles) want = p.n_tiles;
    p.tiles_per_chunk = (int)((p.n_tiles + want - 1) / want);
    p.n_chunks = (p.n_tiles + p.tiles_per_chunk - 1) / p.tiles_per_chunk;
    p.workspace_bytes = p.n_chunks > 1 ? sizeof(float) * (size_t)items * (size_t)p.n_chunks * kRec : 0;
    return p;
}

hipError_t launch_mqa(int U, int T, int H, int W, int64_t N, int K, const void *q, int q_bf16,
                      const int64_t *q_pos, double theta, const uint16_t *raw, const uint16_t *comp,
                      const int32_t *idx, float scale, float *out, void *workspace,
                      hipStream_t stream)
{
    const MqaPlan p = plan_mqa(U, T, H, W, K);
    const int lds = kLdsBytes + 4 * kTile * p.tiles_per_chunk;
    static int attr_bytes = 0;
    if (lds > attr_bytes) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(sparse_mqa_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        attr_bytes = lds;
    }
    MqaArgs a;
    a.T = T; a.H = H; a.W = W; a.K = K; a.n_hg = p.n_hg; a.n_tiles = p.n_tiles;
    a.tiles_per_chunk = p.tiles_per_chunk; a.n_chunks = p.n_chunks;
    a.N = N;
    a.n_items = (int64_t)U * T * p.n_chunks;
    a.q = q; a.q_bf16 = q_bf16; a.pos = q_pos; a.raw = raw; a.comp = comp; a.idx = idx;
    a.scale = scale; a.out = out; a.part = static_cast<float *>(workspace);
    fill_inv_freq(theta, a.inv_freq);
    const int64_t blocks = (a.n_items + kXcd - 1) / kXcd * kXcd * p.n_hg;
    hipLaunchKernelGGL(sparse_mqa_kernel, dim3((unsigned)blocks), dim3(kThreads), lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_chunks == 1) return e;
    hipLaunchKernelGGL(mqa_merge_kernel, dim3((unsigned)((int64_t)U * T * p.n_hg)), dim3(256), 0, stream,
                       H, p.n_hg, p.n_chunks, static_cast<const float *>(workspace), out);
    return hipGetLastError();
}

hipError_t launch_rope(int U, int T, int H, const void *q, int q_bf16, const int64_t *q_pos,
                       double theta, float *q_out, hipStream_t stream)
{
    MqaArgs a = {};
    a.T = T; a.H = H; a.q = q; a.q_bf16 = q_bf16; a.pos = q_pos;
    fill_inv_freq(theta, a.inv_freq);
    const int64_t total8 = (int64_t)U * T * H * (kD / 8);
    hipLaunchKernelGGL(rope_q_kernel, dim3((unsigned)((total8 + 255) / 256)), dim3(256), 0, stream, a, total8, q_out);
    return hipGetLastError();
}

}  // namespace ds4a
