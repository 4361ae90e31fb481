/* ds4attn.h — C ABI of libds4attn: one layer's compressed sparse attention step
 * on an AMD Instinct MI355X (gfx950).
 *
 * The step, as "Reading the architecture of DwarfStar (ds4.c), part 1/8"
 * (Qiita) describes it: in layers with compression ratio 4, a thin indexer
 * scores every compressed KV row and keeps the best n_indexer_top_k of them
 * (section 3-3); the main attention then runs its query heads against one
 * shared 512-dim KV head over the recent raw window plus the selected rows
 * (sections 2 and 3), with RoPE on the last n_rot = 64 dims (section 2).
 *
 * Conventions (all calls):
 *   - Pointers are DEVICE pointers unless stated otherwise; the caller owns every
 *     buffer, including the workspace (size it with ds4a_workspace_bytes).  The
 *     library never allocates or frees device memory.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and performs no host synchronisation.
 *   - Arguments are validated before anything is enqueued.  On a non-zero
 *     status nothing is enqueued, outputs are untouched, and ds4a_last_error()
 *     describes the problem.  A launch failure reported by the runtime maps to
 *     DS4A_E_HIP.  Faults inside kernels surface at the caller's next sync.
 *     There is no fallback path: unsupported shapes return DS4A_E_UNSUPPORTED.
 *   - Device pointers must be 16-byte aligned.  Rows are dense and row-major.
 *   - bf16 / f16 tensors hold IEEE bfloat16 / binary16 bit patterns.
 *   - Inputs must be finite; the library does not scan data.  Device-side
 *     integers are clamped to be safe: n_vis to [0, N]; idx values outside
 *     [0, N) are treated as -1 (skipped).
 *   - Calls on distinct streams are thread-safe.  Calls that share a
 *     workspace must be ordered on one stream.
 */
#ifndef DS4ATTN_H
#define DS4ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: raw_vis in the attention calls; 3: ds4a_indexer_topk_mqa(_fp8) */
#define DS4A_VERSION 3

typedef enum {
    DS4A_OK = 0,
    DS4A_E_NULL = -1,        /* a required pointer is NULL                          */
    DS4A_E_SHAPE = -2,       /* a size is negative, zero where it may not be, or too large */
    DS4A_E_UNSUPPORTED = -3, /* a valid shape this library does not implement        */
    DS4A_E_ALIGN = -4,       /* a device pointer is not 16-byte aligned              */
    DS4A_E_WORKSPACE = -5,   /* workspace missing or smaller than ds4a_workspace_bytes */
    DS4A_E_DTYPE = -6,       /* unknown dtype code                                   */
    DS4A_E_HIP = -7          /* the HIP runtime rejected a launch                   */
} ds4a_status;

typedef enum { DS4A_F32 = 0, DS4A_BF16 = 1, DS4A_F16 = 2 } ds4a_dtype;

/* Supported shapes. */
#define DS4A_INDEXER_HEADS 64     /* Hi: n_indexer_head (section 2)             */
#define DS4A_INDEXER_DIM 128      /* Di: n_indexer_head_dim (section 2)         */
#define DS4A_HEAD_DIM 512         /* D : n_head_dim (section 2)                 */
#define DS4A_ROPE_DIMS 64         /* n_rot (section 2)                          */
#define DS4A_MAX_HEADS 128        /* H : a multiple of 16 up to 128 (Flash 64, Pro 128) */
#define DS4A_MAX_TOPK 2048        /* K : 1..2048 (Flash 512, Pro 1024)          */
#define DS4A_MAX_WINDOW 1024      /* W : a multiple of 32 up to 1024 (n_swa = 128) */
#define DS4A_MAX_DENSE_ROWS (1 << 20) /* N of ds4a_dense_mqa: 0..2^20 compressed rows  */
#define DS4A_MAX_ATTN_ROWS ((1 << 22) - 1) /* N of ds4a_sparse_mqa(_fp8): rows a unit's cache may hold
                                            (4 GiB of bf16 rows, addressed with 32-bit offsets) */
#define DS4A_MAX_COMPRESS_WIDTH 1024  /* width of ds4a_compress_rows (512 KV, 128 indexer)  */
#define DS4A_MAX_COMPRESS_RATIO 1024  /* ratio of ds4a_compress_rows (4 or 128 in Flash)   */

/* A1 — indexer scores (section 3-3: the indexer's own thin query scores every
 * compressed row).  For unit u, query t and row j < n_vis[u][t]:
 *     scores[u][t][j] = sum_h idx_w[u][t][h] * max(0, sum_d idx_q[u][t][h][d] * idx_k[u][j][d])
 * and scores[u][t][j] = -INFINITY for n_vis[u][t] <= j < N.  The nonlinearity
 * (ReLU) and the head weighting are this library's reading; the page names only
 * the head count, head dim and top-k.  Products are exact bf16 x bf16 in fp32,
 * accumulated in fp32; the head sum is fp32.
 *   U, T     : units (layers or sessions) and query tokens per unit, >= 1
 *   N        : compressed rows per unit, >= 1, U*T*N < 2^40, N < 2^31
 *   Hi, Di   : must be 64 and 128
 *   idx_q    : bf16 [U][T][Hi][Di]      idx_w : f32 [U][T][Hi]
 *   idx_k    : bf16 [U][N][Di]          n_vis : int32 [U][T], or NULL for "all N"
 *   scores   : f32 [U][T][N] (output)
 */
int ds4a_indexer_score(int U, int T, int64_t N, int Hi, int Di,
                       const void *idx_q, const float *idx_w, const void *idx_k,
                       const int32_t *n_vis, float *scores, void *stream);

/* A2 — top-k selection (section 3-3: only the n_indexer_top_k best-scoring
 * rows reach the main attention; 512 for Flash, 1024 for Pro per section 2).
 * For each (u, t): the set of min(K, n_vis) rows j < n_vis with the largest
 * scores; equal scores (compared as IEEE floats, so -0 == +0) go to the lower j.
 * idx[u][t][*] receives that set in ascending row order, padded with -1.
 *   K        : 1..DS4A_MAX_TOPK
 *   scores   : f32 [U][T][N] (finite for j < n_vis)     n_vis : int32 [U][T] or NULL
 *   idx      : int32 [U][T][K] (output)
 *   workspace: ds4a_workspace_bytes(0, U, T, N, K, 0, 0) bytes of device memory
 */
int ds4a_topk_select(int U, int T, int64_t N, int K, const float *scores,
                     const int32_t *n_vis, int32_t *idx,
                     void *workspace, size_t workspace_bytes, void *stream);

/* A1 + A2 in one call (section 3-3: the indexer's scores serve only to pick the
 * rows that reach the main attention).  idx receives exactly the set that
 * ds4a_topk_select returns on the scores of ds4a_indexer_score for the same
 * arguments (the scores are computed by the same device code, bit for bit).
 * With T < 4 and at least 128 chunk workgroups in the call (chunks of 2,048 to
 * 8,192 rows, sized per call so that the busiest CU carries the least), the scores
 * never reach memory: each chunk of a query is scored and its top-K selected on
 * chip, and only (score, row) candidates are kept in the workspace; otherwise the
 * scores are written to the workspace and selected from there.
 * Arguments as for ds4a_indexer_score and ds4a_topk_select.
 *   workspace: ds4a_workspace_bytes(2, U, T, N, K, 0, 0) bytes (0 -> NULL allowed)
 */
int ds4a_indexer_topk(int U, int T, int64_t N, int Hi, int Di, int K,
                      const void *idx_q, const float *idx_w, const void *idx_k,
                      const int32_t *n_vis, int32_t *idx,
                      void *workspace, size_t workspace_bytes, void *stream);

/* A1 and A1 + A2 on FP8-stored indexer keys.  The compressor that emits the
 * indexer's keys rounds each row to FP8 (section 3-2 of "Reading the architecture
 * of DwarfStar (ds4.c), part 1/8"; format as at ds4a_compress_rows: OCP E4M3FN with
 * one power-of-two scale per row), so keeping the codes and the scale instead of
 * bf16 values loses nothing and halves the bytes the indexer streams per row
 * (256 -> 128, plus 4 for the scale).  As ds4a_indexer_score / ds4a_indexer_topk
 * with idx_k replaced by
 *   idx_k8      : uint8 [U][N][128] E4M3FN codes (the NaN codes 0x7F, 0xFF not allowed)
 *   idx_k_scale : f32 [U][N], finite and > 0
 * where the key of row j is code value * idx_k_scale[u][j].  The score is taken as
 *   s[j] = idx_k_scale[u][j] * sum_h w[h] * max(0, <qI[h], code values of row j>)
 * (a positive factor passes through the ReLU); the code values are widened to bf16
 * exactly and the products run on the same bf16 MFMAs as the bf16 entry points.
 * With power-of-two scales (as the compressor emits them) every score is bit-identical
 * to the bf16 entry point's score on keys code value * scale, so idx is identical too.
 * Routing (fused or score + select) and workspace sizes are those of the bf16 calls:
 *   workspace: ds4a_workspace_bytes(2, U, T, N, K, 0, 0) bytes (topk; 0 -> NULL allowed)
 */
int ds4a_indexer_score_fp8(int U, int T, int64_t N, int Hi, int Di,
                           const void *idx_q, const float *idx_w, const uint8_t *idx_k8,
                           const float *idx_k_scale, const int32_t *n_vis, float *scores, void *stream);
int ds4a_indexer_topk_fp8(int U, int T, int64_t N, int Hi, int Di, int K,
                          const void *idx_q, const float *idx_w, const uint8_t *idx_k8,
                          const float *idx_k_scale, const int32_t *n_vis, int32_t *idx,
                          void *workspace, size_t workspace_bytes, void *stream);

/* A3-A6 — sparse multi-query attention over the raw window plus the selected
 * rows (sections 2 and 3; the raw window keeps f16-rounded values, section 3-1).
 * For unit u, query t, head h:
 *   q'      = q[u][t][h] with dims D-n_rot+2i, D-n_rot+2i+1 rotated by the angle
 *             q_pos[u][t] * rope_theta^(-2i/n_rot)   (A3; stored rows are already
 *             rotated, so only the query is rotated here)
 *   union   = raw rows raw_kv[u][t + r], r = 0..W_t-1, then comp_kv[u][idx[u][t][k]]
 *             for every idx entry in [0, N) (no de-duplication)
 *   l_r     = scale * <q', row_r>                  (A4; each row is key and value)
 *   out     = sum_r softmax(l)_r * row_r           (A5, A6: one softmax over the union)
 * An empty union gives zeros.  Rows enter the MFMAs in their stored type (bf16
 * compressed rows, f16 raw rows); the query and the probabilities are carried as
 * hi + lo pairs of that type (a bf16 query only in its rotated tail); accumulation
 * is fp32.
 *   H        : query heads, a multiple of 16 up to 128      D, n_rot : 512, 64
 *   W        : raw window rows, a multiple of 32, 0..1024     K : 1..DS4A_MAX_TOPK
 *   q        : [U][T][H][D], q_dtype DS4A_F32 or DS4A_BF16 (pre-RoPE)
 *   q_pos    : int64 [U][T] absolute positions          rope_theta : > 0 (10000 in the tests)
 *   raw_kv   : f16 [U][T+W-1][D]   (query t uses rows t..t+W-1)
 *   raw_vis  : int32 [U][T] or NULL: W_t = raw_vis[u][t] clamped to [0, W] raw rows take
 *              part (a window that is not yet full at the start of a session: the first
 *              rows of the window, as ds4a_push_raw fills it); NULL: W_t = W
 *   comp_kv  : bf16 [U][N][D], 1 <= N <= DS4A_MAX_ATTN_ROWS
 *   idx      : int32 [U][T][K] (from ds4a_topk_select)
 *   out      : f32 [U][T][H][D] (output)
 *   workspace: ds4a_workspace_bytes(1, U, T, N, K, H, W) bytes (0 -> NULL allowed).  When
 *              the union of each query is split over several workgroups (few queries per
 *              call), the workspace begins with arrival counters: they must be zero before
 *              a workspace's first use (allocate it zero-filled), and every call leaves
 *              them zero again.  Calls that share a workspace must be ordered on one stream.
 */
int ds4a_sparse_mqa(int U, int T, int H, int D, int n_rot, int W, int64_t N, int K,
                    const void *q, int q_dtype, const int64_t *q_pos, double rope_theta,
                    const void *raw_kv, const int32_t *raw_vis, const void *comp_kv,
                    const int32_t *idx, float scale, float *out,
                    void *workspace, size_t workspace_bytes, void *stream);

/* ds4a_sparse_mqa for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same call with no workspace argument.
 * Where a split union needs counters and records, they live in the library's own scratch,
 * a static device array of DS4A_SCRATCH_BYTES per GPU (the first DS4A_SCRATCH_COUNT_BYTES
 * hold the counters: zero when the library loads, left zero by every call), held until the
 * process ends.  The call allocates nothing (no hipMalloc, no library allocation); its first
 * call on a device looks the array's address up once.  A call whose split needs more
 * counters or records than the scratch holds returns DS4A_E_WORKSPACE (decode, Pro decode
 * and long-context session shapes fit many times over).  Every call on one GPU shares that
 * GPU's scratch: calls that may overlap on one GPU (different streams, or host threads
 * without ordering) race; order them on one stream.  Arguments, results and other errors as
 * for ds4a_sparse_mqa.
 */
#define DS4A_SCRATCH_BYTES (16u << 20)
#define DS4A_SCRATCH_COUNT_BYTES (64u << 10)
int ds4a_sparse_mqa_noalloc(int U, int T, int H, int D, int n_rot, int W, int64_t N, int K,
                            const void *q, int q_dtype, const int64_t *q_pos, double rope_theta,
                            const void *raw_kv, const int32_t *raw_vis, const void *comp_kv,
                            const int32_t *idx, float scale, float *out, void *stream);

/* A1 + A2 + A3-A6 in one call: ds4a_indexer_topk on (idx_q, idx_w, idx_k, n_vis) followed by
 * ds4a_sparse_mqa on the selected rows, with the same results bit for bit (sections 3-1 to 3-3
 * of "Reading the architecture of DwarfStar (ds4.c), part 1/8": the indexer picks the rows
 * that the main attention then reads).  In decode shapes (T < 4, at least 128 chunk
 * workgroups for the fused select, few enough queries for the 16-head attention kernel, and a
 * union of at most 1,536 rows) the last merge level of the top-k runs inside the attention
 * kernel: each workgroup selects its query's rows from the chunks' candidates itself (when the
 * union is split over several workgroups, each selects the whole set and attends its part), so
 * the selection needs no launch and no round trip through memory of its own.  Otherwise the
 * call launches what the two calls would.
 * Arguments as for ds4a_indexer_topk (Hi, Di, K, idx_q, idx_w, idx_k, n_vis) and
 * ds4a_sparse_mqa (H, D, n_rot, W, q, q_dtype, q_pos, rope_theta, raw_kv, raw_vis, comp_kv,
 * scale, out), with N the rows of both caches, and
 *   idx      : int32 [U][T][K] receiving the selected rows, or NULL
 *   workspace: ds4a_workspace_bytes(4, U, T, N, K, H, W) bytes, zero-filled before its first
 *              use (it holds the attention's arrival counters, which every call leaves zero);
 *              calls that share a workspace must be ordered on one stream
 */
int ds4a_indexer_topk_mqa(int U, int T, int64_t N, int Hi, int Di, int K,
                          const void *idx_q, const float *idx_w, const void *idx_k,
                          const int32_t *n_vis, int H, int D, int n_rot, int W,
                          const void *q, int q_dtype, const int64_t *q_pos, double rope_theta,
                          const void *raw_kv, const int32_t *raw_vis, const void *comp_kv,
                          float scale, int32_t *idx, float *out,
                          void *workspace, size_t workspace_bytes, void *stream);
/* The same on FP8-stored indexer keys and compressed rows (formats as at ds4a_indexer_topk_fp8
 * and ds4a_sparse_mqa_fp8); the results are those of those two calls, bit for bit. */
int ds4a_indexer_topk_mqa_fp8(int U, int T, int64_t N, int Hi, int Di, int K,
                              const void *idx_q, const float *idx_w, const uint8_t *idx_k8,
                              const float *idx_k_scale, const int32_t *n_vis, int H, int D,
                              int n_rot, int W, const void *q, int q_dtype, const int64_t *q_pos,
                              double rope_theta, const void *raw_kv, const int32_t *raw_vis,
                              const uint8_t *comp_kv8, const float *comp_scale, float scale,
                              int32_t *idx, float *out,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Dense attention for the layers that have no indexer (section 3-2 of the same
 * page: ratio-128 layers fold 128 tokens into one row and are few enough to be
 * read whole; ratio-0 layers, the first two of Flash, keep only the raw window).
 * As ds4a_sparse_mqa, with the union
 *   union   = raw rows raw_kv[u][t + r], r = 0..W_t-1, then comp_kv[u][j] for every
 *             j < n_vis[u][t] (all N if n_vis is NULL), in row order
 * and the same arithmetic (same device code, chosen at compile time).
 *   N        : compressed rows per unit, 0..DS4A_MAX_DENSE_ROWS (0: raw window
 *              only, comp_kv may then be NULL); W + N >= 1
 *   n_vis    : int32 [U][T] or NULL; values are clamped to [0, N]
 *   workspace: ds4a_workspace_bytes(3, U, T, N, 0, H, W) bytes (0 -> NULL allowed)
 * Other arguments and errors as for ds4a_sparse_mqa; DS4A_E_UNSUPPORTED also when
 * the call would need 2^31 or more workgroups.
 */
int ds4a_dense_mqa(int U, int T, int H, int D, int n_rot, int W, int64_t N,
                   const void *q, int q_dtype, const int64_t *q_pos, double rope_theta,
                   const void *raw_kv, const int32_t *raw_vis, const void *comp_kv,
                   const int32_t *n_vis, float scale, float *out,
                   void *workspace, size_t workspace_bytes, void *stream);

/* A3-A6 and the dense attention over compressed rows stored as FP8 (the compressor's output
 * format, section 3-2 of "Reading the architecture of DwarfStar (ds4.c), part 1/8"; the
 * stored form of DS4A_ROW_E4M3 rows from ds4a_compress_append).  As ds4a_sparse_mqa /
 * ds4a_dense_mqa with comp_kv replaced by
 *   comp_kv8   : uint8 [U][N][512] E4M3FN codes (NaN codes not allowed)
 *   comp_scale : f32 [U][N], finite and > 0
 * where compressed row j is code value * comp_scale[u][j] (raw rows stay f16).  Codes widen to
 * bf16 exactly on the way into LDS and use the same bf16 MFMAs as the bf16 entry points; a
 * row's scale multiplies its logit and, for the weighted sum, its probability (fp32).  With
 * power-of-two scales the output is bit-identical to the bf16 entry point's on rows
 * code value * scale.  Workspace sizes are those of the bf16 calls (which = 1 and 3).
 */
int ds4a_sparse_mqa_fp8(int U, int T, int H, int D, int n_rot, int W, int64_t N, int K,
                        const void *q, int q_dtype, const int64_t *q_pos, double rope_theta,
                        const void *raw_kv, const int32_t *raw_vis, const uint8_t *comp_kv8,
                        const float *comp_scale, const int32_t *idx, float scale, float *out,
                        void *workspace, size_t workspace_bytes, void *stream);
int ds4a_dense_mqa_fp8(int U, int T, int H, int D, int n_rot, int W, int64_t N,
                       const void *q, int q_dtype, const int64_t *q_pos, double rope_theta,
                       const void *raw_kv, const int32_t *raw_vis, const uint8_t *comp_kv8,
                       const float *comp_scale, const int32_t *n_vis, float scale, float *out,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Compressor row emission (section 3-2: tokens older than the raw window are folded,
 * `ratio` at a time, into one compressed row by a learned pooling; the indexer has its own
 * compressor of the same form).  For each unit u (a layer or a session), from its frontier
 * of `ratio` rows (each token's KV row and its score row, the score already carrying the
 * positional bias):
 *   pooled[j] = sum_r e^(s[r][j] - m[j]) kv[r][j] / sum_r e^(s[r][j] - m[j]),  m[j] = max_r s[r][j]
 *   y         = pooled / sqrt(mean_j pooled[j]^2 + eps) * gain[u]             (RMS norm)
 *   y         = y with its last n_rot dims rotated as the query's tail is rotated
 *               (adjacent pairs, angle row_pos[u] * rope_theta^(-2i/n_rot))
 *   y         = FP8 round trip of y when fp8 = 1
 *   out[u * out_stride + j] = bf16(y[j])
 * Readings of what the page leaves open: the norm's form (epsilon and a per-channel gain
 * are inputs); the rotation's position (an input: row_pos); the FP8 format: OCP E4M3FN
 * with one power-of-two scale per row, the smallest that brings max|y| to <= 448, values
 * rounded to nearest (ties to even) and clipped, then scaled back (exact in bf16).
 * Arithmetic is fp32 except the rotation angle (fp64, as for the query).
 *   width    : a multiple of 4, 4..DS4A_MAX_COMPRESS_WIDTH (512 for KV rows, 128 for
 *              indexer keys)
 *   ratio    : 1..DS4A_MAX_COMPRESS_RATIO       n_rot : even, 0..min(width, 512)
 *   state_kv, state_score : f32 [U][ratio][width]     gain : f32 [U][width]
 *   eps      : >= 0 (finite)                     row_pos : int64 [U]
 *   fp8      : 0 or 1                            out : bf16 [U][out_stride], row u at u * out_stride
 *   out_stride : elements between units' rows, >= width (e.g. N * width to append the row
 *              to a [U][N][width] cache at row n: out = cache + n * width)
 * Errors as for the other calls; no workspace.
 */
int ds4a_compress_rows(int U, int width, int ratio, const float *state_kv, const float *state_score,
                       const float *gain, float eps, int n_rot, const int64_t *row_pos, double rope_theta,
                       int fp8, void *out, int64_t out_stride, void *stream);

/* Formats of an emitted compressed row (ds4a_compress_append). */
#define DS4A_ROW_BF16 0        /* bf16 values, no FP8 step                                 */
#define DS4A_ROW_BF16_FP8RT 1  /* bf16 values after the FP8 round trip (as compress_rows fp8=1) */
#define DS4A_ROW_E4M3 2        /* the FP8 row as stored: E4M3FN codes plus the row's f32 scale */

/* Compressed-row append, the compressor's last step for one decode token per unit (section
 * 3-2: at the ratio boundary one row is emitted into the unit's compressed cache).  Unit u
 * emits only when its token closes a group, pos[u] mod ratio == ratio - 1 (the frontier then
 * holds the group's `ratio` tokens); the row is that of ds4a_compress_rows (same device code)
 * and goes to row n_comp[u] of the unit's cache, after which n_comp[u] is incremented.  A
 * row past cap is not written but still counted, so n_comp[u] > cap after the call tells
 * the caller the cache was full.  Other units are left untouched.
 *   pos      : int64 [U] the token's position            row_pos : int64 [U] (RoPE position)
 *   format   : DS4A_ROW_BF16, DS4A_ROW_BF16_FP8RT, DS4A_ROW_E4M3
 *   comp     : bf16 [U][cap][width] (formats 0, 1) or uint8 [U][cap][width] codes (format 2)
 *   comp_scale : f32 [U][cap] (format 2 only; the row's power-of-two scale, decoded value =
 *              code value * scale)
 *   n_comp   : int32 [U] device counters, read and written by the call
 * Other arguments as for ds4a_compress_rows.  U * cap * width <= 2^40.
 */
int ds4a_compress_append(int U, int width, int ratio, const float *state_kv, const float *state_score,
                         const float *gain, float eps, int n_rot, const int64_t *pos, const int64_t *row_pos,
                         double rope_theta, int format, void *comp, float *comp_scale, int64_t cap,
                         int32_t *n_comp, void *stream);

/* Raw sliding-window push (section 3-1: the last n_swa = 128 tokens keep their KV rows, each
 * value rounded to f16 when it enters; a full window slides down by one row per token).  For
 * each unit u, the T rows kv[u][0..T-1] enter the window raw[u] in order, exactly as T single
 * pushes: while the window holds fewer than cap rows the row is stored at row n_raw[u] and
 * n_raw[u] grows; once full, the rows move down by one (row 0 leaves) and the new row is
 * stored at row cap - 1.  Rows at or past n_raw[u] are never read.  n_raw values outside
 * [0, cap] are clamped.
 *   kv       : f32 [U][T][D]                 raw : f16 [U][cap][D] (read and written)
 *   n_raw    : int32 [U] device counters      D  : a multiple of 8, 8..4096
 *   cap      : 1..DS4A_MAX_WINDOW (128 in Flash and Pro)
 * The window a decode query attends (raw_kv of ds4a_sparse_mqa with T = 1, W = cap) is raw[u]
 * once it is full.
 */
int ds4a_push_raw(int U, int T, int D, int cap, const float *kv, void *raw, int32_t *n_raw, void *stream);

/* A token entering the compressor's frontier (section 3-2: the score row gets the positional
 * bias of the token's place in its group, and both rows are written to the frontier): for
 * each unit u, with r = pos[u] mod ratio (taken in [0, ratio)),
 *   state_kv[u][r][j]    = kv[u][j]
 *   state_score[u][r][j] = score[u][j] + ape[r][j]     (f32 add)
 *   kv, score : f32 [U][width]      ape : f32 [ratio][width]      pos : int64 [U]
 *   state_kv, state_score : f32 [U][ratio][width]   width: a multiple of 4 up to
 *   DS4A_MAX_COMPRESS_WIDTH; ratio: 1..DS4A_MAX_COMPRESS_RATIO
 * Reading: the bias row is the one of the token's place pos mod ratio, the row it is written to.
 */
int ds4a_frontier_push(int U, int width, int ratio, const float *kv, const float *score, const float *ape,
                       const int64_t *pos, float *state_kv, float *state_score, void *stream);

/* A3 alone, for inspection: writes the rotated query as f32 [U][T][H][D], using
 * the same device code as ds4a_sparse_mqa's prologue (fp64 angle and rotation,
 * rounded once to f32).  Same argument rules as ds4a_sparse_mqa. */
int ds4a_rope_q(int U, int T, int H, int D, int n_rot, const void *q, int q_dtype,
                const int64_t *q_pos, double rope_theta, float *q_out, void *stream);

/* Workspace bytes for `which` = 0 (ds4a_topk_select; H and W ignored),
 * 1 (ds4a_sparse_mqa), 2 (ds4a_indexer_topk; H and W ignored), 3
 * (ds4a_dense_mqa; K ignored, N may be 0) or 4 (ds4a_indexer_topk_mqa and its FP8
 * form; never 0 for valid arguments).  0 means no workspace is needed (NULL is
 * accepted), or that the arguments are invalid.
 * Host-only, never touches the GPU. */
size_t ds4a_workspace_bytes(int which, int U, int T, int64_t N, int K, int H, int W);

/* Text of the last non-zero status returned on the calling thread (host memory
 * owned by the library, valid until the thread's next call). */
const char *ds4a_last_error(void);

/* DS4A_VERSION of the loaded library. */
int ds4a_version(void);

#ifdef __cplusplus
}
#endif
#endif
