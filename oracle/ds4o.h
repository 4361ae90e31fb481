/* ds4o.h — plain scalar CPU oracle for one layer's compressed sparse attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may call this library.  It shares no code, header, table or
 * helper with the GPU library (libds4attn) and must never be used as a fallback
 * for it.
 *
 * What it computes follows "Reading the architecture of DwarfStar (ds4.c),
 * part 1/8" (Qiita), sections 2 and 3:
 *   - section 2 (model shape): 64 query heads (Pro: 128), one KV head of 512
 *     dims, RoPE on the last n_rot = 64 dims, 128-row raw window, indexer with
 *     64 heads x 128 dims and top-k 512 (Pro: 1024);
 *   - section 3-1: raw-window values are rounded to f16 when pushed;
 *   - section 3-2: the compressor folds `ratio` recent tokens into one row by
 *     a per-channel softmax-weighted pooling, then normalises, rotates the
 *     tail and round-trips the row through FP8;
 *   - section 3-3: a thin indexer scores the compressed rows and only the
 *     top-k of them reach the main attention;
 *   - section 3 (overview): attention runs over the raw window plus the
 *     selected compressed rows.
 * Readings of points the article leaves open (ReLU between the per-head dot
 * product and the weighted head sum, interleaved RoPE pairs, rows stored
 * already rotated, key = value, one softmax over the concatenated union)
 * are stated beside each function in ds4o.c.
 *
 * All arithmetic is IEEE double; stored inputs are read as the exact real
 * values of their dtypes (bf16 / f16 bit patterns passed as uint16_t).
 */
#ifndef DS4O_H
#define DS4O_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exact value of an IEEE binary16 / bfloat16 bit pattern. */
double ds4o_f16_to_f64(uint16_t h);
double ds4o_bf16_to_f64(uint16_t b);

/* Round a float to IEEE binary16, round-to-nearest-even, gradual underflow,
 * overflow to infinity, NaN kept (quiet).  Returns the bit pattern. */
uint16_t ds4o_round_f16(float x);

/* Indexer scores of one query over rows 0..N-1:
 *   s[j] = sum_h w[h] * max(0, sum_d qI[h][d] * kI[j][d])   for j <  n_vis
 *   s[j] = -infinity                                         for j >= n_vis
 * qI: bf16 [Hi][Di], w: f32 [Hi], kI: bf16 [N][Di], s: double [N]. */
void ds4o_indexer_score(int64_t N, int Hi, int Di, const uint16_t *qI, const float *w,
                        const uint16_t *kI, int64_t n_vis, double *s);

/* Top-k of one query: rows 0..n_vis-1 sorted by (score descending, index
 * ascending); the first min(K, n_vis) indices are written to idx[0..], the
 * remaining slots are -1.  Returns the number of real entries. */
int ds4o_topk(int64_t n_vis, int K, const double *s, int32_t *idx);

/* RoPE on the tail of every head of one query at absolute position pos:
 * pairs (D-n_rot+2i, D-n_rot+2i+1), angle pos * theta^(-2i/n_rot). */
void ds4o_rope_q(int H, int D, int n_rot, int64_t pos, double theta,
                 const double *q_in, double *q_out);

/* Attention of one query.  Union = W raw rows (f16 [W][D]) followed by the
 * compressed rows comp[idx[k]] (bf16 [*][D]) for idx[k] >= 0.  One softmax over
 * the union per head; each row is both key and value.
 * q_rot: double [H][D] (already rotated), out: double [H][D].
 * An empty union gives zeros.  Returns the union size. */
int ds4o_sparse_mqa(int H, int D, int W, int K, const double *q_rot,
                    const uint16_t *raw, const uint16_t *comp, const int32_t *idx,
                    double scale, double *out);

/* As ds4o_sparse_mqa, with the compressed rows stored as FP8 (the compressor's round trip,
 * "Reading the architecture of DwarfStar (ds4.c), part 1/8", section 3-2): row j is the
 * E4M3FN value of each code times comp_scale[j].  comp8: uint8 [*][D]; comp_scale: f32 [*]. */
int ds4o_sparse_mqa_fp8(int H, int D, int W, int K, const double *q_rot,
                        const uint16_t *raw, const uint8_t *comp8, const float *comp_scale,
                        const int32_t *idx, double scale, double *out);

/* Whole step for U units x T queries (the layout of the GPU library's calls),
 * on nthreads host threads over independent (unit, query) pairs:
 *   q      : [U][T][H][D]  f32 (q_is_bf16 = 0) or bf16 bits (q_is_bf16 = 1)
 *   pos    : [U][T] int64      raw : f16 [U][T+W-1][D]  (query t uses rows t..t+W-1)
 *   comp   : bf16 [U][N][D]    kI  : bf16 [U][N][Di]    qI : bf16 [U][T][Hi][Di]
 *   w      : f32 [U][T][Hi]    n_vis : int32 [U][T]
 * Outputs (any may be NULL): scores double [U][T][N], idx int32 [U][T][K],
 * out double [U][T][H][D].  Only the pairs listed in sel (flattened u*T+t,
 * n_sel of them) are computed; sel = NULL means all.  Returns 0 on success. */
int ds4o_step(int U, int T, int64_t N, int H, int D, int n_rot, int W, int Hi, int Di, int K,
              const void *q, int q_is_bf16, const int64_t *pos, double theta,
              const uint16_t *raw, const uint16_t *comp, const uint16_t *kI,
              const uint16_t *qI, const float *w, const int32_t *n_vis, double scale,
              const int64_t *sel, int64_t n_sel, int nthreads,
              double *scores, int32_t *idx, double *out);

/* ------------------------------------------------------------ compressor */

/* Nearest bfloat16 of a double (round to nearest, ties to even), gradual underflow,
 * overflow to infinity.  Returns the bit pattern. */
uint16_t ds4o_round_bf16(double x);

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 fraction bits, no infinities,
 * S.1111.111 is NaN, largest finite 448, subnormals m/8 * 2^-6. */
double ds4o_e4m3_to_f64(uint8_t c);

/* Nearest E4M3FN value of x, ties to the even code; magnitudes above 448 saturate to
 * +-448, NaN gives 0x7f.  Returns the code. */
uint8_t ds4o_round_e4m3(double x);

/* Indexer scores of one query over FP8-stored keys: the key of row j is the E4M3FN value
 * of each code times the row's scale (the compressor's round trip, "Reading the
 * architecture of DwarfStar (ds4.c), part 1/8", section 3-2), then as ds4o_indexer_score:
 *   s[j] = sum_h w[h] * max(0, sum_d qI[h][d] * e4m3(k8[j][d]) * scale[j])   for j < n_vis
 *   s[j] = -infinity                                                        for j >= n_vis
 * qI: bf16 [Hi][Di], w: f32 [Hi], k8: E4M3FN codes [N][Di], scale: f32 [N], s: double [N]. */
void ds4o_indexer_score_fp8(int64_t N, int Hi, int Di, const uint16_t *qI, const float *w,
                            const uint8_t *k8, const float *scale, int64_t n_vis, double *s);

/* One compressed row from the compressor's frontier (section 3-2 of the article):
 *   pooled[j] = sum_r softmax_r(state_score[r][j]) * state_kv[r][j]   (r < ratio)
 *   y         = pooled / sqrt(mean_j pooled[j]^2 + eps) * gain          (RMS norm)
 *   y         = y with its last n_rot dims rotated at position pos     (tail RoPE)
 *   y8        = FP8 round trip of y if fp8 (E4M3FN, one power-of-two scale per row)
 *   out_bf16  = bf16(y8)
 * state_kv, state_score: f32 [ratio][width]; gain: f32 [width].  y_pre (double [width],
 * y before the FP8 step) and scale (the row's FP8 scale, 1 without FP8) may be NULL.
 * Returns 0, or -1 on bad sizes. */
int ds4o_compress_row(int width, int ratio, const float *state_kv, const float *state_score,
                      const float *gain, double eps, int n_rot, int64_t pos, double theta, int fp8,
                      double *y_pre, double *scale, uint16_t *out_bf16);

/* The E4M3FN codes of the row ds4o_compress_row emits with fp8 = 1 (the same steps; codes
 * = round_e4m3(y[j] / scale), the form in which the row can be stored with its scale).
 * codes: uint8 [width]; scale as above.  Returns 0, or -1 on bad sizes. */
int ds4o_compress_row_e4m3(int width, int ratio, const float *state_kv, const float *state_score,
                           const float *gain, double eps, int n_rot, int64_t pos, double theta,
                           uint8_t *codes, double *scale);

/* Raw sliding-window push ("Reading the architecture of DwarfStar (ds4.c), part 1/8",
 * section 3-1): the window keeps the most recent tokens, each value rounded to f16.  After
 * T rows kv f32 [T][D] arrive in a window of cap rows (f16 bit patterns [cap][D] holding
 * *n_raw rows, oldest first), it holds the last min(cap, *n_raw + T) rows of the sequence
 * "current rows, then the new rows", oldest first, and *n_raw is that count; rows past it
 * are untouched. */
void ds4o_push_raw(int cap, int D, int T, const float *kv, uint16_t *raw, int32_t *n_raw);

/* One token entering the compressor's frontier (the same page, section 3-2, steps 2 and
 * 3): its score row plus the positional bias ape[pos % ratio][*] (f32 adds), and its KV row,
 * are written to frontier row pos % ratio.  kv, score: f32 [width]; ape: f32
 * [ratio][width]; state_kv, state_score: f32 [ratio][width]. */
void ds4o_frontier_push(int width, int ratio, int64_t pos, const float *kv, const float *score,
                        const float *ape, float *state_kv, float *state_score);

#ifdef __cplusplus
}
#endif
#endif
