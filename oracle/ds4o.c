/* ds4o.c — plain scalar CPU oracle for one layer's compressed sparse attention step.
 *
 * TEST INFRASTRUCTURE ONLY: called by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library.  Slow on purpose:
 * straight loops in IEEE double, no blocking, no SIMD, no BLAS, one full sort
 * for the top-k.  Threads run only across independent (unit, query) pairs.
 *
 * Source of the method: "Reading the architecture of DwarfStar (ds4.c),
 * part 1/8" (Qiita), sections 2, 3, 3-1, 3-2 and 3-3 (cited per function below).
 */
#define _GNU_SOURCE
#include "ds4o.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- dtypes */

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double ds4o_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* zero / subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double ds4o_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Section 3-1 of the article: each raw-window value is stored as
 * f16_to_f32(f32_to_f16(x)).  The rounding rule is not printed; the reading
 * taken is IEEE round-to-nearest-even with gradual underflow and overflow to
 * infinity.  Done in double: the quantum of x's binade is a power of two, so
 * x / quantum is exact and rint() (ties to even in the default mode) rounds it. */
uint16_t ds4o_round_f16(float xf)
{
    double x = (double)xf;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7e00);
    if (isinf(x))
        return (uint16_t)(sign | 0x7c00);
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);                 /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    if (E < -14)
        E = -14;                   /* subnormal binade: quantum 2^-24 */
    double quantum = ldexp(1.0, E - 10);
    double r = rint(a / quantum) * quantum;
    if (r >= 65536.0)              /* the largest finite f16 is 65504 */
        return (uint16_t)(sign | 0x7c00);
    if (r < ldexp(1.0, -14))       /* stays subnormal (or rounds to zero) */
        return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
    frexp(r, &e2);                 /* rounding may have carried into the next binade */
    E = e2 - 1;
    uint16_t frac = (uint16_t)(r / ldexp(1.0, E - 10) - 1024.0);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | frac);
}

/* --------------------------------------------------------------- indexer */

/* Section 3-3 of the article: ratio-4 layers keep an indexer with its own
 * thin query (64 heads of 128 dims) that scores every compressed row; the
 * scores pick the rows the main attention sees.  The article does not print
 * the score formula.  Reading taken: per-head dot product, ReLU, then a sum
 * weighted by per-head weights (without a per-head nonlinearity the 64 heads
 * would collapse into one 128-dim query).  No scale factor: a positive global
 * scale does not change the selection. */
void ds4o_indexer_score(int64_t N, int Hi, int Di, const uint16_t *qI, const float *w,
                        const uint16_t *kI, int64_t n_vis, double *s)
{
    for (int64_t j = 0; j < N; j++) {
        if (j >= n_vis) {
            s[j] = -INFINITY;
            continue;
        }
        double total = 0.0;
        for (int h = 0; h < Hi; h++) {
            double dot = 0.0;
            for (int d = 0; d < Di; d++)
                dot += ds4o_bf16_to_f64(qI[(int64_t)h * Di + d]) * ds4o_bf16_to_f64(kI[j * Di + d]);
            double relu = dot > 0.0 ? dot : 0.0;
            total += (double)w[h] * relu;
        }
        s[j] = total;
    }
}

/* ------------------------------------------------------------------ top-k */

typedef struct {
    double score;
    int64_t index;
} scored_row;

/* Higher score first; equal scores: lower row index first. */
static int by_score_then_index(const void *pa, const void *pb)
{
    const scored_row *a = (const scored_row *)pa, *b = (const scored_row *)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    if (a->index < b->index) return -1;
    if (a->index > b->index) return 1;
    return 0;
}

/* Section 3-3 of the article: only the n_indexer_top_k best-scoring compressed
 * rows (512; Pro 1024, section 2) go on to the main attention.  Brute force:
 * sort all visible rows, keep the first min(K, n_vis). */
int ds4o_topk(int64_t n_vis, int K, const double *s, int32_t *idx)
{
    if (n_vis < 0)
        n_vis = 0;
    scored_row *rows = (scored_row *)malloc((size_t)(n_vis > 0 ? n_vis : 1) * sizeof *rows);
    for (int64_t j = 0; j < n_vis; j++) {
        rows[j].score = s[j];
        rows[j].index = j;
    }
    qsort(rows, (size_t)n_vis, sizeof *rows, by_score_then_index);
    int taken = (int)(n_vis < K ? n_vis : K);
    for (int k = 0; k < K; k++)
        idx[k] = k < taken ? (int32_t)rows[k].index : -1;
    free(rows);
    return taken;
}

/* ------------------------------------------------------------------- RoPE */

/* Section 2 of the article: n_rot = 64, RoPE applies to the last 64 of the
 * 512 head dims only.  Section 3-2 shows compressed rows rotated ("tail
 * RoPE") when they are emitted, so stored rows are already rotated and only
 * the query is rotated here.  Readings for what is not printed: adjacent
 * pairs (D-n_rot+2i, D-n_rot+2i+1), frequency theta^(-2i/n_rot), angle
 * pos * frequency, no frequency scaling. */
void ds4o_rope_q(int H, int D, int n_rot, int64_t pos, double theta,
                 const double *q_in, double *q_out)
{
    int first = D - n_rot;
    for (int h = 0; h < H; h++) {
        const double *x = q_in + (int64_t)h * D;
        double *y = q_out + (int64_t)h * D;
        for (int d = 0; d < first; d++)
            y[d] = x[d];
        for (int i = 0; i < n_rot / 2; i++) {
            double freq = pow(theta, -2.0 * (double)i / (double)n_rot);
            double angle = (double)pos * freq;
            double c = cos(angle), sn = sin(angle);
            double a = x[first + 2 * i], b = x[first + 2 * i + 1];
            y[first + 2 * i] = a * c - b * sn;
            y[first + 2 * i + 1] = a * sn + b * c;
        }
    }
}

/* -------------------------------------------------------------- attention */

/* Section 2 of the article: 64 query heads share one KV head of 512 dims
 * (multi-query attention).  Section 3: the attention reads the recent raw
 * window at full precision plus the compressed rows the indexer selected.
 * Readings: each stored row is both key and value (the cache holds one
 * 512-vector per token, section 3-1); the union is the concatenation of the
 * raw rows and the selected rows, with no de-duplication; one softmax over
 * the whole union; no sink or bias terms.  Plain two-pass softmax. */
/* One softmax over the n_union rows (doubles, rows[r][d]) for each of the H heads; each row
 * is key and value.  n_union >= 1. */
static void attend_rows(int H, int D, int n_union, const double *rows, const double *q_rot, double scale,
                        double *out)
{
    double *logit = (double *)malloc(sizeof(double) * (size_t)n_union);
    for (int h = 0; h < H; h++) {
        const double *qh = q_rot + (int64_t)h * D;
        double m = -INFINITY;
        for (int r = 0; r < n_union; r++) {
            double dot = 0.0;
            for (int d = 0; d < D; d++)
                dot += qh[d] * rows[(int64_t)r * D + d];
            logit[r] = scale * dot;
            if (logit[r] > m)
                m = logit[r];
        }
        double z = 0.0;
        for (int r = 0; r < n_union; r++) {
            logit[r] = exp(logit[r] - m);   /* now the unnormalised probability */
            z += logit[r];
        }
        double *oh = out + (int64_t)h * D;
        for (int d = 0; d < D; d++) {
            double acc = 0.0;
            for (int r = 0; r < n_union; r++)
                acc += logit[r] * rows[(int64_t)r * D + d];
            oh[d] = acc / z;
        }
    }
    free(logit);
}

/* The union as doubles: the W raw rows, then compressed row idx[k] for each idx[k] >= 0,
 * decoded from bf16 (comp8 == NULL) or from E4M3 codes times the row's scale. */
static int union_mqa(int H, int D, int W, int K, const double *q_rot, const uint16_t *raw,
                     const uint16_t *comp, const uint8_t *comp8, const float *comp_scale,
                     const int32_t *idx, double scale, double *out)
{
    int n_union = W;
    for (int k = 0; k < K; k++)
        if (idx[k] >= 0)
            n_union++;
    if (n_union == 0) {
        memset(out, 0, sizeof(double) * (size_t)H * (size_t)D);
        return 0;
    }
    double *rows = (double *)malloc(sizeof(double) * (size_t)n_union * (size_t)D);
    int r = 0;
    for (int i = 0; i < W; i++, r++)
        for (int d = 0; d < D; d++)
            rows[(int64_t)r * D + d] = ds4o_f16_to_f64(raw[(int64_t)i * D + d]);
    for (int k = 0; k < K; k++) {
        if (idx[k] < 0)
            continue;
        const int64_t j = idx[k];
        for (int d = 0; d < D; d++)
            rows[(int64_t)r * D + d] = comp8 ? ds4o_e4m3_to_f64(comp8[j * D + d]) * (double)comp_scale[j]
                                             : ds4o_bf16_to_f64(comp[j * D + d]);
        r++;
    }
    attend_rows(H, D, n_union, rows, q_rot, scale, out);
    free(rows);
    return n_union;
}

int ds4o_sparse_mqa(int H, int D, int W, int K, const double *q_rot,
                    const uint16_t *raw, const uint16_t *comp, const int32_t *idx,
                    double scale, double *out)
{
    return union_mqa(H, D, W, K, q_rot, raw, comp, NULL, NULL, idx, scale, out);
}

int ds4o_sparse_mqa_fp8(int H, int D, int W, int K, const double *q_rot,
                        const uint16_t *raw, const uint8_t *comp8, const float *comp_scale,
                        const int32_t *idx, double scale, double *out)
{
    return union_mqa(H, D, W, K, q_rot, raw, NULL, comp8, comp_scale, idx, scale, out);
}

/* ------------------------------------------------------------- whole step */

typedef struct {
    int U, T, H, D, n_rot, W, Hi, Di, K, q_is_bf16;
    int64_t N;
    const void *q;
    const int64_t *pos;
    double theta, scale;
    const uint16_t *raw, *comp, *kI, *qI;
    const float *w;
    const int32_t *n_vis;
    const int64_t *sel;
    int64_t n_items;
    double *scores;
    int32_t *idx;
    double *out;
    int64_t next;
    pthread_mutex_t lock;
} step_job;

static void run_one(step_job *j, int64_t item)
{
    int64_t ut = j->sel ? j->sel[item] : item;
    int64_t u = ut / j->T, t = ut % j->T;
    int H = j->H, D = j->D, W = j->W, K = j->K, Hi = j->Hi, Di = j->Di;
    int64_t N = j->N;

    double *s = j->scores ? j->scores + item * N : (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    int32_t *ix = j->idx ? j->idx + item * K : (int32_t *)malloc(sizeof(int32_t) * (size_t)K);

    ds4o_indexer_score(N, Hi, Di, j->qI + (u * j->T + t) * (int64_t)Hi * Di, j->w + (u * j->T + t) * Hi,
                       j->kI + u * N * Di, j->n_vis[u * j->T + t], s);
    ds4o_topk(j->n_vis[u * j->T + t], K, s, ix);

    if (j->out) {
        double *q64 = (double *)malloc(sizeof(double) * (size_t)H * D);
        double *qr = (double *)malloc(sizeof(double) * (size_t)H * D);
        int64_t qoff = (u * j->T + t) * (int64_t)H * D;
        for (int64_t e = 0; e < (int64_t)H * D; e++)
            q64[e] = j->q_is_bf16 ? ds4o_bf16_to_f64(((const uint16_t *)j->q)[qoff + e])
                                  : (double)((const float *)j->q)[qoff + e];
        ds4o_rope_q(H, D, j->n_rot, j->pos[u * j->T + t], j->theta, q64, qr);
        const uint16_t *raw_rows = j->raw + (u * (int64_t)(j->T + W - 1) + t) * D;
        ds4o_sparse_mqa(H, D, W, K, qr, raw_rows, j->comp + u * N * D, ix, j->scale,
                        j->out + item * (int64_t)H * D);
        free(qr);
        free(q64);
    }
    if (!j->scores)
        free(s);
    if (!j->idx)
        free(ix);
}

static void *worker(void *arg)
{
    step_job *j = (step_job *)arg;
    for (;;) {
        pthread_mutex_lock(&j->lock);
        int64_t item = j->next++;
        pthread_mutex_unlock(&j->lock);
        if (item >= j->n_items)
            return NULL;
        run_one(j, item);
    }
}

int ds4o_step(int U, int T, int64_t N, int H, int D, int n_rot, int W, int Hi, int Di, int K,
              const void *q, int q_is_bf16, const int64_t *pos, double theta,
              const uint16_t *raw, const uint16_t *comp, const uint16_t *kI,
              const uint16_t *qI, const float *w, const int32_t *n_vis, double scale,
              const int64_t *sel, int64_t n_sel, int nthreads,
              double *scores, int32_t *idx, double *out)
{
    if (U < 0 || T < 0 || N < 0 || H <= 0 || D <= 0 || n_rot < 0 || n_rot > D || (n_rot & 1) ||
        W < 0 || Hi <= 0 || Di <= 0 || K <= 0)
        return -1;
    step_job j;
    memset(&j, 0, sizeof j);
    j.U = U; j.T = T; j.N = N; j.H = H; j.D = D; j.n_rot = n_rot; j.W = W;
    j.Hi = Hi; j.Di = Di; j.K = K; j.q_is_bf16 = q_is_bf16;
    j.q = q; j.pos = pos; j.theta = theta; j.scale = scale;
    j.raw = raw; j.comp = comp; j.kI = kI; j.qI = qI; j.w = w; j.n_vis = n_vis;
    j.sel = sel;
    j.n_items = sel ? n_sel : (int64_t)U * T;
    j.scores = scores; j.idx = idx; j.out = out;
    for (int64_t i = 0; i < j.n_items; i++) {
        int64_t ut = sel ? sel[i] : i;
        if (ut < 0 || ut >= (int64_t)U * T)
            return -1;
    }
    pthread_mutex_init(&j.lock, NULL);
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int i = 1; i < nthreads; i++)
        if (pthread_create(&th[started], NULL, worker, &j) == 0)
            started++;
    worker(&j);
    for (int i = 0; i < started; i++)
        pthread_join(th[i], NULL);
    pthread_mutex_destroy(&j.lock);
    return 0;
}

/* ------------------------------------------------------------ compressor */

/* Round |x| to a multiple of 2^q_exp by rint (ties to even multiple) in double; exact while
 * |x| / 2^q_exp stays below 2^53. */
static double round_to_quantum(double a, int q_exp)
{
    return ldexp(rint(ldexp(a, -q_exp)), q_exp);
}

/* bfloat16: 8 significant bits, exponent range of binary32 (normals down to 2^-126,
 * subnormal quantum 2^-133), largest finite (2 - 2^-7) * 2^127. */
uint16_t ds4o_round_bf16(double x)
{
    if (isnan(x))
        return 0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);                                  /* a = f * 2^e, 0.5 <= f < 1 */
    int binade = e - 1;                            /* 2^binade <= a < 2^(binade+1) */
    if (binade < -126)
        binade = -126;
    double r = round_to_quantum(a, binade - 7);
    if (r >= ldexp(2.0 - ldexp(1.0, -8), 127))     /* at or past the halfway point to 2^128 */
        return (uint16_t)(sign | 0x7f80);
    float f = (float)r;                            /* exact: 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

double ds4o_e4m3_to_f64(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xf;
    int m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                  /* m/8 * 2^-6 */
    else
        v = ldexp((double)(8 + m), e - 10);        /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

uint8_t ds4o_round_e4m3(double x)
{
    if (isnan(x))
        return 0x7f;
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7e);             /* saturate: 1.75 * 2^8 */
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);
    int binade = e - 1;
    if (binade < -6)
        binade = -6;                               /* subnormals share the quantum 2^-9 */
    double r = round_to_quantum(a, binade - 3);
    if (r >= 448.0)
        return (uint8_t)(sign | 0x7e);
    if (r == 0.0)
        return sign;
    frexp(r, &e);
    binade = e - 1;
    if (binade < -6)                               /* subnormal: r = m * 2^-9 */
        return (uint8_t)(sign | (int)ldexp(r, 9));
    int m = (int)ldexp(r, -binade + 3) - 8;        /* r = (8 + m) * 2^(binade-3) */
    return (uint8_t)(sign | ((binade + 7) << 3) | m);
}

/* Section 3-2 of the article: at every ratio boundary the compressor pools its frontier of
 * `ratio` (kv, score) rows into one row, channel by channel, with the scores as softmax
 * logits (a row of weight e^(s - max) each, divided by their sum), then applies an RMS
 * normalisation, the tail RoPE and an FP8 quantise-dequantise round trip, in that order.
 * Readings for what the article leaves open: the norm is x / sqrt(mean(x^2) + eps) times a
 * per-channel gain; the tail RoPE is the one the query gets (adjacent pairs of the last n_rot
 * dims, angle pos * theta^(-2i/n_rot)) at the position the caller gives; the FP8 format is
 * E4M3FN with one power-of-two scale per row, the smallest that brings max|y| to <= 448,
 * values rounded to nearest (ties to even) and clipped; the row is then stored as bf16 (an
 * E4M3 value times a power of two is exact in bf16). */
int ds4o_compress_row(int width, int ratio, const float *state_kv, const float *state_score,
                      const float *gain, double eps, int n_rot, int64_t pos, double theta, int fp8,
                      double *y_pre, double *scale, uint16_t *out_bf16)
{
    if (width < 2 || ratio < 1 || n_rot < 0 || n_rot > width || (n_rot & 1))
        return -1;
    double *pooled = malloc(sizeof(double) * (size_t)width);
    double *y = malloc(sizeof(double) * (size_t)width);
    if (!pooled || !y) {
        free(pooled);
        free(y);
        return -1;
    }
    /* softmax-weighted pooling over the frontier rows, per channel: the weight of frontier
     * row r is exp(s_r - LSE), LSE = log(sum_r exp(s_r)) taken about the largest score so
     * that no exponential overflows; the weights sum to one (scores are finite). */
    for (int j = 0; j < width; j++) {
        const float *sc = state_score + j, *kv = state_kv + j;
        double top = (double)sc[0];
        for (int r = 1; r < ratio; r++)
            top = fmax(top, (double)sc[(int64_t)r * width]);
        double mass = 0.0;
        for (int r = 0; r < ratio; r++)
            mass += exp((double)sc[(int64_t)r * width] - top);
        const double lse = top + log(mass);
        double mean = 0.0;
        for (int r = 0; r < ratio; r++)
            mean += exp((double)sc[(int64_t)r * width] - lse) * (double)kv[(int64_t)r * width];
        pooled[j] = mean;
    }
    /* RMS normalisation */
    double ms = 0.0;
    for (int j = 0; j < width; j++)
        ms += pooled[j] * pooled[j];
    ms /= (double)width;
    double inv = 1.0 / sqrt(ms + eps);
    for (int j = 0; j < width; j++)
        pooled[j] = pooled[j] * inv * (double)gain[j];
    /* tail RoPE, as for a query of one head */
    ds4o_rope_q(1, width, n_rot, pos, theta, pooled, y);
    if (y_pre)
        memcpy(y_pre, y, sizeof(double) * (size_t)width);
    double s = 1.0;
    if (fp8) {
        double amax = 0.0;
        for (int j = 0; j < width; j++)
            if (fabs(y[j]) > amax)
                amax = fabs(y[j]);
        if (amax > 0.0)
            s = ldexp(1.0, (int)ceil(log2(amax / 448.0)));
        for (int j = 0; j < width; j++)
            y[j] = ds4o_e4m3_to_f64(ds4o_round_e4m3(y[j] / s)) * s;
    }
    if (scale)
        *scale = s;
    for (int j = 0; j < width; j++)
        out_bf16[j] = ds4o_round_bf16(y[j]);
    free(pooled);
    free(y);
    return 0;
}

void ds4o_indexer_score_fp8(int64_t N, int Hi, int Di, const uint16_t *qI, const float *w,
                            const uint8_t *k8, const float *scale, int64_t n_vis, double *s)
{
    double *key = (double *)malloc(sizeof(double) * (size_t)Di);
    for (int64_t j = 0; j < N; j++) {
        if (j >= n_vis) {
            s[j] = -INFINITY;
            continue;
        }
        for (int d = 0; d < Di; d++)
            key[d] = ds4o_e4m3_to_f64(k8[j * Di + d]) * (double)scale[j];
        double total = 0.0;
        for (int h = 0; h < Hi; h++) {
            double dot = 0.0;
            for (int d = 0; d < Di; d++)
                dot += ds4o_bf16_to_f64(qI[(int64_t)h * Di + d]) * key[d];
            double relu = dot > 0.0 ? dot : 0.0;
            total += (double)w[h] * relu;
        }
        s[j] = total;
    }
    free(key);
}

int ds4o_compress_row_e4m3(int width, int ratio, const float *state_kv, const float *state_score,
                           const float *gain, double eps, int n_rot, int64_t pos, double theta,
                           uint8_t *codes, double *scale)
{
    double *y = malloc(sizeof(double) * (size_t)width);
    uint16_t *tmp = malloc(sizeof(uint16_t) * (size_t)width);
    double s = 1.0;
    int rc = (y && tmp) ? ds4o_compress_row(width, ratio, state_kv, state_score, gain, eps, n_rot, pos,
                                            theta, 1, y, &s, tmp)
                        : -1;
    if (rc == 0) {
        for (int j = 0; j < width; j++)
            codes[j] = ds4o_round_e4m3(y[j] / s);
        if (scale)
            *scale = s;
    }
    free(y);
    free(tmp);
    return rc;
}

/* ---------------------------------------------------------- cache upkeep */

void ds4o_push_raw(int cap, int D, int T, const float *kv, uint16_t *raw, int32_t *n_raw)
{
    /* The window after the push holds the last min(cap, n + T) rows of the sequence
     * (its n current rows, then the T new rows rounded to f16): one computed slide. */
    const int64_t n = *n_raw, total = n + T;
    const int64_t keep = total < cap ? total : cap;
    const int64_t first = total - keep;             /* sequence index of the window's row 0 */
    uint16_t *win = malloc(sizeof(uint16_t) * (size_t)(keep > 0 ? keep : 1) * (size_t)D);
    if (!win)
        return;
    for (int64_t i = 0; i < keep; i++) {
        const int64_t s = first + i;
        for (int d = 0; d < D; d++)
            win[i * D + d] = s < n ? raw[s * D + d] : ds4o_round_f16(kv[(s - n) * D + d]);
    }
    memcpy(raw, win, sizeof(uint16_t) * (size_t)keep * (size_t)D);
    free(win);
    *n_raw = (int32_t)keep;
}

void ds4o_frontier_push(int width, int ratio, int64_t pos, const float *kv, const float *score,
                        const float *ape, float *state_kv, float *state_score)
{
    const int64_t row = pos % ratio;
    for (int j = 0; j < width; j++) {
        state_kv[row * width + j] = kv[j];
        state_score[row * width + j] = score[j] + ape[row * width + j];   /* f32 add */
    }
}
