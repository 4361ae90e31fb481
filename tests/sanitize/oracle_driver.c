/* Drives every function of the CPU oracle (oracle/ds4o.c) on small and edge-case inputs,
 * for a build under AddressSanitizer and UndefinedBehaviorSanitizer.  Prints "ok" and
 * returns 0 when every call finished; the sanitizers abort the process on the first error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/ds4o.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static double urand(void) { /* splitmix64 -> [0, 1) */
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (double)((z ^ (z >> 31)) >> 11) * 0x1.0p-53;
}

static float nrand(void) { return (float)((urand() + urand() + urand() - 1.5) * 2.0); }

#define ALLOC(T, n) ((T *)calloc((size_t)(n) > 0 ? (size_t)(n) : 1, sizeof(T)))

static void check(int cond, const char *what) {
    if (!cond) {
        fprintf(stderr, "check failed: %s\n", what);
        exit(2);
    }
}

static void run_attention(int H, int W, int N, int K, int fp8) {
    const int D = 512;
    uint16_t *raw = ALLOC(uint16_t, W * D), *comp = ALLOC(uint16_t, N * D);
    uint8_t *comp8 = ALLOC(uint8_t, N * D);
    float *cs = ALLOC(float, N);
    double *q = ALLOC(double, H * D), *qr = ALLOC(double, H * D), *out = ALLOC(double, H * D);
    int32_t *idx = ALLOC(int32_t, K);
    for (int i = 0; i < W * D; i++) raw[i] = ds4o_round_f16(nrand());
    for (int i = 0; i < N * D; i++) {
        comp[i] = ds4o_round_bf16(nrand());
        comp8[i] = ds4o_round_e4m3(nrand() * 100.0);
    }
    for (int i = 0; i < N; i++) cs[i] = (float)(0.5 + urand());
    for (int i = 0; i < H * D; i++) q[i] = nrand();
    for (int k = 0; k < K; k++) idx[k] = N ? (int32_t)(urand() * N) : -1;
    if (K > 2) idx[1] = -1;
    ds4o_rope_q(H, D, 64, 1048575, 10000.0, q, qr);
    int n = fp8 ? ds4o_sparse_mqa_fp8(H, D, W, K, qr, raw, comp8, cs, idx, 1.0 / sqrt(512.0), out)
                : ds4o_sparse_mqa(H, D, W, K, qr, raw, comp, idx, 1.0 / sqrt(512.0), out);
    check(n >= 0 && n <= W + K, "union size");
    for (int i = 0; i < H * D; i++) check(isfinite(out[i]), "finite attention output");
    free(raw); free(comp); free(comp8); free(cs); free(q); free(qr); free(out); free(idx);
}

int main(void) {
    /* conversions, all 2^16 patterns and edges */
    for (uint32_t b = 0; b < 65536; b++) {
        (void)ds4o_f16_to_f64((uint16_t)b);
        (void)ds4o_bf16_to_f64((uint16_t)b);
    }
    const double edges[] = {0.0, -0.0, 1e-45, 6e-8, 65504.0, 65520.0, 1e30, -1e30, INFINITY, -INFINITY, NAN, 448.0,
                            464.0, 1e-10, 3.4e38};
    for (size_t i = 0; i < sizeof edges / sizeof edges[0]; i++) {
        (void)ds4o_round_f16((float)edges[i]);
        (void)ds4o_round_bf16(edges[i]);
        (void)ds4o_round_e4m3(edges[i]);
    }
    for (int c = 0; c < 256; c++) (void)ds4o_e4m3_to_f64((uint8_t)c);

    /* indexer + top-k: N from 1, n_vis 0 .. N, K above and below n_vis */
    const int Hi = 64, Di = 128;
    for (int N = 1; N <= 600; N += 199) {
        uint16_t *qI = ALLOC(uint16_t, Hi * Di), *kI = ALLOC(uint16_t, N * Di);
        uint8_t *k8 = ALLOC(uint8_t, N * Di);
        float *w = ALLOC(float, Hi), *ks = ALLOC(float, N);
        double *s = ALLOC(double, N);
        for (int i = 0; i < Hi * Di; i++) qI[i] = ds4o_round_bf16(nrand());
        for (int i = 0; i < N * Di; i++) {
            kI[i] = ds4o_round_bf16(nrand());
            k8[i] = ds4o_round_e4m3(nrand() * 50.0);
        }
        for (int h = 0; h < Hi; h++) w[h] = (float)urand();
        for (int j = 0; j < N; j++) ks[j] = 0.01f;
        const int64_t nvs[] = {0, 1, N / 2, N};
        for (int a = 0; a < 4; a++) {
            ds4o_indexer_score(N, Hi, Di, qI, w, kI, nvs[a], s);
            ds4o_indexer_score_fp8(N, Hi, Di, qI, w, k8, ks, nvs[a], s);
            const int Ks[] = {1, 7, 512};
            for (int b = 0; b < 3; b++) {
                int32_t *idx = ALLOC(int32_t, Ks[b]);
                int got = ds4o_topk(nvs[a], Ks[b], s, idx);
                check(got == (nvs[a] < Ks[b] ? nvs[a] : Ks[b]), "top-k count");
                free(idx);
            }
        }
        free(qI); free(kI); free(k8); free(w); free(ks); free(s);
    }

    /* attention: raw only, compressed only, both, Pro heads, FP8 rows, empty union */
    run_attention(64, 128, 300, 64, 0);
    run_attention(16, 0, 50, 8, 0);
    run_attention(128, 32, 1, 3, 1);
    run_attention(64, 128, 0, 1, 0);
    {
        double q[512] = {0}, out[512];
        uint16_t r[512] = {0};
        int32_t none[2] = {-1, -1};
        check(ds4o_sparse_mqa(1, 512, 0, 2, q, r, r, none, 1.0, out) == 0, "empty union");
    }

    /* whole step, decode and a small prefill with causal visibility, several threads */
    {
        const int U = 2, T = 3, H = 16, D = 512, W = 32, K = 40;
        const int64_t N = 100;
        float *q = ALLOC(float, U * T * H * D), *w = ALLOC(float, U * T * Hi);
        int64_t pos[6] = {0, 1, 2, 1000, 1001, 1002};
        uint16_t *raw = ALLOC(uint16_t, U * (T + W - 1) * D), *comp = ALLOC(uint16_t, U * N * D);
        uint16_t *kI = ALLOC(uint16_t, U * N * Di), *qI = ALLOC(uint16_t, U * T * Hi * Di);
        int32_t nv[6] = {0, 50, 100, 100, 3, 40};
        for (int i = 0; i < U * T * H * D; i++) q[i] = nrand();
        for (int i = 0; i < U * T * Hi; i++) w[i] = (float)urand();
        for (int i = 0; i < U * (T + W - 1) * D; i++) raw[i] = ds4o_round_f16(nrand());
        for (int i = 0; i < U * N * D; i++) comp[i] = ds4o_round_bf16(nrand());
        for (int i = 0; i < U * N * Di; i++) kI[i] = ds4o_round_bf16(nrand());
        for (int i = 0; i < U * T * Hi * Di; i++) qI[i] = ds4o_round_bf16(nrand());
        double *sc = ALLOC(double, U * T * N), *out = ALLOC(double, U * T * H * D);
        int32_t *idx = ALLOC(int32_t, U * T * K);
        check(ds4o_step(U, T, N, H, D, 64, W, Hi, Di, K, q, 0, pos, 10000.0, raw, comp, kI, qI, w, nv,
                        1.0 / sqrt(512.0), NULL, 0, 3, sc, idx, out) == 0, "step");
        int64_t sel[2] = {5, 0};
        check(ds4o_step(U, T, N, H, D, 64, W, Hi, Di, K, q, 0, pos, 10000.0, raw, comp, kI, qI, w, nv,
                        1.0 / sqrt(512.0), sel, 2, 1, sc, idx, out) == 0, "step over a selection");
        free(q); free(w); free(raw); free(comp); free(kI); free(qI); free(sc); free(out); free(idx);
    }

    /* compressor and cache upkeep */
    {
        const int widths[] = {4, 128, 512};
        const int ratios[] = {1, 4, 128};
        for (int a = 0; a < 3; a++)
            for (int b = 0; b < 3; b++) {
                const int width = widths[a], ratio = ratios[b];
                float *kv = ALLOC(float, ratio * width), *sc = ALLOC(float, ratio * width), *g = ALLOC(float, width);
                for (int i = 0; i < ratio * width; i++) {
                    kv[i] = nrand();
                    sc[i] = nrand() * 30.0f;
                }
                for (int i = 0; i < width; i++) g[i] = (float)(0.5 + urand());
                uint16_t *out = ALLOC(uint16_t, width);
                uint8_t *codes = ALLOC(uint8_t, width);
                double *y = ALLOC(double, width), s;
                const int n_rot = width >= 64 ? 64 : 0;
                check(ds4o_compress_row(width, ratio, kv, sc, g, 1e-6, n_rot, 12345, 10000.0, 1, y, &s, out) == 0,
                      "compress");
                check(ds4o_compress_row_e4m3(width, ratio, kv, sc, g, 1e-6, n_rot, 7, 10000.0, codes, &s) == 0,
                      "compress e4m3");
                float *skv = ALLOC(float, ratio * width), *ssc = ALLOC(float, ratio * width);
                float *ape = ALLOC(float, ratio * width);
                for (int64_t p = 0; p < 2 * ratio + 1; p++)
                    ds4o_frontier_push(width, ratio, p, kv, sc, ape, skv, ssc);
                free(kv); free(sc); free(g); free(out); free(codes); free(y); free(skv); free(ssc); free(ape);
            }
        check(ds4o_compress_row(0, 4, NULL, NULL, NULL, 0.0, 0, 0, 1.0, 0, NULL, NULL, NULL) == -1, "bad width");
        const int caps[] = {1, 4, 128};
        for (int a = 0; a < 3; a++)
            for (int T = 1; T <= 300; T += 149)
                for (int n0 = 0; n0 <= caps[a]; n0 += caps[a] > 2 ? caps[a] / 2 : 1) {
                    const int cap = caps[a], D = 64;
                    uint16_t *raw = ALLOC(uint16_t, cap * D);
                    float *kv = ALLOC(float, T * D);
                    for (int i = 0; i < T * D; i++) kv[i] = nrand() * 1e4f;
                    int32_t n = n0;
                    ds4o_push_raw(cap, D, T, kv, raw, &n);
                    check(n == (n0 + T < cap ? n0 + T : cap), "window count");
                    free(raw); free(kv);
                }
    }
    puts("ok");
    return 0;
}
