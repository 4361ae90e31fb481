// Drives the host side of libds4attn (argument validation, plans and workspace sizes) under
// AddressSanitizer and UndefinedBehaviorSanitizer, with no GPU: every call below is one that
// the library must refuse before it touches the HIP runtime, plus the size queries over a
// sweep of shapes up to the documented limits.  Prints "ok" and returns 0 when every status
// is the documented one; a sanitizer report aborts the process first.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ds4attn.h"

static int g_fail = 0;

#define EXPECT(call, code)                                                                          \
    do {                                                                                            \
        const int rc_ = (call);                                                                     \
        if (rc_ != (code)) {                                                                        \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d (%s)\n", __FILE__, __LINE__, #call, rc_, \
                    (int)(code), ds4a_last_error());                                                \
            g_fail = 1;                                                                             \
        } else if (rc_ != 0 && strlen(ds4a_last_error()) == 0) {                                    \
            fprintf(stderr, "%s:%d: no error text\n", __FILE__, __LINE__);                         \
            g_fail = 1;                                                                             \
        }                                                                                           \
    } while (0)

int main() {
    alignas(256) static unsigned char buf[1 << 16];
    void *p = buf;                      // a stand-in pointer: never dereferenced on these paths
    void *odd = buf + 1;                // misaligned
    float *pf = reinterpret_cast<float *>(buf);
    int32_t *pi = reinterpret_cast<int32_t *>(buf);
    int64_t *pl = reinterpret_cast<int64_t *>(buf);
    uint8_t *pb = buf;

    // ---- size queries over the documented ranges (no overflow, no out-of-range shifts)
    const int Us[] = {1, 43, 4096, 1 << 24};
    const int Ts[] = {1, 3, 2048, 1 << 24};
    const int64_t Ns[] = {0, 1, 511, 8192, 65536, 262144, 1 << 20, (int64_t(1) << 31) - 1, int64_t(1) << 31};
    const int Ks[] = {0, 1, 512, 1024, 2048, 2049};
    const int Hs[] = {0, 16, 64, 128, 144};
    const int Wsz[] = {-32, 0, 32, 128, 1024, 1056};
    size_t acc = 0;
    for (int which = -1; which <= 4; ++which)
        for (int U : Us)
            for (int T : Ts)
                for (int64_t N : Ns)
                    for (int K : Ks)
                        for (int H : Hs)
                            for (int W : Wsz) acc += ds4a_workspace_bytes(which, U, T, N, K, H, W);
    if (ds4a_workspace_bytes(7, 1, 1, 1, 1, 64, 128) != 0) g_fail = 1;

    // ---- A1 / A2 / A1 + A2: every rule refused before anything runs
    EXPECT(ds4a_indexer_score(0, 1, 10, 64, 128, p, pf, p, nullptr, pf, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_indexer_score(1, 1, 0, 64, 128, p, pf, p, nullptr, pf, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_indexer_score(1, 1, int64_t(1) << 31, 64, 128, p, pf, p, nullptr, pf, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_indexer_score(1 << 20, 1 << 20, 10, 64, 128, p, pf, p, nullptr, pf, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_indexer_score(1 << 12, 1 << 12, int64_t(1) << 30, 64, 128, p, pf, p, nullptr, pf, nullptr),
           DS4A_E_SHAPE);
    EXPECT(ds4a_indexer_score(1, 1, 10, 32, 128, p, pf, p, nullptr, pf, nullptr), DS4A_E_UNSUPPORTED);
    EXPECT(ds4a_indexer_score(1, 1, 10, 64, 128, nullptr, pf, p, nullptr, pf, nullptr), DS4A_E_NULL);
    EXPECT(ds4a_indexer_score(1, 1, 10, 64, 128, odd, pf, p, nullptr, pf, nullptr), DS4A_E_ALIGN);
    EXPECT(ds4a_indexer_score(1, 1, 10, 64, 128, p, pf, p, reinterpret_cast<int32_t *>(buf + 4), pf, nullptr),
           DS4A_E_ALIGN);
    EXPECT(ds4a_indexer_score_fp8(1, 1, 10, 64, 128, p, pf, pb, nullptr, nullptr, pf, nullptr), DS4A_E_NULL);
    EXPECT(ds4a_topk_select(1, 1, 10, 0, pf, nullptr, pi, nullptr, 0, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_topk_select(1, 1, 10, 4096, pf, nullptr, pi, nullptr, 0, nullptr), DS4A_E_UNSUPPORTED);
    EXPECT(ds4a_topk_select(1, 1, 10, 5, nullptr, nullptr, pi, nullptr, 0, nullptr), DS4A_E_NULL);
    EXPECT(ds4a_topk_select(43, 1, 65536, 512, pf, nullptr, pi, nullptr, 0, nullptr), DS4A_E_WORKSPACE);
    EXPECT(ds4a_topk_select(43, 1, 65536, 512, pf, nullptr, pi, p, 16, nullptr), DS4A_E_WORKSPACE);
    EXPECT(ds4a_indexer_topk(43, 1, 65536, 64, 128, 512, p, pf, p, nullptr, pi, nullptr, 0, nullptr),
           DS4A_E_WORKSPACE);
    EXPECT(ds4a_indexer_topk(43, 1, 65536, 64, 128, 512, p, pf, p, nullptr, pi, odd, size_t(1) << 40, nullptr),
           DS4A_E_ALIGN);
    EXPECT(ds4a_indexer_topk_fp8(1, 1, 10, 64, 128, 0, p, pf, pb, pf, nullptr, pi, nullptr, 0, nullptr),
           DS4A_E_SHAPE);

    // ---- A3-A6 and the dense attention
    const double th = 10000.0;
    const float sc = 0.0442f;
    EXPECT(ds4a_sparse_mqa(1, 1, 64, 256, 64, 128, 100, 64, p, DS4A_F32, pl, th, p, nullptr, p, pi, sc, pf, nullptr, 0,
                           nullptr), DS4A_E_UNSUPPORTED);
    EXPECT(ds4a_sparse_mqa(1, 1, 64, 512, 32, 128, 100, 64, p, DS4A_F32, pl, th, p, nullptr, p, pi, sc, pf, nullptr, 0,
                           nullptr), DS4A_E_UNSUPPORTED);
    EXPECT(ds4a_sparse_mqa(1, 1, 48 + 1, 512, 64, 128, 100, 64, p, DS4A_F32, pl, th, p, nullptr, p, pi, sc, pf,
                           nullptr, 0, nullptr), DS4A_E_UNSUPPORTED);
    EXPECT(ds4a_sparse_mqa(1, 1, 64, 512, 64, 100, 100, 64, p, DS4A_F32, pl, th, p, nullptr, p, pi, sc, pf, nullptr, 0,
                           nullptr), DS4A_E_UNSUPPORTED);
    EXPECT(ds4a_sparse_mqa(1, 1, 64, 512, 64, 128, 100, 64, p, DS4A_F16, pl, th, p, nullptr, p, pi, sc, pf, nullptr, 0,
                           nullptr), DS4A_E_UNSUPPORTED);
    EXPECT(ds4a_sparse_mqa(1, 1, 64, 512, 64, 128, 100, 64, p, 9, pl, th, p, nullptr, p, pi, sc, pf, nullptr, 0,
                           nullptr), DS4A_E_DTYPE);
    EXPECT(ds4a_sparse_mqa(1, 1, 64, 512, 64, 128, 100, 64, p, DS4A_F32, pl, -1.0, p, nullptr, p, pi, sc, pf, nullptr,
                           0, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_sparse_mqa(1, 1, 64, 512, 64, 128, 100, 64, p, DS4A_F32, pl, th, p, nullptr, p, pi, 1.0f / 0.0f, pf,
                           nullptr, 0, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_sparse_mqa(1, 1, 64, 512, 64, 128, 100, 64, p, DS4A_F32, pl, th, nullptr, nullptr, p, pi, sc, pf,
                           nullptr, 0, nullptr), DS4A_E_NULL);
    if (ds4a_workspace_bytes(1, 43, 1, 65536, 512, 64, 128) > 0)
        EXPECT(ds4a_sparse_mqa(43, 1, 64, 512, 64, 128, 65536, 512, p, DS4A_F32, pl, th, p, nullptr, p, pi, sc, pf,
                               nullptr, 0, nullptr), DS4A_E_WORKSPACE);
    EXPECT(ds4a_sparse_mqa_fp8(1, 1, 64, 512, 64, 128, 100, 64, p, DS4A_F32, pl, th, p, nullptr, pb, nullptr, pi, sc,
                               pf, nullptr, 0, nullptr), DS4A_E_NULL);
    EXPECT(ds4a_dense_mqa(1, 1, 64, 512, 64, 0, 0, p, DS4A_F32, pl, th, nullptr, nullptr, nullptr, nullptr, sc, pf,
                          nullptr, 0, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_dense_mqa(1, 1, 64, 512, 64, 128, (1 << 20) + 1, p, DS4A_F32, pl, th, p, nullptr, p, nullptr, sc, pf,
                          nullptr, 0, nullptr), DS4A_E_UNSUPPORTED);
    EXPECT(ds4a_dense_mqa(1 << 24, 1, 128, 512, 64, 1024, 1 << 20, p, DS4A_F32, pl, th, p, nullptr, p, nullptr, sc,
                          pf, nullptr, 0, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_dense_mqa_fp8(1, 1, 64, 512, 64, 128, 10, p, DS4A_BF16, pl, th, p, nullptr, pb, nullptr, nullptr, sc,
                              pf, nullptr, 0, nullptr), DS4A_E_NULL);
    EXPECT(ds4a_rope_q(1, 1, 64, 512, 64, nullptr, DS4A_F32, pl, th, pf, nullptr), DS4A_E_NULL);

    // ---- compressor and cache upkeep
    EXPECT(ds4a_compress_rows(1, 6, 4, pf, pf, pf, 1e-6f, 2, pl, th, 1, p, 6, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_compress_rows(1, 2048, 4, pf, pf, pf, 1e-6f, 64, pl, th, 1, p, 2048, nullptr), DS4A_E_UNSUPPORTED);
    EXPECT(ds4a_compress_rows(1, 512, 4, pf, pf, pf, -1.f, 64, pl, th, 1, p, 512, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_compress_rows(1, 512, 4, pf, pf, pf, 1e-6f, 64, pl, th, 2, p, 512, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_compress_rows(1, 512, 4, pf, pf, pf, 1e-6f, 64, pl, th, 1, p, 256, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_compress_append(1, 512, 4, pf, pf, pf, 1e-6f, 64, pl, pl, th, 7, p, pf, 100, pi, nullptr),
           DS4A_E_DTYPE);
    EXPECT(ds4a_compress_append(1 << 24, 1024, 4, pf, pf, pf, 1e-6f, 64, pl, pl, th, 0, p, pf, (int64_t(1) << 31) - 1,
                                pi, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_compress_append(1, 512, 4, pf, pf, pf, 1e-6f, 64, pl, pl, th, DS4A_ROW_E4M3, p, nullptr, 100, pi,
                                nullptr), DS4A_E_NULL);
    EXPECT(ds4a_push_raw(1, 1, 12, 128, pf, p, pi, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_push_raw(1, 1, 512, 2048, pf, p, pi, nullptr), DS4A_E_UNSUPPORTED);
    EXPECT(ds4a_push_raw(1 << 24, 1 << 24, 4096, 128, pf, p, pi, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_push_raw(1, 1, 512, 128, pf, odd, pi, nullptr), DS4A_E_ALIGN);
    EXPECT(ds4a_frontier_push(1, 512, 0, pf, pf, pf, pl, pf, pf, nullptr), DS4A_E_SHAPE);
    EXPECT(ds4a_frontier_push(1, 512, 4, pf, pf, nullptr, pl, pf, pf, nullptr), DS4A_E_NULL);

    if (ds4a_version() < 2) g_fail = 1;
    printf("%s (%zu)\n", g_fail ? "FAILED" : "ok", acc);
    return g_fail;
}
