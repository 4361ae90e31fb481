// api.hip — the extern "C" boundary of libds4attn (declared in include/ds4attn.h).
//
// Every entry point validates its arguments on the host, before any HIP call,
// and returns a status; on error nothing is enqueued and ds4a_last_error()
// holds a message.  Validation is pure host code, so it can be exercised on a
// machine without a GPU.  Fail closed: unsupported shapes are rejected, there
// is no alternative code path.
#include "../../include/ds4attn.h"
#include "launch.hpp"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

namespace {

thread_local char g_err[512];

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = 0;
    return DS4A_OK;
}

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

#define REQUIRE_PTR(p)                                                              \
    do {                                                                            \
        if (!(p)) return fail(DS4A_E_NULL, "%s: %s is NULL", fn, #p);               \
        if (misaligned(p)) return fail(DS4A_E_ALIGN, "%s: %s is not 16-byte aligned", fn, #p); \
    } while (0)

#define REQUIRE_PTR_AS(p, name)                                                     \
    do {                                                                            \
        if (!(p)) return fail(DS4A_E_NULL, "%s: %s is NULL", fn, name);             \
        if (misaligned(p)) return fail(DS4A_E_ALIGN, "%s: %s is not 16-byte aligned", fn, name); \
    } while (0)

#define OPTIONAL_PTR(p)                                                             \
    do {                                                                            \
        if ((p) && misaligned(p)) return fail(DS4A_E_ALIGN, "%s: %s is not 16-byte aligned", fn, #p); \
    } while (0)

constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxElems = int64_t(1) << 40;

int check_units(const char *fn, int U, int T, int64_t N) {
    if (U < 1 || T < 1) return fail(DS4A_E_SHAPE, "%s: U=%d and T=%d must be >= 1", fn, U, T);
    if (N < 1 || N > kMaxRows) return fail(DS4A_E_SHAPE, "%s: N=%lld must be in [1, 2^31-1]", fn, (long long)N);
    if ((int64_t)U * T > (int64_t(1) << 24)) return fail(DS4A_E_SHAPE, "%s: U*T=%lld too large", fn, (long long)U * T);
    if ((int64_t)U * T * N > kMaxElems) return fail(DS4A_E_SHAPE, "%s: U*T*N too large", fn);
    return DS4A_OK;
}

int check_attn_shape(const char *fn, int U, int T, int H, int D, int n_rot, int W, int64_t N, int K, int q_dtype,
                     double theta) {
    if (int rc = check_units(fn, U, T, N)) return rc;
    if (q_dtype != DS4A_F32 && q_dtype != DS4A_BF16) {
        if (q_dtype == DS4A_F16) return fail(DS4A_E_UNSUPPORTED, "%s: f16 queries are not supported", fn);
        return fail(DS4A_E_DTYPE, "%s: unknown q_dtype %d", fn, q_dtype);
    }
    if (H < 1 || D < 1 || n_rot < 0 || W < 0 || K < 1)
        return fail(DS4A_E_SHAPE, "%s: H=%d D=%d n_rot=%d W=%d K=%d out of range", fn, H, D, n_rot, W, K);
    if (D != DS4A_HEAD_DIM) return fail(DS4A_E_UNSUPPORTED, "%s: D=%d (only %d)", fn, D, DS4A_HEAD_DIM);
    if (n_rot != DS4A_ROPE_DIMS) return fail(DS4A_E_UNSUPPORTED, "%s: n_rot=%d (only %d)", fn, n_rot, DS4A_ROPE_DIMS);
    if (H % 16 != 0 || H > DS4A_MAX_HEADS)
        return fail(DS4A_E_UNSUPPORTED, "%s: H=%d (multiples of 16 up to %d)", fn, H, DS4A_MAX_HEADS);
    if (W % 32 != 0 || W > DS4A_MAX_WINDOW)
        return fail(DS4A_E_UNSUPPORTED, "%s: W=%d (multiples of 32 up to %d)", fn, W, DS4A_MAX_WINDOW);
    if (K > DS4A_MAX_TOPK) return fail(DS4A_E_UNSUPPORTED, "%s: K=%d (at most %d)", fn, K, DS4A_MAX_TOPK);
    if (!(theta > 0.0) || theta != theta) return fail(DS4A_E_SHAPE, "%s: rope_theta must be > 0", fn);
    return DS4A_OK;
}

int hip_status(const char *fn, hipError_t e) {
    if (e == hipSuccess) return ok();
    return fail(DS4A_E_HIP, "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of ds4a_indexer_topk_mqa: idx when the caller passes none, then the top-k's, then
// the attention's (whose counters must start at zero).
struct StepLayout {
    size_t idx, topk, attn, total;
};
StepLayout step_layout(int U, int T, int64_t N, int K, int H, int W) {
    StepLayout l;
    l.idx = round256((size_t)U * (size_t)T * (size_t)K * 4);
    l.topk = round256(ds4a::indexer_topk_workspace_bytes(U, T, N, K));
    l.attn = ds4a::plan_attn(U, T, H, W, K).workspace_bytes;
    l.total = l.idx + l.topk + l.attn;
    return l;
}

}  // namespace

extern "C" {

int ds4a_version(void) { return DS4A_VERSION; }

const char *ds4a_last_error(void) { return g_err; }

size_t ds4a_workspace_bytes(int which, int U, int T, int64_t N, int K, int H, int W) {
    if (which == 3) {                        // ds4a_dense_mqa: K ignored, N >= 0
        if (U < 1 || T < 1 || (int64_t)U * T > (int64_t(1) << 24) || N < 0 || N > DS4A_MAX_DENSE_ROWS) return 0;
        if (H < 16 || H % 16 || H > DS4A_MAX_HEADS || W < 0 || W % 32 || W > DS4A_MAX_WINDOW || W + N < 1) return 0;
        return ds4a::plan_attn(U, T, H, W, (int)N).workspace_bytes;
    }
    if (U < 1 || T < 1 || N < 1 || N > kMaxRows || K < 1 || K > DS4A_MAX_TOPK) return 0;
    if (which == 0) return ds4a::topk_workspace_bytes((int64_t)U * T, N, K);
    if (which == 2) return ds4a::indexer_topk_workspace_bytes(U, T, N, K);
    if (which == 4) {
        if (H < 16 || H % 16 || H > DS4A_MAX_HEADS || W < 0 || W % 32 || W > DS4A_MAX_WINDOW) return 0;
        return step_layout(U, T, N, K, H, W).total;
    }
    if (which == 1) {
        if (H < 16 || H % 16 || H > DS4A_MAX_HEADS || W < 0 || W % 32 || W > DS4A_MAX_WINDOW) return 0;
        return ds4a::plan_attn(U, T, H, W, K).workspace_bytes;
    }
    return 0;
}

namespace {

// Key rows of the bf16 (fp8 false) or E4M3 entry points, checked in argument order.
#define REQUIRE_KEYS(keys, fp8)                                                     \
    do {                                                                            \
        REQUIRE_PTR_AS((keys).k, (fp8) ? "idx_k8" : "idx_k");                       \
        if (fp8) REQUIRE_PTR_AS((keys).scale, "idx_k_scale");                       \
    } while (0)

static int indexer_score(const char *fn, int U, int T, int64_t N, int Hi, int Di, const void *idx_q, const float *idx_w,
                  ds4a::KeyRows idx_k, bool fp8, const int32_t *n_vis, float *scores, void *stream) {
    if (int rc = check_units(fn, U, T, N)) return rc;
    if (Hi != DS4A_INDEXER_HEADS || Di != DS4A_INDEXER_DIM)
        return fail(DS4A_E_UNSUPPORTED, "%s: Hi=%d Di=%d (only %d x %d)", fn, Hi, Di, DS4A_INDEXER_HEADS,
                    DS4A_INDEXER_DIM);
    REQUIRE_PTR(idx_q);
    REQUIRE_PTR(idx_w);
    REQUIRE_KEYS(idx_k, fp8);
    REQUIRE_PTR(scores);
    OPTIONAL_PTR(n_vis);
    return hip_status(fn, ds4a::launch_indexer(U, T, N, static_cast<const uint16_t *>(idx_q), idx_w, idx_k, n_vis,
                                               scores, static_cast<hipStream_t>(stream)));
}

static int indexer_topk(const char *fn, int U, int T, int64_t N, int Hi, int Di, int K, const void *idx_q,
                 const float *idx_w, ds4a::KeyRows idx_k, bool fp8, const int32_t *n_vis, int32_t *idx,
                 void *workspace, size_t workspace_bytes, void *stream) {
    if (int rc = check_units(fn, U, T, N)) return rc;
    if (Hi != DS4A_INDEXER_HEADS || Di != DS4A_INDEXER_DIM)
        return fail(DS4A_E_UNSUPPORTED, "%s: Hi=%d Di=%d (only %d x %d)", fn, Hi, Di, DS4A_INDEXER_HEADS,
                    DS4A_INDEXER_DIM);
    if (K < 1) return fail(DS4A_E_SHAPE, "%s: K=%d must be >= 1", fn, K);
    if (K > DS4A_MAX_TOPK) return fail(DS4A_E_UNSUPPORTED, "%s: K=%d (at most %d)", fn, K, DS4A_MAX_TOPK);
    REQUIRE_PTR(idx_q);
    REQUIRE_PTR(idx_w);
    REQUIRE_KEYS(idx_k, fp8);
    REQUIRE_PTR(idx);
    OPTIONAL_PTR(n_vis);
    const size_t need = ds4a::indexer_topk_workspace_bytes(U, T, N, K);
    if (need) {
        if (!workspace || workspace_bytes < need)
            return fail(DS4A_E_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                        workspace ? workspace_bytes : (size_t)0);
        if (misaligned(workspace)) return fail(DS4A_E_ALIGN, "%s: workspace is not 16-byte aligned", fn);
    }
    return hip_status(fn, ds4a::launch_indexer_topk(U, T, N, K, static_cast<const uint16_t *>(idx_q), idx_w, idx_k,
                                                    n_vis, idx, workspace, static_cast<hipStream_t>(stream)));
}

}  // namespace

int ds4a_indexer_score(int U, int T, int64_t N, int Hi, int Di, const void *idx_q, const float *idx_w,
                       const void *idx_k, const int32_t *n_vis, float *scores, void *stream) {
    return indexer_score("ds4a_indexer_score", U, T, N, Hi, Di, idx_q, idx_w, ds4a::KeyRows{idx_k, nullptr}, false,
                         n_vis, scores, stream);
}

int ds4a_indexer_score_fp8(int U, int T, int64_t N, int Hi, int Di, const void *idx_q, const float *idx_w,
                           const uint8_t *idx_k8, const float *idx_k_scale, const int32_t *n_vis, float *scores,
                           void *stream) {
    return indexer_score("ds4a_indexer_score_fp8", U, T, N, Hi, Di, idx_q, idx_w,
                         ds4a::KeyRows{idx_k8, idx_k_scale}, true, n_vis, scores, stream);
}

int ds4a_topk_select(int U, int T, int64_t N, int K, const float *scores, const int32_t *n_vis, int32_t *idx,
                     void *workspace, size_t workspace_bytes, void *stream) {
    const char *fn = "ds4a_topk_select";
    if (int rc = check_units(fn, U, T, N)) return rc;
    if (K < 1) return fail(DS4A_E_SHAPE, "%s: K=%d must be >= 1", fn, K);
    if (K > DS4A_MAX_TOPK) return fail(DS4A_E_UNSUPPORTED, "%s: K=%d (at most %d)", fn, K, DS4A_MAX_TOPK);
    REQUIRE_PTR(scores);
    REQUIRE_PTR(idx);
    OPTIONAL_PTR(n_vis);
    const size_t need = ds4a::topk_workspace_bytes((int64_t)U * T, N, K);
    if (need) {
        if (!workspace || workspace_bytes < need)
            return fail(DS4A_E_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                        workspace ? workspace_bytes : (size_t)0);
        if (misaligned(workspace)) return fail(DS4A_E_ALIGN, "%s: workspace is not 16-byte aligned", fn);
    }
    return hip_status(fn, ds4a::launch_topk((int64_t)U * T, N, K, scores, n_vis, idx, workspace,
                                            static_cast<hipStream_t>(stream)));
}

int ds4a_indexer_topk(int U, int T, int64_t N, int Hi, int Di, int K, const void *idx_q, const float *idx_w,
                      const void *idx_k, const int32_t *n_vis, int32_t *idx, void *workspace,
                      size_t workspace_bytes, void *stream) {
    return indexer_topk("ds4a_indexer_topk", U, T, N, Hi, Di, K, idx_q, idx_w, ds4a::KeyRows{idx_k, nullptr}, false,
                        n_vis, idx, workspace, workspace_bytes, stream);
}

int ds4a_indexer_topk_fp8(int U, int T, int64_t N, int Hi, int Di, int K, const void *idx_q, const float *idx_w,
                          const uint8_t *idx_k8, const float *idx_k_scale, const int32_t *n_vis, int32_t *idx,
                          void *workspace, size_t workspace_bytes, void *stream) {
    return indexer_topk("ds4a_indexer_topk_fp8", U, T, N, Hi, Di, K, idx_q, idx_w,
                        ds4a::KeyRows{idx_k8, idx_k_scale}, true, n_vis, idx, workspace, workspace_bytes, stream);
}

namespace {

// Compressed rows of the bf16 (comp_scale unused) or E4M3 (fp8) attention entry points,
// checked in argument order.
#define REQUIRE_COMP(comp, comp_scale, fp8)                                         \
    do {                                                                            \
        REQUIRE_PTR_AS(comp, (fp8) ? "comp_kv8" : "comp_kv");                       \
        if (fp8) REQUIRE_PTR_AS(comp_scale, "comp_scale");                          \
    } while (0)

// The allocation-free attention's scratch: counters at the start (zero when the code object
// loads, left zero by every call), records after them.  Each device holds its own copy; host
// code uses the device address looked up per device, never the symbol itself.
static __device__ __align__(256) unsigned char scratch[DS4A_SCRATCH_BYTES];

// scratch's address on the current device (looked up once per device).
static hipError_t scratch_on_device(unsigned char **out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static unsigned char *addr[kMaxDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = static_cast<unsigned char *>(p);
    }
    *out = addr[dev];
    return hipSuccess;
}

// noalloc: the workspace is the library's scratch (workspace and workspace_bytes unused).
static int sparse_mqa(const char *fn, int U, int T, int H, int D, int n_rot, int W, int64_t N, int K, const void *q,
               int q_dtype, const int64_t *q_pos, double rope_theta, const void *raw_kv, const int32_t *raw_vis,
               const void *comp_kv, const float *comp_scale, bool fp8, const int32_t *idx, float scale, float *out,
               void *workspace, size_t workspace_bytes, void *stream, bool noalloc = false) {
    if (int rc = check_attn_shape(fn, U, T, H, D, n_rot, W, N, K, q_dtype, rope_theta)) return rc;
    if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
        return fail(DS4A_E_SHAPE, "%s: scale must be finite", fn);
    if (N > DS4A_MAX_ATTN_ROWS)
        return fail(DS4A_E_UNSUPPORTED, "%s: N=%lld (at most %d rows per unit)", fn, (long long)N, DS4A_MAX_ATTN_ROWS);
    REQUIRE_PTR(q);
    REQUIRE_PTR(q_pos);
    if (W > 0) REQUIRE_PTR(raw_kv);
    OPTIONAL_PTR(raw_vis);
    REQUIRE_COMP(comp_kv, comp_scale, fp8);
    REQUIRE_PTR(idx);
    REQUIRE_PTR(out);
    const ds4a::AttnPlan plan = ds4a::plan_attn(U, T, H, W, K);
    if (noalloc) {
        const size_t records = plan.workspace_bytes - plan.count_bytes;
        if (plan.count_bytes > DS4A_SCRATCH_COUNT_BYTES || records > DS4A_SCRATCH_BYTES - DS4A_SCRATCH_COUNT_BYTES)
            return fail(DS4A_E_WORKSPACE,
                        "%s: this call needs %zu bytes of counters and %zu of records; the library's scratch "
                        "holds %u and %u", fn, plan.count_bytes, records, (unsigned)DS4A_SCRATCH_COUNT_BYTES,
                        (unsigned)(DS4A_SCRATCH_BYTES - DS4A_SCRATCH_COUNT_BYTES));
        unsigned char *base = nullptr;
        if (hipError_t e = scratch_on_device(&base); e != hipSuccess) return hip_status(fn, e);
        return hip_status(fn, ds4a::launch_attn_parts(U, T, H, W, N, K, q, q_dtype == DS4A_BF16, q_pos, rope_theta,
                                                      static_cast<const uint16_t *>(raw_kv), comp_kv,
                                                      fp8 ? comp_scale : nullptr, idx, nullptr, raw_vis, scale, out,
                                                      reinterpret_cast<uint32_t *>(base),
                                                      reinterpret_cast<float *>(base + DS4A_SCRATCH_COUNT_BYTES),
                                                      static_cast<hipStream_t>(stream)));
    }
    const size_t need = plan.workspace_bytes;
    if (need) {
        if (!workspace || workspace_bytes < need)
            return fail(DS4A_E_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                        workspace ? workspace_bytes : (size_t)0);
        if (misaligned(workspace)) return fail(DS4A_E_ALIGN, "%s: workspace is not 16-byte aligned", fn);
    }
    return hip_status(fn, ds4a::launch_attn(U, T, H, W, N, K, q, q_dtype == DS4A_BF16, q_pos, rope_theta,
                                           static_cast<const uint16_t *>(raw_kv), comp_kv, fp8 ? comp_scale : nullptr,
                                           idx, nullptr, raw_vis, scale, out, workspace,
                                           static_cast<hipStream_t>(stream)));
}

static int dense_mqa(const char *fn, int U, int T, int H, int D, int n_rot, int W, int64_t N, const void *q, int q_dtype,
              const int64_t *q_pos, double rope_theta, const void *raw_kv, const int32_t *raw_vis,
              const void *comp_kv, const float *comp_scale, bool fp8, const int32_t *n_vis, float scale, float *out,
              void *workspace, size_t workspace_bytes, void *stream) {
    if (U < 1 || T < 1) return fail(DS4A_E_SHAPE, "%s: U=%d and T=%d must be >= 1", fn, U, T);
    if ((int64_t)U * T > (int64_t(1) << 24)) return fail(DS4A_E_SHAPE, "%s: U*T=%lld too large", fn, (long long)U * T);
    if (N < 0) return fail(DS4A_E_SHAPE, "%s: N=%lld must be >= 0", fn, (long long)N);
    if (N > DS4A_MAX_DENSE_ROWS)
        return fail(DS4A_E_UNSUPPORTED, "%s: N=%lld (at most %d)", fn, (long long)N, DS4A_MAX_DENSE_ROWS);
    // the shape rules of ds4a_sparse_mqa, with K standing for the N dense rows (>= 1 there)
    if (int rc = check_attn_shape(fn, U, T, H, D, n_rot, W, N > 0 ? N : 1, 1, q_dtype, rope_theta)) return rc;
    if (W + N < 1) return fail(DS4A_E_SHAPE, "%s: W=%d and N=0: nothing to attend", fn, W);
    if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
        return fail(DS4A_E_SHAPE, "%s: scale must be finite", fn);
    REQUIRE_PTR(q);
    REQUIRE_PTR(q_pos);
    if (W > 0) REQUIRE_PTR(raw_kv);
    OPTIONAL_PTR(raw_vis);
    if (N > 0) REQUIRE_COMP(comp_kv, comp_scale, fp8);
    OPTIONAL_PTR(n_vis);
    REQUIRE_PTR(out);
    const ds4a::AttnPlan plan = ds4a::plan_attn(U, T, H, W, (int)N);
    if (plan.blocks >= (int64_t(1) << 31))
        return fail(DS4A_E_UNSUPPORTED, "%s: U*T=%lld queries over %lld rows is more than one launch holds", fn,
                    (long long)U * T, (long long)N);
    const size_t need = plan.workspace_bytes;
    if (need) {
        if (!workspace || workspace_bytes < need)
            return fail(DS4A_E_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                        workspace ? workspace_bytes : (size_t)0);
        if (misaligned(workspace)) return fail(DS4A_E_ALIGN, "%s: workspace is not 16-byte aligned", fn);
    }
    return hip_status(fn, ds4a::launch_attn(U, T, H, W, N, (int)N, q, q_dtype == DS4A_BF16, q_pos, rope_theta,
                                           static_cast<const uint16_t *>(raw_kv), comp_kv, fp8 ? comp_scale : nullptr,
                                           nullptr, n_vis, raw_vis, scale, out, workspace,
                                           static_cast<hipStream_t>(stream)));
}

}  // namespace

int ds4a_sparse_mqa(int U, int T, int H, int D, int n_rot, int W, int64_t N, int K, const void *q, int q_dtype,
                    const int64_t *q_pos, double rope_theta, const void *raw_kv, const int32_t *raw_vis,
                    const void *comp_kv, const int32_t *idx, float scale, float *out, void *workspace,
                    size_t workspace_bytes, void *stream) {
    return sparse_mqa("ds4a_sparse_mqa", U, T, H, D, n_rot, W, N, K, q, q_dtype, q_pos, rope_theta, raw_kv, raw_vis,
                      comp_kv, nullptr, false, idx, scale, out, workspace, workspace_bytes, stream);
}

int ds4a_sparse_mqa_noalloc(int U, int T, int H, int D, int n_rot, int W, int64_t N, int K, const void *q,
                            int q_dtype, const int64_t *q_pos, double rope_theta, const void *raw_kv,
                            const int32_t *raw_vis, const void *comp_kv, const int32_t *idx, float scale, float *out,
                            void *stream) {
    return sparse_mqa("ds4a_sparse_mqa_noalloc", U, T, H, D, n_rot, W, N, K, q, q_dtype, q_pos, rope_theta, raw_kv,
                      raw_vis, comp_kv, nullptr, false, idx, scale, out, nullptr, 0, stream, true);
}

int ds4a_sparse_mqa_fp8(int U, int T, int H, int D, int n_rot, int W, int64_t N, int K, const void *q,
                        int q_dtype, const int64_t *q_pos, double rope_theta, const void *raw_kv,
                        const int32_t *raw_vis, const uint8_t *comp_kv8, const float *comp_scale, const int32_t *idx,
                        float scale, float *out, void *workspace, size_t workspace_bytes, void *stream) {
    return sparse_mqa("ds4a_sparse_mqa_fp8", U, T, H, D, n_rot, W, N, K, q, q_dtype, q_pos, rope_theta, raw_kv,
                      raw_vis, comp_kv8, comp_scale, true, idx, scale, out, workspace, workspace_bytes, stream);
}

namespace {

// A1 + A2 + A3-A6 in one call.  Where the fused select runs with several chunks per query and
// the attention's 16-head kernel takes whole unions, the last merge level runs inside the
// attention kernel; otherwise the two calls' launches, one after the other.
static int indexer_topk_mqa(const char *fn, int U, int T, int64_t N, int Hi, int Di, int K, const void *idx_q,
                            const float *idx_w, ds4a::KeyRows idx_k, bool fp8k, const int32_t *n_vis, int H, int D,
                            int n_rot, int W, const void *q, int q_dtype, const int64_t *q_pos, double rope_theta,
                            const void *raw_kv, const int32_t *raw_vis, const void *comp_kv, const float *comp_scale,
                            bool fp8r, float scale, int32_t *idx, float *out, void *workspace, size_t workspace_bytes,
                            void *stream) {
    if (int rc = check_attn_shape(fn, U, T, H, D, n_rot, W, N, K, q_dtype, rope_theta)) return rc;
    if (Hi != DS4A_INDEXER_HEADS || Di != DS4A_INDEXER_DIM)
        return fail(DS4A_E_UNSUPPORTED, "%s: Hi=%d Di=%d (only %d x %d)", fn, Hi, Di, DS4A_INDEXER_HEADS,
                    DS4A_INDEXER_DIM);
    if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
        return fail(DS4A_E_SHAPE, "%s: scale must be finite", fn);
    if (N > DS4A_MAX_ATTN_ROWS)
        return fail(DS4A_E_UNSUPPORTED, "%s: N=%lld (at most %d rows per unit)", fn, (long long)N, DS4A_MAX_ATTN_ROWS);
    REQUIRE_PTR(idx_q);
    REQUIRE_PTR(idx_w);
    REQUIRE_KEYS(idx_k, fp8k);
    OPTIONAL_PTR(n_vis);
    REQUIRE_PTR(q);
    REQUIRE_PTR(q_pos);
    if (W > 0) REQUIRE_PTR(raw_kv);
    OPTIONAL_PTR(raw_vis);
    REQUIRE_COMP(comp_kv, comp_scale, fp8r);
    OPTIONAL_PTR(idx);
    REQUIRE_PTR(out);
    const StepLayout l = step_layout(U, T, N, K, H, W);
    if (!workspace || workspace_bytes < l.total)
        return fail(DS4A_E_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, l.total,
                    workspace ? workspace_bytes : (size_t)0);
    if (misaligned(workspace)) return fail(DS4A_E_ALIGN, "%s: workspace is not 16-byte aligned", fn);
    char *ws = static_cast<char *>(workspace);
    void *ws_topk = ws + l.idx;
    void *ws_attn = ws + l.idx + l.topk;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const uint16_t *iq = static_cast<const uint16_t *>(idx_q);
    const uint16_t *raw = static_cast<const uint16_t *>(raw_kv);
    const float *cs = fp8r ? comp_scale : nullptr;
    const ds4a::AttnPlan plan = ds4a::plan_attn(U, T, H, W, K);
    if (ds4a::indexer_candidates_apply(U, T, N, K) && ds4a::attn_dq_merge_apply(plan, 0)) {
        ds4a::CandList cl;
        hipError_t e = ds4a::launch_indexer_candidates(U, T, N, K, iq, idx_w, idx_k, n_vis, ws_topk,
                                                       ds4a::kAttnMergeMax, &cl, st);
        if (e != hipSuccess) return hip_status(fn, e);
        uint32_t *count = static_cast<uint32_t *>(ws_attn);
        float *part = reinterpret_cast<float *>(static_cast<char *>(ws_attn) + plan.count_bytes);
        return hip_status(fn, ds4a::launch_attn_dq_merge(plan, U, T, H, W, N, K, q, q_dtype == DS4A_BF16, q_pos,
                                                         rope_theta, raw, comp_kv, cs, cl, n_vis, raw_vis, scale, idx,
                                                         out, count, part, st));
    }
    int32_t *ix = idx ? idx : reinterpret_cast<int32_t *>(ws);
    hipError_t e = ds4a::launch_indexer_topk(U, T, N, K, iq, idx_w, idx_k, n_vis, ix, ws_topk, st);
    if (e != hipSuccess) return hip_status(fn, e);
    return hip_status(fn, ds4a::launch_attn(U, T, H, W, N, K, q, q_dtype == DS4A_BF16, q_pos, rope_theta, raw, comp_kv,
                                           cs, ix, nullptr, raw_vis, scale, out, ws_attn, st));
}

}  // namespace

int ds4a_indexer_topk_mqa(int U, int T, int64_t N, int Hi, int Di, int K, const void *idx_q, const float *idx_w,
                          const void *idx_k, const int32_t *n_vis, int H, int D, int n_rot, int W, const void *q,
                          int q_dtype, const int64_t *q_pos, double rope_theta, const void *raw_kv,
                          const int32_t *raw_vis, const void *comp_kv, float scale, int32_t *idx, float *out,
                          void *workspace, size_t workspace_bytes, void *stream) {
    return indexer_topk_mqa("ds4a_indexer_topk_mqa", U, T, N, Hi, Di, K, idx_q, idx_w, ds4a::KeyRows{idx_k, nullptr},
                            false, n_vis, H, D, n_rot, W, q, q_dtype, q_pos, rope_theta, raw_kv, raw_vis, comp_kv,
                            nullptr, false, scale, idx, out, workspace, workspace_bytes, stream);
}

int ds4a_indexer_topk_mqa_fp8(int U, int T, int64_t N, int Hi, int Di, int K, const void *idx_q,
                              const float *idx_w, const uint8_t *idx_k8, const float *idx_k_scale,
                              const int32_t *n_vis, int H, int D, int n_rot, int W, const void *q, int q_dtype,
                              const int64_t *q_pos, double rope_theta, const void *raw_kv, const int32_t *raw_vis,
                              const uint8_t *comp_kv8, const float *comp_scale, float scale, int32_t *idx, float *out,
                              void *workspace, size_t workspace_bytes, void *stream) {
    return indexer_topk_mqa("ds4a_indexer_topk_mqa_fp8", U, T, N, Hi, Di, K, idx_q, idx_w,
                            ds4a::KeyRows{idx_k8, idx_k_scale}, true, n_vis, H, D, n_rot, W, q, q_dtype, q_pos,
                            rope_theta, raw_kv, raw_vis, comp_kv8, comp_scale, true, scale, idx, out, workspace,
                            workspace_bytes, stream);
}

int ds4a_dense_mqa(int U, int T, int H, int D, int n_rot, int W, int64_t N, const void *q, int q_dtype,
                   const int64_t *q_pos, double rope_theta, const void *raw_kv, const int32_t *raw_vis,
                   const void *comp_kv, const int32_t *n_vis, float scale, float *out, void *workspace,
                   size_t workspace_bytes, void *stream) {
    return dense_mqa("ds4a_dense_mqa", U, T, H, D, n_rot, W, N, q, q_dtype, q_pos, rope_theta, raw_kv, raw_vis,
                     comp_kv, nullptr, false, n_vis, scale, out, workspace, workspace_bytes, stream);
}

int ds4a_dense_mqa_fp8(int U, int T, int H, int D, int n_rot, int W, int64_t N, const void *q, int q_dtype,
                       const int64_t *q_pos, double rope_theta, const void *raw_kv, const int32_t *raw_vis,
                       const uint8_t *comp_kv8, const float *comp_scale, const int32_t *n_vis, float scale,
                       float *out, void *workspace, size_t workspace_bytes, void *stream) {
    return dense_mqa("ds4a_dense_mqa_fp8", U, T, H, D, n_rot, W, N, q, q_dtype, q_pos, rope_theta, raw_kv, raw_vis,
                     comp_kv8, comp_scale, true, n_vis, scale, out, workspace, workspace_bytes, stream);
}

int ds4a_compress_rows(int U, int width, int ratio, const float *state_kv, const float *state_score,
                       const float *gain, float eps, int n_rot, const int64_t *row_pos, double rope_theta, int fp8,
                       void *out, int64_t out_stride, void *stream) {
    const char *fn = "ds4a_compress_rows";
    if (U < 1 || U > (1 << 24)) return fail(DS4A_E_SHAPE, "%s: U=%d must be in [1, 2^24]", fn, U);
    if (width < 4 || width % 4 || ratio < 1 || n_rot < 0 || n_rot % 2 || n_rot > width)
        return fail(DS4A_E_SHAPE, "%s: width=%d ratio=%d n_rot=%d out of range", fn, width, ratio, n_rot);
    if (width > DS4A_MAX_COMPRESS_WIDTH || ratio > DS4A_MAX_COMPRESS_RATIO || n_rot > 512)
        return fail(DS4A_E_UNSUPPORTED, "%s: width=%d ratio=%d n_rot=%d (width <= %d, ratio <= %d, n_rot <= 512)",
                    fn, width, ratio, n_rot, DS4A_MAX_COMPRESS_WIDTH, DS4A_MAX_COMPRESS_RATIO);
    if (!(eps >= 0.f) || eps == INFINITY) return fail(DS4A_E_SHAPE, "%s: eps must be finite and >= 0", fn);
    if (!(rope_theta > 0.0) || rope_theta != rope_theta) return fail(DS4A_E_SHAPE, "%s: rope_theta must be > 0", fn);
    if (fp8 != 0 && fp8 != 1) return fail(DS4A_E_SHAPE, "%s: fp8 must be 0 or 1", fn);
    if (out_stride < width) return fail(DS4A_E_SHAPE, "%s: out_stride=%lld < width", fn, (long long)out_stride);
    REQUIRE_PTR(state_kv);
    REQUIRE_PTR(state_score);
    REQUIRE_PTR(gain);
    REQUIRE_PTR(row_pos);
    REQUIRE_PTR(out);
    const ds4a::RowDest dst = {fp8 ? DS4A_ROW_BF16_FP8RT : DS4A_ROW_BF16, out, nullptr, out_stride, 1, nullptr,
                               nullptr};
    return hip_status(fn, ds4a::launch_compress(U, width, ratio, state_kv, state_score, gain, eps, n_rot, row_pos,
                                                rope_theta, dst, static_cast<hipStream_t>(stream)));
}

int ds4a_compress_append(int U, int width, int ratio, const float *state_kv, const float *state_score,
                         const float *gain, float eps, int n_rot, const int64_t *pos, const int64_t *row_pos,
                         double rope_theta, int format, void *comp, float *comp_scale, int64_t cap, int32_t *n_comp,
                         void *stream) {
    const char *fn = "ds4a_compress_append";
    if (U < 1 || U > (1 << 24)) return fail(DS4A_E_SHAPE, "%s: U=%d must be in [1, 2^24]", fn, U);
    if (width < 4 || width % 4 || ratio < 1 || n_rot < 0 || n_rot % 2 || n_rot > width)
        return fail(DS4A_E_SHAPE, "%s: width=%d ratio=%d n_rot=%d out of range", fn, width, ratio, n_rot);
    if (width > DS4A_MAX_COMPRESS_WIDTH || ratio > DS4A_MAX_COMPRESS_RATIO || n_rot > 512)
        return fail(DS4A_E_UNSUPPORTED, "%s: width=%d ratio=%d n_rot=%d (width <= %d, ratio <= %d, n_rot <= 512)",
                    fn, width, ratio, n_rot, DS4A_MAX_COMPRESS_WIDTH, DS4A_MAX_COMPRESS_RATIO);
    if (!(eps >= 0.f) || eps == INFINITY) return fail(DS4A_E_SHAPE, "%s: eps must be finite and >= 0", fn);
    if (!(rope_theta > 0.0) || rope_theta != rope_theta) return fail(DS4A_E_SHAPE, "%s: rope_theta must be > 0", fn);
    if (format != DS4A_ROW_BF16 && format != DS4A_ROW_BF16_FP8RT && format != DS4A_ROW_E4M3)
        return fail(DS4A_E_DTYPE, "%s: format=%d (DS4A_ROW_BF16, DS4A_ROW_BF16_FP8RT or DS4A_ROW_E4M3)", fn, format);
    if (cap < 1 || cap > kMaxRows || cap * (int64_t)width > kMaxElems / U)
        return fail(DS4A_E_SHAPE, "%s: cap=%lld out of range (U * cap * width <= 2^40)", fn, (long long)cap);
    REQUIRE_PTR(state_kv);
    REQUIRE_PTR(state_score);
    REQUIRE_PTR(gain);
    REQUIRE_PTR(pos);
    REQUIRE_PTR(row_pos);
    REQUIRE_PTR(comp);
    if (format == DS4A_ROW_E4M3) REQUIRE_PTR(comp_scale);
    REQUIRE_PTR(n_comp);
    const ds4a::RowDest dst = {format, comp, format == DS4A_ROW_E4M3 ? comp_scale : nullptr, cap * width, cap, pos,
                               n_comp};
    return hip_status(fn, ds4a::launch_compress(U, width, ratio, state_kv, state_score, gain, eps, n_rot, row_pos,
                                                rope_theta, dst, static_cast<hipStream_t>(stream)));
}

int ds4a_push_raw(int U, int T, int D, int cap, const float *kv, void *raw, int32_t *n_raw, void *stream) {
    const char *fn = "ds4a_push_raw";
    if (U < 1 || U > (1 << 24) || T < 1 || T > (1 << 24))
        return fail(DS4A_E_SHAPE, "%s: U=%d T=%d must be in [1, 2^24]", fn, U, T);
    if (D < 8 || D % 8 || cap < 1) return fail(DS4A_E_SHAPE, "%s: D=%d cap=%d out of range", fn, D, cap);
    if (D > 4096 || cap > DS4A_MAX_WINDOW)
        return fail(DS4A_E_UNSUPPORTED, "%s: D=%d cap=%d (D <= 4096, cap <= %d)", fn, D, cap, DS4A_MAX_WINDOW);
    if ((int64_t)U * T * D > kMaxElems) return fail(DS4A_E_SHAPE, "%s: U*T*D too large", fn);
    REQUIRE_PTR(kv);
    REQUIRE_PTR(raw);
    REQUIRE_PTR(n_raw);
    return hip_status(fn, ds4a::launch_push_raw(U, T, D, cap, kv, static_cast<uint16_t *>(raw), n_raw,
                                                static_cast<hipStream_t>(stream)));
}

int ds4a_frontier_push(int U, int width, int ratio, const float *kv, const float *score, const float *ape,
                       const int64_t *pos, float *state_kv, float *state_score, void *stream) {
    const char *fn = "ds4a_frontier_push";
    if (U < 1 || U > (1 << 24)) return fail(DS4A_E_SHAPE, "%s: U=%d must be in [1, 2^24]", fn, U);
    if (width < 4 || width % 4 || ratio < 1) return fail(DS4A_E_SHAPE, "%s: width=%d ratio=%d out of range", fn, width, ratio);
    if (width > DS4A_MAX_COMPRESS_WIDTH || ratio > DS4A_MAX_COMPRESS_RATIO)
        return fail(DS4A_E_UNSUPPORTED, "%s: width=%d ratio=%d (width <= %d, ratio <= %d)", fn, width, ratio,
                    DS4A_MAX_COMPRESS_WIDTH, DS4A_MAX_COMPRESS_RATIO);
    REQUIRE_PTR(kv);
    REQUIRE_PTR(score);
    REQUIRE_PTR(ape);
    REQUIRE_PTR(pos);
    REQUIRE_PTR(state_kv);
    REQUIRE_PTR(state_score);
    return hip_status(fn, ds4a::launch_frontier_push(U, width, ratio, kv, score, ape, pos, state_kv, state_score,
                                                     static_cast<hipStream_t>(stream)));
}

int ds4a_rope_q(int U, int T, int H, int D, int n_rot, const void *q, int q_dtype, const int64_t *q_pos,
                double rope_theta, float *q_out, void *stream) {
    const char *fn = "ds4a_rope_q";
    if (int rc = check_attn_shape(fn, U, T, H, D, n_rot, 0, 1, 1, q_dtype, rope_theta)) return rc;
    REQUIRE_PTR(q);
    REQUIRE_PTR(q_pos);
    REQUIRE_PTR(q_out);
    return hip_status(fn, ds4a::launch_rope(U, T, H, q, q_dtype == DS4A_BF16, q_pos, rope_theta, q_out,
                                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"
