// launch.hpp — internal launchers behind the C ABI (validated arguments only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ds4attn.h"

namespace ds4a {

// Units with at least this many queries take the many-queries (prefill) indexer.
constexpr int kIndexerManyQueries = 4;

// Indexer key rows as stored: bf16 [U][N][128] (scale == nullptr), or OCP E4M3FN codes
// [U][N][128] with one positive f32 scale per row [U][N] (the key is code value * scale).
struct KeyRows {
    const void *k;
    const float *scale;
};

// A1: scores f32 [Q][N], Q = U*T.
hipError_t launch_indexer(int U, int T, int64_t N, const uint16_t *idx_q, const float *idx_w, KeyRows idx_k,
                          const int32_t *n_vis, float *scores, hipStream_t stream);

// A2
size_t topk_workspace_bytes(int64_t Q, int64_t N, int K);
hipError_t launch_topk(int64_t Q, int64_t N, int K, const float *scores, const int32_t *n_vis,
                       int32_t *idx, void *workspace, hipStream_t stream);
// Chunked select: level-1 candidate lists ((key, row) pairs, K slots per chunk of `chunk` rows)
// at the start of the workspace, then the merge levels down to idx.
size_t topk_cand_workspace_bytes(int64_t Q, int64_t chunks, int K);
void topk_level1_buffers(void *workspace, int64_t Q, int64_t chunks, int K, uint32_t **keys, int32_t **ids);
hipError_t launch_topk_merge(int64_t Q, int64_t N, int K, int chunk, int64_t chunks, const int32_t *n_vis,
                             int32_t *idx, void *workspace, hipStream_t stream);
// A candidate list per query: query q's candidates are the first count(n_vis[q]) entries of
// keys/ids[q * stride ...], where count follows the chunk sizes of the levels that produced the
// list (first level on rows: each chunk of a level keeps min(K, its size)).
struct CandList {
    static constexpr int kMaxLevels = 12;
    const uint32_t *keys;
    const int32_t *ids;
    int64_t stride;
    int n_levels;
    int level_rows[kMaxLevels];
};
// The merge levels of the chunked select short of the last one: stops at the first list of
// at most max_last slots per query and describes it.
hipError_t launch_topk_merge_levels(int64_t Q, int64_t N, int K, int chunk, int64_t chunks, const int32_t *n_vis,
                                    void *workspace, int64_t max_last, CandList *list, hipStream_t stream);

// A1 + A2 fused: the selected set without materialising scores (decode shapes), or through
// scores kept in the workspace (many queries per unit).
size_t indexer_topk_workspace_bytes(int U, int T, int64_t N, int K);
hipError_t launch_indexer_topk(int U, int T, int64_t N, int K, const uint16_t *idx_q, const float *idx_w,
                               KeyRows idx_k, const int32_t *n_vis, int32_t *idx, void *workspace,
                               hipStream_t stream);
// A1 + A2 short of the last merge level, for a consumer that selects from the final list
// itself: only where the fused select runs with more than one chunk per query (same workspace
// as launch_indexer_topk).
bool indexer_candidates_apply(int U, int T, int64_t N, int K);
hipError_t launch_indexer_candidates(int U, int T, int64_t N, int K, const uint16_t *idx_q, const float *idx_w,
                                     KeyRows idx_k, const int32_t *n_vis, void *workspace, int64_t max_last,
                                     CandList *list, hipStream_t stream);

// A3-A6
// A3-A6.  Two kernels: attn.hip, workgroups of (query, 64-head group, union chunk), for many
// queries; attn_dq.hip, workgroups of (query, 16-head group, union chunk) with the dims split
// over the waves, for few.  comp: bf16 rows [U][N][512] (comp_scale == nullptr) or E4M3 codes
// [U][N][512] with f32 row scales [U][N].  raw_vis: int32 [U][T] raw rows of each query's
// window that take part (rows r < raw_vis, clamped to [0, W]), or nullptr for all W.  A split
// union keeps per-(query, 16-head group) arrival counters at the start of the workspace, zero
// before the first call and returned to zero by every call, then the records.
struct AttnPlan {
    bool dq = false;       // the 16-head kernel
    int n_hg;              // head groups (of 64, or of 16 for the 16-head kernel)
    int n_steps;           // union steps of 32 rows
    int steps_per_chunk;
    int n_chunks;
    size_t count_bytes;    // counters (0 when the union is not split)
    size_t workspace_bytes;
    int64_t blocks;        // grid size (padded to whole rounds of the 8 XCDs)
};
AttnPlan plan_attn(int U, int T, int H, int W, int K);        // chooses the kernel
AttnPlan plan_attn_wide(int U, int T, int H, int W, int K);
AttnPlan plan_attn_dq(int U, int T, int H, int W, int K);
hipError_t launch_attn_wide(const AttnPlan &p, int U, int T, int H, int W, int64_t N, int K, const void *q, int q_bf16,
                            const int64_t *q_pos, double theta, const uint16_t *raw, const void *comp,
                            const float *comp_scale, const int32_t *idx, const int32_t *n_vis, const int32_t *raw_vis,
                            float scale, float *out, uint32_t *count, float *part, hipStream_t stream);
hipError_t launch_attn_dq(const AttnPlan &p, int U, int T, int H, int W, int64_t N, int K, const void *q, int q_bf16,
                          const int64_t *q_pos, double theta, const uint16_t *raw, const void *comp,
                          const float *comp_scale, const int32_t *idx, const int32_t *n_vis, const int32_t *raw_vis,
                          float scale, float *out, uint32_t *count, float *part, hipStream_t stream);
// The 16-head kernel with the last top-k merge level inside (sparse unions of at most 48 steps,
// lists of at most 6,144 candidates per query): the rows of each query are selected from cl by
// the workgroups themselves (the set the top-k kernels would write; a workgroup of a split
// union selects them all and attends its chunk's), and written to idx_out when it is not null.
// cand_nvis: the indexer's visible rows per query (NULL: all N).  count, part: as for
// launch_attn_parts (used when the union is split).
constexpr int64_t kAttnMergeMax = 6144;      // candidates per query the in-kernel merge takes
bool attn_dq_merge_apply(const AttnPlan &p, int64_t list_stride);
hipError_t launch_attn_dq_merge(const AttnPlan &p, int U, int T, int H, int W, int64_t N, int K, const void *q,
                                int q_bf16, const int64_t *q_pos, double theta, const uint16_t *raw, const void *comp,
                                const float *comp_scale, const CandList &cl, const int32_t *cand_nvis,
                                const int32_t *raw_vis, float scale, int32_t *idx_out, float *out, uint32_t *count,
                                float *part, hipStream_t stream);
// As launch_attn with the counters and the records given apart (count: plan.count_bytes,
// zero before the call and left zero; part: plan.workspace_bytes - plan.count_bytes).
hipError_t launch_attn_parts(int U, int T, int H, int W, int64_t N, int K, const void *q, int q_bf16,
                             const int64_t *q_pos, double theta, const uint16_t *raw, const void *comp,
                             const float *comp_scale, const int32_t *idx, const int32_t *n_vis, const int32_t *raw_vis,
                             float scale, float *out, uint32_t *count, float *part, hipStream_t stream);
hipError_t launch_attn(int U, int T, int H, int W, int64_t N, int K, const void *q, int q_bf16,
                       const int64_t *q_pos, double theta, const uint16_t *raw, const void *comp,
                       const float *comp_scale, const int32_t *idx, const int32_t *n_vis, const int32_t *raw_vis,
                       float scale, float *out, void *workspace, hipStream_t stream);
// Where an emitted compressed row goes.  format (DS4A_ROW_* in the public header): bf16
// values, bf16 values after the FP8 round trip, or E4M3 codes (uint8) plus the row's scale.
// The row of unit u is row n_rows[u] (0 if n_rows is null) of a cache whose units are
// unit_stride elements apart and hold cap rows of `width` elements; scales (E4M3) at
// scale[u * cap + row].  With emit_pos, only units with emit_pos[u] mod ratio == ratio - 1
// emit, and n_rows counts the rows emitted (also past cap, where nothing is written).
struct RowDest {
    int format;
    void *out;
    float *scale;
    int64_t unit_stride;
    int64_t cap;
    const int64_t *emit_pos;
    int32_t *n_rows;
};
hipError_t launch_compress(int U, int width, int ratio, const float *state_kv, const float *state_score,
                           const float *gain, float eps, int n_rot, const int64_t *row_pos, double theta,
                           const RowDest &dst, hipStream_t stream);
// Cache upkeep: raw-window push (kv f32 [U][T][D] into f16 [U][cap][D], counts n_raw [U]) and
// the compressor frontier push (row pos mod ratio of f32 [U][ratio][width]).
hipError_t launch_push_raw(int U, int T, int D, int cap, const float *kv, uint16_t *raw, int32_t *n_raw,
                           hipStream_t stream);
hipError_t launch_frontier_push(int U, int width, int ratio, const float *kv, const float *score, const float *ape,
                                const int64_t *pos, float *state_kv, float *state_score, hipStream_t stream);
hipError_t launch_rope(int U, int T, int H, const void *q, int q_bf16, const int64_t *q_pos,
                       double theta, float *q_out, hipStream_t stream);

}  // namespace ds4a
