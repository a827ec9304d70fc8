// Internal declarations shared by the HIP translation units of libspec.
// Not part of the public ABI (that is include/spec.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spec {

// ---------------------------------------------------------------- qmv ----
// Work decomposition of one qmv call.  It depends on (N, K) only, never on
// M, so row m of an M-row call reduces in exactly the same order as a
// one-row call.
struct QmvPlan {
    int n_blocks;        // 64-row blocks along N (one workgroup column each)
    int n_pairs;         // 128-wide K steps ("pairs" of two 64-groups)
    int splits;          // K splits across workgroups (1 = no partials)
    int pairs_per_split; // K steps per split
    size_t lds_bytes;    // dynamic LDS per workgroup
};

QmvPlan qmv_plan(int N, int K);
size_t qmv_workspace_bytes(const QmvPlan &p, int M, int N);
int qmv_max_rows();  // largest N a workspace's counter area supports
hipError_t launch_qmv(int bits, const void *w, const uint16_t *scales,
                      const uint16_t *biases, const uint16_t *x, float *y,
                      int M, int N, int K, const QmvPlan &plan, void *ws,
                      hipStream_t stream);

// ------------------------------------------------------------ sampling ----
struct SamplingParams {
    float scale;     // log2(e) / T, used as exp2((z - max) * scale)
    int k_eff;       // kept candidates before top-p (1 = greedy)
    float top_p;     // applied when use_p
    bool use_p;
    bool candidates; // true: distributions live on <= 256 sorted candidates
};

struct AcceptPlan {
    int B, D, V;
    int rows;        // B * (2D + 1)
    int chunks;      // vocabulary chunks per row in the statistics pass
    int chunk_len;   // elements per chunk
    int chunks3;     // vocabulary chunks per sequence in the draw pass
    int chunk3_len;
    size_t ws_bytes;
    // workspace offsets
    size_t off_row_cnt, off_seq_cnt, off_chunk_stats, off_chunk_keys,
        off_row_final, off_row_keys, off_seq_sums;
};

AcceptPlan accept_plan(int B, int D, int V, int k_eff, bool candidates);
SamplingParams sampling_params(float temperature, int top_k, float top_p, int V);

// Enqueue the full verification (statistics pass + acceptance/draw pass).
// draft_* may be null when D == 0.  accepted_len, p_draft, q_draft nullable.
hipError_t launch_accept(const float *target, const float *draft,
                         const int32_t *draft_tokens, const float *uniforms,
                         const AcceptPlan &plan, const SamplingParams &sp,
                         int32_t *accepted_len, int32_t *next_token,
                         float *p_draft, float *q_draft, void *ws,
                         hipStream_t stream);

// Statistics pass then a dense write of every row's distribution.
hipError_t launch_probs(const float *logits, const AcceptPlan &plan,
                        const SamplingParams &sp, float *probs, void *ws,
                        hipStream_t stream);

} // namespace spec
