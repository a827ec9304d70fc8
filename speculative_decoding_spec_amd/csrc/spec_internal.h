// Internal declarations shared by the HIP translation units of libspec.
// Not part of the public ABI (that is include/spec.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spec {

// ---------------------------------------------------------------- qmv ----
// Work decomposition of one qmv call: one workgroup per 16 weight rows, its
// waves splitting K.  It depends on (bits, N, K) only, never on M, so row m of an
// M-row call reduces in exactly the same order as a one-row call.
struct QmvPlan {
    int n_tiles;          // 16-row tiles
    int n_pairs;          // 128-wide K steps (pairs of 64-groups)
    int waves;            // waves per workgroup (K split inside the workgroup)
    int tiles_per_wave;   // tiles each workgroup (and each of its waves) serves
    int stages;           // pairs in flight per wave (one pair per load stage)
};

QmvPlan qmv_plan(int bits, int N, int K);
size_t qmv_packed_bytes(int bits, int N, int K);
size_t qmv_packed_sb_bytes(int N, int K);
// Packs one matrix (w2 == nullptr) or a gate/up pair with alternating
// 16-row tiles (N = rows of each, packed as gate_up_rows(N) rows).
hipError_t launch_pack(int bits, const void *w, const uint16_t *scales,
                       const uint16_t *biases, const void *w2,
                       const uint16_t *scales2, const uint16_t *biases2, int N,
                       int K, void *w_packed, void *sb_packed, hipStream_t stream);
int gate_up_rows(int F);
// Draft-only 4-bit copy (G = 64) of a bf16 [N][K] matrix, interchange layout.
hipError_t launch_requantize_w4(const uint16_t *w, int N, int K, uint32_t *w4,
                                uint16_t *scales, uint16_t *biases, hipStream_t stream);
// interchange = false: w / sb are the packed tiles and scale/bias words of
// launch_pack (biases unused); true: w is the caller's row-major codes,
// sb the fp16 scales and biases the fp16 biases, each [N][K/64].
hipError_t launch_qmv(int bits, bool interchange, const void *w, const void *sb,
                      const uint16_t *biases, const uint16_t *x, float *y, int M, int N,
                      int K, hipStream_t stream);
// h (bf16 [M][F]) = silu(x G^T) * (x U^T) from a gate/up pair packed with
// alternating tiles.
hipError_t launch_qmv_gate_up_silu(int bits, const void *w_packed, const void *sb_packed,
                                   const uint16_t *x, uint16_t *h, int M, int F, int K,
                                   hipStream_t stream);
// The vector-ALU comparison variant on packed W4 weights, M = 1..4: y fp32
// [M][N] (F == 0), or the gated activation h bf16 [M][F] of a gate/up pair
// packed as N = gate_up_rows(F) rows (F > 0).
hipError_t launch_qmv_valu(const void *w_packed, const void *sb_packed, const uint16_t *x,
                           void *out, int M, int N, int K, int F, hipStream_t stream);

// ------------------------------------------------------------ sampling ----
struct SamplingParams {
    float scale;     // log2(e) / T, used as exp2((z - max) * scale)
    int k_eff;       // kept candidates before top-p (1 = greedy)
    float top_p;     // applied when use_p
    bool use_p;
    bool candidates; // true: distributions live on <= 256 sorted candidates
    bool block_stats; // full vocabulary, V % 4 == 0: the statistics pass also
                      // leaves each target row's 256-token block (max, sum of
                      // exponentials), so the draw need not re-read the row
    int merge_chunks; // > 0: full-vocabulary rows span this many chunks and the
                      // draw kernels merge their statistics themselves
    int chunk_blocks; // 256-token blocks per statistics chunk (block_stats)
};

struct AcceptPlan {
    int B, D, V;
    int rows;        // B * (2D + 1)
    int chunks;      // vocabulary chunks per row in the statistics pass
    int chunk_len;   // elements per chunk
    int nblocks;     // 256-token draw blocks per row
    int chunks3;     // draw-sum workgroups per sequence
    bool fused_draw;    // one fused decide/sum/draw workgroup per sequence
    int blocks_per_chunk3;
    size_t ws_bytes;
    // workspace offsets
    size_t off_chunk_stats, off_chunk_keys, off_row_final, off_row_keys, off_block_sums,
        off_block_stats;
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

// -------------------------------------------------------------- greedy ----
struct GreedyPlan {
    int B, D, V;
    int rows;        // B * (D + 1) target rows
    int chunks;      // vocabulary chunks per row
    int chunk_len;   // elements per chunk
    size_t ws_bytes;
};

GreedyPlan greedy_plan(int B, int D, int V);

// Enqueue greedy verification: the argmax pass over the target rows, then
// the per-sequence match.  draft_tokens may be null when D == 0.
hipError_t launch_greedy(const float *target, const int32_t *draft_tokens,
                         const GreedyPlan &plan, int32_t *accepted_len,
                         int32_t *next_token, void *ws, hipStream_t stream);

// ----------------------------------------------------------- recurrent ----
// Gated-delta-rule state (dk = dv = 128) over T steps with the innovation
// tape, and the commit of the first n[b] steps from the tape.
hipError_t launch_gdn_record(const float *S0, const float *q, const float *k, const float *v,
                             const float *alpha, const float *beta, int B, int T, int H,
                             float *o, float *delta, float *S_final, hipStream_t stream);
hipError_t launch_gdn_commit(float *S, const float *alpha, const float *k, const float *delta,
                             const int32_t *n_steps, int B, int T, int H, hipStream_t stream);
hipError_t launch_gdn_commit_record(float *S, const float *prev_alpha, const float *prev_k,
                                    const float *prev_delta, const int32_t *n_steps, int Tp,
                                    const float *q, const float *k, const float *v,
                                    const float *alpha, const float *beta, int B, int T, int H,
                                    float *o, float *delta, float *S_final, hipStream_t stream);

// ----------------------------------------------------------- measurement ----
// A plain streaming read of `bytes` (a multiple of 16) with `groups`
// workgroups; sink[g] receives the XOR of the 32-bit words workgroup g read.
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, int groups,
                              hipStream_t stream);

} // namespace spec
