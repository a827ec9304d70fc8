/*
 * spec.h -- C ABI of the MI355X (gfx950) speculative-decoding hot path.
 *
 * Two parts, as described by the MTPLX announcement (molayo1419.me) and its
 * Japanese re-post (ai-navigate-news):
 *
 *  1. The target model's verify pass over M = D + 1 positions (one per draft
 *     token plus the bonus position), whose linear layers are small-M
 *     group-quantized matrix-vector products ("Layer 0: MLX Runtime": the
 *     stock quantized matrix-vector kernel stalls at M = 3..6; the verify
 *     block over D + 1 positions is laid out in the savepearlharbor.com
 *     llama.cpp MTP article, section on how speculative decoding works).
 *  2. The probability-ratio (Leviathan-Chen) acceptance in fp32 per
 *     position, with residual (p - q)+ resampling on the first rejection and
 *     a bonus token when every draft is accepted ("Layer 2: Speculative
 *     cycle (the hot loop)").
 *
 * Conventions shared by every entry point:
 *  - All array pointers are device memory owned by the caller; the library
 *    never allocates, frees or retains them.  Layouts are row-major and
 *    contiguous.
 *  - Calls are asynchronous and stream ordered on `stream` (NULL = the
 *    default stream).  The library keeps no mutable global state beyond the
 *    per-GPU address of the fixed workspace of spec_verify_accept_noalloc;
 *    calls on different streams may run concurrently as long as they do not
 *    share a workspace (which all spec_verify_accept_noalloc calls on one GPU
 *    do).
 *  - Arguments are validated on the host first.  On failure the call returns
 *    SPEC_ERR_INVALID / SPEC_ERR_UNSUPPORTED / SPEC_ERR_WORKSPACE and
 *    enqueues nothing.  SPEC_ERR_DEVICE means a HIP call failed.
 *  - Workspaces: the caller allocates `*_workspace_size(...)` bytes of device
 *    memory, 256-byte aligned.  Its contents need no initialization and
 *    carry nothing from one call to the next (every call writes what it
 *    reads), so a workspace can be reused by any later call whose size query
 *    is not larger.  Calls sharing one workspace must be ordered on one
 *    stream.  No kernel of the library waits for another workgroup: there
 *    are no counters, spin waits or device-scope fences.
 */
#ifndef SPEC_H
#define SPEC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spec_status {
    SPEC_OK = 0,
    SPEC_ERR_INVALID = 1,     /* NULL pointer where one is required, size out of range */
    SPEC_ERR_UNSUPPORTED = 2, /* well formed but not implemented (group size, M > 16, alignment) */
    SPEC_ERR_WORKSPACE = 3,   /* workspace missing or smaller than its size query */
    SPEC_ERR_DEVICE = 4       /* a HIP runtime call failed */
} spec_status;

/* Static, NUL-terminated name of a status code ("SPEC_OK", ...). */
const char *spec_status_str(spec_status s);

/* Library version, major * 10000 + minor * 100 + patch. */
int spec_version(void);

/* ------------------------------------------------------------------ */
/* Verify qmv: y = x * W^T with affine group-quantized W.               */
/* ------------------------------------------------------------------ */
/*
 * Computes y[m][n] = sum_k x[m][k] * (s[n][k/G] * q[n][k] + b[n][k/G]) for
 * m < M, n < N: every weight of the target's linear layer is streamed once
 * and serves all M = D + 1 verify rows (affine group quantization as in the
 * mlxcel manual's "MTP and DFlash" page, draft block width section; MTPLX
 * "Layer 0: MLX Runtime", the small-M quantized matrix-vector product on the
 * model's own quantized weights).
 *
 * spec_qmv_w4 / spec_qmv_w8 read the weights as stored (interchange layout):
 *  w       W4: uint32 [N][K/8]; element k of row n is bits 4*(k%8)..4*(k%8)+3
 *          of word k/8 (unsigned code 0..15).  16-byte aligned.
 *          W8: uint8 [N][K]; one unsigned code 0..255 per byte.  16-byte aligned.
 *  scales  fp16 bit patterns [N][K/G]  (s), 2-byte aligned
 *  biases  fp16 bit patterns [N][K/G]  (b), 2-byte aligned
 *  x       bf16 bit patterns [M][K], 16-byte aligned
 *  y       fp32 [M][N], written (never read), 4-byte aligned
 *  M       1..16 rows (0 is a no-op).  Up to 8 rows fill the verify blocks of
 *          MTP depths D <= 7; 9..16 rows cover the 16-wide blocks of DFlash
 *          drafters (mlxcel manual, "MTP and DFlash": the comparison table's
 *          typical width, and split-mtp's block size of at most 16).
 *  N >= 0, 0 <= K < 2^24 with K % G == 0, G == 64, N <= 2^28
 *          (SPEC_ERR_UNSUPPORTED otherwise; a misaligned w or x is
 *          SPEC_ERR_UNSUPPORTED, a misaligned scales, biases or y
 *          SPEC_ERR_INVALID).
 *
 * spec_qmv_w4_packed / spec_qmv_w8_packed compute the same products from a
 * copy of the weights that spec_pack_w4 / spec_pack_w8 rearranged once, at
 * load time, into the order the kernel streams (tiles of 16 rows x 128 k,
 * each read by one wave as contiguous 1 KB runs; scale and bias interleaved
 * in one 32-bit word).  Both forms give bitwise the same y; the packed form
 * is the faster one on the verify shapes (a load instruction reads 1 KB of
 * contiguous memory instead of 64 or 128 bytes from each of 16 rows), at the
 * cost of a second copy of the weights.
 *  w_packed   spec_qmv_packed_weight_bytes(bits, N, K, G) bytes, 16-byte aligned
 *  sb_packed  spec_qmv_packed_sb_bytes(N, K, G) bytes, 4-byte aligned
 *  spec_pack_* take w, scales and biases in the interchange layout above.
 *
 * Results are deterministic, and row m of an M-row call is bitwise equal to
 * the one-row call on x[m] (the reduction order does not depend on M, also
 * across the 8-row boundary).
 */
spec_status spec_qmv_w4(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                        const uint16_t *x, float *y, int M, int N, int K, int G,
                        hipStream_t stream);

spec_status spec_qmv_w8(const uint8_t *w, const uint16_t *scales, const uint16_t *biases,
                        const uint16_t *x, float *y, int M, int N, int K, int G,
                        hipStream_t stream);

size_t spec_qmv_packed_weight_bytes(int bits, int N, int K, int G);
size_t spec_qmv_packed_sb_bytes(int N, int K, int G);

spec_status spec_pack_w4(const uint32_t *w, const uint16_t *scales,
                         const uint16_t *biases, int N, int K, int G,
                         void *w_packed, void *sb_packed, hipStream_t stream);

spec_status spec_pack_w8(const uint8_t *w, const uint16_t *scales,
                         const uint16_t *biases, int N, int K, int G,
                         void *w_packed, void *sb_packed, hipStream_t stream);

spec_status spec_qmv_w4_packed(const void *w_packed, const void *sb_packed,
                               const uint16_t *x, float *y, int M, int N, int K,
                               int G, hipStream_t stream);

spec_status spec_qmv_w8_packed(const void *w_packed, const void *sb_packed,
                               const uint16_t *x, float *y, int M, int N, int K,
                               int G, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Draft-only 4-bit copy of a weight matrix                             */
/* ------------------------------------------------------------------ */
/*
 * The target keeps its LM head at model precision; a separate 4-bit copy is
 * built in memory and used only for drafting (MTPLX announcement, "Layer 0"
 * custom kernels: draft-only requantised LM head, 29% less draft time).  The
 * quantizer is the min/max affine fit of the qmv path's format (a reading):
 * per row and group of G = 64 along K,
 *   b = min w,  s = (max w - min w) / 15  (fp32, rounded to nearest-even fp16),
 *   q = round_half_even((w - b) / s) with the fp16 s and b, in fp32,
 *       clamped to 0..15 (0 where s is 0 or not finite).
 *  w_bf16  bf16 bit patterns [N][K], 16-byte aligned; K % 64 == 0
 *  w4      uint32 [N][K/8] out (element k at bits 4*(k%8) of word k/8),
 *          16-byte aligned: the interchange layout of spec_pack_w4
 *  scales, biases  fp16 bit patterns [N][K/64] out
 * Results are bitwise deterministic (the codes are integer decisions taken
 * in fp32 with correctly rounded operations).
 */
spec_status spec_requantize_w4(const uint16_t *w_bf16, int N, int K, int G, uint32_t *w4,
                               uint16_t *scales, uint16_t *biases, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Gated MLP activation: h = silu(x G^T) * (x U^T), one launch           */
/* ------------------------------------------------------------------ */
/*
 * The MLP block dominates verify time (MTPLX re-post, "3) MLX verify
 * bottleneck"); in the Qwen target it is down(silu(gate(x)) * up(x)) (the
 * SiLU-gated form is a reading: the pages do not spell it out).  Gate and up
 * share x, so they stream as one launch, and the activation between the two
 * halves of the block is applied to their fp32 results in the same launch:
 *   h[m][f] = bf16( silu(g) * u ),  g = (x G^T)[m][f], u = (x U^T)[m][f],
 *   silu(g) = g / (1 + exp(-g)), rounded to nearest-even bf16,
 * which is the x of the down projection.  g and u are computed exactly as
 * spec_qmv_* computes each (bitwise the same fp32 values).
 *
 * spec_pack_gate_up packs G and U (each in the interchange layout of
 * spec_pack_w4 / spec_pack_w8 with N = F rows) into one buffer with
 * alternating 16-row tiles.  Its packed buffers have the sizes of an
 * R-row matrix, R = spec_gate_up_packed_rows(F) = 32 * ceil(F / 16):
 *   w_packed   spec_qmv_packed_weight_bytes(bits, R, K, G) bytes, 16-byte aligned
 *   sb_packed  spec_qmv_packed_sb_bytes(R, K, G) bytes, 4-byte aligned
 * spec_qmv_gate_up_silu reads them:
 *  bits    4 or 8, as packed
 *  x       bf16 [M][K], 16-byte aligned; M 0..16
 *  h       bf16 [M][F] out, 2-byte aligned
 *  F, K, G as packed (K % G == 0, G == 64)
 * Errors as for spec_qmv_*.
 */
int spec_gate_up_packed_rows(int F);

spec_status spec_pack_gate_up(int bits, const void *gate_w, const uint16_t *gate_scales,
                              const uint16_t *gate_biases, const void *up_w,
                              const uint16_t *up_scales, const uint16_t *up_biases,
                              int F, int K, int G, void *w_packed, void *sb_packed,
                              hipStream_t stream);

spec_status spec_qmv_gate_up_silu(int bits, const void *w_packed, const void *sb_packed,
                                  const uint16_t *x, uint16_t *h, int M, int F, int K,
                                  int G, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Vector-ALU comparison variants (W4, M = 1..4)                        */
/* ------------------------------------------------------------------ */
/*
 * The small-M product of spec_qmv_w4_packed and of spec_qmv_gate_up_silu
 * (bits 4) with the multiply-accumulate on the vector ALU
 * (v_dot2c_f32_bf16, two bf16 products per instruction) instead of the
 * matrix cores: the same packed weights, loads, x staging, affine fold and
 * reduction order over waves, kept to measure the one against the other at
 * the small M where most of each MFMA's A rows are zero (the MTPLX
 * announcement, "Layer 0: MLX Runtime", fixes its stock small-M kernel with
 * wider SIMD groups and unrolling, i.e. on the vector units).  Results obey
 * the same parity bound as spec_qmv_*, but are not bitwise equal to them
 * (the products are summed in another order).  Arguments, layouts and
 * errors as for spec_qmv_w4_packed and spec_qmv_gate_up_silu, except:
 *  M  0..4 (SPEC_ERR_UNSUPPORTED above)
 */
spec_status spec_qmv_w4_packed_valu(const void *w_packed, const void *sb_packed,
                                    const uint16_t *x, float *y, int M, int N, int K,
                                    int G, hipStream_t stream);

spec_status spec_qmv_gate_up_silu_w4_valu(const void *w_packed, const void *sb_packed,
                                          const uint16_t *x, uint16_t *h, int M, int F,
                                          int K, int G, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Sampling distribution                                                */
/* ------------------------------------------------------------------ */
/*
 * The filtered sampling distribution of a logits row (MTPLX "QWEN 3.6 27B @
 * 63 TPS": exact temperature sampling with top_p and top_k, not greedy-only;
 * greedy when T <= 0 or top_k == 1 as in the mlxcel manual's DFlash-family
 * drafter table):
 *   greedy            one-hot at the first maximum logit;
 *   otherwise         pi = softmax((z - max z) / T), then
 *   top-k             if 1 <= top_k < V: keep the top_k logits (ties to the
 *                     lower index), renormalize;
 *   top-p             if top_p < 1: keep the shortest prefix, in the same rank
 *                     order, whose mass reaches top_p (at least one token),
 *                     renormalize.
 * top_p < 1 requires 1 <= min(top_k, V) <= 256 (SPEC_ERR_UNSUPPORTED otherwise).
 * temperature must be finite (SPEC_ERR_INVALID otherwise).
 * A row holding NaN or +inf, or no finite logit, is invalid: its outputs are
 * NaN (probs) or -1 (tokens).
 */
size_t spec_sample_workspace_size(int R, int V, int top_k);

/* probs [R][V] fp32 = the distribution of each logits row [R][V]. */
spec_status spec_sample_probs(const float *logits, int R, int V,
                              float temperature, int top_k, float top_p,
                              float *probs, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* tokens [R] int32 = inverse-CDF draw (vocabulary order, first token whose
 * cumulative mass exceeds u * total) from each row with uniforms [R] in [0, 1). */
spec_status spec_sample_tokens(const float *logits, int R, int V,
                               float temperature, int top_k, float top_p,
                               const float *uniforms, int32_t *tokens,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Verification: ratio acceptance, residual resampling, bonus token     */
/* ------------------------------------------------------------------ */
/*
 * For each of B sequences with D drafts (MTPLX "Layer 2: Speculative cycle";
 * savepearlharbor.com article, how verification works):
 *   P_i = distribution of target row i (i = 0..D), Q_i = of draft row i
 *   (i < D), both with the same temperature / top_k / top_p;
 *   for i = 0..D-1: a_i = P_i(d_i) / Q_i(d_i) in fp32; accept d_i iff
 *   u_i < a_i; at the first rejection draw the next token from the
 *   residual max(0, P_i - Q_i) (from P_i if that residual is all zero);
 *   if all D are accepted draw the bonus token from P_D with u_D.
 * Draws are inverse-CDF draws in vocabulary order (the first token whose
 * cumulative weight exceeds u times the total).  The residual (the pages
 * name it, not its sampler) is drawn:
 *   - with top-k / top-p / greedy filters, by inverse CDF with u_D;
 *   - over the full vocabulary, by rejection from P_i: candidate k =
 *     0, 1, ... is the inverse-CDF draw from P_i with v_k and is kept iff
 *     a_k < (P_i - Q_i) / P_i at it (fp32); v_k, a_k are outputs 2k, 2k + 1
 *     of the SplitMix64 stream seeded with u_D's bit pattern (z = seed +
 *     (i + 1) * 0x9E3779B97F4A7C15, then the published mix; uniform = the
 *     top 24 bits * 2^-24); after 64 candidates none of which is kept, the
 *     residual's inverse CDF with output 128.  This has exactly the
 *     residual's distribution and reads one block of each row per
 *     candidate instead of the rows again.
 * The sequence emits draft_tokens[b][0..accepted_len-1] then next_token.
 *
 *  target_logits  fp32 [B][D+1][V]
 *  draft_logits   fp32 [B][D][V] (may be NULL when D == 0)
 *  draft_tokens   int32 [B][D]   (may be NULL when D == 0)
 *  uniforms       fp32 [B][D+1] in [0, 1): tests u_0..u_{D-1}, final draw
 *                 (or the residual's stream seed) u_D
 *  B >= 0, 0 <= D <= 15, 2 <= V < 2^24
 *  accepted_len   int32 [B] out: 0..D
 *  next_token     int32 [B] out
 *  p_draft, q_draft  fp32 [B][D] out, nullable: P_i(d_i) and Q_i(d_i)
 * A sequence with an invalid row or a draft token outside [0, V) gets
 * accepted_len = next_token = -1 (and NaN in p_draft / q_draft); other
 * sequences are unaffected.
 */
size_t spec_verify_accept_workspace(int B, int D, int V, int top_k);

spec_status spec_verify_accept(const float *target_logits,
                               const float *draft_logits,
                               const int32_t *draft_tokens,
                               const float *uniforms, int B, int D, int V,
                               float temperature, int top_k, float top_p,
                               int32_t *accepted_len, int32_t *next_token,
                               float *p_draft, float *q_draft, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * spec_verify_accept_noalloc: the same call for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): no workspace argument, and no allocation.  Its
 * workspace is a fixed array of SPEC_NOALLOC_SCRATCH_BYTES in device memory
 * that the library holds on each GPU it runs on until the process ends (its
 * device address is looked up once per GPU, on the first call there).
 *  - Arguments, results and errors as spec_verify_accept; a call whose
 *    workspace (spec_verify_accept_workspace for its B, D, V, top_k is an
 *    upper bound) would exceed SPEC_NOALLOC_SCRATCH_BYTES returns
 *    SPEC_ERR_WORKSPACE and enqueues nothing.
 *  - `stream` must belong to the current device (SPEC_ERR_INVALID
 *    otherwise); NULL is the current device's default stream.
 *  - Every call on one GPU uses the same array: calls that overlap on one
 *    GPU (on different streams, or from several host threads) race and give
 *    wrong results.  Calls ordered on one stream are safe; the array keeps
 *    the last call's contents, which no call reads.
 */
#define SPEC_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

spec_status spec_verify_accept_noalloc(const float *target_logits,
                                       const float *draft_logits,
                                       const int32_t *draft_tokens,
                                       const float *uniforms, int B, int D, int V,
                                       float temperature, int top_k, float top_p,
                                       int32_t *accepted_len, int32_t *next_token,
                                       float *p_draft, float *q_draft, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Greedy verification: match the drafts against the target's argmax   */
/* ------------------------------------------------------------------ */
/*
 * The sample-and-match loop with a greedy sampler (savepearlharbor.com
 * llama.cpp MTP article, how speculative decoding works; greedy means
 * T <= 0 or top_k == 1, mlxcel manual, DFlash-family drafter table).  For
 * each of B sequences, with t_i the first index of the largest logit of
 * target row i (i = 0..D):
 *   keep d_i while d_i == t_i; at the first mismatch accepted_len = i and
 *   next_token = t_i; if all D match, accepted_len = D, next_token = t_D.
 * Only the target logits are read.  For valid draft rows this is exactly
 * what spec_verify_accept returns with top_k = 1.
 *
 *  target_logits  fp32 [B][D+1][V]; 16-byte aligned when V % 4 == 0
 *  draft_tokens   int32 [B][D] (may be NULL when D == 0)
 *  B >= 0, 0 <= D <= 15, 2 <= V < 2^24, B * (D + 1) <= 2^23
 *  accepted_len   int32 [B] out: 0..D
 *  next_token     int32 [B] out
 * A sequence with an invalid target row (a NaN, a +inf, or no finite
 * logit) or a draft token outside [0, V) gets accepted_len = next_token =
 * -1; other sequences are unaffected.  The workspace holds one 16-byte
 * record per (row, vocabulary chunk).
 */
size_t spec_verify_greedy_workspace(int B, int D, int V);

spec_status spec_verify_greedy(const float *target_logits,
                               const int32_t *draft_tokens, int B, int D, int V,
                               int32_t *accepted_len, int32_t *next_token,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Recurrent (GDN) layer state: innovation tape capture and commit      */
/* ------------------------------------------------------------------ */
/*
 * The MTPLX announcement ("Layer 0" custom kernels: innovation-tape GDN
 * capture; "Layer 2": the tape commits accepted GDN state deltas and rolls
 * back rejected ones) keeps the recurrent state of the target out of
 * per-position snapshots during a speculative cycle.  Each verify position
 * records a small tuple; after acceptance only the accepted steps are
 * applied to the committed state.  The update is the gated delta rule, per
 * head (the pages name GDN without writing it out; this form is a reading):
 *     delta_t = beta_t * (v_t - alpha_t * S_{t-1} k_t)
 *     S_t     = alpha_t * S_{t-1} + delta_t k_t^T
 *     o_t     = S_t q_t
 * Layouts, all fp32, row-major:
 *  S0, S, S_final  [B][H][dv][dk], 16-byte aligned
 *  q, k            [B][T][H][dk] (the caller normalizes them), 16-byte aligned
 *  v, o, delta     [B][T][H][dv]
 *  alpha, beta     [B][T][H]
 *  dk = dv = 128, 0 <= T <= 16 (D + 1 verify positions), B * H < 2^28
 *
 * spec_gdn_record runs the T steps from S0 (left untouched), writes o and
 * the tape delta, and S_T to S_final when it is not NULL.
 * spec_gdn_commit rebuilds, in place in S (holding S0), the state after the
 * first n_steps[b] steps of sequence b from the tape (alpha, k, delta) alone;
 * after verification n_steps[b] = accepted_len[b] + 1 (the position of the
 * last committed token and the accepted drafts).  n_steps[b] <= 0 leaves S
 * unchanged (so accepted_len = -1 commits nothing), values above T count as
 * T.  Committing n steps reproduces bitwise the S_final that spec_gdn_record
 * returns when run for n steps.
 */
spec_status spec_gdn_record(const float *S0, const float *q, const float *k, const float *v,
                            const float *alpha, const float *beta, int B, int T, int H,
                            int dk, int dv, float *o, float *delta, float *S_final,
                            hipStream_t stream);

spec_status spec_gdn_commit(float *S, const float *alpha, const float *k, const float *delta,
                            const int32_t *n_steps, int B, int T, int H, int dk, int dv,
                            hipStream_t stream);

/*
 * spec_gdn_commit_record joins the two calls of a cycle boundary (the same
 * "Layer 2" cycle: commit the accepted steps, then capture the next verify
 * block) in one pass over the state.  In place in S it commits the first
 * n_steps[b] steps of the previous cycle's tape (prev_alpha [B][T_prev][H],
 * prev_k [B][T_prev][H][dk], prev_delta [B][T_prev][H][dv]) exactly as
 * spec_gdn_commit does, then records the T steps of the next verify block
 * from the committed state (q, k, v, alpha, beta -> o, delta, and S_T to
 * S_final when it is not NULL) exactly as spec_gdn_record does.  S is read
 * and written once, where the two calls read it twice and write it once.
 * Every output is bitwise the one of spec_gdn_commit followed by
 * spec_gdn_record on the same arguments.
 * T_prev = 0 commits nothing (then prev_* and n_steps may be NULL); T = 0
 * records nothing (then q, k, v, alpha, beta, o, delta may be NULL);
 * 0 <= T_prev, T <= 16.  Other workgroups read what one writes, so no
 * output (S, o, delta, S_final) may share memory with any other argument:
 * the previous and the next tape live in separate buffers
 * (SPEC_ERR_INVALID otherwise).  Layouts and alignment as above.
 */
spec_status spec_gdn_commit_record(float *S, const float *prev_alpha, const float *prev_k,
                                   const float *prev_delta, const int32_t *n_steps, int T_prev,
                                   const float *q, const float *k, const float *v,
                                   const float *alpha, const float *beta, int B, int T, int H,
                                   int dk, int dv, float *o, float *delta, float *S_final,
                                   hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Measurement: attainable HBM read rate                                */
/* ------------------------------------------------------------------ */
/*
 * The llama.cpp MTP article (section on the theoretical maximum of
 * generation speed) bounds token generation by memory bandwidth -- memory
 * speed over the bytes of the active weights -- and sets measured rates
 * beside that bound.  spec_stream_read is the measured side on this GPU: a
 * plain read of `bytes` bytes at `src` (16-byte aligned, bytes a multiple
 * of 16; every byte read once, with the 16-byte non-temporal loads the hot
 * kernels stream with), so a kernel's rate can be given as a share of the
 * published peak and of what a plain read attains.  SPEC_STREAM_READ_GROUPS
 * workgroups each fold the 32-bit words they read by XOR into sink[g]
 * (SPEC_STREAM_READ_GROUPS uint32 words, 4-byte aligned, overwritten), so
 * the XOR of all sink words is the XOR of all 32-bit words of src: no load
 * is dead, and a caller can check that all were read.  bytes = 0 writes
 * zeros.
 */
#define SPEC_STREAM_READ_GROUPS 2048

spec_status spec_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_H */
