/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the speculative-decoding hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no
 * source, header, table or constant with the HIP library, and the HIP
 * library never calls it.
 *
 * What it computes, and where the pages define it:
 *
 *   qmv       y[m][n] = sum_k x[m][k] * (s[n][k/G] * q[n][k] + b[n][k/G])
 *             Affine group-quantized weights ("4-bit MLX", "affine-quantized
 *             target"): mlxcel manual page "MTP and DFlash", section on the
 *             draft block width; MTPLX announcement (molayo1419.me), section
 *             "Layer 0: MLX Runtime" (small-M quantized matrix-vector kernel).
 *             Plain definition: dequantize every weight, then an fp64 dot
 *             product summed sequentially in k order.
 *
 *   gate_up_silu
 *             h = silu(x W_gate^T) * (x W_up^T), rounded to bf16: the MLP
 *             block's activation between its projections (MTPLX re-post,
 *             "3) MLX verify bottleneck": MLP operations dominate verify;
 *             the SiLU-gated form of the Qwen target is a reading).
 *
 *   probs     The sampling distribution at temperature T with top-k and
 *             top-p: MTPLX announcement, "QWEN 3.6 27B @ 63 TPS" (T 0.6,
 *             top_p 0.95, top_k 20; exact temperature sampling, not greedy).
 *             Greedy when T <= 0 or top_k == 1: mlxcel manual, DFlash-family
 *             drafter table (LFM2 DSpark row: sampling means T > 0 and
 *             top_k != 1).
 *
 *   accept    Probability-ratio (Leviathan-Chen) acceptance per position in
 *             fp32, residual (p - q)+ on the first rejection, bonus token
 *             when every draft is accepted: MTPLX announcement, "Layer 2:
 *             Speculative cycle (the hot loop)"; the same in the Japanese
 *             re-post (ai-navigate-news), "Layer 2".  D accepted drafts give
 *             D + 1 tokens and a full rejection still gives one:
 *             savepearlharbor.com llama.cpp MTP article, section on how
 *             speculative decoding works.
 *
 *   gdn       Innovation-tape capture and commit of the recurrent (GDN)
 *             state: MTPLX announcement, "Layer 0" custom kernels and
 *             "Layer 2" (the tape commits accepted state deltas); the gated
 *             delta rule is a reading.
 *
 *   requantize_w4
 *             The draft-only 4-bit LM head: MTPLX announcement, "Layer 0"
 *             custom kernels; the min/max affine fit is a reading.
 *
 *   greedy    Verification with greedy sampling: keep each draft while it
 *             equals the target's argmax at its position, emit the target's
 *             argmax at the first mismatch (or at the bonus position):
 *             savepearlharbor.com llama.cpp MTP article, how speculative
 *             decoding works; greedy is T <= 0 or top_k == 1 (mlxcel manual,
 *             DFlash-family drafter table).
 *
 * Readings taken where the pages are silent are listed in the repository's
 * design notes; each is restated at the function that takes it.
 *
 * Build: gcc -O2 -fPIC -shared -ffp-contract=off oracle.c -o liboracle.so -lm
 * (no fused multiply-add, no fast-math: every operation is a plain IEEE op).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Number formats, decoded from their IEEE definitions.                 */
/* ------------------------------------------------------------------ */

/* IEEE 754 binary16 bit pattern -> double (exact). */
static double half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25); /* (1024 + f) * 2^(e - 15 - 10) */
    return sign ? -v : v;
}

/* bfloat16 bit pattern -> double: bf16 is the upper half of a binary32. */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_half_to_double(uint16_t h) { return half_to_double(h); }
double oracle_bf16_to_double(uint16_t b) { return bf16_to_double(b); }

/* ------------------------------------------------------------------ */
/* qmv                                                                  */
/* ------------------------------------------------------------------ */

/* Quantized code of weight (n, k).
 * W4: uint32 words, row-major [N][K/8]; element k sits in bits 4*(k%8)..+3
 *     of word k/8 (little-endian nibble order within the word).
 * W8: one byte per element, row-major [N][K]. */
static unsigned code_at(int bits, const void *w, long K, long n, long k)
{
    if (bits == 4) {
        const uint32_t *w4 = (const uint32_t *)w;
        uint32_t word = w4[n * (K / 8) + k / 8];
        return (word >> (4 * (k % 8))) & 0xFu;
    }
    return ((const uint8_t *)w)[n * K + k];
}

/* One output: y[m][n] = sum_k xhat[m][k] * what[n][k], sequential in k,
 * with what = s * q + b decoded exactly in fp64 (s, b are fp16; q <= 255 so
 * s * q + b is exact in a double).  Also returns sum_k |xhat * what|, the
 * magnitude the tolerance of a near-zero output is scaled by. */
static double qmv_one(int bits, const void *w, const uint16_t *scales,
                      const uint16_t *biases, const uint16_t *x, long K, long G,
                      long m, long n, double *abs_sum)
{
    long ng = K / G;
    double acc = 0.0, mag = 0.0;
    for (long k = 0; k < K; ++k) {
        double s = half_to_double(scales[n * ng + k / G]);
        double b = half_to_double(biases[n * ng + k / G]);
        double q = (double)code_at(bits, w, K, n, k);
        double what = s * q + b;
        double xh = bf16_to_double(x[m * K + k]);
        acc += xh * what;
        mag += fabs(xh * what);
    }
    if (abs_sum)
        *abs_sum = mag;
    return acc;
}

/* Returns 0, or -1 on an argument error (nothing written). */
static int qmv_args_ok(int bits, long M, long N, long K, long G)
{
    if (bits != 4 && bits != 8)
        return 0;
    if (M < 0 || N < 0 || K < 0 || G <= 0 || K % G != 0)
        return 0;
    if (bits == 4 && K % 8 != 0)
        return 0;
    return 1;
}

/* Rows n0..n1-1 of all M outputs: y[m][n - n0], y laid out [M][n1 - n0].
 * abs_sum (nullable) gets sum_k |xhat * what| with the same layout. */
int oracle_qmv(int bits, const void *w, const uint16_t *scales,
               const uint16_t *biases, const uint16_t *x, long M, long N,
               long K, long G, long n0, long n1, double *y, double *abs_sum)
{
    if (!qmv_args_ok(bits, M, N, K, G) || n0 < 0 || n1 > N || n0 > n1)
        return -1;
    long w_out = n1 - n0;
    for (long m = 0; m < M; ++m)
        for (long n = n0; n < n1; ++n) {
            double mag;
            y[m * w_out + (n - n0)] =
                qmv_one(bits, w, scales, biases, x, K, G, m, n, &mag);
            if (abs_sum)
                abs_sum[m * w_out + (n - n0)] = mag;
        }
    return 0;
}

/* Selected outputs (m_idx[i], n_idx[i]) one by one, for sampled checks of
 * shapes too large to compute whole. */
int oracle_qmv_points(int bits, const void *w, const uint16_t *scales,
                      const uint16_t *biases, const uint16_t *x, long M,
                      long N, long K, long G, const long *m_idx,
                      const long *n_idx, long count, double *y,
                      double *abs_sum)
{
    if (!qmv_args_ok(bits, M, N, K, G))
        return -1;
    for (long i = 0; i < count; ++i) {
        if (m_idx[i] < 0 || m_idx[i] >= M || n_idx[i] < 0 || n_idx[i] >= N)
            return -1;
    }
    for (long i = 0; i < count; ++i) {
        double mag;
        y[i] = qmv_one(bits, w, scales, biases, x, K, G, m_idx[i], n_idx[i],
                       &mag);
        if (abs_sum)
            abs_sum[i] = mag;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* SiLU-gated MLP activation                                            */
/* ------------------------------------------------------------------ */

/* Round-to-nearest-even of a double to bfloat16 (8 significant bits, the
 * exponent range of binary32, subnormals included), as its bit pattern.
 * Direct from the double, so there is no double rounding. */
uint16_t oracle_double_to_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0;
    if (v == 0.0)
        return signbit(v) ? 0x8000 : 0x0000;
    int e;
    frexp(fabs(v), &e);                 /* |v| = f * 2^e, f in [0.5, 1) */
    int ulp_exp = e - 8;                /* 8 significant bits */
    if (ulp_exp < -133)                 /* below the normal range: fixed ulp */
        ulp_exp = -133;
    double q = ldexp(v, -ulp_exp);      /* exact: a power-of-two scaling */
    double r = nearbyint(q);            /* ties to even (default rounding) */
    double rv = ldexp(r, ulp_exp);
    if (fabs(rv) >= ldexp(1.0, 128))
        return v > 0 ? 0x7F80 : 0xFF80;
    float f = (float)rv;                /* exact: rv has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* The gated activation of the MLP block: h[m][n] = silu(g) * u with
 * g = (x W_gate^T)[m][n], u = (x W_up^T)[m][n] (each the plain qmv of this
 * file, in fp64) and silu(g) = g / (1 + exp(-g)).  The pages put the MLP at
 * about half of verify time (MTPLX re-post, "3) MLX verify bottleneck")
 * without spelling out its form; the target is a Qwen model, whose MLP is
 * this SiLU-gated product followed by the down projection (a reading).  h
 * feeds the down projection as bf16, like every qmv input, so h_bf16 is h
 * rounded to nearest-even bf16.  Rows n0..n1-1, laid out [M][n1 - n0];
 * either output may be NULL. */
int oracle_gate_up_silu(int bits, const void *gw, const uint16_t *gs,
                        const uint16_t *gb, const void *uw, const uint16_t *us,
                        const uint16_t *ub, const uint16_t *x, long M, long F,
                        long K, long G, long n0, long n1, double *h,
                        uint16_t *h_bf16)
{
    if (!qmv_args_ok(bits, M, F, K, G) || n0 < 0 || n1 > F || n0 > n1)
        return -1;
    long w_out = n1 - n0;
    for (long m = 0; m < M; ++m)
        for (long n = n0; n < n1; ++n) {
            double g = qmv_one(bits, gw, gs, gb, x, K, G, m, n, NULL);
            double u = qmv_one(bits, uw, us, ub, x, K, G, m, n, NULL);
            double v = g / (1.0 + exp(-g)) * u;
            if (h)
                h[m * w_out + (n - n0)] = v;
            if (h_bf16)
                h_bf16[m * w_out + (n - n0)] = oracle_double_to_bf16(v);
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Sampling distribution                                                */
/* ------------------------------------------------------------------ */

/* Rank order used by both filters: logit descending, then index ascending.
 * Softmax is monotone in the logit, so this is the probability order with a
 * fixed tie-break (lower index first).  Records carry their own logit, so
 * sorting needs no shared state and the oracle is safe to call from several
 * threads at once. */
typedef struct {
    float z;
    long idx;
} ranked;

static int rank_cmp(const void *pa, const void *pb)
{
    const ranked *a = (const ranked *)pa, *b = (const ranked *)pb;
    if (a->z > b->z)
        return -1;
    if (a->z < b->z)
        return 1;
    return (a->idx < b->idx) ? -1 : (a->idx > b->idx);
}

/* A row is usable when it has no NaN, no +inf and at least one finite
 * logit (-inf entries are allowed and get probability zero). */
static int row_valid(const float *z, long V)
{
    int finite = 0;
    for (long i = 0; i < V; ++i) {
        if (isnan(z[i]) || (isinf(z[i]) && z[i] > 0))
            return 0;
        if (isfinite(z[i]))
            finite = 1;
    }
    return finite;
}

/* Filtered sampling distribution of one logits row, in fp64.
 *   1. Greedy when !(T > 0) or top_k == 1: one-hot at the first maximum.
 *   2. pi = exp((z - max z) / T) / sum, with T taken at its fp32 value.
 *   3. top-k when 1 <= top_k < V: keep the top_k tokens in rank order,
 *      renormalize.
 *   4. top-p when top_p < 1: over the kept tokens in rank order, keep the
 *      shortest prefix whose mass reaches top_p (at least one token),
 *      renormalize.
 * The order temperature -> top-k -> top-p is a reading: the pages name the
 * three settings together but never their order.
 * Returns 0, or -1 for an invalid row (out untouched). */
int oracle_probs(const float *z, long V, float T, int top_k, float top_p,
                 double *out)
{
    if (V < 1 || !row_valid(z, V))
        return -1;
    long amax = 0;
    for (long i = 1; i < V; ++i)
        if (z[i] > z[amax])
            amax = i;
    if (!(T > 0.0f) || top_k == 1) {
        for (long i = 0; i < V; ++i)
            out[i] = 0.0;
        out[amax] = 1.0;
        return 0;
    }

    double t = (double)T, zmax = (double)z[amax], sum = 0.0;
    for (long i = 0; i < V; ++i) {
        out[i] = exp(((double)z[i] - zmax) / t);
        sum += out[i];
    }
    for (long i = 0; i < V; ++i)
        out[i] /= sum;

    int use_k = (top_k >= 1 && (long)top_k < V);
    int use_p = (top_p < 1.0f);
    if (!use_k && !use_p)
        return 0;

    ranked *rec = (ranked *)malloc(sizeof(ranked) * (size_t)V);
    long *order = (long *)malloc(sizeof(long) * (size_t)V);
    if (!rec || !order) {
        free(rec);
        free(order);
        return -2;
    }
    for (long i = 0; i < V; ++i) {
        rec[i].z = z[i];
        rec[i].idx = i;
    }
    qsort(rec, (size_t)V, sizeof(ranked), rank_cmp);
    for (long i = 0; i < V; ++i)
        order[i] = rec[i].idx;
    free(rec);

    long kept = V;
    if (use_k) {
        kept = top_k;
        double s = 0.0;
        for (long j = 0; j < kept; ++j)
            s += out[order[j]];
        for (long j = kept; j < V; ++j)
            out[order[j]] = 0.0;
        for (long j = 0; j < kept; ++j)
            out[order[j]] /= s;
    }
    if (use_p) {
        double cum = 0.0, tp = (double)top_p;
        long cut = kept;
        for (long j = 0; j < kept; ++j) {
            cum += out[order[j]];
            if (cum >= tp) {
                cut = j + 1;
                break;
            }
        }
        double s = 0.0;
        for (long j = 0; j < cut; ++j)
            s += out[order[j]];
        for (long j = cut; j < kept; ++j)
            out[order[j]] = 0.0;
        for (long j = 0; j < cut; ++j)
            out[order[j]] /= s;
    }
    free(order);
    return 0;
}

/* Inverse CDF in vocabulary order: c_x = sum_{y <= x} w_y (fp64), and the
 * draw is the first x with c_x > u * c_{V-1}.  The strict comparison means a
 * zero-weight token is never drawn.  Returns -1 if the weights sum to zero.
 * margin (nullable) receives the distance of u * c_{V-1} to the nearer
 * boundary of the drawn token's interval, relative to c_{V-1}: a draw whose
 * margin is below a rounding tolerance may come out as a neighbour under
 * another summation order. */
static long inv_cdf_margin(const double *wts, long V, float u, double *margin)
{
    double total = 0.0;
    for (long x = 0; x < V; ++x)
        total += wts[x];
    if (margin)
        *margin = INFINITY;
    if (!(total > 0.0))
        return -1;
    double target = (double)u * total, c = 0.0;
    long last_pos = -1;
    for (long x = 0; x < V; ++x) {
        const double before = c;
        c += wts[x];
        if (wts[x] > 0.0)
            last_pos = x;
        if (c > target) {
            if (margin)
                *margin = fmin(c - target, target - before) / total;
            return x;
        }
    }
    if (margin)
        *margin = 0.0;
    return last_pos; /* unreachable for u < 1; guards rounding at the end */
}

static long inv_cdf(const double *wts, long V, float u)
{
    return inv_cdf_margin(wts, V, u, NULL);
}

/* SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014), used as a counter-based generator:
 * output i of the stream with seed s is the finalizer applied to
 * s + (i + 1) * 0x9E3779B97F4A7C15 (mod 2^64). */
uint64_t oracle_splitmix64(uint64_t seed, uint64_t i)
{
    uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Output i of the stream as a uniform on [0, 1): its top 24 bits times 2^-24,
 * an exact fp32 value. */
float oracle_stream_uniform(uint64_t seed, uint64_t i)
{
    return (float)(oracle_splitmix64(seed, i) >> 40) * 0x1p-24f;
}

/* One token drawn from the filtered distribution of a row with uniform u. */
long oracle_sample(const float *z, long V, float T, int top_k, float top_p,
                   float u)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    if (!p)
        return -2;
    long tok = -1;
    if (oracle_probs(z, V, T, top_k, top_p, p) == 0)
        tok = inv_cdf(p, V, u);
    free(p);
    return tok;
}

/* Many rows at once: tokens[r] drawn from row r with uniform u[r]. */
int oracle_sample_rows(const float *z, long R, long V, float T, int top_k,
                       float top_p, const float *u, int32_t *tokens)
{
    for (long r = 0; r < R; ++r)
        tokens[r] = (int32_t)oracle_sample(z + r * V, V, T, top_k, top_p, u[r]);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Acceptance                                                           */
/* ------------------------------------------------------------------ */

/* Verification of one block of B sequences.
 *
 * Per sequence b, with P_i = probs(target row i) for i = 0..D and
 * Q_i = probs(draft row i) for i = 0..D-1:
 *   for i = 0..D-1:
 *       a_i = P_i(d_i) / Q_i(d_i), both rounded to fp32 and divided in fp32
 *             (the pages decide each position in fp32); a_i = 0 when
 *             P_i(d_i) = 0, +inf when only Q_i(d_i) = 0;
 *       accept d_i iff u_i < a_i (fp32 compare), i.e. with probability
 *             min(1, P_i(d_i) / Q_i(d_i));
 *       on the first rejection: next is drawn from r = max(0, P_i - Q_i)
 *             (fp64; r = P_i if it sums to zero), accepted = i, stop;
 *   if all D are accepted: next = InvCDF(P_D, u_D), accepted = D (bonus).
 * The emitted tokens are d_0..d_{accepted-1} followed by next.
 *
 * How next is drawn from r (a reading; the pages name the residual, not
 * the way it is sampled):
 *   - with top-k or top-p active (and for greedy sampling), r's support is
 *     a few kept tokens: next = InvCDF(r, u_D);
 *   - over the full vocabulary, by rejection from P_i, which never needs r
 *     in full: candidate k = 0, 1, ... is j_k = InvCDF(P_i, v_k), kept iff
 *     a_k < (P - Q) / P at j_k, with P, Q rounded to fp32 and the quotient
 *     taken in fp32 (as the ratio test); the first kept candidate is next.
 *     A candidate j is kept with probability max(0, 1 - Q(j)/P(j)), so next
 *     has exactly the distribution r / sum(r).  v_k and a_k are outputs 2k
 *     and 2k + 1 of the SplitMix64 stream seeded with u_D's bit pattern;
 *     after kCandidates candidates none of which is kept, next =
 *     InvCDF(r, output 2 * kCandidates).
 *
 * Uniform layout (a reading): u[b][0..D-1] are the D tests, u[b][D] is the
 * single final draw (or the seed of its stream).  Any row that is invalid,
 * or a draft token outside [0, V), makes the whole sequence invalid:
 * accepted = next = -1.
 *
 * p_draft / q_draft (nullable) receive P_i(d_i), Q_i(d_i) in fp64 for every
 * i (NaN for an invalid sequence).  draw_row (nullable) receives, per
 * sequence, the position whose distribution the final draw used (i for a
 * residual at i, D for the bonus, -1 if invalid).  draw_margin (nullable)
 * receives, per sequence, the smallest relative distance to a decision
 * boundary met while drawing next: over every inverse-CDF draw made, the
 * target's distance to its interval's boundaries over the total, and over
 * every candidate test up to the kept one, |a_k - (P - Q)/P|.  A draw whose
 * margin is below a rounding tolerance may come out differently under
 * another (correct) summation order. */
enum { kCandidates = 64 };

int oracle_accept(const float *target_logits, const float *draft_logits,
                  const int32_t *draft_tokens, const float *uniforms, long B,
                  long D, long V, float T, int top_k, float top_p,
                  int32_t *accepted_len, int32_t *next_token, double *p_draft,
                  double *q_draft, int32_t *draw_row, double *draw_margin)
{
    /* filtered (candidate) mode, as the sampling settings define it */
    const int greedy = !(T > 0.0f) || top_k == 1;
    const int k_eff = greedy ? 1 : ((top_k >= 1 && top_k < V) ? top_k : (int)V);
    const int filtered = k_eff < V || (!greedy && top_p < 1.0f);
    if (B < 0 || D < 0 || V < 1)
        return -1;
    double *P = (double *)malloc(sizeof(double) * (size_t)((D + 1) * V));
    double *Q = (double *)malloc(sizeof(double) * (size_t)((D > 0 ? D : 1) * V));
    double *r = (double *)malloc(sizeof(double) * (size_t)V);
    if (!P || !Q || !r) {
        free(P); free(Q); free(r);
        return -2;
    }
    for (long b = 0; b < B; ++b) {
        const float *tl = target_logits + b * (D + 1) * V;
        const float *dl = draft_logits ? draft_logits + b * D * V : NULL;
        const int32_t *dt = draft_tokens ? draft_tokens + b * D : NULL;
        const float *u = uniforms + b * (D + 1);
        int ok = 1;
        for (long i = 0; i <= D && ok; ++i)
            ok = (oracle_probs(tl + i * V, V, T, top_k, top_p, P + i * V) == 0);
        for (long i = 0; i < D && ok; ++i)
            ok = (oracle_probs(dl + i * V, V, T, top_k, top_p, Q + i * V) == 0);
        for (long i = 0; i < D && ok; ++i)
            ok = (dt[i] >= 0 && dt[i] < V);
        if (!ok) {
            accepted_len[b] = next_token[b] = -1;
            if (draw_row)
                draw_row[b] = -1;
            if (draw_margin)
                draw_margin[b] = INFINITY;
            for (long i = 0; i < D; ++i) {
                if (p_draft) p_draft[b * D + i] = NAN;
                if (q_draft) q_draft[b * D + i] = NAN;
            }
            continue;
        }
        for (long i = 0; i < D; ++i) {
            if (p_draft) p_draft[b * D + i] = P[i * V + dt[i]];
            if (q_draft) q_draft[b * D + i] = Q[i * V + dt[i]];
        }
        long i;
        for (i = 0; i < D; ++i) {
            float pf = (float)P[i * V + dt[i]];
            float qf = (float)Q[i * V + dt[i]];
            float a = (pf == 0.0f) ? 0.0f : pf / qf;
            if (!(u[i] < a))
                break;
        }
        long tok = -1;
        double margin = INFINITY, mk;
        if (i < D) {
            const double *Pi = P + i * V, *Qi = Q + i * V;
            double tot = 0.0;
            for (long x = 0; x < V; ++x) {
                double d = Pi[x] - Qi[x];
                r[x] = d > 0.0 ? d : 0.0;
                tot += r[x];
            }
            if (!(tot > 0.0))
                memcpy(r, Pi, sizeof(double) * (size_t)V);
            if (filtered) {
                tok = inv_cdf_margin(r, V, u[D], &margin);
            } else {
                uint32_t ubits;
                memcpy(&ubits, &u[D], sizeof ubits);
                const uint64_t seed = ubits;
                for (long c = 0; c < kCandidates && tok < 0; ++c) {
                    const float v = oracle_stream_uniform(seed, 2 * (uint64_t)c);
                    const float a = oracle_stream_uniform(seed, 2 * (uint64_t)c + 1);
                    const long j = inv_cdf_margin(Pi, V, v, &mk);
                    margin = fmin(margin, mk);
                    const float pf = (float)Pi[j], qf = (float)Qi[j];
                    const float thr = (pf - qf) / pf;
                    margin = fmin(margin, fabs((double)a - (double)thr));
                    if (a < thr)
                        tok = j;
                }
                if (tok < 0) {
                    tok = inv_cdf_margin(r, V, oracle_stream_uniform(seed, 2 * (uint64_t)kCandidates), &mk);
                    margin = fmin(margin, mk);
                }
            }
        } else {
            tok = inv_cdf_margin(P + D * V, V, u[D], &margin);
        }
        accepted_len[b] = (int32_t)i;
        next_token[b] = (int32_t)tok;
        if (draw_row)
            draw_row[b] = (int32_t)i;
        if (draw_margin)
            draw_margin[b] = margin;
    }
    free(P); free(Q); free(r);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Greedy verification                                                  */
/* ------------------------------------------------------------------ */

/* Greedy verification of B sequences: the sample-and-match loop of the
 * savepearlharbor.com llama.cpp MTP article (how speculative decoding
 * works), with the greedy sampler of the mlxcel manual's DFlash-family
 * drafter table (sampling only when T > 0 and top_k != 1).
 *
 * Per sequence b, with t_i = the first index of the largest logit of
 * target row i (i = 0..D):
 *   for i = 0..D-1: keep d_i while d_i == t_i; at the first mismatch emit
 *       t_i and stop (accepted = i, next = t_i);
 *   if all D match: accepted = D, next = t_D.
 * Only the target rows are read.  A target row that is invalid (NaN, +inf,
 * or no finite logit, as for sampling) or a draft token outside [0, V) makes
 * the sequence invalid: accepted = next = -1.  draft_tokens may be NULL when
 * D == 0. */
int oracle_verify_greedy(const float *target_logits, const int32_t *draft_tokens,
                         long B, long D, long V, int32_t *accepted_len,
                         int32_t *next_token)
{
    if (B < 0 || D < 0 || V < 1)
        return -1;
    for (long b = 0; b < B; ++b) {
        const float *tl = target_logits + b * (D + 1) * V;
        const int32_t *dt = draft_tokens ? draft_tokens + b * D : NULL;
        int ok = 1;
        for (long i = 0; i <= D && ok; ++i)
            ok = row_valid(tl + i * V, V);
        for (long i = 0; i < D && ok; ++i)
            ok = (dt[i] >= 0 && dt[i] < V);
        if (!ok) {
            accepted_len[b] = next_token[b] = -1;
            continue;
        }
        long i = 0;
        long t = 0;
        for (;; ++i) {
            const float *z = tl + i * V;
            t = 0;
            for (long x = 1; x < V; ++x)
                if (z[x] > z[t])
                    t = x;
            if (i == D || dt[i] != t)
                break;
        }
        accepted_len[b] = (int32_t)i;
        next_token[b] = (int32_t)t;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Recurrent (GDN) state: innovation tape capture and commit            */
/* ------------------------------------------------------------------ */

/* The recurrent layers of the target keep a per-head state S (dv x dk).
 * During a speculative cycle the state is not snapshotted per position;
 * each step records a small tuple instead, and after verification only the
 * accepted steps are committed (MTPLX announcement, "Layer 0" custom kernels:
 * innovation-tape GDN capture of (token, gate, state-delta) tuples, replayed
 * on rejection instead of restoring the whole recurrent state; "Layer 2":
 * the tape commits accepted GDN state deltas and rolls back rejected ones).
 *
 * The pages do not write out the GDN update; the reading is the gated delta
 * rule of Gated DeltaNet, one head at a time:
 *   innovation  delta_t = beta_t * (v_t - alpha_t * S_{t-1} k_t)      (dv)
 *   state       S_t     = alpha_t * S_{t-1} + delta_t k_t^T
 *   output      o_t     = S_t q_t                                    (dv)
 * so the tape tuple of a step is (alpha_t, delta_t) with k_t: the state
 * delta is the rank-1 delta_t k_t^T, the gate alpha_t.
 *
 * Layouts (row-major): S0, S_final [B][H][dv][dk]; q, k [B][T][H][dk];
 * v [B][T][H][dv]; alpha, beta [B][T][H]; o, delta [B][T][H][dv].  Inputs
 * are fp32 as a kernel sees them, everything else fp64.  S_final (nullable)
 * gets S_T. */
int oracle_gdn_record(const float *S0, const float *q, const float *k,
                      const float *v, const float *alpha, const float *beta,
                      long B, long T, long H, long dk, long dv, double *o,
                      double *delta, double *S_final)
{
    if (B < 0 || T < 0 || H < 0 || dk < 1 || dv < 1)
        return -1;
    double *S = (double *)malloc(sizeof(double) * (size_t)(dv * dk));
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!S || !u) {
        free(S); free(u);
        return -2;
    }
    for (long b = 0; b < B; ++b)
        for (long h = 0; h < H; ++h) {
            const float *s0 = S0 + (b * H + h) * dv * dk;
            for (long e = 0; e < dv * dk; ++e)
                S[e] = (double)s0[e];
            for (long t = 0; t < T; ++t) {
                const long bth = (b * T + t) * H + h;
                const float *kt = k + bth * dk, *qt = q + bth * dk, *vt = v + bth * dv;
                const double a = (double)alpha[bth], be = (double)beta[bth];
                double *dt = delta + bth * dv, *ot = o + bth * dv;
                for (long i = 0; i < dv; ++i) {          /* u = S_{t-1} k_t */
                    double acc = 0.0;
                    for (long c = 0; c < dk; ++c)
                        acc += S[i * dk + c] * (double)kt[c];
                    u[i] = acc;
                }
                for (long i = 0; i < dv; ++i)            /* the innovation */
                    dt[i] = be * ((double)vt[i] - a * u[i]);
                for (long i = 0; i < dv; ++i)            /* gated rank-1 update */
                    for (long c = 0; c < dk; ++c)
                        S[i * dk + c] = a * S[i * dk + c] + dt[i] * (double)kt[c];
                for (long i = 0; i < dv; ++i) {          /* readout */
                    double acc = 0.0;
                    for (long c = 0; c < dk; ++c)
                        acc += S[i * dk + c] * (double)qt[c];
                    ot[i] = acc;
                }
            }
            if (S_final)
                for (long e = 0; e < dv * dk; ++e)
                    S_final[(b * H + h) * dv * dk + e] = S[e];
        }
    free(S); free(u);
    return 0;
}

/* Commit after verification: S_out = the state after the first n[b] steps
 * of sequence b, rebuilt from S0 and the tape alone:
 *   S_t = alpha_t * S_{t-1} + delta_t k_t^T,   t = 0 .. n[b] - 1,
 * with 0 <= n[b] <= T (n[b] = 0 keeps S0: nothing committed).  delta is the
 * tape as fp32 (what a kernel stored).  n[b] < 0 or > T is an error. */
int oracle_gdn_commit(const float *S0, const float *alpha, const float *k,
                      const float *delta, const int32_t *n, long B, long T,
                      long H, long dk, long dv, double *S_out)
{
    if (B < 0 || T < 0 || H < 0 || dk < 1 || dv < 1)
        return -1;
    for (long b = 0; b < B; ++b)
        if (n[b] < 0 || n[b] > T)
            return -1;
    for (long b = 0; b < B; ++b)
        for (long h = 0; h < H; ++h) {
            double *S = S_out + (b * H + h) * dv * dk;
            const float *s0 = S0 + (b * H + h) * dv * dk;
            for (long e = 0; e < dv * dk; ++e)
                S[e] = (double)s0[e];
            for (long t = 0; t < n[b]; ++t) {
                const long bth = (b * T + t) * H + h;
                const double a = (double)alpha[bth];
                for (long i = 0; i < dv; ++i)
                    for (long c = 0; c < dk; ++c)
                        S[i * dk + c] = a * S[i * dk + c] +
                                        (double)delta[bth * dv + i] * (double)k[bth * dk + c];
            }
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Draft-only 4-bit LM head: requantization                             */
/* ------------------------------------------------------------------ */

/* The target keeps its LM head at model precision; a separate 4-bit copy is
 * built in memory for drafting only (MTPLX announcement, "Layer 0" custom
 * kernels: draft-only requantised LM head, draft time down 29%).  The pages
 * do not give the quantizer; the reading is the affine group quantization
 * the qmv path reads (ŵ = s q + b, groups of G along K, codes 0..15), with
 * the usual min/max fit per group:
 *   b = min_g w,  s = (max_g w - min_g w) / 15   (fp32, then to fp16, nearest even)
 *   q = round_half_even((w - b16) / s16) clamped to 0..15   (fp32)
 *   q = 0 where s16 is 0 or not finite.
 * The code is an integer decided by floating point, so it is decided in the
 * kernel's precision (fp32 subtraction and division, correctly rounded), not
 * in fp64.  Source: bf16 bit patterns [N][K]; outputs in the interchange
 * layout of the qmv path: W4 words [N][K/8] (element k at bits 4*(k%8) of
 * word k/8), fp16 scales and biases [N][K/G]. */
/* Nearest-even binary16 bit pattern of a float (11 significant bits,
 * normal exponents -14..15, subnormal ulp 2^-24, overflow to infinity). */
static uint16_t float_to_half_bits(float f)
{
    double v = (double)f;
    if (isnan(v))
        return 0x7E00;
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    v = fabs(v);
    if (v == 0.0)
        return sign;
    int e;
    frexp(v, &e);                       /* v = m * 2^e, m in [0.5, 1) */
    int ulp_exp = e - 11;
    if (ulp_exp < -24)
        ulp_exp = -24;
    double r = ldexp(nearbyint(ldexp(v, -ulp_exp)), ulp_exp);
    if (r >= 65536.0)
        return sign | 0x7C00;
    if (r < ldexp(1.0, -14))            /* subnormal (or rounded up to 2^-14) */
        return sign | (uint16_t)ldexp(r, 24);
    frexp(r, &e);
    int E = e - 1;                      /* r = 1.f * 2^E */
    uint16_t mant = (uint16_t)(ldexp(r, -E) * 1024.0 - 1024.0);
    return sign | (uint16_t)((E + 15) << 10) | mant;
}

uint16_t oracle_float_to_half(float f) { return float_to_half_bits(f); }

int oracle_requantize_w4(const uint16_t *w_bf16, long N, long K, long G,
                         uint32_t *w4, uint16_t *scales, uint16_t *biases)
{
    if (N < 0 || K < 0 || G <= 0 || K % G != 0 || K % 8 != 0)
        return -1;
    long ng = K / G;
    for (long n = 0; n < N; ++n) {
        for (long k8 = 0; k8 < K / 8; ++k8)
            w4[n * (K / 8) + k8] = 0;
        for (long g = 0; g < ng; ++g) {
            float lo = INFINITY, hi = -INFINITY;
            for (long k = g * G; k < (g + 1) * G; ++k) {
                float v = (float)bf16_to_double(w_bf16[n * K + k]);
                if (v < lo) lo = v;
                if (v > hi) hi = v;
            }
            float sf = (hi - lo) / 15.0f;
            uint16_t s16 = float_to_half_bits(sf), b16 = float_to_half_bits(lo);
            scales[n * ng + g] = s16;
            biases[n * ng + g] = b16;
            float s = (float)half_to_double(s16), b = (float)half_to_double(b16);
            for (long k = g * G; k < (g + 1) * G; ++k) {
                unsigned q = 0;
                if (s != 0.0f && isfinite(s)) {
                    float v = (float)bf16_to_double(w_bf16[n * K + k]);
                    float r = nearbyintf((v - b) / s);
                    q = r < 0.0f ? 0u : (r > 15.0f ? 15u : (unsigned)r);
                }
                w4[n * (K / 8) + k / 8] |= (uint32_t)q << (4 * (k % 8));
            }
        }
    }
    return 0;
}
