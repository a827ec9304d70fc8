// Verification kernels for gfx950: the target/draft sampling distributions,
// the per-position probability-ratio test, and the residual or bonus draw.
//
// The rule (MTPLX announcement, "Layer 2: Speculative cycle (the hot
// loop)"; Japanese re-post, same section): each draft d_i is accepted in
// fp32 with probability min(1, p_i(d_i) / q_i(d_i)); the first rejection
// emits a fresh token from the residual (p - q)+, and when every draft is
// accepted the last target position yields a bonus token.  The savepearl-
// harbor.com llama.cpp MTP article (how verification works) fixes the
// output count: D accepted drafts give D + 1 tokens, a full rejection still
// gives one.  Sampling uses the temperature / top-k / top-p settings of the
// MTPLX benchmark ("QWEN 3.6 27B @ 63 TPS").
//
// Kernels:
//  1. row_stats  -- grid (row, chunk).  One streaming pass over every fp32
//     logit.  Full-vocabulary mode: per-chunk running max and sum of
//     exp2((z - max) * log2(e)/T).  Candidate mode (top-k active, top-p, or
//     greedy): the chunk's top-k (logit, index) keys by radix select.  The
//     workgroup that finishes a row last merges its chunks in chunk order
//     into the row's final statistics (max, normalizer, kept candidates).
//  2. accept     -- grid (sequence, chunk).  Every workgroup recomputes the
//     D ratio tests from the row statistics (a handful of gathers), then
//     sums the draw distribution (residual at the rejected position, or the
//     bonus row) over its vocabulary chunk.  The last workgroup of the
//     sequence turns u_D into a target mass, finds the chunk that holds it
//     and scans that chunk in vocabulary order: an inverse-CDF draw with no
//     sort.  In candidate mode one workgroup does the draw over <= 256
//     candidates.
//  3. probs      -- dense write of the distributions (spec_sample_probs).
//
// Every reduction runs in a fixed order, so results are deterministic.
#include "spec_internal.h"

#include <algorithm>
#include <cfloat>
#include <cmath>

namespace spec {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxCand = 256;       // top-k cap in candidate mode
constexpr int kCandChunk = 4096;    // logits per workgroup in candidate mode
constexpr int kTargetBlocks = 1024;

constexpr int kInvalid = 1;         // row flag: NaN / +inf / no finite logit

// The workspace starts with two fixed counter areas (rows, then sequences)
// that no plan uses for anything else, so calls of any shape can share one
// workspace: every call leaves its counters at zero.  Row statistics are
// launched in batches of at most kRowSlots rows when a row spans several
// chunks; sequences only use counters when the batch is small.
constexpr int kRowSlots = 131072;
constexpr int kSeqSlots = 131072;

// Release: make this workgroup's earlier global writes visible device-wide
// before the counter increment.  Acquire: after observing the last
// increment, see every other workgroup's writes.
__device__ __forceinline__ void release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

struct RowFinal {
    float m;      // max logit
    float inv;    // 1 / normalizer (full vocabulary, or of the kept candidates)
    int n_kept;   // candidate mode: kept candidates (rank order)
    int flags;
};

struct ChunkStat {
    float m;
    float S;
    int bad;      // saw NaN or +inf
    int finite;   // saw a finite logit
};

struct Rows {
    const float *target;
    const float *draft;
    int D;
    int V;
    __device__ __forceinline__ const float *row(int r) const {
        const int per = 2 * D + 1;
        const int b = r / per;
        const int i = r - b * per;
        if (i <= D)
            return target + ((size_t)b * (D + 1) + i) * V;
        return draft + ((size_t)b * D + (i - D - 1)) * V;
    }
    __device__ __forceinline__ int target_row(int b, int i) const { return b * (2 * D + 1) + i; }
    __device__ __forceinline__ int draft_row(int b, int i) const { return b * (2 * D + 1) + D + 1 + i; }
};

struct Ws {
    unsigned *row_cnt;
    unsigned *seq_cnt;
    ChunkStat *chunk_stats;     // [rows][chunks]
    uint64_t *chunk_keys;       // [rows][chunks][k]  (candidate mode)
    RowFinal *row_final;        // [rows]
    uint64_t *row_keys;         // [rows][k]          (candidate mode)
    float2 *seq_sums;           // [B][chunks3]  (residual mass, target mass)
};

// ---------------------------------------------------------------- keys ----
// A 64-bit rank key: larger = better rank.  High word: the logit mapped to an
// unsigned order-preserving code (-0 folded onto +0); low word: the bitwise
// complement of the index, so equal logits rank the lower index first.
__device__ __forceinline__ uint32_t ordered_code(float z) {
    const uint32_t u = __float_as_uint(z + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float code_to_float(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ uint64_t make_key(float z, int idx) {
    return ((uint64_t)ordered_code(z) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ float key_logit(uint64_t k) { return code_to_float((uint32_t)(k >> 32)); }
__device__ __forceinline__ int key_index(uint64_t k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

__device__ __forceinline__ float weight(float z, float m, float scale) {
    return __builtin_amdgcn_exp2f((z - m) * scale);
}

// ------------------------------------------------------ block reductions ----
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v |= __shfl_xor(v, o);
    return v;
}

// Fixed-order block sum: butterfly inside each wave, then waves 0..3.
__device__ float block_sum(float v, float *sh) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        sh[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = sh[0];
    for (int w = 1; w < kWaves; ++w)
        s += sh[w];
    return s;
}
__device__ int block_or(int v, int *sh) {
    v = wave_or(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        sh[threadIdx.x >> 6] = v;
    __syncthreads();
    int s = 0;
    for (int w = 0; w < kWaves; ++w)
        s |= sh[w];
    return s;
}

// Merge of two (max, sum of exp2((z - max) * scale)) summaries.
__device__ __forceinline__ void merge_ms(float &m, float &S, float m2, float S2, float scale) {
    const float mn = fmaxf(m, m2);
    const float e1 = (m == mn) ? 1.0f : weight(m, mn, scale);
    const float e2 = (m2 == mn) ? 1.0f : weight(m2, mn, scale);
    S = S * e1 + S2 * e2;
    m = mn;
}
__device__ void wave_merge_ms(float &m, float &S, float scale) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float m2 = __shfl_xor(m, o);
        const float S2 = __shfl_xor(S, o);
        merge_ms(m, S, m2, S2, scale);
    }
}

// Inclusive scan of one int per thread, in thread order.
__device__ int block_incl_scan(int v, int *sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o);
        if (lane >= o)
            v += t;
    }
    __syncthreads();
    if (lane == 63)
        sh[wave] = v;
    __syncthreads();
    for (int w = 0; w < wave; ++w)
        v += sh[w];
    return v;
}
// Same for floats (fixed order: Hillis-Steele inside the wave, then waves).
__device__ float block_incl_scan_f(float v, float *sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float t = __shfl_up(v, o);
        if (lane >= o)
            v += t;
    }
    __syncthreads();
    if (lane == 63)
        sh[wave] = v;
    __syncthreads();
    float base = 0.0f;
    for (int w = 0; w < wave; ++w)
        base += sh[w];
    return base + v;
}

// ------------------------------------------------------- radix selection ----
struct SelectShared {
    unsigned hist[256];
    int scan[kWaves];
    int bin, above, count, out_n;
};

// Selects the `k` largest keys among the keys visited by `each` (a functor
// calling f(key) for every key this thread owns; keys are unique).  Writes
// them to out[] (any order) and returns how many were written (min(k, n)).
template <class Each>
__device__ int block_select_topk(Each each, int n, int k, uint64_t *out, int cap,
                                 SelectShared &sh) {
    const int want = min(k, n);
    uint64_t prefix = 0, mask = 0;
    if (want < n) {
        int remaining = want;
        for (int d = 7; d >= 0; --d) {
            sh.hist[threadIdx.x] = 0;
            if (threadIdx.x == 0) {
                sh.bin = 0;
                sh.above = 0;
                sh.count = 0;
            }
            __syncthreads();
            each([&](uint64_t key) {
                if ((key & mask) == prefix)
                    atomicAdd(&sh.hist[(unsigned)(key >> (8 * d)) & 0xFFu], 1u);
            });
            __syncthreads();
            // thread t owns bin 255 - t: scan counts from the top bin down
            const int c = (int)sh.hist[255 - threadIdx.x];
            const int incl = block_incl_scan(c, sh.scan);
            const int excl = incl - c;
            if (excl < remaining && incl >= remaining) {
                sh.bin = 255 - threadIdx.x;
                sh.above = excl;
                sh.count = c;
            }
            __syncthreads();
            remaining -= sh.above;
            prefix |= (uint64_t)sh.bin << (8 * d);
            mask |= (uint64_t)0xFF << (8 * d);
            const bool done = (sh.count == remaining);
            __syncthreads();
            if (done)
                break;
        }
    }
    if (threadIdx.x == 0)
        sh.out_n = 0;
    __syncthreads();
    each([&](uint64_t key) {
        if ((key & mask) >= prefix) {
            const int slot = atomicAdd(&sh.out_n, 1);
            if (slot < cap)
                out[slot] = key;
        }
    });
    __syncthreads();
    return min(want, min(sh.out_n, cap));
}

// Bitonic sort of n <= 256 keys in LDS, descending (padding with 0 keys).
__device__ void block_sort_desc(uint64_t *keys, int n) {
    int P = 1;
    while (P < n)
        P <<= 1;
    for (int i = n + (int)threadIdx.x; i < P; i += kThreads)
        keys[i] = 0;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < P; i += kThreads) {
                const int partner = i ^ stride;
                if (partner > i) {
                    const bool desc = ((i & size) == 0);
                    const uint64_t a = keys[i], b = keys[partner];
                    if (desc ? (a < b) : (a > b)) {
                        keys[i] = b;
                        keys[partner] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
}

// ------------------------------------------------------------- kernel 1 ----
struct StatsShared {
    SelectShared sel;
    uint64_t keys[kMaxCand * 2];
    float fsh[kWaves];
    float fsh2[kWaves];
    int ish[kWaves];
    int last;
};

__global__ __launch_bounds__(kThreads) void row_stats_kernel(
    Rows rows, int row0, int chunks, int chunk_len, SamplingParams sp, Ws ws) {
    __shared__ StatsShared sh;
    const int r = row0 + blockIdx.x;
    const int c = blockIdx.y;
    const int V = rows.V;
    const float *z = rows.row(r);
    const int lo = c * chunk_len;
    const int hi = min(V, lo + chunk_len);
    const float scale = sp.scale;
    int bad = 0, finite = 0;

    if (!sp.candidates) {
        // ---- running max and normalizer over the chunk ----
        float m = -INFINITY, S = 0.0f;
        const bool vec = ((V & 3) == 0);
        if (vec) {
            const float4 *z4 = reinterpret_cast<const float4 *>(z);
            for (int base = lo + threadIdx.x * 4; base < hi; base += kThreads * 16) {
                // Branch-free: clamp each load into the chunk and mask the
                // lanes past its end to -inf (which adds nothing below).
                float v[16];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int e = base + u * kThreads * 4;
                    const float4 t = z4[min(e, hi - 4) >> 2];
                    const bool in = e < hi;
                    v[4 * u + 0] = in ? t.x : -INFINITY;
                    v[4 * u + 1] = in ? t.y : -INFINITY;
                    v[4 * u + 2] = in ? t.z : -INFINITY;
                    v[4 * u + 3] = in ? t.w : -INFINITY;
                }
                float bm = m;
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    bad |= (v[q] != v[q]) | (v[q] == INFINITY);
                    finite |= (v[q] > -INFINITY) & (v[q] < INFINITY);
                    bm = fmaxf(bm, v[q]);
                }
                if (bm > -INFINITY) {
                    float s = (m == bm) ? S : S * weight(m, bm, scale);
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        s += weight(v[q], bm, scale);
                    S = s;
                    m = bm;
                }
            }
        } else {
            for (int e = lo + threadIdx.x; e < hi; e += kThreads) {
                const float v = z[e];
                bad |= (v != v) | (v == INFINITY);
                finite |= (v > -INFINITY) & (v < INFINITY);
                const float bm = fmaxf(m, v);
                if (bm > -INFINITY) {
                    S = ((m == bm) ? S : S * weight(m, bm, scale)) + weight(v, bm, scale);
                    m = bm;
                }
            }
        }
        wave_merge_ms(m, S, scale);
        __syncthreads();
        if ((threadIdx.x & 63) == 0) {
            sh.fsh[threadIdx.x >> 6] = m;
            sh.fsh2[threadIdx.x >> 6] = S;
        }
        bad = block_or(bad, sh.ish);
        finite = block_or(finite, sh.ish);
        if (threadIdx.x == 0) {
            float mm = sh.fsh[0], SS = sh.fsh2[0];
            for (int w = 1; w < kWaves; ++w)
                merge_ms(mm, SS, sh.fsh[w], sh.fsh2[w], scale);
            ws.chunk_stats[(size_t)r * chunks + c] = ChunkStat{mm, SS, bad, finite};
        }
    } else {
        // ---- candidate mode: the chunk's top-k keys ----
        constexpr int E = kCandChunk / kThreads;  // 16 keys per thread
        uint64_t mine[E];
#pragma unroll
        for (int q = 0; q < E; ++q) {
            const int e = lo + q * kThreads + threadIdx.x;
            if (e < hi) {
                const float v = z[e];
                bad |= (v != v) | (v == INFINITY);
                finite |= (v > -INFINITY) & (v < INFINITY);
                mine[q] = make_key(v, e);
            } else {
                mine[q] = 0;  // below every real key; never selected (see n)
            }
        }
        const int n = hi - lo;
        auto each = [&](auto f) {
#pragma unroll
            for (int q = 0; q < E; ++q)
                if (lo + q * kThreads + (int)threadIdx.x < hi)
                    f(mine[q]);
        };
        const int got = block_select_topk(each, n, sp.k_eff, sh.keys, kMaxCand, sh.sel);
        uint64_t *dst = ws.chunk_keys + ((size_t)r * chunks + c) * sp.k_eff;
        for (int i = threadIdx.x; i < sp.k_eff; i += kThreads)
            dst[i] = (i < got) ? sh.keys[i] : 0;
        bad = block_or(bad, sh.ish);
        finite = block_or(finite, sh.ish);
        if (threadIdx.x == 0)
            ws.chunk_stats[(size_t)r * chunks + c] = ChunkStat{0.0f, 0.0f, bad, finite};
    }

    // ---- the last chunk of this row merges all chunks in chunk order ----
    if (chunks > 1) {
        release_agent();
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned prev = atomicAdd(&ws.row_cnt[blockIdx.x], 1u);
            sh.last = (prev == (unsigned)(chunks - 1));
        }
        __syncthreads();
        if (!sh.last)
            return;
        acquire_agent();
    } else {
        __syncthreads();
    }

    int rbad = 0, rfin = 0;
    for (int cc = 0; cc < chunks; ++cc) {
        const ChunkStat st = ws.chunk_stats[(size_t)r * chunks + cc];
        rbad |= st.bad;
        rfin |= st.finite;
    }
    const int flags = (rbad || !rfin) ? kInvalid : 0;

    if (!sp.candidates) {
        if (threadIdx.x == 0) {
            float m = -INFINITY, S = 0.0f;
            for (int cc = 0; cc < chunks; ++cc) {
                const ChunkStat st = ws.chunk_stats[(size_t)r * chunks + cc];
                merge_ms(m, S, st.m, st.S, scale);
            }
            ws.row_final[r] = RowFinal{m, 1.0f / S, 0, flags};
            if (chunks > 1)
                atomicExch(&ws.row_cnt[blockIdx.x], 0u);
        }
        return;
    }

    const int k = sp.k_eff;
    const uint64_t *ck = ws.chunk_keys + (size_t)r * chunks * k;
    const int total = chunks * k;
    auto each_g = [&](auto f) {
        for (int i = threadIdx.x; i < total; i += kThreads) {
            const uint64_t key = __builtin_nontemporal_load(&ck[i]);
            if (key != 0)
                f(key);
        }
    };
    // number of real keys: min(k, chunk length) per chunk
    int n_real = 0;
    for (int cc = 0; cc < chunks; ++cc)
        n_real += min(k, min(V, (cc + 1) * chunk_len) - cc * chunk_len);
    const int got = block_select_topk(each_g, n_real, k, sh.keys, kMaxCand, sh.sel);
    block_sort_desc(sh.keys, got);
    if (threadIdx.x == 0) {
        const float m = key_logit(sh.keys[0]);
        float cum = 0.0f;
        for (int i = 0; i < got; ++i)
            cum += weight(key_logit(sh.keys[i]), m, scale);
        const float S_all = cum;
        int kept = got;
        float S_kept = S_all;
        if (sp.use_p) {
            cum = 0.0f;
            for (int i = 0; i < got; ++i) {
                cum += weight(key_logit(sh.keys[i]), m, scale);
                if (cum / S_all >= sp.top_p) {
                    kept = i + 1;
                    break;
                }
            }
            if (kept == got) {
                cum = S_all;
            }
            S_kept = cum;
        }
        ws.row_final[r] = RowFinal{m, 1.0f / S_kept, kept, flags};
        if (chunks > 1)
            atomicExch(&ws.row_cnt[blockIdx.x], 0u);
    }
    uint64_t *rk = ws.row_keys + (size_t)r * k;
    for (int i = threadIdx.x; i < k; i += kThreads)
        rk[i] = (i < got) ? sh.keys[i] : 0;
}

// ------------------------------------------------------------- kernel 2 ----
// Probability of token x under row r's final distribution, given its logit.
__device__ __forceinline__ float row_prob(const RowFinal &f, const uint64_t *keys,
                                          bool candidates, float scale, float zx, int x) {
    if (candidates && make_key(zx, x) < keys[f.n_kept - 1])
        return 0.0f;
    return weight(zx, f.m, scale) * f.inv;
}

struct AcceptShared {
    float fsh[kWaves];
    int ish[kWaves];
    int last;
    int seq_L;
    int seq_ok;
    float2 sums[64];
    // candidate draw
    uint64_t ckey[kMaxCand];   // (index-major key for sorting) index << 32 | float bits of r
    float cw[kMaxCand];
    float cp[kMaxCand];
    int found;
};

// Decisions of sequence b from the row statistics: returns L (0..D) or -1.
__device__ int decide(const Rows &rows, const Ws &ws, const SamplingParams &sp,
                      const int32_t *draft_tokens, const float *uniforms, int b,
                      float *p_out, float *q_out) {
    const int D = rows.D, V = rows.V;
    for (int i = 0; i <= D; ++i)
        if (ws.row_final[rows.target_row(b, i)].flags)
            return -1;
    for (int i = 0; i < D; ++i) {
        if (ws.row_final[rows.draft_row(b, i)].flags)
            return -1;
        const int d = draft_tokens[(size_t)b * D + i];
        if (d < 0 || d >= V)
            return -1;
    }
    int L = D;
    for (int i = 0; i < D; ++i) {
        const int d = draft_tokens[(size_t)b * D + i];
        const int tr = rows.target_row(b, i), dr = rows.draft_row(b, i);
        const RowFinal ft = ws.row_final[tr], fd = ws.row_final[dr];
        const float zt = rows.row(tr)[d], zd = rows.row(dr)[d];
        const float p = row_prob(ft, ws.row_keys + (size_t)tr * sp.k_eff, sp.candidates, sp.scale, zt, d);
        const float q = row_prob(fd, ws.row_keys + (size_t)dr * sp.k_eff, sp.candidates, sp.scale, zd, d);
        if (p_out) p_out[i] = p;
        if (q_out) q_out[i] = q;
        const float a = (p == 0.0f) ? 0.0f : p / q;
        if (L == D && !(uniforms[(size_t)b * (D + 1) + i] < a))
            L = i;
    }
    return L;
}

__global__ __launch_bounds__(kThreads) void accept_kernel(
    Rows rows, SamplingParams sp, const int32_t *__restrict__ draft_tokens,
    const float *__restrict__ uniforms, int chunks3, int chunk3_len,
    int32_t *__restrict__ accepted_len, int32_t *__restrict__ next_token,
    float *__restrict__ p_draft, float *__restrict__ q_draft, Ws ws) {
    __shared__ AcceptShared sh;
    const int b = blockIdx.x;
    const int c = blockIdx.y;
    const int D = rows.D, V = rows.V;
    const float scale = sp.scale;

    if (threadIdx.x == 0) {
        float pv[16], qv[16];
        const int L = decide(rows, ws, sp, draft_tokens, uniforms, b, pv, qv);
        sh.seq_L = L;
        if (c == 0) {
            for (int i = 0; i < D; ++i) {
                if (p_draft) p_draft[(size_t)b * D + i] = (L < 0) ? NAN : pv[i];
                if (q_draft) q_draft[(size_t)b * D + i] = (L < 0) ? NAN : qv[i];
            }
            if (L < 0) {
                if (accepted_len) accepted_len[b] = -1;
                next_token[b] = -1;
            }
        }
    }
    __syncthreads();
    const int L = sh.seq_L;
    if (L < 0)
        return;
    const float u = uniforms[(size_t)b * (D + 1) + D];
    const bool residual = (L < D);
    const int tr = rows.target_row(b, L);
    const RowFinal ft = ws.row_final[tr];
    const float *zt = rows.row(tr);
    const uint64_t *kt = ws.row_keys + (size_t)tr * sp.k_eff;
    const int dr = residual ? rows.draft_row(b, L) : 0;
    const RowFinal fd = residual ? ws.row_final[dr] : RowFinal{0.0f, 1.0f, 0, 0};
    const float *zd = residual ? rows.row(dr) : nullptr;
    const uint64_t *kd = residual ? ws.row_keys + (size_t)dr * sp.k_eff : nullptr;

    if (sp.candidates) {
        // ---- draw over the kept candidates of the target row (c == 0 only) ----
        if (c != 0)
            return;
        const int n = ft.n_kept;
        for (int i = threadIdx.x; i < kMaxCand; i += kThreads) {
            if (i < n) {
                const uint64_t key = kt[i];
                const int x = key_index(key);
                const float p = weight(key_logit(key), ft.m, scale) * ft.inv;
                float w = p;
                if (residual) {
                    const float q = row_prob(fd, kd, true, scale, zd[x], x);
                    w = fmaxf(p - q, 0.0f);
                }
                // sort key: index ascending -> store index in the high word
                sh.ckey[i] = ((uint64_t)(uint32_t)x << 32) | (uint32_t)i;
                sh.cw[i] = w;
                sh.cp[i] = p;
            } else {
                sh.ckey[i] = ~(uint64_t)0;  // sorts last in ascending order
            }
        }
        __syncthreads();
        // ascending sort by index: sort descending the complemented keys
        for (int i = threadIdx.x; i < kMaxCand; i += kThreads)
            sh.ckey[i] = ~sh.ckey[i];
        __syncthreads();
        block_sort_desc(sh.ckey, kMaxCand);
        if (threadIdx.x == 0) {
            float tot = 0.0f;
            for (int i = 0; i < n; ++i)
                tot += sh.cw[(uint32_t)~sh.ckey[i]];
            const bool use_p = !(tot > 0.0f);
            if (use_p) {
                tot = 0.0f;
                for (int i = 0; i < n; ++i)
                    tot += sh.cp[(uint32_t)~sh.ckey[i]];
            }
            const float target = u * tot;
            float cum = 0.0f;
            int pick = -1, last_pos = -1;
            for (int i = 0; i < n; ++i) {
                const int slot = (int)(uint32_t)~sh.ckey[i];
                const float w = use_p ? sh.cp[slot] : sh.cw[slot];
                const int x = (int)((~sh.ckey[i]) >> 32);
                cum += w;
                if (w > 0.0f)
                    last_pos = x;
                if (cum > target) {
                    pick = x;
                    break;
                }
            }
            if (pick < 0)
                pick = last_pos;
            if (accepted_len) accepted_len[b] = L;
            next_token[b] = pick;
        }
        return;
    }

    // ---- full-vocabulary draw: chunk sums ----
    const int lo = c * chunk3_len;
    const int hi = min(V, lo + chunk3_len);
    float wr = 0.0f, wp = 0.0f;
    if ((V & 3) == 0) {
        // float4 loads, clamped into the chunk; lanes past its end add 0
        const float4 *zt4 = reinterpret_cast<const float4 *>(zt);
        const float4 *zd4 = residual ? reinterpret_cast<const float4 *>(zd) : zt4;
        for (int base = lo + threadIdx.x * 4; base < hi; base += kThreads * 8) {
            float4 a[2], q4[2];
            bool in[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int e = base + u * kThreads * 4;
                in[u] = e < hi;
                const int ec = min(e, hi - 4) >> 2;
                a[u] = zt4[ec];
                q4[u] = zd4[ec];
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const float tv[4] = {a[u].x, a[u].y, a[u].z, a[u].w};
                const float dv[4] = {q4[u].x, q4[u].y, q4[u].z, q4[u].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float p = in[u] ? weight(tv[q], ft.m, scale) * ft.inv : 0.0f;
                    wp += p;
                    if (residual) {
                        const float qq = weight(dv[q], fd.m, scale) * fd.inv;
                        wr += in[u] ? fmaxf(p - qq, 0.0f) : 0.0f;
                    }
                }
            }
        }
    } else {
        for (int x = lo + threadIdx.x; x < hi; x += kThreads) {
            const float p = weight(zt[x], ft.m, scale) * ft.inv;
            wp += p;
            if (residual) {
                const float q = weight(zd[x], fd.m, scale) * fd.inv;
                wr += fmaxf(p - q, 0.0f);
            }
        }
    }
    wr = block_sum(wr, sh.fsh);
    wp = block_sum(wp, sh.fsh);
    if (threadIdx.x == 0)
        ws.seq_sums[(size_t)b * chunks3 + c] = make_float2(residual ? wr : wp, wp);

    if (chunks3 > 1) {
        release_agent();
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned prev = atomicAdd(&ws.seq_cnt[b], 1u);
            sh.last = (prev == (unsigned)(chunks3 - 1));
        }
        __syncthreads();
        if (!sh.last)
            return;
        acquire_agent();
    } else {
        __syncthreads();
    }

    // ---- last chunk: locate the target mass, then scan one chunk ----
    __shared__ int s_chunk;
    __shared__ float s_before, s_target;
    __shared__ int s_use_p;
    if (threadIdx.x == 0) {
        float tot = 0.0f;
        for (int cc = 0; cc < chunks3; ++cc)
            tot += __builtin_nontemporal_load(&ws.seq_sums[(size_t)b * chunks3 + cc].x);
        int use_p = !(tot > 0.0f);
        if (use_p) {
            tot = 0.0f;
            for (int cc = 0; cc < chunks3; ++cc)
                tot += __builtin_nontemporal_load(&ws.seq_sums[(size_t)b * chunks3 + cc].y);
        }
        const float target = u * tot;
        float cum = 0.0f, before = 0.0f;
        int pick = -1, last_pos = -1;
        float last_before = 0.0f;
        for (int cc = 0; cc < chunks3; ++cc) {
            const float2 s2 = ws.seq_sums[(size_t)b * chunks3 + cc];
            const float w = use_p ? s2.y : s2.x;
            before = cum;
            cum += w;
            if (w > 0.0f) {
                last_pos = cc;
                last_before = before;
            }
            if (cum > target) {
                pick = cc;
                break;
            }
        }
        if (pick < 0) {
            pick = last_pos;
            before = last_before;
        }
        s_chunk = pick;
        s_before = before;
        s_target = target;
        s_use_p = use_p;
        if (chunks3 > 1)
            atomicExch(&ws.seq_cnt[b], 0u);
    }
    __syncthreads();
    const int cs = s_chunk;
    const bool use_p = s_use_p != 0;
    const float tgt = s_target - s_before;
    const int clo = cs * chunk3_len;
    const int chi = min(V, clo + chunk3_len);
    const int seg = (chi - clo + kThreads - 1) / kThreads;
    const int slo = clo + threadIdx.x * seg;
    const int shi = min(chi, slo + seg);
    auto wt = [&](int x) -> float {
        const float p = weight(zt[x], ft.m, scale) * ft.inv;
        if (!residual || use_p)
            return p;
        const float q = weight(zd[x], fd.m, scale) * fd.inv;
        return fmaxf(p - q, 0.0f);
    };
    float mysum = 0.0f;
    int mylast = -1;
    for (int x = slo; x < shi; ++x) {
        const float w = wt(x);
        mysum += w;
        if (w > 0.0f)
            mylast = x;
    }
    const float incl = block_incl_scan_f(mysum, sh.fsh);
    const float excl = incl - mysum;
    if (threadIdx.x == 0)
        sh.found = 0x7FFFFFFF;
    __syncthreads();
    if (incl > tgt && excl <= tgt)
        atomicMin(&sh.found, (int)threadIdx.x);
    __syncthreads();
    int owner = sh.found;
    if (owner == 0x7FFFFFFF) {
        // rounding left the target at or past the chunk end: last positive
        // token of the chunk
        __syncthreads();
        if (threadIdx.x == 0)
            sh.found = -1;
        __syncthreads();
        if (mylast >= 0)
            atomicMax(&sh.found, (int)threadIdx.x);
        __syncthreads();
        owner = sh.found;
        if ((int)threadIdx.x == owner) {
            if (accepted_len) accepted_len[b] = L;
            next_token[b] = mylast;
        }
        return;
    }
    if ((int)threadIdx.x == owner) {
        float cum = excl;
        int pick = -1, last_pos = -1;
        for (int x = slo; x < shi; ++x) {
            const float w = wt(x);
            cum += w;
            if (w > 0.0f)
                last_pos = x;
            if (cum > tgt) {
                pick = x;
                break;
            }
        }
        if (pick < 0)
            pick = last_pos;
        if (accepted_len) accepted_len[b] = L;
        next_token[b] = pick;
    }
}

// ------------------------------------------------------------- kernel 3 ----
__global__ __launch_bounds__(kThreads) void probs_kernel(
    Rows rows, SamplingParams sp, int chunk_len, float *__restrict__ probs, Ws ws) {
    const int r = blockIdx.x;
    const int c = blockIdx.y;
    const int V = rows.V;
    const float *z = rows.row(r);
    const RowFinal f = ws.row_final[r];
    const uint64_t *keys = ws.row_keys + (size_t)r * sp.k_eff;
    float *out = probs + (size_t)r * V;
    const int lo = c * chunk_len, hi = min(V, lo + chunk_len);
    for (int x = lo + threadIdx.x; x < hi; x += kThreads)
        out[x] = f.flags ? NAN : row_prob(f, keys, sp.candidates, sp.scale, z[x], x);
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

hipError_t launch_row_stats(const Rows &rows, const AcceptPlan &plan,
                            const SamplingParams &sp, const Ws &w, hipStream_t stream) {
    // One launch when rows finish without counters; otherwise batches of at
    // most kRowSlots rows, each batch reusing the same counter slots.
    const int batch = plan.chunks > 1 ? kRowSlots : plan.rows;
    for (int r0 = 0; r0 < plan.rows; r0 += batch) {
        const int n = std::min(batch, plan.rows - r0);
        row_stats_kernel<<<dim3(n, plan.chunks), kThreads, 0, stream>>>(
            rows, r0, plan.chunks, plan.chunk_len, sp, w);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

Ws carve(const AcceptPlan &p, void *base) {
    unsigned char *b = reinterpret_cast<unsigned char *>(base);
    Ws w;
    w.row_cnt = reinterpret_cast<unsigned *>(b + p.off_row_cnt);
    w.seq_cnt = reinterpret_cast<unsigned *>(b + p.off_seq_cnt);
    w.chunk_stats = reinterpret_cast<ChunkStat *>(b + p.off_chunk_stats);
    w.chunk_keys = reinterpret_cast<uint64_t *>(b + p.off_chunk_keys);
    w.row_final = reinterpret_cast<RowFinal *>(b + p.off_row_final);
    w.row_keys = reinterpret_cast<uint64_t *>(b + p.off_row_keys);
    w.seq_sums = reinterpret_cast<float2 *>(b + p.off_seq_sums);
    return w;
}

} // namespace

SamplingParams sampling_params(float temperature, int top_k, float top_p, int V) {
    SamplingParams sp{};
    const bool greedy = !(temperature > 0.0f) || top_k == 1;
    int k_eff = V;
    if (greedy)
        k_eff = 1;
    else if (top_k >= 1 && top_k < V)
        k_eff = top_k;
    sp.k_eff = k_eff;
    sp.use_p = !greedy && (top_p < 1.0f);
    sp.top_p = top_p;
    sp.candidates = (k_eff < V) || sp.use_p;
    float scale = greedy ? 1.0f : (float)(1.4426950408889634 / (double)temperature);
    if (!(scale <= FLT_MAX))
        scale = FLT_MAX;
    sp.scale = scale;
    return sp;
}

AcceptPlan accept_plan(int B, int D, int V, int k_eff, bool candidates) {
    AcceptPlan p{};
    p.B = B;
    p.D = D;
    p.V = V;
    p.rows = B * (2 * D + 1);
    if (candidates) {
        p.chunk_len = kCandChunk;
    } else {
        int C = (kTargetBlocks + std::max(p.rows, 1) - 1) / std::max(p.rows, 1);
        C = std::max(1, std::min(C, (V + 2047) / 2048));
        int len = (V + C - 1) / C;
        p.chunk_len = ((len + 1023) / 1024) * 1024;
    }
    p.chunks = std::max(1, (V + p.chunk_len - 1) / p.chunk_len);
    if (candidates) {
        p.chunks3 = 1;
        p.chunk3_len = V;
    } else {
        int C3 = (kTargetBlocks + std::max(B, 1) - 1) / std::max(B, 1);
        C3 = std::max(1, std::min(C3, std::min(64, (V + 2047) / 2048)));
        if (B > kSeqSlots)
            C3 = 1;
        int len = (V + C3 - 1) / C3;
        p.chunk3_len = ((len + 1023) / 1024) * 1024;
        p.chunks3 = std::max(1, (V + p.chunk3_len - 1) / p.chunk3_len);
    }
    const int k = candidates ? k_eff : 0;
    size_t off = 0;
    p.off_row_cnt = off;     off += (size_t)kRowSlots * sizeof(unsigned);
    p.off_seq_cnt = off;     off += (size_t)kSeqSlots * sizeof(unsigned);
    p.off_chunk_stats = off; off += align256((size_t)p.rows * p.chunks * sizeof(ChunkStat));
    p.off_chunk_keys = off;  off += align256((size_t)p.rows * p.chunks * k * sizeof(uint64_t));
    p.off_row_final = off;   off += align256((size_t)p.rows * sizeof(RowFinal));
    p.off_row_keys = off;    off += align256((size_t)p.rows * k * sizeof(uint64_t));
    p.off_seq_sums = off;    off += align256((size_t)B * p.chunks3 * sizeof(float2));
    p.ws_bytes = off;
    return p;
}

hipError_t launch_accept(const float *target, const float *draft,
                         const int32_t *draft_tokens, const float *uniforms,
                         const AcceptPlan &plan, const SamplingParams &sp,
                         int32_t *accepted_len, int32_t *next_token,
                         float *p_draft, float *q_draft, void *ws,
                         hipStream_t stream) {
    if (plan.B == 0)
        return hipSuccess;
    Rows rows{target, draft, plan.D, plan.V};
    Ws w = carve(plan, ws);
    hipError_t e = launch_row_stats(rows, plan, sp, w, stream);
    if (e != hipSuccess)
        return e;
    accept_kernel<<<dim3(plan.B, plan.chunks3), kThreads, 0, stream>>>(
        rows, sp, draft_tokens, uniforms, plan.chunks3, plan.chunk3_len,
        accepted_len, next_token, p_draft, q_draft, w);
    return hipGetLastError();
}

hipError_t launch_probs(const float *logits, const AcceptPlan &plan,
                        const SamplingParams &sp, float *probs, void *ws,
                        hipStream_t stream) {
    if (plan.B == 0)
        return hipSuccess;
    Rows rows{logits, nullptr, 0, plan.V};
    Ws w = carve(plan, ws);
    hipError_t e = launch_row_stats(rows, plan, sp, w, stream);
    if (e != hipSuccess)
        return e;
    const int pc = (plan.V + 4095) / 4096;
    probs_kernel<<<dim3(plan.rows, pc), kThreads, 0, stream>>>(rows, sp, 4096, probs, w);
    return hipGetLastError();
}

} // namespace spec
