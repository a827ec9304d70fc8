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
// Kernels (no workgroup ever waits for, or signals, another: each step's
// results reach the next through the kernel boundary, so there are no
// fences, counters or spin waits):
//  1. row_stats / row_chunk -- grid (row, chunk).  One streaming pass over
//     every fp32 logit.  Full-vocabulary mode (row_stats_kernel; rows that
//     are not 16-byte aligned go to row_chunk_kernel<false>): per-chunk
//     running max and sum of exp2((z - max) * log2(e)/T), and on target rows
//     every 256-token block's sum relative to the chunk's max.  Candidate
//     mode (top-k active, top-p, or greedy; row_chunk_kernel<true>): the
//     chunk's top-k (logit, index) keys.  A row that is a single chunk is
//     finalized right here.
//  2. row_merge  -- grid (row), candidate rows that span several chunks (and
//     every such row for the dense probabilities): merges the chunks into
//     the row's final statistics.  The draw kernels merge full-vocabulary
//     rows of their own sequence themselves.
//  3. draw_sums  -- grid (sequence, chunk), full-vocabulary rows without
//     block sums (not 16-byte aligned): recomputes the D ratio tests and sums
//     the target row's mass over every 256-token block.
//  4. draw_final -- grid (sequence): decisions, then the draw.  Bonus: the
//     inverse CDF over the target row's block masses, then one block scanned
//     in vocabulary order.  Residual: candidates drawn from the target row
//     and kept with probability (p - q)/p (falling back to the residual's
//     inverse CDF).  In candidate mode the draw runs over the <= 256 kept
//     candidates instead.
//     draw_fused    -- the same in one 1024-thread workgroup per sequence,
//     for every full-vocabulary batch whose rows have block sums, and for
//     the others from 128 sequences on (same masses, same draw).
//  5. probs      -- dense write of the distributions (spec_sample_probs).
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
// Batches whose rows lack block sums (not 16-byte aligned) are drawn by the
// fused kernel from this many sequences on (half the CUs busy); below, the
// block sums are spread over a launch of their own first.
constexpr int kFusedMinB = 128;
// Statistics pass over 16-byte aligned rows: workgroup size and 16-byte
// loads per thread in flight (measured: 256 x 8 slightly ahead of 256 x 4
// and 512 x 4; 128-thread workgroups 4-5% slower).
constexpr int kStatsThreads = 256;
constexpr int kStatsLoads = 8;
constexpr int kBlock = 256;         // tokens per draw block (64 lanes x 4)
// Block statistics of one statistics chunk are gathered in LDS and written
// out once, contiguously (single-lane scattered 8-byte stores measured 20 us
// slower over 1536 rows of 151936 logits); full-vocabulary chunks hold at
// most this many blocks.
constexpr int kStatsLdsBlocks = 1024;

constexpr int kInvalid = 1;         // row flag: NaN / +inf / no finite logit
constexpr int kMaxDepth = 15;       // drafts per sequence at most (the ABI's limit)

// Logit loads of the statistics pass are non-temporal: every logit is read
// once there, and keeping it out of the caches measured 12% faster for the
// pass plus the draw that follows (which then re-read one or two rows per
// sequence with ordinary loads; it now reads one 256-token block per
// candidate, and whole rows only on the residual's fallback).
typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_once(const float4 *p) {
    const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float load_once(const float *p) {
    return __builtin_nontemporal_load(p);
}

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
    ChunkStat *chunk_stats;     // [rows][chunks]
    uint64_t *chunk_keys;       // [rows][chunks][k]  (candidate mode)
    RowFinal *row_final;        // [rows]
    uint64_t *row_keys;         // [rows][k]          (candidate mode)
    float2 *block_sums;         // [B][nblocks]  (draw mass, target mass)
    float *block_stats;         // [B][D + 1][nblocks]  target blocks' sums of
                                // exponentials relative to their chunk's max
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
// Wave reductions by DPP lane moves (no LDS round trip per step): neighbour
// pairs, quads, half rows and rows of 16 lanes, then the row broadcasts fold
// row 0 into row 1, row 2 into row 3, and rows 0-1 into rows 2-3, leaving the
// total in lane 63, which every lane reads back.  A fixed tree, so the sum is
// deterministic.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <class Op>
__device__ __forceinline__ float wave_reduce_tree(float v, Op op, float identity) {
    v = op(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]
    v = op(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
    v = op(v, dpp_f<0x141>(v));   // row_half_mirror
    v = op(v, dpp_f<0x140>(v));   // row_mirror
    // row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3; the
    // other rows take the identity
    v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(
                  __float_as_int(identity), __float_as_int(v), 0x142, 0xA, 0xF, false)));
    v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(
                  __float_as_int(identity), __float_as_int(v), 0x143, 0xC, 0xF, false)));
    return v;   // the total in lane 63
}
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op, float identity) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_reduce_tree(v, op, identity)), 63));
}
// The wave's sum in lane 63 only (other lanes hold partial sums).
__device__ __forceinline__ float wave_sum_lane63(float v) {
    return wave_reduce_tree(v, [](float a, float b) { return a + b; }, 0.0f);
}
// Orders one wave's LDS writes before its following LDS reads (and reads
// before later writes): a wave's LDS operations run in program order, so
// only the compiler must not move them across this point.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__device__ __forceinline__ float wave_sum(float v) {
    return wave_reduce(v, [](float a, float b) { return a + b; }, 0.0f);
}
__device__ __forceinline__ float wave_max(float v) {
    return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); }, -INFINITY);
}
// The same tree on unsigned 32-bit words (max; 0 is the identity), to every
// lane.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0xB1, 0xF>(v));
    v = max(v, dpp_u32<0x4E, 0xF>(v));
    v = max(v, dpp_u32<0x141, 0xF>(v));
    v = max(v, dpp_u32<0x140, 0xF>(v));
    v = max(v, dpp_u32<0x142, 0xA>(v));
    v = max(v, dpp_u32<0x143, 0xC>(v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// Largest key of the wave, to every lane: the largest high word first (the
// logit's code), then, only if several lanes hold it, the largest low word
// among them; otherwise the one lane's low word is read directly.  The same
// result as a 64-bit tree, in about a third of the instructions.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    const uint32_t hi = (uint32_t)(v >> 32);
    const uint32_t mh = wave_max_u32(hi);
    const unsigned long long at = __ballot(hi == mh);
    uint32_t lo;
    if (__popcll(at) == 1)
        lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, __ffsll((long long)at) - 1);
    else
        lo = wave_max_u32(hi == mh ? (uint32_t)v : 0u);
    return ((uint64_t)mh << 32) | lo;
}
// The k-th largest (1 <= k <= 64) of the wave's 64 distinct keys, to every
// lane: k rounds of the wave max, each retiring the lane that holds it.
__device__ __forceinline__ uint64_t wave_kth_largest(uint64_t v, int k) {
    uint64_t top = 0;
    for (int i = 0; i < k; ++i) {
        top = wave_max_u64(v);
        if (v == top)
            v = 0;
    }
    return top;
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

// Inclusive scan of one int per thread, in thread order.  Inside the wave
// by DPP: shifts by 1, 2, 4, 8 within each row of 16 lanes, then the row
// broadcasts carry row totals into the rows above (no LDS round trips).
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_shift_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
__device__ int block_incl_scan(int v, int *sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v += dpp_shift_i<0x111, 0xF>(v);   // row_shr:1
    v += dpp_shift_i<0x112, 0xF>(v);   // row_shr:2
    v += dpp_shift_i<0x114, 0xF>(v);   // row_shr:4
    v += dpp_shift_i<0x118, 0xF>(v);   // row_shr:8
    v += dpp_shift_i<0x142, 0xA>(v);   // row_bcast:15 into rows 1, 3
    v += dpp_shift_i<0x143, 0xC>(v);   // row_bcast:31 into rows 2, 3
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

// Gathers the nonzero keys at or above theta among those `each` visits
// (a functor calling f(key) for every key this thread owns) into out[], in
// thread order, and returns how many there are (only the first cap are
// stored).  Positions come from one block-wide scan of the per-thread
// counts, so no two threads contend for a counter.  sh: kWaves ints.
template <class Each>
__device__ int block_gather_ge(Each each, uint64_t theta, uint64_t *out, int cap, int *sh) {
    int cnt = 0;
    each([&](uint64_t key) { cnt += (key != 0 && key >= theta) ? 1 : 0; });
    int pos = block_incl_scan(cnt, sh) - cnt;
    int total = 0;
    for (int w = 0; w < kWaves; ++w)
        total += sh[w];
    each([&](uint64_t key) {
        if (key != 0 && key >= theta) {
            if (pos < cap)
                out[pos] = key;
            ++pos;
        }
    });
    return total;
}

// Sorts keys[0..n) in LDS (n <= kThreads, keys unique) into descending
// order, in place, by rank: thread t's key moves to the number of keys
// greater than it.  n broadcast reads per thread (issued eight at a time, so
// their latencies overlap) and two barriers -- far fewer steps than a
// sorting network for the short lists sorted here.
__device__ void block_sort_desc(uint64_t *keys, int n) {
    __syncthreads();   // the caller's writes to keys
    const int t = threadIdx.x;
    uint64_t mine = 0;
    int rank = 0;
    if (t < n) {
        mine = keys[t];
        int j = 0;
        for (; j + 8 <= n; j += 8) {
            uint64_t v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                v[q] = keys[j + q];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                rank += v[q] > mine;
        }
        for (; j < n; ++j)
            rank += keys[j] > mine;
    }
    __syncthreads();
    if (t < n)
        keys[rank] = mine;
    __syncthreads();
}

// ------------------------------------------------------- row statistics ----
struct StatsShared {
    SelectShared sel;
    uint64_t keys[kMaxCand * 2];
    uint64_t kth[kWaves];
    float fsh[kWaves];
    float fsh2[kWaves];
    int ish[kWaves];
};

// Reads lane l's value of v (l uniform).
__device__ __forceinline__ float lane_value(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Sorted candidates -> the row's final statistics (top-p cut, normalizer).
// keys[0..got) sorted by rank, in LDS; called by all threads.  Wave 0 does
// the work: lane l computes the weights of candidates l, l + 64, ..., then
// the cumulative sums run in rank order, one addition at a time (the order
// fixes their rounding), each lane keeping the sums at its own candidates;
// the top-p cut is the first candidate whose cumulative share reaches
// top_p, found by one division per lane and a ballot.
__device__ void finalize_candidates(const uint64_t *keys, int got, int flags,
                                    const SamplingParams &sp, int r, Ws &ws) {
    constexpr int Q = kMaxCand / 64;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const float m = key_logit(keys[0]);
        float w[Q], cs[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int i = lane + 64 * q;
            w[q] = i < got ? weight(key_logit(keys[i]), m, sp.scale) : 0.0f;
            cs[q] = 0.0f;
        }
        float cum = 0.0f;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int cnt = min(64, got - 64 * q);
            for (int l = 0; l < cnt; ++l) {
                cum += lane_value(w[q], l);
                cs[q] = lane == l ? cum : cs[q];
            }
        }
        const float S_all = cum;
        int kept = got;
        float S_kept = S_all;
        if (sp.use_p) {
#pragma unroll
            for (int q = Q - 1; q >= 0; --q) {
                const int i = lane + 64 * q;
                const unsigned long long hit = __ballot(i < got && cs[q] / S_all >= sp.top_p);
                if (hit) {
                    const int l = __ffsll((long long)hit) - 1;
                    kept = 64 * q + l + 1;
                    S_kept = lane_value(cs[q], l);
                }
            }
            if (kept == got)
                S_kept = S_all;
        }
        if (lane == 0)
            ws.row_final[r] = RowFinal{m, 1.0f / S_kept, kept, flags};
    }
    uint64_t *rk = ws.row_keys + (size_t)r * sp.k_eff;
    for (int i = threadIdx.x; i < sp.k_eff; i += kThreads)
        rk[i] = (i < got) ? keys[i] : 0;
}

// CAND: candidate mode (top-k / top-p / greedy).  The two modes are separate
// instantiations so the full-vocabulary pass is not held to the register
// budget of the radix selection (fewer registers, more waves per CU).
template <bool CAND>
__global__ __launch_bounds__(kThreads) void row_chunk_kernel(
    Rows rows, int chunks, int chunk_len, SamplingParams sp, Ws ws) {
    __shared__ StatsShared sh;
    const int r = blockIdx.x;
    const int c = blockIdx.y;
    const int V = rows.V;
    const float *z = rows.row(r);
    const int lo = c * chunk_len;
    const int hi = min(V, lo + chunk_len);
    const float scale = sp.scale;
    int bad = 0, finite = 0;

    if (!CAND) {
        // ---- running max and normalizer over the chunk ----
        float m = -INFINITY, S = 0.0f;
        // rows not 16-byte aligned (aligned rows go to row_stats_kernel)
        for (int e = lo + threadIdx.x; e < hi; e += kThreads) {
            const float v = load_once(&z[e]);
            bad |= !(v < INFINITY);   // NaN or +inf
            const float bm = fmaxf(m, v);
            if (bm > -INFINITY) {
                S = ((m == bm) ? S : S * weight(m, bm, scale)) + weight(v, bm, scale);
                m = bm;
            }
        }
        // A finite logit was seen iff the running max left -inf (a +inf
        // sets bad as well, and NaN never enters the max).
        finite = m > -INFINITY;
        wave_merge_ms(m, S, scale);
        __syncthreads();
        if ((threadIdx.x & 63) == 0) {
            sh.fsh[threadIdx.x >> 6] = m;
            sh.fsh2[threadIdx.x >> 6] = S;
        }
        {
            const int f = block_or((bad ? 1 : 0) | (finite ? 2 : 0), sh.ish);
            bad = f & 1;
            finite = (f >> 1) & 1;
        }
        if (threadIdx.x == 0) {
            float mm = sh.fsh[0], SS = sh.fsh2[0];
            for (int w = 1; w < kWaves; ++w)
                merge_ms(mm, SS, sh.fsh[w], sh.fsh2[w], scale);
            if (chunks == 1)
                ws.row_final[r] = RowFinal{mm, 1.0f / SS, 0, (bad || !finite) ? kInvalid : 0};
            else
                ws.chunk_stats[(size_t)r * chunks + c] = ChunkStat{mm, SS, bad, finite};
        }
        return;
    }

    // ---- candidate mode: the chunk's top-k keys ----
    constexpr int E = kCandChunk / kThreads;  // 16 keys per thread
    uint64_t mine[E];
#pragma unroll
    for (int q = 0; q < E; ++q) {
        const int e = lo + q * kThreads + threadIdx.x;
        if (e < hi) {
            const float v = load_once(&z[e]);
            bad |= (v != v) | (v == INFINITY);
            finite |= (v > -INFINITY) & (v < INFINITY);
            mine[q] = make_key(v, e);
        } else {
            mine[q] = 0;  // below every real key; never visited (see each)
        }
    }
    const int n = hi - lo;
    auto each = [&](auto f) {
#pragma unroll
        for (int q = 0; q < E; ++q)
            if (lo + q * kThreads + (int)threadIdx.x < hi)
                f(mine[q]);
    };
    const int want = min(sp.k_eff, n);
    int got = -1;
    if (n >= kThreads && want < kThreads) {
        // Every thread holds a key.  Each wave finds the ceil(want / 4)-th
        // largest of its 64 per-thread maxima; the smallest of those four is
        // at most the want-th largest key (at least want distinct keys lie
        // at or above it), so the keys at or above it hold the whole top-k.
        // Those few are sorted by rank: no radix passes.
        uint64_t tmax = 0;
#pragma unroll
        for (int q = 0; q < E; ++q)
            tmax = max(tmax, mine[q]);
        const uint64_t kth = wave_kth_largest(tmax, (want + kWaves - 1) / kWaves);
        if ((threadIdx.x & 63) == 0)
            sh.kth[threadIdx.x >> 6] = kth;
        __syncthreads();
        uint64_t theta = sh.kth[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            theta = min(theta, sh.kth[w]);
        uint64_t *cand = sh.keys + kMaxCand;   // second half; the result goes to the first
        const int C = block_gather_ge(each, theta, cand, kMaxCand, sh.sel.scan);
        __syncthreads();
        if (C <= kMaxCand) {   // else (many equal-valued... or spread keys): the general select
            block_sort_desc(cand, C);
            for (int i = threadIdx.x; i < want; i += kThreads)
                sh.keys[i] = cand[i];
            got = want;
        }
        __syncthreads();
    }
    const bool sorted = got >= 0;
    if (!sorted)   // few keys, or too many above the bound: select among all
        got = block_select_topk(each, n, sp.k_eff, sh.keys, kMaxCand, sh.sel);
    // the chunk's keys leave sorted (descending), so a small-k merge can walk
    // the chunks' lists from their heads
    if (!sorted)
        block_sort_desc(sh.keys, got);
    {
        const int f = block_or((bad ? 1 : 0) | (finite ? 2 : 0), sh.ish);
        bad = f & 1;
        finite = (f >> 1) & 1;
    }
    if (chunks == 1) {
        finalize_candidates(sh.keys, got, (bad || !finite) ? kInvalid : 0, sp, r, ws);
        return;
    }
    uint64_t *dst = ws.chunk_keys + ((size_t)r * chunks + c) * sp.k_eff;
    for (int i = threadIdx.x; i < sp.k_eff; i += kThreads)
        dst[i] = (i < got) ? sh.keys[i] : 0;
    if (threadIdx.x == 0)
        ws.chunk_stats[(size_t)r * chunks + c] = ChunkStat{0.0f, 0.0f, bad, finite};
}

// The full-vocabulary statistics pass on its own (rows of 16-byte aligned
// logits, no per-block output): NT threads, NV 16-byte loads per thread in
// flight per step, the same per-thread online update as row_chunk_kernel,
// then the waves merged in index order.
template <int NT, int NV>
__global__ __launch_bounds__(NT) void row_stats_kernel(
    Rows rows, int chunks, int chunk_len, SamplingParams sp, Ws ws) {
    constexpr int NW = NT / 64;
    __shared__ float s_m[NW], s_S[NW];
    __shared__ int s_flags[NW];
    static_assert(NV == 8, "the block-sum transpose reads two float4 per lane: 8 blocks");
    __shared__ __align__(16) float s_red[NW][NV][64];
    __shared__ float2 s_bst[kStatsLdsBlocks];
    const int r = blockIdx.x;
    const int c = blockIdx.y;
    const int V = rows.V;
    const float4 *z4 = reinterpret_cast<const float4 *>(rows.row(r));
    const int lo = c * chunk_len;
    const int hi = min(V, lo + chunk_len);
    const float scale = sp.scale;
    // Target rows of a full-vocabulary draw also leave, per 256-token block,
    // the block's sum of exp2((z - M) * scale) with M the chunk's max, so the
    // draw needs no second pass over the row.  For each u, the 64 lanes of a
    // wave hold one whole block (chunks start on 1024-token boundaries).
    const int per_seq = 2 * rows.D + 1;
    const int seq = r / per_seq, pos = r - seq * per_seq;
    const bool emit = sp.block_stats && pos <= rows.D;
    const int nblocks = (V + kBlock - 1) / kBlock;
    float *bstat = ws.block_stats + ((size_t)seq * (rows.D + 1) + pos) * nblocks;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float m = -INFINITY, S = 0.0f;
    // Loads are clamped into the chunk and lanes past its end masked to
    // -inf, which adds nothing below.
    auto load = [&](int base, float *v) {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int e = base + u * NT * 4;
            const float4 t = load_once(&z4[min(e, hi - 4) >> 2]);
            const bool in = e < hi;
            v[4 * u + 0] = in ? t.x : -INFINITY;
            v[4 * u + 1] = in ? t.y : -INFINITY;
            v[4 * u + 2] = in ? t.z : -INFINITY;
            v[4 * u + 3] = in ? t.w : -INFINITY;
        }
    };
    // Invalid logits (NaN, +inf) are not tested one by one: either enters
    // the sum of exponentials as NaN (a NaN's weight is NaN; a +inf makes
    // the running max +inf and its own weight exp2(NaN)), which stays NaN
    // through every rescale and merge.  Only a NaN among values that are
    // otherwise all -inf skips the sum, and is looked for there.
    int hidden_nan = 0;
    // The running max is kept per wave, so one set of exponentials serves
    // the normalizer and, on target rows, the block sums: block u of an
    // iteration is stored as (the wave's running max M, its sum of
    // exp2((z - M) * scale)).  The lanes' four-token partial sums of the
    // wave's NV blocks pass through LDS (transposed: each lane picks up four
    // partials of two blocks), then 16-lane DPP folds finish them.  Target and draft rows are
    // summed alike, so identical rows get identical statistics.  The loop
    // bound is the same for every thread, so each wave reduces whole blocks.
    float(*red)[64] = s_red[wave];
    for (int base0 = lo; base0 < hi; base0 += NT * 4 * NV) {
        float v[4 * NV];
        load(base0 + threadIdx.x * 4, v);
        float lm = m;
#pragma unroll
        for (int q = 0; q < 4 * NV; ++q)
            lm = fmaxf(lm, v[q]);
        const float bm = wave_max(lm);
        float t0 = 0.0f, t1 = 0.0f;
        if (bm > -INFINITY) {
            float s = (m == bm) ? S : S * weight(m, bm, scale);
#pragma unroll
            for (int u = 0; u < NV; ++u) {
                float sb = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sb += weight(v[4 * u + q], bm, scale);
                s += sb;
                if (emit)
                    red[u][lane] = sb;
            }
            S = s;
            m = bm;
            if (emit) {
                // Lane l reads 16 consecutive bytes at l and at 64 + l (no
                // bank conflicts): four partials of block l / 16 and four of
                // block 4 + l / 16; each row of 16 lanes then folds its two.
                wave_lds_sync();
                const float4 *rp = reinterpret_cast<const float4 *>(&red[0][0]);
                const float4 a = rp[lane], c = rp[64 + lane];
                t0 = (a.x + a.y) + (a.z + a.w);
                t1 = (c.x + c.y) + (c.z + c.w);
                t0 += dpp_f<0xB1>(t0);  t1 += dpp_f<0xB1>(t1);    // quad_perm [1,0,3,2]
                t0 += dpp_f<0x4E>(t0);  t1 += dpp_f<0x4E>(t1);    // quad_perm [2,3,0,1]
                t0 += dpp_f<0x141>(t0); t1 += dpp_f<0x141>(t1);   // row_half_mirror
                t0 += dpp_f<0x140>(t0); t1 += dpp_f<0x140>(t1);   // row_mirror
                wave_lds_sync();        // the reads above precede the next writes
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4 * NV; ++q)
                hidden_nan |= v[q] != v[q];
        }
        if (emit && (lane & 15) < 2) {
            const int u = (lane >> 4) + 4 * (lane & 1);
            const int lblk = (base0 - lo) / kBlock + wave + u * (NT * 4 / kBlock);
            if (lo + lblk * kBlock < hi)
                s_bst[lblk] = make_float2(bm, (lane & 1) ? t1 : t0);
        }
    }
    const int bad = hidden_nan | !(S == S);
    // a finite logit was seen iff the running max left -inf
    int flags = bad | ((m > -INFINITY) ? 2 : 0);
    wave_merge_ms(m, S, scale);
    flags = wave_or(flags);
    if ((threadIdx.x & 63) == 0) {
        s_m[threadIdx.x >> 6] = m;
        s_S[threadIdx.x >> 6] = S;
        s_flags[threadIdx.x >> 6] = flags;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float mm = s_m[0], SS = s_S[0];
        int f = s_flags[0];
        for (int w = 1; w < NW; ++w) {
            merge_ms(mm, SS, s_m[w], s_S[w], scale);
            f |= s_flags[w];
        }
        const int rbad = f & 1, rfin = (f >> 1) & 1;
        if (chunks == 1)
            ws.row_final[r] = RowFinal{mm, 1.0f / SS, 0, (rbad || !rfin) ? kInvalid : 0};
        else
            ws.chunk_stats[(size_t)r * chunks + c] = ChunkStat{mm, SS, rbad, rfin};
        s_m[0] = mm;
    }
    if (emit) {
        // The block sums, rescaled to the chunk's max, written out once,
        // contiguously and non-temporally: 4 bytes per block (HBM writes
        // measured costly while the pass streams: about 2 us per MB).
        __syncthreads();
        const float mm = s_m[0];
        const int nb = (hi - lo + kBlock - 1) / kBlock;
        for (int k = threadIdx.x; k < nb; k += NT) {
            const float2 st = s_bst[k];
            __builtin_nontemporal_store(st.y > 0.0f ? st.y * weight(st.x, mm, scale) : 0.0f,
                                        &bstat[lo / kBlock + k]);
        }
    }
}

// Final statistics of row r from its C chunk statistics, by one wave: lane
// l folds chunks l, l + 64, ... in order, then the lanes merge in a fixed
// butterfly.  Called by all 64 lanes; every lane returns the result.
__device__ RowFinal wave_row_final(const Ws &ws, int r, int C, float scale) {
    const int lane = threadIdx.x & 63;
    float m = -INFINITY, S = 0.0f;
    int f = 0;
    for (int cc = lane; cc < C; cc += 64) {
        const ChunkStat st = ws.chunk_stats[(size_t)r * C + cc];
        merge_ms(m, S, st.m, st.S, scale);
        f |= (st.bad ? 1 : 0) | (st.finite ? 2 : 0);
    }
    wave_merge_ms(m, S, scale);
    f = wave_or(f);
    return RowFinal{m, 1.0f / S, 0, ((f & 1) || !(f & 2)) ? kInvalid : 0};
}

// Chunk keys per thread held in registers by the merge (totals up to
// kThreads x this; larger totals are re-read from memory each round).
constexpr int kMergeRegKeys = 4;
// The k-way merge of sorted chunk lists: for k up to kMergeWalkK, at most
// 64 chunks (one per lane), and at most kMergeWalkMax keys in all (in LDS).
constexpr int kMergeWalkK = 64;
constexpr int kMergeWalkMax = 4096;

struct MergeShared : StatsShared {
    uint64_t walk[kMergeWalkMax];
};

__global__ __launch_bounds__(kThreads) void row_merge_kernel(
    Rows rows, int chunks, int chunk_len, SamplingParams sp, Ws ws) {
    __shared__ MergeShared sh;
    const int r = blockIdx.x;
    const int V = rows.V;
    const int k = sp.k_eff;
    const uint64_t *ck = ws.chunk_keys + (size_t)r * chunks * k;
    const int total = chunks * k;
    // Small k: the chunks' sorted lists are merged by a walk over their
    // heads (below).  Their loads go out first, beside the chunk flags'.
    const bool walk = sp.candidates && k <= kMergeWalkK && chunks <= 64 && total <= kMergeWalkMax;
    uint64_t staged[kMergeWalkMax / kThreads];
    if (walk) {
#pragma unroll
        for (int q = 0; q < kMergeWalkMax / kThreads; ++q) {
            const int i = q * kThreads + (int)threadIdx.x;
            staged[q] = i < total ? ck[i] : 0;
        }
    }
    // row flags: thread t folds chunks t, t + kThreads, ...
    int fl = 0;
    for (int cc = threadIdx.x; cc < chunks; cc += kThreads) {
        const ChunkStat st = ws.chunk_stats[(size_t)r * chunks + cc];
        fl |= (st.bad ? 1 : 0) | (st.finite ? 2 : 0);
    }
    fl = block_or(fl, sh.ish);
    const int flags = ((fl & 1) || !(fl & 2)) ? kInvalid : 0;
    if (!sp.candidates) {
        // the same merge the draw kernels do for themselves (wave_row_final)
        if (threadIdx.x < 64) {
            const RowFinal f = wave_row_final(ws, r, chunks, sp.scale);
            if (threadIdx.x == 0)
                ws.row_final[r] = f;
        }
        return;
    }
    // number of real keys: min(k, chunk length) per chunk
    int n_real = 0;
    for (int cc = 0; cc < chunks; ++cc)
        n_real += min(k, min(V, (cc + 1) * chunk_len) - cc * chunk_len);
    int got;
    if (walk) {
        got = min(k, n_real);
        // The row's top-k lie at or above a bound found as in the chunk
        // pass: each wave takes the ceil(got / 4)-th largest of its threads'
        // largest staged keys, and the smallest of the four is at most the
        // got-th largest key.  The keys at or above it are gathered and
        // sorted by rank: the same keys in the same order as the walk below,
        // which runs only when more than kMaxCand keys reach the bound.
        {
            uint64_t tmax = 0;
#pragma unroll
            for (int q = 0; q < kMergeWalkMax / kThreads; ++q)
                tmax = max(tmax, staged[q]);
            const uint64_t kth = wave_kth_largest(tmax, (got + kWaves - 1) / kWaves);
            if ((threadIdx.x & 63) == 0)
                sh.kth[threadIdx.x >> 6] = kth;
            __syncthreads();
            uint64_t theta = sh.kth[0];
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                theta = min(theta, sh.kth[w]);
            auto each_s = [&](auto f) {
#pragma unroll
                for (int q = 0; q < kMergeWalkMax / kThreads; ++q)
                    f(staged[q]);
            };
            uint64_t *cand = sh.keys + kMaxCand;
            const int C = block_gather_ge(each_s, theta, cand, kMaxCand, sh.sel.scan);
            if (C <= kMaxCand) {
                block_sort_desc(cand, C);
                for (int i = threadIdx.x; i < got; i += kThreads)
                    sh.keys[i] = cand[i];
                __syncthreads();
                finalize_candidates(sh.keys, got, flags, sp, r, ws);
                return;
            }
        }
        // The chunks' lists arrive sorted, so the row's top-k is a k-way
        // merge.  The lists are staged in LDS; wave 0 keeps list c's head in
        // lane c and k times takes the largest head (keys are unique) and
        // advances that list.  Each lane also holds the key after its head,
        // so an advance takes the held key and its LDS read (for the key
        // after that) has a whole step to arrive.
        uint64_t *lists = sh.walk;
#pragma unroll
        for (int q = 0; q < kMergeWalkMax / kThreads; ++q) {
            const int i = q * kThreads + (int)threadIdx.x;
            if (i < total)
                lists[i] = staged[q];
        }
        __syncthreads();
        if (threadIdx.x < 64) {
            const int lane = threadIdx.x;
            int pos = 0;
            uint64_t head = lane < chunks ? lists[lane * k] : 0;
            uint64_t next = (lane < chunks && k > 1) ? lists[lane * k + 1] : 0;
            for (int i = 0; i < got; ++i) {
                const uint64_t top = wave_max_u64(head);
                if (lane == 0)
                    sh.keys[i] = top;
                if (head == top) {   // the one list holding it
                    ++pos;
                    head = next;
                    next = pos + 1 < k ? lists[lane * k + pos + 1] : 0;
                }
            }
        }
        __syncthreads();
        finalize_candidates(sh.keys, got, flags, sp, r, ws);
        return;
    }
    if (total <= kThreads * kMergeRegKeys) {
        // Few keys (small k): each thread holds its share in registers for
        // all the selection rounds instead of re-reading them.
        uint64_t mine[kMergeRegKeys];
#pragma unroll
        for (int q = 0; q < kMergeRegKeys; ++q) {
            const int i = q * kThreads + (int)threadIdx.x;
            mine[q] = i < total ? ck[i] : 0;
        }
        auto each_r = [&](auto f) {
#pragma unroll
            for (int q = 0; q < kMergeRegKeys; ++q)
                if (mine[q] != 0)
                    f(mine[q]);
        };
        got = block_select_topk(each_r, n_real, k, sh.keys, kMaxCand, sh.sel);
    } else {
        auto each_g = [&](auto f) {
            for (int i = threadIdx.x; i < total; i += kThreads) {
                const uint64_t key = ck[i];
                if (key != 0)
                    f(key);
            }
        };
        got = block_select_topk(each_g, n_real, k, sh.keys, kMaxCand, sh.sel);
    }
    block_sort_desc(sh.keys, got);
    finalize_candidates(sh.keys, got, flags, sp, r, ws);
}


// ---------------------------------------------------------- verification ----
// Probability of token x under row r's final distribution, given its logit.
__device__ __forceinline__ float row_prob(const RowFinal &f, const uint64_t *keys,
                                          bool candidates, float scale, float zx, int x) {
#pragma clang fp contract(off)
    if (candidates && make_key(zx, x) < keys[f.n_kept - 1])
        return 0.0f;
    return weight(zx, f.m, scale) * f.inv;   // rounded here, never fused
}

// The final statistics of sequence b's 2D + 1 rows, staged in LDS: rf[i] for
// target position i, rf[D + 1 + i] for draft position i.  Full-vocabulary
// rows that span several chunks are merged here (sp.merge_chunks > 0), so
// no separate merge launch runs before the draw.  Called by all threads.
template <int NW>
__device__ void stage_row_finals(const Rows &rows, const Ws &ws, const SamplingParams &sp, int b,
                                 RowFinal *rf) {
    const int D = rows.D, n = 2 * D + 1;
    for (int i = (int)(threadIdx.x >> 6); i < n; i += NW) {
        const int r = i <= D ? rows.target_row(b, i) : rows.draft_row(b, i - D - 1);
        const RowFinal f = sp.merge_chunks > 0 ? wave_row_final(ws, r, sp.merge_chunks, sp.scale)
                                               : ws.row_final[r];
        if ((threadIdx.x & 63) == 0)
            rf[i] = f;
    }
    __syncthreads();
}

// The inputs of sequence b's D ratio tests that do not depend on the row
// statistics, loaded before those are staged so the two waits overlap:
// lane i < D of wave 0 holds draft token i, its target and draft logits
// (when the token is in range) and its uniform.  Called by all threads.
struct DecideInputs {
    int d;
    float zt, zd, u;
};
__device__ DecideInputs load_decide_inputs(const Rows &rows, const int32_t *draft_tokens,
                                           const float *uniforms, int b) {
    DecideInputs in{-1, 0.0f, 0.0f, 0.0f};
    const int i = threadIdx.x;
    if (i < rows.D) {
        in.d = draft_tokens[(size_t)b * rows.D + i];
        in.u = uniforms[(size_t)b * (rows.D + 1) + i];
        if (in.d >= 0 && in.d < rows.V) {
            in.zt = rows.row(rows.target_row(b, i))[in.d];
            in.zd = rows.row(rows.draft_row(b, i))[in.d];
        }
    }
    return in;
}

// Decisions of sequence b from the row statistics, one position per lane
// of wave 0: returns L (0..D) or -1 for an invalid sequence to every thread
// of the block (through *sh_L).  When p_out / q_out are given, wave 0 also
// writes P_i(d_i), Q_i(d_i) for the sequence (NaN if it is invalid).  Called
// by all threads of the block.
__device__ int decide_block(const Rows &rows, const Ws &ws, const SamplingParams &sp,
                            const RowFinal *rf, const DecideInputs &in, int b, float *p_out,
                            float *q_out, int *sh_L) {
    const int D = rows.D, V = rows.V;
    if (threadIdx.x < 64) {
        const int i = threadIdx.x;
        bool bad = false, rej = false;
        float p = 0.0f, q = 0.0f;
        if (i <= D)
            bad = rf[i].flags != 0;
        if (i < D) {
            const int tr = rows.target_row(b, i), dr = rows.draft_row(b, i);
            const RowFinal ft = rf[i], fd = rf[D + 1 + i];
            const int d = in.d;
            bad = bad || fd.flags != 0 || d < 0 || d >= V;
            if (!bad) {
                p = row_prob(ft, ws.row_keys + (size_t)tr * sp.k_eff, sp.candidates, sp.scale, in.zt, d);
                q = row_prob(fd, ws.row_keys + (size_t)dr * sp.k_eff, sp.candidates, sp.scale, in.zd, d);
                const float a = (p == 0.0f) ? 0.0f : p / q;
                rej = !(in.u < a);
            }
        }
        const unsigned long long any_bad = __ballot(bad);
        const unsigned long long rejects = __ballot(rej);
        const int L = any_bad ? -1 : (rejects ? __ffsll((long long)rejects) - 1 : D);
        if (i < D) {
            if (p_out) p_out[(size_t)b * D + i] = (L < 0) ? NAN : p;
            if (q_out) q_out[(size_t)b * D + i] = (L < 0) ? NAN : q;
        }
        if (i == 0)
            *sh_L = L;
    }
    __syncthreads();
    return *sh_L;
}

// The draw distribution of sequence b once L is known: target row L, and
// for a residual (L < D) the draft row L as well.
struct DrawRows {
    bool residual;
    RowFinal ft, fd;
    const float *zt, *zd;
    const uint64_t *kt, *kd;
};

__device__ DrawRows draw_rows(const Rows &rows, const Ws &ws, const SamplingParams &sp,
                              const RowFinal *rf, int b, int L) {
    DrawRows d;
    d.residual = L < rows.D;
    const int tr = rows.target_row(b, L);
    d.ft = rf[L];
    d.zt = rows.row(tr);
    d.kt = ws.row_keys + (size_t)tr * sp.k_eff;
    if (d.residual) {
        const int dr = rows.draft_row(b, L);
        d.fd = rf[rows.D + 1 + L];
        d.zd = rows.row(dr);
        d.kd = ws.row_keys + (size_t)dr * sp.k_eff;
    } else {
        d.fd = RowFinal{0.0f, 1.0f, 0, 0};
        d.zd = d.zt;
        d.kd = d.kt;
    }
    return d;
}

// The target-row view of a draw: block sums over it are (p, p).
__device__ __forceinline__ DrawRows target_only(const DrawRows &d) {
    DrawRows t = d;
    t.residual = false;
    t.fd = RowFinal{0.0f, 1.0f, 0, 0};
    t.zd = t.zt;
    t.kd = t.kt;
    return t;
}

// The stop row's block statistics (each block's sum of exp2((z - M) *
// scale), M its statistics chunk's max) to its block masses (p, p).
__device__ void stats_to_masses(const Rows &rows, const Ws &ws, const SamplingParams &sp,
                                const DrawRows &d, int b, int L, float2 *dst) {
#pragma clang fp contract(off)
    const int nblocks = (rows.V + kBlock - 1) / kBlock;
    const float *src = ws.block_stats + ((size_t)b * (rows.D + 1) + L) * nblocks;
    const int chunks = max(1, sp.merge_chunks);
    const ChunkStat *cs = ws.chunk_stats + (size_t)rows.target_row(b, L) * chunks;
    for (int k = threadIdx.x; k < nblocks; k += blockDim.x) {
        const float mc = chunks > 1 ? cs[k / sp.chunk_blocks].m : d.ft.m;
        const float mass = src[k] * weight(mc, d.ft.m, sp.scale) * d.ft.inv;
        dst[k] = make_float2(mass, mass);
    }
}

// Weights of token x: (residual max(0, p - q) or p, and p), full vocabulary.
// p and q are each rounded before the subtraction (contraction into a fused
// multiply-add is off here): where the two distributions agree, p - q is then
// exactly zero, as the rule has it, and an all-zero residual is recognized
// (draw from p instead).
__device__ __forceinline__ float2 draw_weight(const DrawRows &d, float scale, float zt, float zd) {
#pragma clang fp contract(off)
    const float p = weight(zt, d.ft.m, scale) * d.ft.inv;
    if (!d.residual)
        return make_float2(p, p);
    const float q = weight(zd, d.fd.m, scale) * d.fd.inv;
    return make_float2(fmaxf(p - q, 0.0f), p);
}

// Sums of the draw weights over 256-token blocks [blk_lo, blk_hi) of
// sequence b's draw rows, into out[blk]: wave w takes blocks w, w + NW, ...
// and each block is summed by one wave (four tokens per lane, then a fixed
// wave reduction), so the sums do not depend on the workgroup size.
template <int NW>
__device__ void block_draw_sums(const DrawRows &d, const SamplingParams &sp, int V, int blk_lo,
                                int blk_hi, float2 *out) {
    constexpr int kW = NW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if ((V & 3) == 0) {
        // kAhead blocks per wave in flight: their loads are all issued
        // before the first is reduced.  (Without a residual only the target
        // row is read.)
        constexpr int kAhead = 4;
        const float4 *zt4 = reinterpret_cast<const float4 *>(d.zt);
        const float4 *zd4 = reinterpret_cast<const float4 *>(d.zd);
        for (int blk0 = blk_lo + wave; blk0 < blk_hi; blk0 += kW * kAhead) {
            float4 t[kAhead], q[kAhead];
#pragma unroll
            for (int k = 0; k < kAhead; ++k) {
                const int blk = min(blk0 + k * kW, blk_hi - 1);
                const int e4 = min(blk * kBlock + 4 * lane, V - 4) >> 2;
                t[k] = load_once(&zt4[e4]);
                q[k] = d.residual ? load_once(&zd4[e4]) : t[k];
            }
#pragma unroll
            for (int k = 0; k < kAhead; ++k) {
                const int blk = blk0 + k * kW;
                if (blk >= blk_hi)
                    break;
                const int e = blk * kBlock + 4 * lane;
                const float zt[4] = {t[k].x, t[k].y, t[k].z, t[k].w};
                const float zd[4] = {q[k].x, q[k].y, q[k].z, q[k].w};
                float wr = 0.0f, wp = 0.0f;
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const float2 wv = draw_weight(d, sp.scale, zt[qq], zd[qq]);
                    const bool in = e + qq < V;
                    wr += in ? wv.x : 0.0f;
                    wp += in ? wv.y : 0.0f;
                }
                wr = wave_sum(wr);
                wp = wave_sum(wp);
                if (lane == 0)
                    out[blk] = make_float2(wr, wp);
            }
        }
        return;
    }
    // rows not 16-byte aligned: scalar loads
    for (int blk = blk_lo + wave; blk < blk_hi; blk += kW) {
        const int e = blk * kBlock + 4 * lane;   // this lane's 4 tokens
        float zt4[4], zd4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            zt4[q] = d.zt[min(e + q, V - 1)];
            zd4[q] = d.residual ? d.zd[min(e + q, V - 1)] : zt4[q];
        }
        float wr = 0.0f, wp = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float2 wv = draw_weight(d, sp.scale, zt4[q], zd4[q]);
            const bool in = e + q < V;
            wr += in ? wv.x : 0.0f;
            wp += in ? wv.y : 0.0f;
        }
        wr = wave_sum(wr);
        wp = wave_sum(wp);
        if (lane == 0)
            out[blk] = make_float2(wr, wp);
    }
}

// Kernel 3: per 256-token block, the target row's mass, for rows the
// statistics pass left no block sums for (not 16-byte aligned) in batches
// below the fused draw (several workgroups per sequence).
__global__ __launch_bounds__(kThreads) void draw_sums_kernel(
    Rows rows, SamplingParams sp, const int32_t *__restrict__ draft_tokens,
    const float *__restrict__ uniforms, int blocks_per_chunk, Ws ws) {
    __shared__ int s_L;
    const int b = blockIdx.x;
    const int c = blockIdx.y;
    const int V = rows.V;
    const int nblocks = (V + kBlock - 1) / kBlock;
    __shared__ RowFinal s_rf[2 * kMaxDepth + 1];
    const DecideInputs din = load_decide_inputs(rows, draft_tokens, uniforms, b);
    stage_row_finals<kWaves>(rows, ws, sp, b, s_rf);
    const int L = decide_block(rows, ws, sp, s_rf, din, b, nullptr, nullptr, &s_L);
    if (L < 0)
        return;
    const DrawRows d = draw_rows(rows, ws, sp, s_rf, b, L);
    const int blk_lo = c * blocks_per_chunk;
    const int blk_hi = min(nblocks, blk_lo + blocks_per_chunk);
    // the target row's block masses: the bonus draws from them, a residual
    // draws candidates from them
    block_draw_sums<kWaves>(target_only(d), sp, V, blk_lo, blk_hi, ws.block_sums + (size_t)b * nblocks);
}

template <int NW>
struct FinalSharedT {
    RowFinal rf[2 * kMaxDepth + 1];   // the sequence's row statistics
    float fsh[NW];
    int ish[NW];
    // rejection draw: inclusive prefix of the target mass per block run,
    // and each wave's candidate of a round
    float run_incl[kThreads];
    int cand[NW];
    int found;
    int L;
    float before, target;
    int use_p, blk;
    // candidate draw
    uint64_t ckey[kMaxCand];
    float cw[kMaxCand];
    float cp[kMaxCand];
};
using FinalShared = FinalSharedT<kWaves>;

// The full-vocabulary inverse-CDF draw of sequence b from its block sums:
// find the 256-token block holding u * total, then scan that block in
// vocabulary order.  The block runs belong to kThreads logical threads; in a
// larger workgroup the other threads own none and only join the barriers.
template <int NW>
__device__ void draw_full_vocab(const Rows &rows, const SamplingParams &sp, const float2 *bs,
                                const DrawRows &d, int b, int L, float u, FinalSharedT<NW> &sh,
                                int32_t *__restrict__ accepted_len,
                                int32_t *__restrict__ next_token) {
    const int V = rows.V;
    const float scale = sp.scale;
    // ---- full vocabulary: find the block holding u * total ----
    const int nblocks = (V + kBlock - 1) / kBlock;
    // Block masses: (residual mass, target mass), or (p, p) without a residual.
    auto mass = [&](int k, bool target_mass) -> float {
        const float2 v = bs[k];
        return target_mass ? v.y : v.x;
    };
    // thread t owns a contiguous run of blocks
    const int per = (nblocks + kThreads - 1) / kThreads;
    const int b_lo = min(nblocks, (int)threadIdx.x * per);
    const int b_hi = min(nblocks, b_lo + per);
    float my_r = 0.0f, my_p = 0.0f;
    for (int k = b_lo; k < b_hi; ++k) {
        my_r += mass(k, false);
        my_p += mass(k, true);
    }
    float incl_r = block_incl_scan_f(my_r, sh.fsh);
    __syncthreads();
    if (threadIdx.x == kThreads - 1)
        sh.use_p = !(incl_r > 0.0f);
    __syncthreads();
    const bool use_p = sh.use_p != 0;
    float incl = incl_r, mine = my_r;
    if (use_p) {
        incl = block_incl_scan_f(my_p, sh.fsh);
        mine = my_p;
    }
    if (threadIdx.x == kThreads - 1)
        sh.target = u * incl;   // u * total
    if (threadIdx.x == 0)
        sh.found = 0x7FFFFFFF;
    __syncthreads();
    const float target = sh.target;
    const float excl = incl - mine;
    if (incl > target && excl <= target)
        atomicMin(&sh.found, (int)threadIdx.x);
    __syncthreads();
    if ((int)threadIdx.x == (sh.found == 0x7FFFFFFF ? -1 : sh.found)) {
        float cum = excl;
        int pick = -1, last_pos = -1;
        float before = excl, last_before = excl;
        for (int k = b_lo; k < b_hi; ++k) {
            const float w = mass(k, use_p);
            before = cum;
            cum += w;
            if (w > 0.0f) {
                last_pos = k;
                last_before = before;
            }
            if (cum > target) {
                pick = k;
                break;
            }
        }
        if (pick < 0) {
            pick = last_pos;
            before = last_before;
        }
        sh.blk = pick;
        sh.before = before;
    }
    if (sh.found == 0x7FFFFFFF && threadIdx.x == 0) {
        // rounding left the target at or past the end: the last block with
        // positive mass
        int k = nblocks - 1;
        while (k > 0 && !(mass(k, use_p) > 0.0f))
            --k;
        sh.blk = k;
        float before = 0.0f;
        for (int kk = 0; kk < k; ++kk)
            before += mass(kk, use_p);
        sh.before = before;
    }
    __syncthreads();
    // ---- scan the chosen block in vocabulary order (one wave) ----
    if (threadIdx.x >= 64)
        return;
    const int lane = threadIdx.x;
    const int blk = sh.blk;
    const int e = blk * kBlock + 4 * lane;
    float w4[4];
    int last_local = -1;
    float lane_sum = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int x = e + q;
        float w = 0.0f;
        if (x < V) {
            const float2 wv = draw_weight(d, scale, d.zt[x], d.residual ? d.zd[x] : 0.0f);
            w = use_p ? wv.y : wv.x;
        }
        w4[q] = w;
        lane_sum += w;
        if (w > 0.0f)
            last_local = x;
    }
    // inclusive scan of the lane sums in lane order
    float incl_l = lane_sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float t = __shfl_up(incl_l, o);
        if (lane >= o)
            incl_l += t;
    }
    const float tgt = target - sh.before;
    const float excl_l = incl_l - lane_sum;
    int pick = -1;
    {
        float cum = excl_l;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            cum += w4[q];
            if (pick < 0 && w4[q] > 0.0f && cum > tgt)
                pick = e + q;
        }
    }
    // first lane (in vocabulary order) whose run crosses the target
    const unsigned long long hit = __ballot(pick >= 0);
    const unsigned long long pos = __ballot(last_local >= 0);
    if (hit) {
        const int first = __ffsll(hit) - 1;
        if (lane == first) {
            if (accepted_len) accepted_len[b] = L;
            next_token[b] = pick;
        }
    } else {
        // rounding: the target sits at the block end -- last positive token
        const int lastl = 63 - __clzll(pos);
        if (lane == lastl) {
            if (accepted_len) accepted_len[b] = L;
            next_token[b] = last_local;
        }
    }
}

// The residual draw over the full vocabulary, by rejection from the
// target distribution P of the stop row (MTPLX announcement, "Layer 2":
// the residual (p - q)+ replaces a rejected draft; the way it is sampled is
// this library's reading): candidate k is the inverse-CDF draw from P with
// uniform v_k, kept iff a_k < (P - Q) / P at it (P and Q in fp32, the
// quotient in fp32).  A candidate j is kept with probability
// max(0, 1 - Q(j)/P(j)), so the first kept one has exactly the residual's
// distribution -- and needs P's block masses (one pass over the target row)
// and one 256-token block per candidate, not the residual over both rows.
// v_k and a_k are outputs 2k and 2k + 1 of the SplitMix64 stream (Steele,
// Lea and Flood, "Fast splittable pseudorandom number generators", OOPSLA
// 2014) seeded with the bit pattern of the sequence's final uniform; after
// kCandidates candidates none of which is kept, the inverse CDF of the
// residual with output 2 kCandidates decides.
constexpr int kCandidates = 64;

__device__ __forceinline__ float stream_uniform(uint64_t seed, uint64_t i) {
    uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (float)(uint32_t)(z >> 40) * 0x1p-24f;
}

// Inclusive wave scan (lane order) of one float per lane.
__device__ __forceinline__ float wave_incl_scan_f(float v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float t = __shfl_up(v, o);
        if (lane >= o)
            v += t;
    }
    return v;
}

// One candidate, by one wave (every lane returns it): the first token x in
// vocabulary order whose cumulative target mass exceeds `target`, from the
// block masses bs[k].y (runs of `per` blocks per logical thread, their
// inclusive prefixes in run_incl) and the block's own tokens.  Where rounding
// leaves no crossing, the last position with positive mass is taken, as in
// the single draw.
__device__ int wave_candidate(const DrawRows &d, float scale, int V, const float2 *bs,
                              const float *run_incl, int per, float target) {
    const int lane = threadIdx.x & 63;
    const int nblocks = (V + kBlock - 1) / kBlock;
    // the run holding the target
    int t = -1;
    for (int c = 0; c < kThreads && t < 0; c += 64) {
        const unsigned long long m = __ballot(run_incl[c + lane] > target);
        if (m)
            t = c + __ffsll((long long)m) - 1;
    }
    if (t < 0) {   // past the end: the last run with positive mass
        for (int c = kThreads - 64; c >= 0 && t < 0; c -= 64) {
            const int tt = c + lane;
            const float ex = tt > 0 ? run_incl[tt - 1] : 0.0f;
            const unsigned long long m = __ballot(run_incl[tt] > ex);
            if (m)
                t = c + 63 - __clzll(m);
        }
        t = max(t, 0);
    }
    // the block within the run
    const int lo = min(nblocks, t * per), hi = min(nblocks, lo + per);
    float carry = t > 0 ? run_incl[t - 1] : 0.0f;
    int blk = -1, last_blk = -1;
    float before = carry, last_before = carry;
    for (int c0 = lo; c0 < hi && blk < 0; c0 += 64) {
        const int k = c0 + lane;
        const float m = k < hi ? bs[k].y : 0.0f;
        const float incl = wave_incl_scan_f(m) + carry;
        const unsigned long long hit = __ballot(m > 0.0f && incl > target);
        const unsigned long long pos = __ballot(m > 0.0f);
        if (hit) {
            const int f = __ffsll((long long)hit) - 1;
            blk = c0 + f;
            before = __shfl(incl - m, f);
        } else if (pos) {
            const int f = 63 - __clzll(pos);
            last_blk = c0 + f;
            last_before = __shfl(incl - m, f);
        }
        carry = __shfl(incl, 63);
    }
    if (blk < 0) {
        blk = max(last_blk, lo);
        before = last_blk >= 0 ? last_before : carry;
    }
    // the token within the block
    const int e = blk * kBlock + 4 * lane;
    float w4[4];
    float lane_sum = 0.0f;
    int last_local = -1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int x = e + q;
        const float w = x < V ? weight(d.zt[x], d.ft.m, scale) * d.ft.inv : 0.0f;
        w4[q] = w;
        lane_sum += w;
        if (w > 0.0f)
            last_local = x;
    }
    const float incl_l = wave_incl_scan_f(lane_sum);
    const float tgt = target - before;
    int pick = -1;
    {
        float cum = incl_l - lane_sum;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            cum += w4[q];
            if (pick < 0 && w4[q] > 0.0f && cum > tgt)
                pick = e + q;
        }
    }
    const unsigned long long hit = __ballot(pick >= 0);
    if (hit)
        return __shfl(pick, __ffsll((long long)hit) - 1);
    const unsigned long long pos = __ballot(last_local >= 0);
    return pos ? __shfl(last_local, 63 - __clzll(pos)) : blk * kBlock;
}

// The rejection draw of one sequence (d: a residual draw; bs: the block
// masses of its target row, (p, p) per block).  Called by all threads;
// returns the kept token to every thread, or -1 if no candidate was kept.
template <int NW>
__device__ int rejection_draw(const Rows &rows, const SamplingParams &sp, const float2 *bs,
                              const DrawRows &d, uint64_t seed, FinalSharedT<NW> &sh) {
#pragma clang fp contract(off)
    const int V = rows.V;
    const float scale = sp.scale;
    const int nblocks = (V + kBlock - 1) / kBlock;
    // runs of blocks per logical thread (kThreads of them, as the single
    // draw has), their target masses summed in order, then scanned
    const int per = (nblocks + kThreads - 1) / kThreads;
    const int b_lo = min(nblocks, (int)threadIdx.x * per);
    const int b_hi = min(nblocks, b_lo + per);
    float mine = 0.0f;
    for (int k = b_lo; k < b_hi; ++k)
        mine += bs[k].y;
    const float incl = block_incl_scan_f(mine, sh.fsh);
    if (threadIdx.x < kThreads)
        sh.run_incl[threadIdx.x] = incl;
    __syncthreads();
    const float total = sh.run_incl[kThreads - 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int k0 = 0; k0 < kCandidates; k0 += NW) {
        const uint64_t k = (uint64_t)(k0 + wave);
        const float v = stream_uniform(seed, 2 * k), a = stream_uniform(seed, 2 * k + 1);
        const int j = wave_candidate(d, scale, V, bs, sh.run_incl, per, v * total);
        const float pf = weight(d.zt[j], d.ft.m, scale) * d.ft.inv;
        const float qf = weight(d.zd[j], d.fd.m, scale) * d.fd.inv;
        const float thr = (pf - qf) / pf;
        if (lane == 0)
            sh.cand[wave] = (k0 + wave < kCandidates && a < thr) ? j : -1;
        __syncthreads();
        int tok = -1;
        for (int w = 0; w < NW && tok < 0; ++w)
            tok = sh.cand[w];
        __syncthreads();
        if (tok >= 0)
            return tok;
    }
    return -1;
}

// Kernel 4: decisions, then the inverse-CDF draw.
__global__ __launch_bounds__(kThreads) void draw_final_kernel(
    Rows rows, SamplingParams sp, const int32_t *__restrict__ draft_tokens,
    const float *__restrict__ uniforms, int32_t *__restrict__ accepted_len,
    int32_t *__restrict__ next_token, float *__restrict__ p_draft,
    float *__restrict__ q_draft, Ws ws) {
    __shared__ FinalShared sh;
    const int b = blockIdx.x;
    const int D = rows.D;
    const float scale = sp.scale;

    const DecideInputs din = load_decide_inputs(rows, draft_tokens, uniforms, b);
    stage_row_finals<kWaves>(rows, ws, sp, b, sh.rf);
    const int L = decide_block(rows, ws, sp, sh.rf, din, b, p_draft, q_draft, &sh.L);
    if (L < 0) {
        if (threadIdx.x == 0) {
            if (accepted_len) accepted_len[b] = -1;
            next_token[b] = -1;
        }
        return;
    }
    const float u = uniforms[(size_t)b * (D + 1) + D];
    const DrawRows d = draw_rows(rows, ws, sp, sh.rf, b, L);

    if (sp.candidates) {
        // ---- draw over the kept candidates of the target row ----
        const int n = d.ft.n_kept;
        for (int i = threadIdx.x; i < kMaxCand; i += kThreads) {
            if (i < n) {
                const uint64_t key = d.kt[i];
                const int x = key_index(key);
                const float p = row_prob(d.ft, d.kt, false, scale, key_logit(key), x);
                float w = p;
                if (d.residual) {
                    const float q = row_prob(d.fd, d.kd, true, scale, d.zd[x], x);
                    w = fmaxf(p - q, 0.0f);
                }
                // index-major sort key, complemented so a descending sort
                // yields ascending vocabulary order
                sh.ckey[i] = ~(((uint64_t)(uint32_t)x << 32) | (uint32_t)i);
                sh.cw[i] = w;
                sh.cp[i] = p;
            } else {
                sh.ckey[i] = 0;  // sorts last
            }
        }
        __syncthreads();
        block_sort_desc(sh.ckey, n);   // entries n.. are zero and stay last
        if (threadIdx.x < 64) {
            // Wave 0: lane l holds the candidates l, l + 64, ... in
            // vocabulary order (token, residual weight, target probability);
            // the totals and the running sum go one addition at a time in
            // that order, each lane keeping the sums at its own candidates;
            // the token is the first whose running sum passes u * total (else
            // the last with positive weight).
            constexpr int Q = kMaxCand / 64;
            const int lane = threadIdx.x;
            int xs[Q];
            float wr[Q], wp[Q], cs[Q];
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int i = lane + 64 * q;
                const uint64_t key = i < n ? ~sh.ckey[i] : 0;
                const int slot = (int)(uint32_t)key;
                xs[q] = (int)(key >> 32);
                wr[q] = i < n ? sh.cw[slot] : 0.0f;
                wp[q] = i < n ? sh.cp[slot] : 0.0f;
                cs[q] = 0.0f;
            }
            float tot = 0.0f;
#pragma unroll
            for (int q = 0; q < Q; ++q)
                for (int l = 0; l < min(64, n - 64 * q); ++l)
                    tot += lane_value(wr[q], l);
            const bool use_p = !(tot > 0.0f);
            if (use_p) {
                tot = 0.0f;
#pragma unroll
                for (int q = 0; q < Q; ++q)
                    for (int l = 0; l < min(64, n - 64 * q); ++l)
                        tot += lane_value(wp[q], l);
            }
            const float target = u * tot;
            float cum = 0.0f;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const float wq = use_p ? wp[q] : wr[q];
                for (int l = 0; l < min(64, n - 64 * q); ++l) {
                    cum += lane_value(wq, l);
                    cs[q] = lane == l ? cum : cs[q];
                }
            }
            int pick = -1, last_pos = -1;
#pragma unroll
            for (int q = Q - 1; q >= 0; --q) {
                const int i = lane + 64 * q;
                const unsigned long long pass = __ballot(i < n && cs[q] > target);
                if (pass)
                    pick = __shfl(xs[q], __ffsll((long long)pass) - 1);
            }
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int i = lane + 64 * q;
                const float wq = use_p ? wp[q] : wr[q];
                const unsigned long long pos = __ballot(i < n && wq > 0.0f);
                if (pos)
                    last_pos = __shfl(xs[q], 63 - __clzll((long long)pos));
            }
            if (pick < 0)
                pick = last_pos;
            if (lane == 0) {
                if (accepted_len) accepted_len[b] = L;
                next_token[b] = pick;
            }
        }
        return;
    }
    const int nblocks = (rows.V + kBlock - 1) / kBlock;
    // the target row's (p, p) block masses, as the block-sum launch left
    // them (rows with block statistics are drawn by draw_fused_kernel)
    float2 *bs = ws.block_sums + (size_t)b * nblocks;
    if (d.residual) {
        const uint32_t ubits = __float_as_uint(u);
        const int tok = rejection_draw(rows, sp, bs, d, (uint64_t)ubits, sh);
        if (tok >= 0) {
            if (threadIdx.x == 0) {
                if (accepted_len) accepted_len[b] = L;
                next_token[b] = tok;
            }
            return;
        }
        // no candidate kept: the residual's own sums, then its inverse CDF
        block_draw_sums<kWaves>(d, sp, rows.V, 0, nblocks, bs);
        __syncthreads();
        draw_full_vocab(rows, sp, bs, d, b, L, stream_uniform(ubits, 2 * kCandidates), sh,
                        accepted_len, next_token);
        return;
    }
    draw_full_vocab(rows, sp, bs, d, b, L, u, sh, accepted_len, next_token);
}

// Kernels 3 and 4 as one (full vocabulary): one 1024-thread workgroup per
// sequence decides (16 waves merge its rows' statistics in parallel), turns
// the target row's block sums into masses in LDS (or sums the blocks itself
// for rows without them), then draws.  Same masses and draw as the
// two-kernel path, one launch and one decision pass fewer.
constexpr int kFusedThreads = 1024;
// Block sums of rows up to this many 256-token blocks (262144 tokens) stay
// in LDS; longer rows use the workspace.
constexpr int kFusedLdsBlocks = 1024;
template <int NW>
struct FusedShared : FinalSharedT<NW> {
    float2 bsum[kFusedLdsBlocks];
};
__global__ __launch_bounds__(kFusedThreads) void draw_fused_kernel(
    Rows rows, SamplingParams sp, const int32_t *__restrict__ draft_tokens,
    const float *__restrict__ uniforms, int32_t *__restrict__ accepted_len,
    int32_t *__restrict__ next_token, float *__restrict__ p_draft,
    float *__restrict__ q_draft, Ws ws) {
    constexpr int NW = kFusedThreads / 64;
    __shared__ FusedShared<NW> sh;
    const int b = blockIdx.x;
    const int D = rows.D, V = rows.V;
    const DecideInputs din = load_decide_inputs(rows, draft_tokens, uniforms, b);
    stage_row_finals<NW>(rows, ws, sp, b, sh.rf);
    const int L = decide_block(rows, ws, sp, sh.rf, din, b, p_draft, q_draft, &sh.L);
    if (L < 0) {
        if (threadIdx.x == 0) {
            if (accepted_len) accepted_len[b] = -1;
            next_token[b] = -1;
        }
        return;
    }
    const float u = uniforms[(size_t)b * (D + 1) + D];
    const DrawRows d = draw_rows(rows, ws, sp, sh.rf, b, L);
    const int nblocks = (V + kBlock - 1) / kBlock;
    float2 *bs = nblocks <= kFusedLdsBlocks ? sh.bsum : ws.block_sums + (size_t)b * nblocks;
    // the target row's block masses (the bonus draws from them, a residual
    // draws candidates from them): from the row's block statistics, or summed
    // here over the row
    if (sp.block_stats)
        stats_to_masses(rows, ws, sp, d, b, L, bs);
    else
        block_draw_sums<NW>(target_only(d), sp, V, 0, nblocks, bs);
    __syncthreads();   // the block masses, written above, are read by other waves below
    if (d.residual) {
        const uint32_t ubits = __float_as_uint(u);
        const int tok = rejection_draw(rows, sp, bs, d, (uint64_t)ubits, sh);
        if (tok >= 0) {
            if (threadIdx.x == 0) {
                if (accepted_len) accepted_len[b] = L;
                next_token[b] = tok;
            }
            return;
        }
        block_draw_sums<NW>(d, sp, V, 0, nblocks, bs);
        __syncthreads();
        draw_full_vocab(rows, sp, bs, d, b, L, stream_uniform(ubits, 2 * kCandidates), sh,
                        accepted_len, next_token);
        return;
    }
    draw_full_vocab(rows, sp, bs, d, b, L, u, sh, accepted_len, next_token);
}

// ----------------------------------------------------------------- probs ----
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

Ws carve(const AcceptPlan &p, void *base) {
    unsigned char *b = reinterpret_cast<unsigned char *>(base);
    Ws w;
    w.chunk_stats = reinterpret_cast<ChunkStat *>(b + p.off_chunk_stats);
    w.chunk_keys = reinterpret_cast<uint64_t *>(b + p.off_chunk_keys);
    w.row_final = reinterpret_cast<RowFinal *>(b + p.off_row_final);
    w.row_keys = reinterpret_cast<uint64_t *>(b + p.off_row_keys);
    w.block_sums = reinterpret_cast<float2 *>(b + p.off_block_sums);
    w.block_stats = reinterpret_cast<float *>(b + p.off_block_stats);
    return w;
}

// merge_full: also merge full-vocabulary rows that span chunks into
// row_final (the draw kernels merge those themselves; the dense probs pass
// reads row_final).  Candidate rows are always merged here.
hipError_t launch_row_stats(const Rows &rows, const AcceptPlan &plan,
                            const SamplingParams &sp, const Ws &w, bool merge_full,
                            hipStream_t stream) {
    if (sp.candidates)
        row_chunk_kernel<true><<<dim3(plan.rows, plan.chunks), kThreads, 0, stream>>>(
            rows, plan.chunks, plan.chunk_len, sp, w);
    else if ((rows.V & 3) == 0)
        row_stats_kernel<kStatsThreads, kStatsLoads><<<dim3(plan.rows, plan.chunks), kStatsThreads, 0, stream>>>(
            rows, plan.chunks, plan.chunk_len, sp, w);
    else
        row_chunk_kernel<false><<<dim3(plan.rows, plan.chunks), kThreads, 0, stream>>>(
            rows, plan.chunks, plan.chunk_len, sp, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.chunks == 1 || !(sp.candidates || merge_full))
        return e;
    row_merge_kernel<<<plan.rows, kThreads, 0, stream>>>(rows, plan.chunks, plan.chunk_len, sp, w);
    return hipGetLastError();
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
        C = std::max(C, (V + kStatsLdsBlocks * kBlock - 1) / (kStatsLdsBlocks * kBlock));
        int len = (V + C - 1) / C;
        p.chunk_len = ((len + 1023) / 1024) * 1024;
    }
    p.chunks = std::max(1, (V + p.chunk_len - 1) / p.chunk_len);
    p.nblocks = (V + kBlock - 1) / kBlock;
    // The draw: one fused 1024-thread workgroup per sequence whenever the
    // statistics pass leaves the target rows' block sums (16-byte aligned
    // rows), and for rows without them from kFusedMinB sequences on; below
    // that, draw-sum workgroups of whole 256-token blocks (about
    // kTargetBlocks in total), then one draw workgroup per sequence.
    p.fused_draw = B >= kFusedMinB || (!candidates && V % 4 == 0);
    int C3 = (kTargetBlocks + std::max(B, 1) - 1) / std::max(B, 1);
    C3 = std::max(1, std::min(C3, (p.nblocks + 31) / 32));
    p.blocks_per_chunk3 = (p.nblocks + C3 - 1) / C3;
    p.chunks3 = (p.nblocks + p.blocks_per_chunk3 - 1) / p.blocks_per_chunk3;
    const int k = candidates ? k_eff : 0;
    size_t off = 0;
    p.off_chunk_stats = off; off += align256((size_t)p.rows * p.chunks * sizeof(ChunkStat));
    p.off_chunk_keys = off;  off += align256((size_t)p.rows * p.chunks * k * sizeof(uint64_t));
    p.off_row_final = off;   off += align256((size_t)p.rows * sizeof(RowFinal));
    p.off_row_keys = off;    off += align256((size_t)p.rows * k * sizeof(uint64_t));
    // full vocabulary: per sequence the draw's block masses, and (rows
    // 16-byte aligned) per target row the block statistics
    const size_t stat_rows = (candidates || V % 4 != 0) ? 0 : (size_t)B * (D + 1);
    p.off_block_sums = off;  off += align256(candidates ? 0 : (size_t)B * p.nblocks * sizeof(float2));
    p.off_block_stats = off; off += align256(stat_rows * p.nblocks * sizeof(float));
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
    SamplingParams spl = sp;
    spl.block_stats = !sp.candidates && (plan.V & 3) == 0;
    spl.merge_chunks = (!sp.candidates && plan.chunks > 1) ? plan.chunks : 0;
    spl.chunk_blocks = plan.chunk_len / kBlock;
    hipError_t e = launch_row_stats(rows, plan, spl, w, false, stream);
    if (e != hipSuccess)
        return e;
    if (!sp.candidates && plan.fused_draw) {
        draw_fused_kernel<<<plan.B, kFusedThreads, 0, stream>>>(
            rows, spl, draft_tokens, uniforms, accepted_len, next_token, p_draft, q_draft, w);
        return hipGetLastError();
    }
    if (!sp.candidates && !spl.block_stats) {
        draw_sums_kernel<<<dim3(plan.B, plan.chunks3), kThreads, 0, stream>>>(
            rows, spl, draft_tokens, uniforms, plan.blocks_per_chunk3, w);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    draw_final_kernel<<<plan.B, kThreads, 0, stream>>>(
        rows, spl, draft_tokens, uniforms, accepted_len, next_token, p_draft, q_draft, w);
    return hipGetLastError();
}

hipError_t launch_probs(const float *logits, const AcceptPlan &plan,
                        const SamplingParams &sp, float *probs, void *ws,
                        hipStream_t stream) {
    if (plan.B == 0)
        return hipSuccess;
    Rows rows{logits, nullptr, 0, plan.V};
    Ws w = carve(plan, ws);
    hipError_t e = launch_row_stats(rows, plan, sp, w, true, stream);
    if (e != hipSuccess)
        return e;
    const int pc = (plan.V + 4095) / 4096;
    probs_kernel<<<dim3(plan.rows, pc), kThreads, 0, stream>>>(rows, sp, 4096, probs, w);
    return hipGetLastError();
}

} // namespace spec
