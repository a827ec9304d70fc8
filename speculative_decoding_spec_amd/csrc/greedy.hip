// Greedy verification for gfx950: the sample-and-match loop over the
// target's argmax.
//
// With a greedy sampler (T <= 0 or top_k == 1: the mlxcel manual's
// DFlash-family drafter table) verification needs no probabilities: the
// savepearlharbor.com llama.cpp MTP article (how speculative decoding works)
// keeps each draft while it equals the target's own token at that position
// and emits the target's token at the first mismatch, or at the bonus
// position when every draft matched.  The probability-ratio rule reduces to
// the same thing when both distributions are one-hot, so this path returns
// what spec_verify_accept returns at top_k = 1 for valid draft rows, while
// reading only the target logits: half the bytes of the sampling path, and
// no exponentials.
//
// Kernels (no workgroup waits for another):
//  1. greedy_rows   -- grid (row, chunk).  One streaming pass over the
//     target logits: the chunk's largest logit and its first index, and
//     whether the chunk holds a NaN or +inf.
//  2. greedy_decide -- grid (sequence).  Merges each row's chunks in chunk
//     order, then one lane per position compares the draft with the row's
//     argmax; a ballot gives the first mismatch.
//
// Ties go to the lowest index everywhere: inside a thread the indices are
// visited in increasing order under a strict comparison, and every merge
// prefers the lower index among equal values.
#include "spec_internal.h"

#include <algorithm>
#include <climits>
#include <cmath>

namespace spec {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTargetBlocks = 1024;

struct GreedyChunk {
    float v;    // largest logit of the chunk (-inf if none is finite)
    int idx;    // its first index (INT_MAX if none)
    int bad;    // the chunk holds a NaN or +inf
    int pad;
};

// Every logit is read exactly once: keep the stream out of the caches.
typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_once(const float4 *p) {
    const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float load_once(const float *p) {
    return __builtin_nontemporal_load(p);
}

// (v, i) beats (best, bi) if larger, or equal with a lower index.
__device__ __forceinline__ void take_better(float &best, int &bi, float v, int i) {
    if (v > best || (v == best && i < bi)) {
        best = v;
        bi = i;
    }
}

__device__ __forceinline__ void wave_argmax(float &best, int &bi) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(best, off);
        const int oi = __shfl_xor(bi, off);
        take_better(best, bi, ov, oi);
    }
}

__device__ __forceinline__ int wave_any(int v) {
    return __ballot(v != 0) != 0ull;
}

__global__ __launch_bounds__(kThreads) void greedy_rows_kernel(
    const float *__restrict__ logits, int V, int chunk_len,
    GreedyChunk *__restrict__ out) {
    __shared__ float s_v[kWaves];
    __shared__ int s_i[kWaves], s_bad[kWaves];
    const int r = blockIdx.x;
    const int c = blockIdx.y;
    const float *z = logits + (size_t)r * V;
    const int lo = c * chunk_len;
    const int hi = min(V, lo + chunk_len);
    float best = -INFINITY;
    int bi = INT_MAX;
    int bad = 0;
    if ((V & 3) == 0) {
        const float4 *z4 = reinterpret_cast<const float4 *>(z);
        for (int base = lo + threadIdx.x * 4; base < hi; base += kThreads * 16) {
            // Branch-free: clamp each load into the chunk (hi is a multiple
            // of 4) and mask the lanes past its end to -inf, which never
            // wins.  A clamped load re-reads real logits of the chunk, so
            // its NaN / +inf check is harmless.
            float4 t[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                t[u] = load_once(&z4[min(base + u * kThreads * 4, hi - 4) >> 2]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = base + u * kThreads * 4;
                const bool in = e < hi;
                const float v[4] = {t[u].x, t[u].y, t[u].z, t[u].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    bad |= !(v[q] < INFINITY);       // NaN or +inf
                    const float x = in ? v[q] : -INFINITY;
                    if (x > best) {
                        best = x;
                        bi = e + q;
                    }
                }
            }
        }
    } else {
        for (int e = lo + threadIdx.x; e < hi; e += kThreads) {
            const float v = load_once(&z[e]);
            bad |= !(v < INFINITY);
            if (v > best) {
                best = v;
                bi = e;
            }
        }
    }
    wave_argmax(best, bi);
    bad = wave_any(bad);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        s_v[wave] = best;
        s_i[wave] = bi;
        s_bad[wave] = bad;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float bv = s_v[0];
        int bx = s_i[0], bb = s_bad[0];
        for (int w = 1; w < kWaves; ++w) {
            take_better(bv, bx, s_v[w], s_i[w]);
            bb |= s_bad[w];
        }
        out[(size_t)r * gridDim.y + c] = GreedyChunk{bv, bx, bb, 0};
    }
}

__global__ __launch_bounds__(kThreads) void greedy_decide_kernel(
    const GreedyChunk *__restrict__ chunk_res, int chunks,
    const int32_t *__restrict__ draft_tokens, int D, int V,
    int32_t *__restrict__ accepted_len, int32_t *__restrict__ next_token) {
    __shared__ int s_idx[16], s_bad[16];
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i = wave; i <= D; i += kWaves) {
        const GreedyChunk *row = chunk_res + ((size_t)b * (D + 1) + i) * chunks;
        float best = -INFINITY;
        int bi = INT_MAX, bad = 0;
        for (int c = lane; c < chunks; c += 64) {
            const GreedyChunk g = row[c];
            bad |= g.bad;
            take_better(best, bi, g.v, g.idx);
        }
        wave_argmax(best, bi);
        bad = wave_any(bad);
        if (lane == 0) {
            s_idx[i] = bi;
            s_bad[i] = bad || !(best > -INFINITY);   // no finite logit
        }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        const int i = threadIdx.x;
        bool invalid = false, miss = false;
        if (i <= D)
            invalid = s_bad[i] != 0;
        if (i < D) {
            const int d = draft_tokens[(size_t)b * D + i];
            invalid = invalid || d < 0 || d >= V;
            miss = d != s_idx[i];
        }
        const unsigned long long any_invalid = __ballot(invalid);
        const unsigned long long misses = __ballot(miss);
        if (i == 0) {
            const int L = any_invalid ? -1 : (misses ? __ffsll((long long)misses) - 1 : D);
            accepted_len[b] = L;
            next_token[b] = (L < 0) ? -1 : s_idx[L];
        }
    }
}

} // namespace

GreedyPlan greedy_plan(int B, int D, int V) {
    GreedyPlan p{};
    p.B = B;
    p.D = D;
    p.V = V;
    p.rows = B * (D + 1);
    int C = (kTargetBlocks + std::max(p.rows, 1) - 1) / std::max(p.rows, 1);
    C = std::max(1, std::min(C, (V + 2047) / 2048));
    const int len = (V + C - 1) / C;
    p.chunk_len = ((len + 1023) / 1024) * 1024;
    p.chunks = std::max(1, (V + p.chunk_len - 1) / p.chunk_len);
    p.ws_bytes = (size_t)p.rows * p.chunks * sizeof(GreedyChunk);
    return p;
}

hipError_t launch_greedy(const float *target, const int32_t *draft_tokens,
                         const GreedyPlan &plan, int32_t *accepted_len,
                         int32_t *next_token, void *ws, hipStream_t stream) {
    if (plan.B == 0)
        return hipSuccess;
    GreedyChunk *chunk_res = static_cast<GreedyChunk *>(ws);
    greedy_rows_kernel<<<dim3(plan.rows, plan.chunks), kThreads, 0, stream>>>(
        target, plan.V, plan.chunk_len, chunk_res);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    greedy_decide_kernel<<<plan.B, kThreads, 0, stream>>>(
        chunk_res, plan.chunks, draft_tokens, plan.D, plan.V, accepted_len, next_token);
    return hipGetLastError();
}

} // namespace spec
