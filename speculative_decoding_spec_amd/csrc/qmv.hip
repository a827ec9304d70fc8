// Small-M affine group-quantized matrix-vector product for gfx950.
//
// y[m][n] = sum_k x[m][k] * (s[n][g] * q[n][k] + b[n][g]),  g = k / 64,
// for the M = D + 1 rows of a verify block (MTPLX announcement, "Layer 0:
// MLX Runtime": the stock quantized matrix-vector kernel stalls at the
// verify shapes M = 3..6; the savepearlharbor.com llama.cpp MTP article,
// section on the theoretical maximum of token generation: decoding is bound
// by streaming every weight once, and extra rows ride on the same fetch).
//
// Design (one pass over the weights, every fetched weight feeds all M rows):
//  * A workgroup of 4 waves owns 64 weight rows (16 per wave) and one K
//    split.  It stages its slice of x in LDS once, already permuted into the
//    per-lane MFMA operand order, together with per-group sums of x.
//  * Each lane streams 16 bytes of packed codes per 128-wide K step ("pair"
//    of two 64-groups): W4 = 32 nibbles, W8 = 2 x 16 bytes.  Four lanes
//    cover 64 (W4) or 128 (W8) contiguous bytes of one row.
//  * Codes become bf16 in registers with no conversion instruction for W4:
//    OR-ing a nibble q into the mantissa of 128.0 (0x4300) gives 128 + q
//    exactly; the 128 offset is removed with the group sum of x.  W8 codes
//    convert with the byte-to-float instructions (exact below 256).
//  * v_mfma_f32_16x16x32_bf16 does the multiply-accumulate: B = 16 weight
//    rows x 32 k, A = the x rows.  The two groups of a pair are kept apart
//    by feeding group 0 through A rows 0..7 and group 1 through A rows
//    8..15 (each zero on the other group's k slots), so M <= 8 rows use the
//    whole 16-row tile and every output of the MFMA belongs to exactly one
//    group.  The per-group affine terms are then applied in fp32:
//        acc += s * C + (b - 128 s) * sum_x            (W4)
//        acc += s * C + b * sum_x                      (W8)
//  * The two group halves meet with one cross-lane add; K splits (when N is
//    too small to fill the GPU) meet in a fixed order in the workgroup that
//    arrives last, so the result is deterministic and independent of M.
#include "spec_internal.h"

namespace spec {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;          // 4 waves of 64
constexpr int kRowsPerBlock = 64;      // 16 rows per wave
constexpr int kMaxPairsPerSplit = 20;  // LDS budget: 20 x 2112 B = 42 KB
constexpr int kFragBytesPerPair = 4 * 32 * 16;  // 4 MFMA steps x 32 lane slots x 16 B
constexpr int kSumBytesPerPair = 2 * 8 * 4;     // 2 groups x 8 rows x fp32
constexpr int kMinPairsPerSplit = 2;
constexpr int kTargetBlocks = 512;
// The workspace starts with a fixed counter area, one counter per 64-row
// block, that no plan ever uses for anything else: calls of any shape can
// then share one workspace, because every call leaves its counters at zero.
constexpr size_t kCounterBytes = 256 * 1024;   // 65536 blocks: N <= 4194304

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float bf16_lo(unsigned v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(unsigned v) { return __uint_as_float(v & 0xFFFF0000u); }

// 8 bf16 of x in k order (x0|x1, x2|x3, x4|x5, x6|x7) -> the order the W4
// unpack produces on the B side: (x0|x4, x1|x5, x2|x6, x3|x7).
__device__ __forceinline__ u32x4 permute_for_w4(u32x4 v) {
    u32x4 o;
    o.x = (v.x & 0xFFFFu) | (v.z << 16);
    o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    o.z = (v.y & 0xFFFFu) | (v.w << 16);
    o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    return o;
}

// One 32-bit word of 8 nibbles -> 8 bf16 values 128 + q, in the order
// (q0, q4, q1, q5, q2, q6, q3, q7).
__device__ __forceinline__ bf16x8 unpack_w4(unsigned d) {
    const unsigned mask = 0x000F000Fu, magic = 0x43004300u;
    u32x4 o;
    o.x = (d & mask) | magic;
    o.y = ((d >> 4) & mask) | magic;
    o.z = ((d >> 8) & mask) | magic;
    o.w = ((d >> 12) & mask) | magic;
    return __builtin_bit_cast(bf16x8, o);
}

// Two words of 4 bytes each -> 8 bf16 values q (exact: q < 256 needs 8
// significant bits, the upper half of the fp32 holds them all).
__device__ __forceinline__ bf16x8 unpack_w8(unsigned d0, unsigned d1) {
    u32x4 o;
    o.x = (__float_as_uint((float)(d0 & 0xFFu)) >> 16) |
          (__float_as_uint((float)((d0 >> 8) & 0xFFu)) & 0xFFFF0000u);
    o.y = (__float_as_uint((float)((d0 >> 16) & 0xFFu)) >> 16) |
          (__float_as_uint((float)(d0 >> 24)) & 0xFFFF0000u);
    o.z = (__float_as_uint((float)(d1 & 0xFFu)) >> 16) |
          (__float_as_uint((float)((d1 >> 8) & 0xFFu)) & 0xFFFF0000u);
    o.w = (__float_as_uint((float)((d1 >> 16) & 0xFFu)) >> 16) |
          (__float_as_uint((float)(d1 >> 24)) & 0xFFFF0000u);
    return __builtin_bit_cast(bf16x8, o);
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void qmv_kernel(
    const void *__restrict__ w, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ x,
    float *__restrict__ y, int M, int N, int K, int pairs_per_split,
    int splits, float *__restrict__ partial, unsigned *__restrict__ counters) {
    extern __shared__ __align__(16) unsigned char lds[];
    u32x4 *xf = reinterpret_cast<u32x4 *>(lds);
    float *xs = reinterpret_cast<float *>(lds + (size_t)pairs_per_split * kFragBytesPerPair);
    __shared__ int s_last;

    const int blk = blockIdx.x;
    const int split = blockIdx.y;
    const int ng = K >> 6;
    const int n_pairs = (ng + 1) >> 1;
    const int p_begin = split * pairs_per_split;
    const int P = min(pairs_per_split, n_pairs - p_begin);

    // ---- stage x: one item = (pair p, half h, row m), 64 values of x ----
    for (int item = threadIdx.x; item < P * 16; item += kThreads) {
        const int p = item >> 4, h = (item >> 3) & 1, m = item & 7;
        if (m >= M)
            continue;
        const int g = 2 * (p_begin + p) + h;
        u32x4 frag[8];
        float sum = 0.0f;
        if (g < ng) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (size_t)m * K + (size_t)g * 64);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const u32x4 v = src[q];
                sum += bf16_lo(v.x); sum += bf16_hi(v.x);
                sum += bf16_lo(v.y); sum += bf16_hi(v.y);
                sum += bf16_lo(v.z); sum += bf16_hi(v.z);
                sum += bf16_lo(v.w); sum += bf16_hi(v.w);
                frag[q] = (BITS == 4) ? permute_for_w4(v) : v;
            }
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q)
                frag[q] = u32x4{0u, 0u, 0u, 0u};
        }
        // 8-value block q = 4 * sub + t feeds MFMA step t of lane slot
        // (half h, sub, row m).
#pragma unroll
        for (int q = 0; q < 8; ++q)
            xf[(p * 4 + (q & 3)) * 32 + 16 * h + 8 * (q >> 2) + m] = frag[q];
        xs[(p * 2 + h) * 8 + m] = sum;
    }
    __syncthreads();

    // ---- lane roles ----
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane >> 4;   // k-slot group of the A/B operands, row group of C
    const int r = lane & 15;   // A row / B and C column
    const int h = j >> 1;      // which group of the pair this lane's k slots hold
    const int sub = j & 1;     // which 32-k half of that group
    const int n = blk * kRowsPerBlock + wave * 16 + r;
    const bool n_ok = n < N;
    // A row r carries x row (r & 7) for half (r >> 3); it is non-zero only on
    // the k slots of that half.
    const bool a_act = (h == (r >> 3)) && ((r & 7) < M);
    const int a_slot = 16 * h + 8 * sub + (r & 7);

    const uint16_t *srow = scales + (size_t)(n_ok ? n : 0) * ng;
    const uint16_t *brow = biases + (size_t)(n_ok ? n : 0) * ng;
    const u32x4 *wrow;
    if (BITS == 4)
        wrow = reinterpret_cast<const u32x4 *>(w) + (size_t)(n_ok ? n : 0) * (K >> 5) + 2 * h + sub;
    else
        wrow = reinterpret_cast<const u32x4 *>(w) + (size_t)(n_ok ? n : 0) * (K >> 4) + 4 * h + 2 * sub;

    const f32x4 *xs4 = reinterpret_cast<const f32x4 *>(xs);
    const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};

    constexpr int U = (BITS == 4) ? 8 : 4;   // pairs in flight per lane
    constexpr int W = BITS / 4;              // 16-byte loads per pair per lane
    for (int p0 = 0; p0 < P; p0 += U) {
        u32x4 raw[U][W];
        uint16_t s16[U], b16[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u;
            const int g = 2 * (p_begin + p) + h;
            if (n_ok && p < P && g < ng) {
#pragma unroll
                for (int v = 0; v < W; ++v)
                    raw[u][v] = wrow[(size_t)(p_begin + p) * (4 * W) + v];
                s16[u] = srow[g];
                b16[u] = brow[g];
            } else {
#pragma unroll
                for (int v = 0; v < W; ++v)
                    raw[u][v] = u32x4{0u, 0u, 0u, 0u};
                s16[u] = 0;
                b16[u] = 0;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u;
            if (p >= P)
                break;
            f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bf16x8 a = a_act ? __builtin_bit_cast(bf16x8, xf[(p * 4 + t) * 32 + a_slot]) : zero8;
                bf16x8 b;
                if (BITS == 4) {
                    b = unpack_w4(raw[u][0][t]);
                } else {
                    const u32x4 &lo = raw[u][(t * 2) >> 2];
                    b = unpack_w8(lo[(t * 2) & 3], lo[(t * 2 + 1) & 3]);
                }
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
            }
            // C row 4*j + i is x row m = 4*sub + i of half h.
            const f32x4 xsum = xs4[(p * 2 + h) * 2 + sub];
            const float s = half_bits_to_float(s16[u]);
            const float b = half_bits_to_float(b16[u]);
            const float bb = (BITS == 4) ? fmaf(-128.0f, s, b) : b;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[i] = fmaf(s, c[i], acc[i]);
                acc[i] = fmaf(bb, xsum[i], acc[i]);
            }
        }
    }

    // Lanes l and l ^ 32 hold the same (m, n) for the two groups of each pair.
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc[i] += __shfl_xor(acc[i], 32);

    if (lane < 32 && n_ok) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * sub + i;
            if (m < M) {
                if (splits == 1)
                    y[(size_t)m * N + n] = acc[i];
                else
                    partial[((size_t)split * M + m) * N + n] = acc[i];
            }
        }
    }
    if (splits == 1)
        return;

    // ---- K splits: the last workgroup of this row block sums them in order ----
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = atomicAdd(&counters[blk], 1u);
        s_last = (prev == (unsigned)(splits - 1));
    }
    __syncthreads();
    if (!s_last)
        return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    for (int e = threadIdx.x; e < M * kRowsPerBlock; e += kThreads) {
        const int m = e / kRowsPerBlock;
        const int nn = blk * kRowsPerBlock + e % kRowsPerBlock;
        if (nn >= N)
            continue;
        float v = __builtin_nontemporal_load(&partial[(size_t)m * N + nn]);
        for (int sp = 1; sp < splits; ++sp)
            v += __builtin_nontemporal_load(&partial[((size_t)sp * M + m) * N + nn]);
        y[(size_t)m * N + nn] = v;
    }
    if (threadIdx.x == 0)
        atomicExch(&counters[blk], 0u);
}

__global__ void fill_zero_kernel(float *__restrict__ y, size_t count) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (size_t)gridDim.x * blockDim.x)
        y[i] = 0.0f;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

} // namespace

QmvPlan qmv_plan(int N, int K) {
    QmvPlan p{};
    p.n_blocks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
    const int ng = K / 64;
    p.n_pairs = (ng + 1) / 2;
    int S = 1;
    if (p.n_pairs > 0 && p.n_blocks > 0) {
        while (p.n_blocks * S < kTargetBlocks &&
               (p.n_pairs + 2 * S - 1) / (2 * S) >= kMinPairsPerSplit)
            S *= 2;
        S = std::max(S, (p.n_pairs + kMaxPairsPerSplit - 1) / kMaxPairsPerSplit);
        p.pairs_per_split = (p.n_pairs + S - 1) / S;
        S = (p.n_pairs + p.pairs_per_split - 1) / p.pairs_per_split;
    } else {
        p.pairs_per_split = 0;
    }
    p.splits = S;
    p.lds_bytes = (size_t)p.pairs_per_split * (kFragBytesPerPair + kSumBytesPerPair);
    return p;
}

size_t qmv_workspace_bytes(const QmvPlan &p, int M, int N) {
    if (p.splits <= 1 || M <= 0 || N <= 0)
        return 0;
    return kCounterBytes + align256((size_t)p.splits * M * N * sizeof(float));
}

int qmv_max_rows() { return (int)(kCounterBytes / sizeof(unsigned)) * kRowsPerBlock; }

hipError_t launch_qmv(int bits, const void *w, const uint16_t *scales,
                      const uint16_t *biases, const uint16_t *x, float *y,
                      int M, int N, int K, const QmvPlan &plan, void *ws,
                      hipStream_t stream) {
    if (M == 0 || N == 0)
        return hipSuccess;
    if (K == 0) {
        const size_t count = (size_t)M * N;
        const int blocks = (int)std::min<size_t>((count + 255) / 256, 4096);
        fill_zero_kernel<<<blocks, 256, 0, stream>>>(y, count);
        return hipGetLastError();
    }
    unsigned *counters = nullptr;
    float *partial = nullptr;
    if (plan.splits > 1) {
        counters = reinterpret_cast<unsigned *>(ws);
        partial = reinterpret_cast<float *>(reinterpret_cast<unsigned char *>(ws) + kCounterBytes);
    }
    dim3 grid(plan.n_blocks, plan.splits);
    if (bits == 4)
        qmv_kernel<4><<<grid, kThreads, plan.lds_bytes, stream>>>(
            w, scales, biases, x, y, M, N, K, plan.pairs_per_split, plan.splits,
            partial, counters);
    else
        qmv_kernel<8><<<grid, kThreads, plan.lds_bytes, stream>>>(
            w, scales, biases, x, y, M, N, K, plan.pairs_per_split, plan.splits,
            partial, counters);
    return hipGetLastError();
}

} // namespace spec
