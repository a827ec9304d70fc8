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
//  * A workgroup owns one 16-row tile of W (the MFMA's 16 columns) and its
//    4 or 8 waves split K, wave w taking every 4th/8th 128-wide step ("pair"
//    of two 64-groups).  Nothing crosses workgroups: no fences, no
//    workspace, and even N = 5120 launches 320 workgroups of 8 waves.
//  * Each lane streams 16 bytes of packed codes per pair (W4: 32 nibbles;
//    W8: two 16-byte loads); four lanes cover 64 (W4) or 128 (W8) contiguous
//    bytes of one row.  Loads are branch-free (indices clamp into range) and
//    double buffered in batches, so a whole batch stays in flight.
//  * Codes become bf16 in registers with no conversion instruction for W4:
//    OR-ing a nibble q into the mantissa of 128.0 (0x4300) gives 128 + q
//    exactly; the 128 offset is removed with the group sum of x.  W8 codes
//    convert with the byte-to-float instructions (exact below 256).
//  * v_mfma_f32_16x16x32_bf16 does the multiply-accumulate: B = 16 weight
//    rows x 32 k, A = the x rows, read straight from global memory (x is a
//    few hundred KB at most and stays in L2).  The two groups of a pair are
//    kept apart by feeding group 0 through A rows 0..7 and group 1 through
//    A rows 8..15 (each zero on the other group's k slots), so M <= 8 rows
//    use the whole 16-row tile and every MFMA output belongs to one group.
//    A second MFMA against a ones operand yields the group sums of x in the
//    same lane layout.  The per-group affine terms are applied in fp32:
//        acc += s * C + (b - 128 s) * sum_x            (W4)
//        acc += s * C + b * sum_x                      (W8)
//  * The two group halves and the waves meet in LDS in a fixed order, so
//    results are deterministic and row m never depends on M.
#include "spec_internal.h"

namespace spec {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Raw (unformatted, stride 0) buffer resource flags for gfx9-family parts,
// and a byte offset beyond any x buffer: loads there return zeros.
constexpr int kBufferFlags = 0x00020000;
constexpr unsigned kOutOfRange = 0x40000000u;

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// One 32-bit word of 8 nibbles q0..q7 (q_i at bits 4i) -> 8 bf16 values
// 128 + q_i in k order.  The even and odd nibbles are first separated into
// bytes (lo = q0 q2 q4 q6, hi = q1 q3 q5 q7), interleaved into k order
// (q0 q1 q2 q3 / q4 q5 q6 q7), and each byte is then paired with the byte
// 0x43: bf16 0x43qq = 128 + q exactly (128 has 7 mantissa bits of ulp 1).
__device__ __forceinline__ bf16x8 unpack_w4(unsigned d) {
    const unsigned lo = d & 0x0F0F0F0Fu;
    const unsigned hi = (d >> 4) & 0x0F0F0F0Fu;
    const unsigned q03 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // q0 q1 q2 q3
    const unsigned q47 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // q4 q5 q6 q7
    const unsigned c43 = 0x43434343u;
    u32x4 o;
    o.x = __builtin_amdgcn_perm(c43, q03, 0x04010400u);   // 0x43 q1 0x43 q0
    o.y = __builtin_amdgcn_perm(c43, q03, 0x04030402u);
    o.z = __builtin_amdgcn_perm(c43, q47, 0x04010400u);
    o.w = __builtin_amdgcn_perm(c43, q47, 0x04030402u);
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

// ---------------------------------------------------------------------------
// Packed layout (written once by pack_kernel, read by qmv_kernel).
//
// W is cut into tiles of 16 rows x 128 k (one "pair" of 64-groups).  Tile
// (t, p) -- rows 16t..16t+15, k = 128p..128p+127 -- is stored contiguously at
// tile index t * n_pairs + p, as 64 lane slots of 16 bytes (W4) or two
// 1 KB halves of 64 x 16 bytes (W8).  Lane slot l = 16 j + r holds row
// 16t + r, k = 128p + 64 (j >> 1) + 32 (j & 1) + [0, 32): exactly the bytes
// the MFMA B operand of lane l needs, in the original code order.  A wave
// therefore reads 1 KB per load instruction and streams a contiguous region.
// Scales and biases become one 32-bit word per (row, group): fp16 scale in
// the low half, fp16 bias in the high half, stored as [t][g][r] with the group
// count padded to 2 * n_pairs.  Rows past N and groups past K/64 are zero, so
// they contribute exactly nothing.
// ---------------------------------------------------------------------------

template <int BITS>
__global__ __launch_bounds__(256) void pack_kernel(
    const void *__restrict__ w, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, u32x4 *__restrict__ wp,
    uint32_t *__restrict__ sbp, int N, int K) {
    const int ng = K >> 6;
    const int n_pairs = (ng + 1) >> 1;
    const int ngp = 2 * n_pairs;
    const int n_tiles = (N + 15) >> 4;
    constexpr int L = BITS / 4;   // 16-byte slots per lane and tile
    const size_t slots = (size_t)n_tiles * n_pairs * 64 * L;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < slots;
         i += (size_t)gridDim.x * blockDim.x) {
        const int lane = (int)(i & 63);
        const size_t rest = i >> 6;
        const int v = (int)(rest % L);            // which 1 KB half (W8)
        const size_t tp = rest / L;               // t * n_pairs + p
        const int p = (int)(tp % n_pairs);
        const int t = (int)(tp / n_pairs);
        const int r = lane & 15, j = lane >> 4;
        const int n = 16 * t + r;
        const int k = 128 * p + 64 * (j >> 1) + 32 * (j & 1) + 16 * v;  // first k of the 16 bytes
        u32x4 val = {0u, 0u, 0u, 0u};
        if (n < N && k < K) {
            if (BITS == 4)
                val = reinterpret_cast<const u32x4 *>(w)[((size_t)n * K + k) >> 5];
            else
                val = reinterpret_cast<const u32x4 *>(w)[((size_t)n * K + k) >> 4];
        }
        wp[i] = val;
    }
    const size_t sb_count = (size_t)n_tiles * ngp * 16;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < sb_count;
         i += (size_t)gridDim.x * blockDim.x) {
        const int r = (int)(i & 15);
        const size_t tg = i >> 4;
        const int g = (int)(tg % ngp);
        const int t = (int)(tg / ngp);
        const int n = 16 * t + r;
        uint32_t val = 0;
        if (n < N && g < ng)
            val = (uint32_t)scales[(size_t)n * ng + g] | ((uint32_t)biases[(size_t)n * ng + g] << 16);
        sbp[i] = val;
    }
}

template <int BITS, int WAVES, int T>
__global__ __launch_bounds__(WAVES * 64) void qmv_kernel(
    const u32x4 *__restrict__ wp, const uint32_t *__restrict__ sbp,
    const uint16_t *__restrict__ x, float *__restrict__ y, int M, int N, int K) {
    __shared__ f32x4 red[WAVES][T][64];

    constexpr int L = BITS / 4;              // 1 KB loads per pair, tile and wave
    const int ng = K >> 6;                   // groups per row
    const int n_pairs = (ng + 1) >> 1;       // 128-wide K steps
    const int ngp = 2 * n_pairs;
    const int n_tiles = (N + 15) >> 4;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane >> 4;   // k-slot group of the A/B operands, row group of C
    const int r = lane & 15;   // A row / B and C column
    const int h = j >> 1;      // which group of the pair this lane's k slots hold
    const int sub = j & 1;     // which 32-k half of that group

    // This wave's contiguous share of the pairs, for each of the T tiles.
    const int ppw = (n_pairs + WAVES - 1) / WAVES;
    const int p_lo = min(n_pairs, wave * ppw);
    const int p_hi = min(n_pairs, p_lo + ppw);

    // Buffer resources: lane-dependent offsets are fixed, per-pair offsets
    // are wave-uniform (scalar registers).  A tile past the last one gets an
    // empty resource, so its loads return zeros.
    __amdgpu_buffer_rsrc_t wres[T], sbres[T];
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
        const int t = blockIdx.x * T + tt;
        const bool there = t < n_tiles;
        wres[tt] = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(wp + (size_t)min(t, n_tiles - 1) * n_pairs * 64 * L), (short)0,
            there ? n_pairs * 1024 * L : 0, kBufferFlags);
        sbres[tt] = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(sbp + (size_t)min(t, n_tiles - 1) * ngp * 16), (short)0,
            there ? ngp * 64 : 0, kBufferFlags);
    }
    // A row r carries x row (r & 7) for half (r >> 3) and is non-zero only on
    // that half's k slots.  Lanes outside that pattern, or with a row >= M,
    // start past the end of x, where buffer loads return zeros.
    const bool a_act = (h == (r >> 3)) && ((r & 7) < M);
    const __amdgpu_buffer_rsrc_t xres =
        __builtin_amdgcn_make_buffer_rsrc((void *)x, (short)0, M * K * 2, kBufferFlags);
    const unsigned xoff = a_act ? (unsigned)(((r & 7) * K + 64 * h + 32 * sub) * 2) : kOutOfRange;
    const unsigned woff = (unsigned)lane * 16u;
    const unsigned sboff = (unsigned)(h * 16 + r) * 4u;

    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    f32x4 acc[T];
#pragma unroll
    for (int tt = 0; tt < T; ++tt)
        acc[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    constexpr int U = (T == 1) ? 4 : (T == 2 ? 2 : 1);   // pairs per batch
    struct Batch {
        u32x4 raw[U][T][L];
        uint32_t sb[U][T];
    };
    auto load_w = [&](Batch &bt, int p0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = min(p0 + u, n_pairs - 1);
#pragma unroll
            for (int tt = 0; tt < T; ++tt) {
#pragma unroll
                for (int v = 0; v < L; ++v)
                    bt.raw[u][tt][v] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres[tt], woff, (p * L + v) * 1024, 0));
                bt.sb[u][tt] = __builtin_amdgcn_raw_buffer_load_b32(sbres[tt], sboff, p * 128, 0);
            }
        }
    };
    auto load_x = [&](u32x4 (&a)[U][4], int p0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = min(p0 + u, n_pairs - 1);
            // the odd last group of a row has no partner: its half reads zeros
            const unsigned off = (2 * p + h < ng) ? xoff : kOutOfRange;
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
                a[u][s4] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, off + s4 * 16u, p * 256, 0));
        }
    };
    auto compute = [&](const Batch &bt, const u32x4 (&a)[U][4], int p0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (p0 + u >= p_hi)
                break;
            f32x4 c[T];
            f32x4 cx = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int tt = 0; tt < T; ++tt)
                c[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const bf16x8 av = __builtin_bit_cast(bf16x8, a[u][s4]);
                cx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, ones, cx, 0, 0, 0);
#pragma unroll
                for (int tt = 0; tt < T; ++tt) {
                    bf16x8 bv;
                    if (BITS == 4) {
                        bv = unpack_w4(bt.raw[u][tt][0][s4]);
                    } else {
                        const u32x4 &lo = bt.raw[u][tt][s4 >> 1];
                        bv = unpack_w8(lo[(s4 * 2) & 3], lo[(s4 * 2 + 1) & 3]);
                    }
                    c[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c[tt], 0, 0, 0);
                }
            }
            // C row 4*j + i is x row m = 4*sub + i of half h; cx holds the
            // same rows' sums of x over the group.
#pragma unroll
            for (int tt = 0; tt < T; ++tt) {
                const float s = half_bits_to_float((uint16_t)(bt.sb[u][tt] & 0xFFFFu));
                const float bias = half_bits_to_float((uint16_t)(bt.sb[u][tt] >> 16));
                const float bb = (BITS == 4) ? fmaf(-128.0f, s, bias) : bias;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[tt][i] = fmaf(s, c[tt][i], acc[tt][i]);
                    acc[tt][i] = fmaf(bb, cx[i], acc[tt][i]);
                }
            }
        }
    };

    // Vector-memory loads complete in issue order, so each batch's x
    // operands (L2 hits) are requested before the next batch of weights
    // (HBM): consuming them never waits for the weights still in flight.
    Batch cur, nxt;
    u32x4 a[U][4];
    if (p_lo < p_hi)
        load_w(cur, p_lo);
    for (int p0 = p_lo; p0 < p_hi; p0 += U) {
        load_x(a, p0);
        if (p0 + U < p_hi)
            load_w(nxt, p0 + U);
        compute(cur, a, p0);
        cur = nxt;
    }

    // Fixed-order reduction: the two groups of a pair (lanes l, l ^ 32), then
    // the waves in index order.  Neither depends on M.
#pragma unroll
    for (int tt = 0; tt < T; ++tt)
        red[wave][tt][lane] = acc[tt];
    __syncthreads();
    if (wave == 0 && lane < 32) {
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            const int n = (blockIdx.x * T + tt) * 16 + r;
            if (n >= N)
                continue;
            f32x4 tot = red[0][tt][lane] + red[0][tt][lane + 32];
            for (int ww = 1; ww < WAVES; ++ww)
                tot += red[ww][tt][lane] + red[ww][tt][lane + 32];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * sub + i;
                if (m < M)
                    y[(size_t)m * N + n] = tot[i];
            }
        }
    }
}

__global__ void fill_zero_kernel(float *__restrict__ y, size_t count) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (size_t)gridDim.x * blockDim.x)
        y[i] = 0.0f;
}

} // namespace

QmvPlan qmv_plan(int bits, int N, int K) {
    QmvPlan p{};
    p.n_tiles = (N + 15) / 16;
    p.n_pairs = (K / 64 + 1) / 2;
    // Enough tiles: each wave serves two (or, for very wide matrices, four)
    // tiles with one x operand, cutting the x traffic by that factor; 4 waves
    // split K.  (W8 streams twice the bytes per x fragment, so two suffice.)  Few tiles: one tile per workgroup and K
    // split over 4 or 8 waves, so even N = 5120 gives >= 2560 waves.  The
    // choice depends on (N, K) only, never on M.
    if (p.n_tiles >= 4096 && bits == 4) {
        p.tiles_per_wave = 4;
        p.waves = 4;
    } else if (p.n_tiles >= 1024) {
        p.tiles_per_wave = 2;
        p.waves = 4;
    } else {
        p.tiles_per_wave = 1;
        p.waves = K >= 8192 ? 8 : 4;
    }
    return p;
}

size_t qmv_packed_bytes(int bits, int N, int K) {
    const QmvPlan p = qmv_plan(bits, N, K);
    return (size_t)p.n_tiles * p.n_pairs * 64 * 16 * (bits / 4);
}

size_t qmv_packed_sb_bytes(int N, int K) {
    const QmvPlan p = qmv_plan(4, N, K);
    return (size_t)p.n_tiles * (2 * p.n_pairs) * 16 * 4;
}

hipError_t launch_pack(int bits, const void *w, const uint16_t *scales,
                       const uint16_t *biases, int N, int K, void *w_packed,
                       void *sb_packed, hipStream_t stream) {
    if (N == 0 || K == 0)
        return hipSuccess;
    const size_t slots = qmv_packed_bytes(bits, N, K) / 16;
    const int blocks = (int)std::min<size_t>((slots + 255) / 256, 65536);
    if (bits == 4)
        pack_kernel<4><<<blocks, 256, 0, stream>>>(w, scales, biases, (u32x4 *)w_packed,
                                                   (uint32_t *)sb_packed, N, K);
    else
        pack_kernel<8><<<blocks, 256, 0, stream>>>(w, scales, biases, (u32x4 *)w_packed,
                                                   (uint32_t *)sb_packed, N, K);
    return hipGetLastError();
}

hipError_t launch_qmv(int bits, const void *w_packed, const void *sb_packed,
                      const uint16_t *x, float *y, int M, int N, int K,
                      hipStream_t stream) {
    if (M == 0 || N == 0)
        return hipSuccess;
    if (K == 0) {
        const size_t count = (size_t)M * N;
        const int blocks = (int)std::min<size_t>((count + 255) / 256, 4096);
        fill_zero_kernel<<<blocks, 256, 0, stream>>>(y, count);
        return hipGetLastError();
    }
    const QmvPlan plan = qmv_plan(bits, N, K);
    const u32x4 *wp = (const u32x4 *)w_packed;
    const uint32_t *sbp = (const uint32_t *)sb_packed;
    const dim3 grid((plan.n_tiles + plan.tiles_per_wave - 1) / plan.tiles_per_wave);
#define SPEC_QMV_LAUNCH(B, W, TT) \
    qmv_kernel<B, W, TT><<<grid, (W) * 64, 0, stream>>>(wp, sbp, x, y, M, N, K)
    if (bits == 4) {
        if (plan.tiles_per_wave == 4)
            SPEC_QMV_LAUNCH(4, 4, 4);
        else if (plan.tiles_per_wave == 2)
            SPEC_QMV_LAUNCH(4, 4, 2);
        else if (plan.waves == 8)
            SPEC_QMV_LAUNCH(4, 8, 1);
        else
            SPEC_QMV_LAUNCH(4, 4, 1);
    } else {
        if (plan.tiles_per_wave == 4)
            SPEC_QMV_LAUNCH(8, 4, 4);
        else if (plan.tiles_per_wave == 2)
            SPEC_QMV_LAUNCH(8, 4, 2);
        else if (plan.waves == 8)
            SPEC_QMV_LAUNCH(8, 8, 1);
        else
            SPEC_QMV_LAUNCH(8, 4, 1);
    }
#undef SPEC_QMV_LAUNCH
    return hipGetLastError();
}

} // namespace spec
