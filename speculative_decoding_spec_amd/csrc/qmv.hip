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
//  * A workgroup owns 1, 2 or 4 16-row tiles of W (the MFMA's 16 columns)
//    and its 4 or 8 waves split K, each wave taking a contiguous run of
//    128-wide steps ("pairs" of two 64-groups) for all of the workgroup's
//    tiles.  Nothing crosses workgroups: no fences, no workspace.
//  * Two weight layouts are streamed by the same kernel:
//      - packed: tiles of 16 rows x 128 k stored as 1 KB (W4) runs in MFMA
//        operand order, so each load instruction of a wave reads 1 KB of
//        contiguous memory (written once by pack_kernel);
//      - interchange: the caller's row-major codes [N][K*bits/8] with fp16
//        scales and biases [N][K/64]; a load instruction then reads 64 bytes
//        (W4) or 128 bytes (W8) from each of 16 rows.
//    In both, lane 16j + r of a wave holds row r of the tile and the 32
//    consecutive k starting at 32j of the pair.
//  * A wave keeps S stages of loads in flight: the codes, scale/bias words
//    and x rows of one pair are issued together while earlier pairs are
//    computed.  Edges use out-of-range buffer offsets (zeros, no memory
//    traffic) instead of branches.
//  * x is read compactly (the M rows of the pair, 16 bytes per lane) and
//    staged through a per-wave 16 x 128 bf16 matrix in LDS in exactly the
//    shape of the MFMA A operand (zero where a row carries no x), from which
//    each lane reads its operand with one 16-byte read per 32-k step.  The
//    16-byte chunks of row r are XOR-swizzled by swz(r), so that neither the
//    writes (one x row, 16 chunks) nor the reads (16 rows, one chunk) meet
//    bank conflicts.
//  * Codes become bf16 in registers with no conversion instruction for W4:
//    a nibble q placed in the top four mantissa bits of bf16 16.0 gives
//    16 + q exactly; the offset is removed per group with the group sum of
//    x.  (It is 16 code steps, so the fold loses little to cancellation; a
//    nibble in the low mantissa bits of 128.0 would put 128 there.)  W8
//    codes convert with the byte-to-float instructions (exact below 256).
//  * v_mfma_f32_16x16x32_bf16 does the multiply-accumulate: B = 16 weight
//    rows x 32 k, A = the x rows.  The two groups of a pair are kept apart by
//    feeding group 0 through A rows 0..7 and group 1 through A rows 8..15
//    (each zero on the other group's k slots), so M <= 8 rows use the whole
//    16-row tile and every MFMA output belongs to one group.  A second MFMA
//    against a ones operand yields the group sums of x in the same lane
//    layout.  Blocks of 9..16 rows (the 16-wide drafter blocks of the mlxcel
//    manual's DFlash section) fill all 16 A rows and run one MFMA per group
//    instead (the wide form, below).  The per-group affine terms are applied in fp32:
//        acc += s * C + (b - 16 s) * sum_x             (W4, C over 16 + q)
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
// and a byte offset beyond any buffer: loads there return zeros.
constexpr int kBufferFlags = 0x00020000;
// Cache policy of the weight loads: non-temporal (each code is read once
// per launch, so it need not displace x and the scale/bias words in L2);
// measured 3-8% faster than the default policy on the verify shapes.
constexpr int kStreamOnce = 2;
// Interchange weights: a load reads 64 bytes (W4) of each of 16 rows, half a
// 128-byte cache line; the next pair's load reads the other half, so these
// loads keep the default policy and the line stays in L2 between the two.
constexpr int kRowHalfLine = 0;
constexpr unsigned kOutOfRange = 0x40000000u;

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// Codes to bf16 for W4.  A code q placed in bits 3..6 (the top four of the
// seven mantissa bits) of bf16 16.0 gives 16 + q exactly, so each output
// register is ((word >> s) & 0x00780078) | 0x41804180: k-slot i of a 32-bit
// word (bits 4i..4i+3) in its low half and k-slot i + 4 in its high half, in
// the k order (k0, k4, k1, k5, k2, k6, k3, k7); the x operand is staged in
// the same order (stage_w4_order).  The shifts are 64-bit, each serving two
// words at once: the bits a 64-bit shift carries across the word boundary
// land outside the mask.  Six VALU operations per 8 codes.  The shift counts
// arrive in scalar registers the compiler cannot see through (opaque_sgpr):
// with constant counts it would prove the carried bits unused and split each
// 64-bit shift back into two 32-bit ones.
struct W4Shifts {
    unsigned l3, r1, r5, r9;
};

// The two 32-bit words 2 half and 2 half + 1 of the 16 bytes of codes a lane
// holds per tile and pair -> the MFMA B operands of 32-k steps 2 half and
// 2 half + 1.
__device__ __forceinline__ void unpack_w4(u32x4 raw, int half, unsigned base, W4Shifts sh,
                                          bf16x8 b[2]) {
    constexpr unsigned kMask = 0x00780078u;
    typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
    const uint64_t w = __builtin_bit_cast(u64x2, raw)[half];
    const uint64_t l3 = w << sh.l3, r1 = w >> sh.r1, r5 = w >> sh.r5, r9 = w >> sh.r9;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int hi = 32 * e;
        u32x4 o;
        o.x = ((unsigned)(l3 >> hi) & kMask) | base;
        o.y = ((unsigned)(r1 >> hi) & kMask) | base;
        o.z = ((unsigned)(r5 >> hi) & kMask) | base;
        o.w = ((unsigned)(r9 >> hi) & kMask) | base;
        b[e] = __builtin_bit_cast(bf16x8, o);
    }
}

// A wave-uniform constant in a scalar register, opaque to the optimizer
// (set once, before the main loop; a scalar move, no vector-register write).
__device__ __forceinline__ unsigned opaque_sgpr(unsigned c) {
    unsigned v;
    asm volatile("s_mov_b32 %0, %1" : "=s"(v) : "i"(c));
    return v;
}

// A value in a vector register the compiler cannot rematerialize: constants
// the loop reads every iteration stay put instead of being rebuilt there
// (with the mask as the one scalar operand, each (v & mask) | base above is
// a single v_and_or_b32).
__device__ __forceinline__ unsigned vgpr_const(unsigned c) {
    unsigned v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "i"(c));
    return v;
}

// Eight consecutive bf16 x values (k0..k7, two per 32-bit word) reordered
// to (k0, k4, k1, k5, k2, k6, k3, k7), the k order of unpack_w4.
__device__ __forceinline__ u32x4 stage_w4_order(u32x4 v) {
    u32x4 o;
    o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
    o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
    o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
    o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
    return o;
}

// Two words of 4 bytes each -> 8 bf16 values q in k order (exact: q < 256
// needs 8 significant bits, the upper half of the fp32 holds them all).
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

// Swizzle of the staged A matrix: 16-byte chunk c of row r is stored at
// chunk c ^ swz(r), swz(r) = 2 (r mod 8) + r / 8, a permutation of 0..15.
// The operand read of one 32-k step (row r = lane mod 16, chunk 4 (lane / 16)
// + s) and the staging write of one x row (chunks 0..7 into row m, 8..15
// into row m + 8) both measure zero bank-conflict cycles with it on gfx950
// (SQ_LDS_BANK_CONFLICT over every lane pattern of the kernel, in a probe);
// unswizzled rows, a 272-byte row pitch and an XOR with r itself each cost
// four conflict cycles per 16-byte read there.
__device__ __forceinline__ int swz(int r) {
    return 2 * (r & 7) + (r >> 3);
}

// ---------------------------------------------------------------------------
// Packed layout (written once by pack_kernel, read by qmv_kernel).
//
// W is cut into tiles of 16 rows x 128 k (one "pair" of 64-groups).  Tile
// (t, p) -- rows 16t..16t+15, k = 128p..128p+127 -- is stored contiguously at
// tile index t * n_pairs + p, as 64 lane slots of 16 bytes (W4) or two
// 1 KB halves of 64 x 16 bytes (W8).  Lane slot l = 16 j + r holds row
// 16t + r, k = 128p + 32 j + [0, 32) (W8 half v: k = 128p + 32 j + 16 v +
// [0, 16)), the codes in their original order: exactly the bytes the MFMA B
// operand of lane l needs.  A wave therefore reads 1 KB per load
// instruction and streams a contiguous region.  Scales and biases become
// one 32-bit word per (row, group): fp16 scale in the low half, fp16 bias in
// the high half, stored as [t][p / 2][h * 16 + r][p % 2] for group
// g = 2p + h, so one 8-byte load gives a lane the words of two pairs.  Rows
// past N and groups past K/64 are zero, so they contribute exactly nothing.
// ---------------------------------------------------------------------------

// With a second matrix (w2, scales2, biases2 non-null: the up projection
// next to the gate projection w) the tiles alternate: tile 2i holds rows
// 16i..16i+15 of the first matrix and tile 2i + 1 the same rows of the
// second, so one workgroup owning two tiles sees both halves of a gated
// product.  N is then the row count of each matrix.
template <int BITS>
__global__ __launch_bounds__(256) void pack_kernel(
    const void *__restrict__ w, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const void *__restrict__ w2,
    const uint16_t *__restrict__ scales2, const uint16_t *__restrict__ biases2,
    u32x4 *__restrict__ wp, uint32_t *__restrict__ sbp, int N, int K) {
    const bool two = w2 != nullptr;
    const int ng = K >> 6;
    const int n_pairs = (ng + 1) >> 1;
    const int n_tiles = two ? 2 * ((N + 15) >> 4) : (N + 15) >> 4;
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
        const int n = two ? 16 * (t >> 1) + r : 16 * t + r;
        const void *src = (two && (t & 1)) ? w2 : w;
        const int k = 128 * p + 32 * j + 16 * v;   // first k of the 16 bytes
        u32x4 val = {0u, 0u, 0u, 0u};
        if (n < N && k < K)
            val = reinterpret_cast<const u32x4 *>(src)[((size_t)n * K + k) / (BITS == 4 ? 32 : 16)];
        wp[i] = val;
    }
    // scale/bias words: [t][p / 2][h * 16 + r][p % 2] for the group g = 2p + h
    const int npp = (n_pairs + 1) >> 1;
    const size_t sb_count = (size_t)n_tiles * npp * 64;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < sb_count;
         i += (size_t)gridDim.x * blockDim.x) {
        const int e = (int)(i & 1);
        const int hr = (int)((i >> 1) & 31);
        const size_t rest = i >> 6;
        const int pp = (int)(rest % npp);
        const int t = (int)(rest / npp);
        const int n = two ? 16 * (t >> 1) + (hr & 15) : 16 * t + (hr & 15);
        const bool second = two && (t & 1);
        const uint16_t *sc = second ? scales2 : scales;
        const uint16_t *bi = second ? biases2 : biases;
        const int g = 2 * (2 * pp + e) + (hr >> 4);
        uint32_t val = 0;
        if (n < N && g < ng)
            val = (uint32_t)sc[(size_t)n * ng + g] | ((uint32_t)bi[(size_t)n * ng + g] << 16);
        sbp[i] = val;
    }
}

// Kernel arguments.  Packed layout: w = tiles, sb = scale/bias words,
// biases unused.  Interchange layout: w = codes [N][K*BITS/8], sb = scales
// [N][K/64], biases [N][K/64] (fp16 bit patterns).
struct QmvArgs {
    const void *w;
    const void *sb;
    const uint16_t *biases;
    const uint16_t *x;
    void *out;
    int M, N, K, n_out;
};

// RM: the interchange (row-major) layout instead of packed tiles.
//
// XH: 16-byte x loads per lane and pair -- 1 when M <= 4 (rows 0..3),
// 2 when M <= 8, 4 when M <= 16.  Rows a launch does not stage hold zeros
// (their MFMA operand rows are zero), so the M <= 4 and M <= 8 variants
// compute bitwise the same.
//
// XH = 4 is the wide form for 9..16 rows: every A row is an x row, so the
// two groups of a pair can no longer share an MFMA through the row split.
// Each 32-k step then runs two MFMAs per tile on the same B operand, with A
// masked to group 0's k slots (lanes j = 0, 1) and to group 1's (j = 2, 3),
// into separate accumulators that get their own group's scale and bias.
// The per-group FMA chains and the final sum are those of the pair form, so
// rows 0..7 of a wide call equal an M <= 8 call bitwise.
//
// GLU: the weights are a gate/up pair packed with alternating tiles (see
// pack_kernel), T is even, and instead of y the kernel writes the gated
// activation h[m][f] = silu(g) * u as bf16 [M][n_out], g and u being the
// outputs of tiles 2i and 2i + 1 for f = 16i + r.  g and u are reduced
// exactly as a plain launch reduces them.
//
// MR: C rows of a lane's 4-row block that can hold an x row (M itself when
// M <= 4, else 4); the per-group affine epilogue skips the others.
//
// SB2 (interchange only): the scales and biases of two pairs come in one
// 8-byte load each (rows of a multiple of 4 groups, 8-byte aligned arrays);
// otherwise two 2-byte loads per pair and group.
//
// VALU (W4, M <= 4): the same loads, staging and fold, with the products on
// the vector ALU instead of the matrix cores -- the comparison variant.
// Lane 16 j + r takes its 32 codes of row r (k slots 32 j ..) against the
// same k of each x row m < MR, two products per v_dot2c_f32_bf16, and the
// x sums over those k the same way; lanes j and j ^ 1 (the two halves of
// one group) are added before the usual reduction.
template <int BITS, bool RM, int WAVES, int T, int S, int XH, bool GLU = false, int MR = 4,
          bool SB2 = true, bool VALU = false>
__global__ __launch_bounds__(WAVES * 64) void qmv_kernel(QmvArgs a) {
    static_assert(XH == 1 || XH == 2 || XH == 4, "x loads per lane and pair");
    static_assert(!VALU || (BITS == 4 && XH == 1), "the vector-ALU variant serves W4 at M <= 4");
    static_assert(!GLU || (T % 2 == 0 && !RM), "a gated launch pairs packed gate and up tiles");
    // packed, or SB2: a two-pair scale/bias block hands over between stage slots
    constexpr bool HANDOFF = !RM || SB2;
    static_assert(!HANDOFF || S % 2 == 0, "scale/bias blocks of two pairs need an even stage count");
    static_assert(MR >= 1 && MR <= 4 && (XH == 1 || MR == 4), "rows per lane block");
    constexpr bool WIDE = XH == 4;  // 9..16 rows: one MFMA per group
    constexpr int NG = WIDE ? 2 : 1;    // groups (accumulators) per lane
    constexpr int L = BITS / 4;     // 16-byte code loads per pair, tile and lane
    // Each wave stages x in its own 16 x 128 slot; the cross-wave reduction
    // reuses the same memory after the main loop.
    union Shared {
        uint16_t xs[WAVES][16][128];
        f32x4 red[WAVES][T][64];
    };
    __shared__ __attribute__((aligned(16))) Shared sh;
    __shared__ __attribute__((aligned(16))) uint16_t xzero[8];

    const int M = a.M, N = a.N, K = a.K;
    const int ng = K >> 6;                   // groups per row
    const int n_pairs = (ng + 1) >> 1;       // 128-wide K steps
    const int npp = (n_pairs + 1) >> 1;      // packed scale/bias blocks of two pairs
    const int n_tiles = (N + 15) >> 4;
    const int lane = threadIdx.x & 63;
    // readfirstlane makes the wave index (and all that derives from it)
    // provably uniform, so buffer offsets stay in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int j = lane >> 4;   // k-slot group of the A/B operands, row group of C
    const int r = lane & 15;   // A row / B and C column
    const int h = j >> 1;      // which group of the pair this lane's k slots hold
    const int sub = j & 1;     // which 32-k half of that group

    // This wave's contiguous share of the pairs (an even count, so a wave's
    // range starts at an even pair, as the packed scale/bias blocks need).
    const int ppw = ((n_pairs + WAVES - 1) / WAVES + 1) & ~1;
    const int p_lo = min(n_pairs, wave * ppw);
    const int p_hi = min(n_pairs, p_lo + ppw);

    // Buffer resources: lane-dependent offsets are fixed, per-pair offsets
    // are wave-uniform (scalar registers).  A tile past the last one (or
    // rows past N) gets an empty range, so its loads return zeros.
    constexpr int kRowBytesPerK = BITS;          // row bytes = K * BITS / 8
    const unsigned row_bytes = (unsigned)(K / 8) * kRowBytesPerK;
    __amdgpu_buffer_rsrc_t wres[T], sres[T], bres[T];
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
        const int t = blockIdx.x * T + tt;
        const int tc = min(t, n_tiles - 1);
        if (!RM) {
            const bool there = t < n_tiles;
            wres[tt] = __builtin_amdgcn_make_buffer_rsrc(
                (void *)((const u32x4 *)a.w + (size_t)tc * n_pairs * 64 * L), (short)0,
                there ? n_pairs * 1024 * L : 0, kBufferFlags);
            sres[tt] = __builtin_amdgcn_make_buffer_rsrc(
                (void *)((const uint32_t *)a.sb + (size_t)tc * npp * 64), (short)0,
                there ? npp * 256 : 0, kBufferFlags);
        } else {
            const int rows = max(0, min(16, N - 16 * t));
            wres[tt] = __builtin_amdgcn_make_buffer_rsrc(
                (void *)((const char *)a.w + (size_t)16 * tc * row_bytes), (short)0,
                rows * row_bytes, kBufferFlags);
            sres[tt] = __builtin_amdgcn_make_buffer_rsrc(
                (void *)((const uint16_t *)a.sb + (size_t)16 * tc * ng), (short)0,
                rows * ng * 2, kBufferFlags);
            bres[tt] = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(a.biases + (size_t)16 * tc * ng), (short)0, rows * ng * 2, kBufferFlags);
        }
    }
    const __amdgpu_buffer_rsrc_t xres =
        __builtin_amdgcn_make_buffer_rsrc((void *)a.x, (short)0, M * K * 2, kBufferFlags);
    // Packed: lane slot l of a tile's pair; interchange: row r, bytes
    // 32 j * BITS / 8 of the pair's k.
    const unsigned woff = RM ? (unsigned)r * row_bytes + (unsigned)j * (4 * BITS) : (unsigned)lane * 16u;
    // Scale/bias offsets.  Pair form: this lane's group h; wide form: both
    // groups of row r.  Packed: the word of (row, group) in a 2-pair block;
    // interchange: the fp16 of (row, group) relative to the pair's first.
    unsigned sboff[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g)
        sboff[g] = RM ? (unsigned)(r * ng + (WIDE ? g : h)) * 2u
                      : (unsigned)((WIDE ? g : h) * 16 + r) * 8u;
    // x is loaded compactly: lane -> row (lane >> 4) + 4 i, 16-byte chunk
    // (lane & 15) of the pair's 128 k; rows >= M read zeros.
    const int xrow0 = lane >> 4, xch = lane & 15;
    // Wide form: lanes read their A row only for the MFMA of their own group.
    bool a_act[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g)
        a_act[g] = h == g;
    // Zero this wave's staged A matrix once: in the pair form, the halves of
    // each row that belong to the other group, and the rows no x row maps
    // to, are never written again.
    {
        u32x4 *slot = reinterpret_cast<u32x4 *>(&sh.xs[wave][0][0]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            slot[lane + 64 * i] = u32x4{0u, 0u, 0u, 0u};
    }
    if (threadIdx.x < 8)
        xzero[threadIdx.x] = 0;
    __syncthreads();

    const bf16x8 ones = __builtin_bit_cast(
        bf16x8, u32x4{vgpr_const(0x3F803F80u), vgpr_const(0x3F803F80u), vgpr_const(0x3F803F80u),
                      vgpr_const(0x3F803F80u)});
    const unsigned w4base = vgpr_const(0x41804180u);
    const W4Shifts w4sh{opaque_sgpr(3), opaque_sgpr(1), opaque_sgpr(5), opaque_sgpr(9)};
    f32x4 acc[T][NG];
#pragma unroll
    for (int tt = 0; tt < T; ++tt)
#pragma unroll
        for (int g = 0; g < NG; ++g)
            acc[tt][g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // A stage is one pair: the T tiles' codes and scale/bias words, and the
    // compact x rows, all issued together.  Pairs outside this wave's range
    // load through an out-of-range offset (zeros, no memory traffic), so no
    // load sits under a branch and the compiler counts outstanding loads
    // exactly.  Packed scale/bias words come two pairs per load: the stage
    // of an even pair (an even stage slot, since a wave's range starts at an
    // even pair and S is even) loads the 8-byte block holding both pairs'
    // words, and its compute hands the odd pair's word on to the next stage
    // (sb_next); the odd stage loads none.  Interchange scales and biases
    // are two 2-byte loads per pair and group.
    struct Stage {
        u32x4 raw[T][L];
        uint32_t sb[T][NG];
        uint32_t sb_odd[T][NG];   // packed: the odd pair's words
        u32x4 xc[XH];
    };
    uint32_t sb_next[T][NG];
    auto issue = [&](Stage &st, int p, int slot) {
        const bool in = p >= p_lo && p < p_hi;
        const int pc = in ? p : 0;
        // interchange: the odd last group of a row has no codes or scales
        const bool gin = !RM || 2 * pc + h < ng;
        const unsigned wv = (in && gin) ? woff : kOutOfRange;
#pragma unroll
        for (int tt = 0; tt < T; ++tt)
#pragma unroll
            for (int v = 0; v < L; ++v)
                st.raw[tt][v] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               wres[tt], wv, RM ? pc * 16 * BITS + 16 * v : (pc * L + v) * 1024,
                               RM ? kRowHalfLine : kStreamOnce));
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                if (RM && !SB2) {
                    const bool gg = in && 2 * pc + (WIDE ? g : h) < ng;
                    const unsigned sv = gg ? sboff[g] : kOutOfRange;
                    const uint32_t s16 = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(sres[tt], sv, pc * 4, 0);
                    const uint32_t b16 = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(bres[tt], sv, pc * 4, 0);
                    st.sb[tt][g] = s16 | (b16 << 16);
                } else if (RM && slot % 2 == 0) {
                    // groups 4q .. 4q + 3 of this lane's row: pair 2q holds
                    // 4q + grp, pair 2q + 1 holds 4q + 2 + grp
                    const int grp = WIDE ? g : h;
                    const unsigned sv = in ? (unsigned)(r * ng) * 2u : kOutOfRange;
                    const auto s4 = __builtin_amdgcn_raw_buffer_load_b64(sres[tt], sv, (pc >> 1) * 8, 0);
                    const auto b4 = __builtin_amdgcn_raw_buffer_load_b64(bres[tt], sv, (pc >> 1) * 8, 0);
                    const unsigned sh16 = 16u * (unsigned)(grp & 1);
                    const unsigned se = (s4[grp >> 1] >> sh16) & 0xFFFFu, so = (s4[1 + (grp >> 1)] >> sh16) & 0xFFFFu;
                    const unsigned be = (b4[grp >> 1] >> sh16) & 0xFFFFu, bo = (b4[1 + (grp >> 1)] >> sh16) & 0xFFFFu;
                    st.sb[tt][g] = se | (be << 16);
                    st.sb_odd[tt][g] = so | (bo << 16);
                } else if (!RM && slot % 2 == 0) {
                    // one load gives this lane's words of both pairs of a block
                    const unsigned sv = in ? sboff[g] : kOutOfRange;
                    const auto v2 = __builtin_amdgcn_raw_buffer_load_b64(sres[tt], sv, (pc >> 1) * 256, 0);
                    st.sb[tt][g] = v2[0];
                    st.sb_odd[tt][g] = v2[1];
                }
            }
        }
        // the odd last group of a row has no partner: its chunks read zeros
        const bool xgin = 2 * pc + (xch >> 3) < ng;
#pragma unroll
        for (int i = 0; i < XH; ++i) {
            const int row = xrow0 + 4 * i;
            const unsigned off = (in && xgin && row < M) ? (unsigned)((row * K + 8 * xch) * 2) : kOutOfRange;
            st.xc[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, off, pc * 256, 0));
        }
    };
    auto compute = [&](const Stage &st, int p, int slot) {
        if (p >= p_hi)
            return;
        // Stage x through this wave's LDS matrix, then read the MFMA A
        // fragments back.  LDS operations of one wave complete in order, so
        // the matrix can be rewritten by the next stage right away.  Pair
        // form: x row m's chunk c goes to A row m (c < 8, group 0) or m + 8
        // (group 1); wide form: A row m.
#pragma unroll
        for (int i = 0; i < XH; ++i) {
            const int m = xrow0 + 4 * i;
            const int arow = WIDE ? m : m + 8 * (xch >> 3);
            const u32x4 v = BITS == 4 ? stage_w4_order(st.xc[i]) : st.xc[i];
            *reinterpret_cast<u32x4 *>(&sh.xs[wave][arow][8 * (xch ^ swz(arow))]) = v;
        }
        f32x4 c[T][NG];
        f32x4 cx[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            cx[g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int tt = 0; tt < T; ++tt)
                c[tt][g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        const int rsw = swz(r);
        if constexpr (VALU) {
            // c[tt][0][m] and cx[0][m]: this lane's 32 k of x row m against
            // the codes of tile tt, and against ones.  x row m of this
            // lane's group h is A row m + 8 h; its 32 k are chunks 4 j ..
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const bf16x2 one2 = __builtin_bit_cast(bf16x2, 0x3F803F80u);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                bf16x8 xv[2][MR];
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        const int ar = m + 8 * h;
                        xv[e][m] = *reinterpret_cast<const bf16x8 *>(
                            &sh.xs[wave][ar][8 * ((4 * j + 2 * half + e) ^ swz(ar))]);
                    }
                // (Words go through named scalars: a bit_cast applied to a
                // vector element directly read element 0 for every index.)
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        const u32x4 xw = __builtin_bit_cast(u32x4, xv[e][m]);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const unsigned xq = xw[q];
                            cx[0][m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xq),
                                                                      one2, cx[0][m], false);
                        }
                    }
#pragma unroll
                for (int tt = 0; tt < T; ++tt) {
                    bf16x8 bv[2];
                    unpack_w4(st.raw[tt][0], half, w4base, w4sh, bv);
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const u32x4 bw = __builtin_bit_cast(u32x4, bv[e]);
#pragma unroll
                        for (int m = 0; m < MR; ++m) {
                            const u32x4 xw = __builtin_bit_cast(u32x4, xv[e][m]);
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const unsigned xq = xw[q], bq = bw[q];
                                c[tt][0][m] = __builtin_amdgcn_fdot2_f32_bf16(
                                    __builtin_bit_cast(bf16x2, xq), __builtin_bit_cast(bf16x2, bq),
                                    c[tt][0][m], false);
                            }
                        }
                    }
                }
            }
        } else {
        // Two 32-k steps at a time: both A fragments, then per tile the two B
        // operands (unpacked right before their MFMAs, so only one tile's are
        // live) -- the same MFMA order per accumulator as step by step.
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8 av[2][NG];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int s4 = 2 * half + e;
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const uint16_t *src =
                        (!WIDE || a_act[g]) ? &sh.xs[wave][r][8 * ((4 * j + s4) ^ rsw)] : xzero;
                    av[e][g] = *reinterpret_cast<const bf16x8 *>(src);
                }
            }
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    cx[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[e][g], ones, cx[g], 0, 0, 0);
#pragma unroll
            for (int tt = 0; tt < T; ++tt) {
                bf16x8 bv[2];
                if (BITS == 4) {
                    unpack_w4(st.raw[tt][0], half, w4base, w4sh, bv);
                } else {
                    const u32x4 &lo = st.raw[tt][half];
                    bv[0] = unpack_w8(lo[0], lo[1]);
                    bv[1] = unpack_w8(lo[2], lo[3]);
                }
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int g = 0; g < NG; ++g)
                        c[tt][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[e][g], bv[e], c[tt][g], 0, 0, 0);
            }
        }
        }
        // Pair form: C row 4*j + i is x row m = 4*sub + i of half h.
        // Wide form: C row 4*j + i is x row 4*j + i, one accumulator per
        // group.  cx holds the same rows' sums of x over the group.
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                uint32_t sbw = st.sb[tt][g];
                if (HANDOFF) {
                    if (slot % 2 == 0)
                        sb_next[tt][g] = st.sb_odd[tt][g];
                    else
                        sbw = sb_next[tt][g];
                }
                const float s = half_bits_to_float((uint16_t)(sbw & 0xFFFFu));
                const float bias = half_bits_to_float((uint16_t)(sbw >> 16));
                const float bb = BITS == 4 ? fmaf(-16.0f, s, bias) : bias;
                // rows i >= MR of this lane's C block hold no x row
#pragma unroll
                for (int i = 0; i < MR; ++i) {
                    acc[tt][g][i] = fmaf(s, c[tt][g][i], acc[tt][g][i]);
                    acc[tt][g][i] = fmaf(bb, cx[g][i], acc[tt][g][i]);
                }
            }
        }
    };

    // S stages in flight: while one is computed the others are loading.  The
    // loop starts one round early with nothing to compute, so the loads the
    // loop header sees are always the previous round's, in issue order, and
    // each compute waits only for its own stage.
    Stage st[S];
    for (int base = p_lo - S; base < p_hi; base += S) {
#pragma unroll
        for (int q = 0; q < S; ++q) {
            if (base + q >= p_lo)
                compute(st[q], base + q, q);
            __builtin_amdgcn_sched_barrier(0);
            issue(st[q], base + q + S, q);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Fixed-order reduction: the two groups of a pair (pair form: lanes l,
    // l ^ 32; wide form: the two accumulators of a lane), then the waves in
    // index order.  Neither depends on M.
    if constexpr (VALU) {
        // the two halves of a group (lanes l, l ^ 16) into the even one; the
        // odd lanes stand for x rows 4..7, which a call of M <= 4 lacks
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            f32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // (the element goes through a named scalar: a bit_cast applied
                // to a vector element directly read element 0 for every i)
                const float ai = acc[tt][0][i];
                o[i] = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, ai), 0x401F));
            }
            acc[tt][0] = sub ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : acc[tt][0] + o;
        }
    }
    __syncthreads();   // every wave is done with its x matrix
#pragma unroll
    for (int tt = 0; tt < T; ++tt)
        sh.red[wave][tt][lane] = WIDE ? acc[tt][0] + acc[tt][NG - 1] : acc[tt][0];
    __syncthreads();
    if (WIDE ? wave == 0 : (wave == 0 && lane < 32)) {
        f32x4 tot[T];
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            tot[tt] = WIDE ? sh.red[0][tt][lane] : sh.red[0][tt][lane] + sh.red[0][tt][lane + 32];
            for (int ww = 1; ww < WAVES; ++ww)
                tot[tt] += WIDE ? sh.red[ww][tt][lane] : sh.red[ww][tt][lane] + sh.red[ww][tt][lane + 32];
        }
        const int m0 = WIDE ? 4 * j : 4 * sub;
        if (!GLU) {
            float *y = static_cast<float *>(a.out);
#pragma unroll
            for (int tt = 0; tt < T; ++tt) {
                const int n = (blockIdx.x * T + tt) * 16 + r;
                if (n >= N)
                    continue;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (m0 + i < M)
                        y[(size_t)(m0 + i) * N + n] = tot[tt][i];
            }
        } else {
            uint16_t *hout = static_cast<uint16_t *>(a.out);
#pragma unroll
            for (int tt = 0; tt < T; tt += 2) {
                const int f = ((blockIdx.x * T + tt) >> 1) * 16 + r;
                if (f >= a.n_out)
                    continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (m0 + i >= M)
                        continue;
                    const float g = tot[tt][i], u = tot[tt + 1][i];
                    const float v = g / (1.0f + expf(-g)) * u;
                    // nearest-even bf16 (finite values and infinities; the
                    // quiet-NaN pattern for NaN)
                    const unsigned bits = __float_as_uint(v);
                    const unsigned rnd = (v != v) ? 0x7FC00000u
                                                  : bits + 0x7FFFu + ((bits >> 16) & 1u);
                    hout[(size_t)(m0 + i) * a.n_out + f] = (uint16_t)(rnd >> 16);
                }
            }
        }
    }
}

// Draft-only 4-bit copy of a weight matrix (MTPLX announcement, "Layer 0"
// custom kernels: the target's LM head stays at model precision, a 4-bit
// copy serves drafting).  One thread per (row, 64-group): min/max fit,
// b = min, s = (max - min) / 15 (fp32, then nearest-even fp16), codes
// round_half_even((w - b16) / s16) clamped to 0..15 (0 where s16 is 0 or
// not finite), in the interchange layout spec_pack_w4 reads.
__global__ __launch_bounds__(256) void requantize_w4_kernel(
    const uint16_t *__restrict__ w, int N, int K, uint32_t *__restrict__ w4,
    uint16_t *__restrict__ scales, uint16_t *__restrict__ biases) {
    const int ng = K >> 6;
    const size_t count = (size_t)N * ng;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (size_t)gridDim.x * blockDim.x) {
        const size_t n = i / ng;
        const int g = (int)(i - n * ng);
        const u32x4 *src = reinterpret_cast<const u32x4 *>(w + n * K + 64 * g);
        u32x4 raw[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
            raw[c] = src[c];
        float lo = INFINITY, hi = -INFINITY;
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = __uint_as_float(raw[c][e] << 16);
                const float b = __uint_as_float(raw[c][e] & 0xFFFF0000u);
                lo = fminf(lo, fminf(a, b));
                hi = fmaxf(hi, fmaxf(a, b));
            }
        const _Float16 s16 = (_Float16)((hi - lo) / 15.0f);
        const _Float16 b16 = (_Float16)lo;
        scales[i] = __builtin_bit_cast(uint16_t, s16);
        biases[i] = __builtin_bit_cast(uint16_t, b16);
        const float sf = (float)s16, bf = (float)b16;
        const bool use = sf != 0.0f && __builtin_isfinite(sf);
        uint32_t *dst = w4 + n * (K >> 3) + 8 * g;
#pragma unroll
        for (int c = 0; c < 8; ++c) {          // 8 codes per output word
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = __uint_as_float(raw[c][e] << 16);
                const float b = __uint_as_float(raw[c][e] & 0xFFFF0000u);
                const float ra = rintf((a - bf) / sf), rb = rintf((b - bf) / sf);
                const uint32_t qa = use ? (uint32_t)fminf(fmaxf(ra, 0.0f), 15.0f) : 0u;
                const uint32_t qb = use ? (uint32_t)fminf(fmaxf(rb, 0.0f), 15.0f) : 0u;
                word |= qa << (8 * e) | qb << (8 * e + 4);
            }
            dst[c] = word;
        }
    }
}

template <typename V>
__global__ void fill_zero_kernel(V *__restrict__ y, size_t count) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (size_t)gridDim.x * blockDim.x)
        y[i] = V(0);
}

template <typename V>
hipError_t fill_zero(V *y, size_t count, hipStream_t stream) {
    const int blocks = (int)std::min<size_t>((count + 255) / 256, 4096);
    fill_zero_kernel<<<blocks, 256, 0, stream>>>(y, count);
    return hipGetLastError();
}

// Launches qmv_kernel for one (bits, layout) at the plan's shape; the x-row
// variant (XH, MR) follows M.
template <int B, bool RM, int W, int TT, int SS, bool GLU, bool SB2 = true>
hipError_t launch_shape(const QmvArgs &a, int blocks, hipStream_t stream) {
    if (a.M == 1)
        qmv_kernel<B, RM, W, TT, SS, 1, GLU, 1, SB2><<<blocks, W * 64, 0, stream>>>(a);
    else if (a.M == 2)
        qmv_kernel<B, RM, W, TT, SS, 1, GLU, 2, SB2><<<blocks, W * 64, 0, stream>>>(a);
    else if (a.M == 3)
        qmv_kernel<B, RM, W, TT, SS, 1, GLU, 3, SB2><<<blocks, W * 64, 0, stream>>>(a);
    else if (a.M == 4)
        qmv_kernel<B, RM, W, TT, SS, 1, GLU, 4, SB2><<<blocks, W * 64, 0, stream>>>(a);
    else if (a.M <= 8)
        qmv_kernel<B, RM, W, TT, SS, 2, GLU, 4, SB2><<<blocks, W * 64, 0, stream>>>(a);
    else
        qmv_kernel<B, RM, W, TT, SS, 4, GLU, 4, SB2><<<blocks, W * 64, 0, stream>>>(a);
    return hipGetLastError();
}

// The vector-ALU variant (W4, M = 1..4) at the plan's shape.
template <int W, int TT, bool GLU>
hipError_t launch_valu_shape(const QmvArgs &a, int blocks, hipStream_t stream) {
    if (a.M == 1)
        qmv_kernel<4, false, W, TT, 2, 1, GLU, 1, true, true><<<blocks, W * 64, 0, stream>>>(a);
    else if (a.M == 2)
        qmv_kernel<4, false, W, TT, 2, 1, GLU, 2, true, true><<<blocks, W * 64, 0, stream>>>(a);
    else if (a.M == 3)
        qmv_kernel<4, false, W, TT, 2, 1, GLU, 3, true, true><<<blocks, W * 64, 0, stream>>>(a);
    else
        qmv_kernel<4, false, W, TT, 2, 1, GLU, 4, true, true><<<blocks, W * 64, 0, stream>>>(a);
    return hipGetLastError();
}

} // namespace

QmvPlan qmv_plan(int bits, int N, int K) {
    QmvPlan p{};
    p.n_tiles = (N + 15) / 16;
    p.n_pairs = (K / 64 + 1) / 2;
    // Launch shape, from (N, K) only (never M, so row m never depends on M),
    // chosen by measurement on the verify shapes: enough waves in flight to
    // cover HBM latency, and as many tiles per wave as that allows, since
    // the tiles served by one x fragment share its staging and its
    // group-sum MFMA.
    //   very tall (LM head, >= 4096 tiles):   4 tiles, 4 waves split K
    //   tall (MLP gate/up, >= 1024 tiles):    2 tiles, 4 waves (W8: 1 tile, 8 waves)
    //   long K (MLP down, >= 96 pairs):       2 tiles, 8 waves
    //   the rest (attention q/k/v/o):         1 tile, 8 waves
    p.stages = 2;
    if (p.n_tiles >= 4096) {
        p.tiles_per_wave = bits == 4 ? 4 : 2;
        p.waves = bits == 4 ? 4 : 8;
    } else if (p.n_tiles >= 1024) {
        p.tiles_per_wave = bits == 4 ? 2 : 1;
        p.waves = bits == 4 ? 4 : 8;
    } else if (p.n_pairs >= 96) {
        p.tiles_per_wave = 2; p.waves = 8;
    } else {
        p.tiles_per_wave = 1; p.waves = 8;
    }
    return p;
}

size_t qmv_packed_bytes(int bits, int N, int K) {
    const QmvPlan p = qmv_plan(bits, N, K);
    return (size_t)p.n_tiles * p.n_pairs * 64 * 16 * (bits / 4);
}

size_t qmv_packed_sb_bytes(int N, int K) {
    const QmvPlan p = qmv_plan(4, N, K);
    return (size_t)p.n_tiles * ((p.n_pairs + 1) / 2) * 256;
}

hipError_t launch_pack(int bits, const void *w, const uint16_t *scales,
                       const uint16_t *biases, const void *w2,
                       const uint16_t *scales2, const uint16_t *biases2, int N,
                       int K, void *w_packed, void *sb_packed, hipStream_t stream) {
    if (N == 0 || K == 0)
        return hipSuccess;
    const int n_rows = w2 ? gate_up_rows(N) : N;
    const size_t slots = qmv_packed_bytes(bits, n_rows, K) / 16;
    const int blocks = (int)std::min<size_t>((slots + 255) / 256, 65536);
    if (bits == 4)
        pack_kernel<4><<<blocks, 256, 0, stream>>>(w, scales, biases, w2, scales2, biases2,
                                                   (u32x4 *)w_packed, (uint32_t *)sb_packed, N, K);
    else
        pack_kernel<8><<<blocks, 256, 0, stream>>>(w, scales, biases, w2, scales2, biases2,
                                                   (u32x4 *)w_packed, (uint32_t *)sb_packed, N, K);
    return hipGetLastError();
}

int gate_up_rows(int F) { return 32 * ((F + 15) / 16); }

hipError_t launch_requantize_w4(const uint16_t *w, int N, int K, uint32_t *w4,
                                uint16_t *scales, uint16_t *biases, hipStream_t stream) {
    if (N == 0 || K == 0)
        return hipSuccess;
    const size_t count = (size_t)N * (K / 64);
    const int blocks = (int)std::min<size_t>((count + 255) / 256, 65536);
    requantize_w4_kernel<<<blocks, 256, 0, stream>>>(w, N, K, w4, scales, biases);
    return hipGetLastError();
}

hipError_t launch_qmv(int bits, bool interchange, const void *w, const void *sb,
                      const uint16_t *biases, const uint16_t *x, float *y, int M, int N,
                      int K, hipStream_t stream) {
    if (M == 0 || N == 0)
        return hipSuccess;
    if (K == 0)
        return fill_zero(y, (size_t)M * N, stream);
    const QmvPlan plan = qmv_plan(bits, N, K);
    const QmvArgs a{w, sb, biases, x, y, M, N, K, 0};
    // Very tall launches (LM heads) at one or two rows take half the tiles
    // per workgroup: x is a small share of their bytes there, and smaller
    // workgroups drain sooner at the end of the launch (W4 M = 1: 65.8
    // against 68.5 us).  The waves, and so every output's arithmetic, are
    // the plan's: results do not depend on the tile count.
    const int T = (plan.n_tiles >= 4096 && M <= 2) ? std::max(1, plan.tiles_per_wave / 2)
                                                   : plan.tiles_per_wave;
    const int blocks = (plan.n_tiles + T - 1) / T;
    // Interchange scales and biases load two pairs' worth (8 bytes) at a time
    // when every row starts 8-byte aligned.
    const bool sb2 = (K / 64) % 4 == 0 &&
                     ((reinterpret_cast<uintptr_t>(sb) | reinterpret_cast<uintptr_t>(biases)) & 7u) == 0;
#define SPEC_QMV_LAUNCH(B, W, TT, SS)                                                    \
    if (bits == B && plan.waves == W && T == TT && plan.stages == SS) \
        return !interchange ? launch_shape<B, false, W, TT, SS, false>(a, blocks, stream) \
               : sb2        ? launch_shape<B, true, W, TT, SS, false, true>(a, blocks, stream) \
                            : launch_shape<B, true, W, TT, SS, false, false>(a, blocks, stream);
#define SPEC_QMV_SHAPES(B) \
    SPEC_QMV_LAUNCH(B, 4, 4, 2) SPEC_QMV_LAUNCH(B, 4, 2, 2) SPEC_QMV_LAUNCH(B, 8, 2, 2) \
    SPEC_QMV_LAUNCH(B, 8, 1, 2)
    SPEC_QMV_SHAPES(4)
    SPEC_QMV_SHAPES(8)
#undef SPEC_QMV_SHAPES
#undef SPEC_QMV_LAUNCH
    return hipErrorInvalidConfiguration;   // no kernel for this plan (unreachable)
}

hipError_t launch_qmv_gate_up_silu(int bits, const void *w_packed, const void *sb_packed,
                                   const uint16_t *x, uint16_t *h, int M, int F, int K,
                                   hipStream_t stream) {
    if (M == 0 || F == 0)
        return hipSuccess;
    if (K == 0)   // g = u = 0, so h = silu(0) * 0 = +0
        return fill_zero(h, (size_t)M * F, stream);
    const int N = gate_up_rows(F);
    const QmvPlan plan = qmv_plan(bits, N, K);
    // The plain launch shape with at least one gate/up tile pair per
    // workgroup: the waves (hence every output's reduction order) are the
    // plain launch's, only the tiles per workgroup may double.
    const int T = std::max(plan.tiles_per_wave, 2);
    const QmvArgs a{w_packed, sb_packed, nullptr, x, h, M, N, K, F};
    // n_tiles is even, so no workgroup splits a gate/up pair; tiles past the
    // end (T = 4) read zeros and write nothing.
    const int blocks = (plan.n_tiles + T - 1) / T;
#define SPEC_QMV_GLU_LAUNCH(B, W, TT)                                          \
    if (bits == B && plan.waves == W && T == TT && plan.stages == 2)           \
        return launch_shape<B, false, W, TT, 2, true>(a, blocks, stream);
    SPEC_QMV_GLU_LAUNCH(4, 4, 4) SPEC_QMV_GLU_LAUNCH(4, 4, 2) SPEC_QMV_GLU_LAUNCH(4, 8, 2)
    SPEC_QMV_GLU_LAUNCH(8, 8, 2)
#undef SPEC_QMV_GLU_LAUNCH
    return hipErrorInvalidConfiguration;   // no kernel for this plan (unreachable)
}

hipError_t launch_qmv_valu(const void *w_packed, const void *sb_packed, const uint16_t *x,
                           void *out, int M, int N, int K, int F, hipStream_t stream) {
    const bool gated = F > 0;
    if (M == 0 || N == 0)
        return hipSuccess;
    if (K == 0)
        return gated ? fill_zero(static_cast<uint16_t *>(out), (size_t)M * F, stream)
                     : fill_zero(static_cast<float *>(out), (size_t)M * N, stream);
    const QmvPlan plan = qmv_plan(4, N, K);
    const int T = gated ? std::max(plan.tiles_per_wave, 2) : plan.tiles_per_wave;
    const QmvArgs a{w_packed, sb_packed, nullptr, x, out, M, N, K, gated ? F : 0};
    const int blocks = (plan.n_tiles + T - 1) / T;
#define SPEC_QMV_VALU_LAUNCH(W, TT)                                                     \
    if (plan.waves == W && T == TT)                                                     \
        return gated ? launch_valu_shape<W, TT, true>(a, blocks, stream)                \
                     : launch_valu_shape<W, TT, false>(a, blocks, stream);
    SPEC_QMV_VALU_LAUNCH(4, 4) SPEC_QMV_VALU_LAUNCH(4, 2) SPEC_QMV_VALU_LAUNCH(8, 2)
#undef SPEC_QMV_VALU_LAUNCH
    if (!gated && plan.waves == 8 && T == 1)
        return launch_valu_shape<8, 1, false>(a, blocks, stream);
    return hipErrorInvalidConfiguration;   // no kernel for this plan (unreachable)
}

} // namespace spec
