// Recurrent-layer state of the target during a speculative cycle, for
// gfx950: capture of an innovation tape over the verify positions, and the
// commit of the accepted steps afterwards.
//
// The MTPLX announcement ("Layer 0" custom kernels; "Layer 2: Speculative
// cycle") keeps the recurrent (GDN) state of the target out of per-position
// snapshots: each step records a small tuple (gate, state delta), and after
// verification the accepted steps are committed from the tape while the
// rejected ones are dropped -- kilobytes per step instead of copies of the
// whole state.  The update is the gated delta rule, per head (a reading; the
// pages name GDN without writing it out):
//     delta_t = beta_t * (v_t - alpha_t * S_{t-1} k_t)     (the innovation)
//     S_t     = alpha_t * S_{t-1} + delta_t k_t^T
//     o_t     = S_t q_t
// with S a dv x dk fp32 matrix (dk = dv = 128), [B][H][dv][dk] in HBM.  The
// tape of a step is (alpha_t, delta_t) together with k_t, which the caller
// already holds from the verify pass.
//
// The rule is separable by rows: row i of S needs only its own v_i and the
// shared k_t, q_t (delta_i = beta (v_i - alpha S_i . k_t)).  So rows are
// spread over lanes with no exchange between rows: 8 lanes per row, each
// holding 16 of its 128 columns (columns 4l + 32j, so every load of S is a
// full 128-byte row segment per 8 lanes), dot products finished by a 3-step
// butterfly inside the 8 lanes.  A 256-thread workgroup owns 32 rows of one
// (sequence, head); the step inputs (k, q, v, gates) are staged in LDS once.
//  1. gdn_record -- reads S_0 once, runs the T steps, writes o and the tape
//     delta, and optionally S_T; S_0 itself is left untouched.
//  2. gdn_commit -- reads S_0 once, applies the first n[b] rank-1 updates
//     from the tape, writes the committed state in place.
//  3. gdn_commit_record -- both at a cycle boundary: commits the previous
//     cycle's tape in place and records the next verify block from the
//     committed rows, so the state crosses HBM once each way instead of
//     three times (commit read and write, then the capture's read).
// All apply the update through the same function, so committing n steps
// reproduces bitwise the state the recording reached after n steps.
#include "spec_internal.h"

#include <type_traits>

namespace spec {
namespace {

constexpr int kD = 128;            // dk = dv
constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 8;   // 32 rows per workgroup
constexpr int kBlocksPerHead = kD / kRowsPerBlock;
constexpr int kMaxT = 16;

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Workgroups are dealt to the 8 XCDs in turn (workgroup w on XCD w % 8).
// The four row blocks of a head read the same k and q, so they are placed
// on one XCD (w, w + 8, w + 16, w + 24) where its L2 serves the repeats.
static_assert(kBlocksPerHead == 4, "head_block deals four row blocks per head");
struct HeadBlock {
    int bh;     // (sequence, head); >= B * H means an idle padding workgroup
    int row0;   // first of the block's 32 rows
};
__device__ __forceinline__ HeadBlock head_block(int w) {
    const int grp = w >> 3;
    return HeadBlock{(grp >> 2) * 8 + (w & 7), (grp & 3) * kRowsPerBlock};
}

__device__ __forceinline__ float4 load_once4(const float *p) {
    const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

// The state update of one element: S <- alpha * S + delta * k, the product
// rounded first, then one fused multiply-add.  Shared by both kernels.
__device__ __forceinline__ float gdn_update(float s, float alpha, float delta, float k) {
    return fmaf(alpha, s, __fmul_rn(delta, k));
}

__device__ __forceinline__ float dot4(const float4 &s, const float4 &x) {
    return fmaf(s.x, x.x, fmaf(s.y, x.y, fmaf(s.z, x.z, __fmul_rn(s.w, x.w))));
}

// Sum over the 8 lanes of a row: swap neighbours, then pairs, then the two
// quads (half-row mirror).  Every lane adds the same two values at each
// step, so all 8 end with the same bits.
// (Every lane is a valid source for these patterns, so the moves are free to
// fold into the adds as DPP operands.)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row8_sum(float x) {
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    x += dpp_f<0x141>(x);
    return x;
}

// Step inputs of a capture of TT steps (TT is a template argument so the
// step loop unrolls fully: no loop-carried register copies of the state).
template <int TT>
struct RecordShared {
    static constexpr int N = TT > 0 ? TT : 1;
    float4 k[N][kD / 4];
    float4 q[N][kD / 4];
    float v[N][kRowsPerBlock];
    float alpha[N];
    float beta[N];
};

struct CommitShared {
    float4 k[kMaxT][kD / 4];
    float d[kMaxT][kRowsPerBlock];
    float alpha[kMaxT];
};

// The block's 32 state rows: lane l8 of row lr holds columns 4 l8 + 32 j.
__device__ __forceinline__ void load_rows(float4 S[4], const float *srow) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        S[j] = load_once4(srow + 32 * j);
}

__device__ __forceinline__ void store_rows(float *srow, const float4 S[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4 *>(srow + 32 * j) = S[j];
}

// Step inputs of the T positions of (b, h) for the block's rows, into LDS.
template <int TT>
__device__ __forceinline__ void stage_record(RecordShared<TT> &sh, const float *q, const float *k,
                                             const float *v, const float *alpha,
                                             const float *beta, int b, int h, int T, int H,
                                             int row0, int t) {
    for (int i = t; i < T * (kD / 4); i += kThreads) {
        const int s = i / (kD / 4), c4 = i - s * (kD / 4);
        const size_t bth = ((size_t)b * T + s) * H + h;
        sh.k[s][c4] = reinterpret_cast<const float4 *>(k + bth * kD)[c4];
        sh.q[s][c4] = reinterpret_cast<const float4 *>(q + bth * kD)[c4];
    }
    for (int i = t; i < T * kRowsPerBlock; i += kThreads) {
        const int s = i / kRowsPerBlock, r = i - s * kRowsPerBlock;
        sh.v[s][r] = v[(((size_t)b * T + s) * H + h) * kD + row0 + r];
    }
    if (t < T) {
        const size_t bth = ((size_t)b * T + t) * H + h;
        sh.alpha[t] = alpha[bth];
        sh.beta[t] = beta[bth];
    }
}

// The first n tape entries of (b, h) (a tape of T positions) for the block's
// rows, into LDS.
__device__ __forceinline__ void stage_commit(CommitShared &sh, const float *alpha,
                                             const float *k, const float *delta, int b, int h,
                                             int n, int T, int H, int row0, int t) {
    for (int i = t; i < n * (kD / 4); i += kThreads) {
        const int s = i / (kD / 4), c4 = i - s * (kD / 4);
        sh.k[s][c4] = reinterpret_cast<const float4 *>(k + (((size_t)b * T + s) * H + h) * kD)[c4];
    }
    for (int i = t; i < n * kRowsPerBlock; i += kThreads) {
        const int s = i / kRowsPerBlock, r = i - s * kRowsPerBlock;
        sh.d[s][r] = delta[(((size_t)b * T + s) * H + h) * kD + row0 + r];
    }
    if (t < n)
        sh.alpha[t] = alpha[((size_t)b * T + t) * H + h];
}

// T steps of the rule on the registers S (row lr, lane l8), writing o_t and
// the innovation delta_t of the row (lane 0 of the row).
template <int TT>
__device__ __forceinline__ void record_steps(float4 S[4], const RecordShared<TT> &sh, int H,
                                             int b, int h, int row, int lr, int l8,
                                             float *__restrict__ o, float *__restrict__ delta) {
    constexpr int T = TT;
#pragma unroll
    for (int s = 0; s < T; ++s) {
        const float a = sh.alpha[s], be = sh.beta[s];
        float4 k4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            k4[j] = sh.k[s][l8 + 8 * j];
        // u_i = S_{t-1}[i] . k_t (two independent chains, then the row sum)
        float u = (dot4(S[0], k4[0]) + dot4(S[2], k4[2])) + (dot4(S[1], k4[1]) + dot4(S[3], k4[3]));
        u = row8_sum(u);
        const float d = be * (sh.v[s][lr] - a * u);
        const size_t off = (((size_t)b * T + s) * H + h) * kD + row;
        if (l8 == 0)
            delta[off] = d;
        // S_t[i] = alpha S_{t-1}[i] + delta_i k_t
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            S[j].x = gdn_update(S[j].x, a, d, k4[j].x);
            S[j].y = gdn_update(S[j].y, a, d, k4[j].y);
            S[j].z = gdn_update(S[j].z, a, d, k4[j].z);
            S[j].w = gdn_update(S[j].w, a, d, k4[j].w);
        }
        // o_t[i] = S_t[i] . q_t
        float ov = (dot4(S[0], sh.q[s][l8]) + dot4(S[2], sh.q[s][l8 + 16])) +
                   (dot4(S[1], sh.q[s][l8 + 8]) + dot4(S[3], sh.q[s][l8 + 24]));
        ov = row8_sum(ov);
        if (l8 == 0)
            o[off] = ov;
    }
}

// The n staged tape steps applied to the registers S.
__device__ __forceinline__ void commit_steps(float4 S[4], const CommitShared &sh, int n, int lr,
                                             int l8) {
    for (int s = 0; s < n; ++s) {
        const float a = sh.alpha[s], d = sh.d[s][lr];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 k4 = sh.k[s][l8 + 8 * j];
            S[j].x = gdn_update(S[j].x, a, d, k4.x);
            S[j].y = gdn_update(S[j].y, a, d, k4.y);
            S[j].z = gdn_update(S[j].z, a, d, k4.z);
            S[j].w = gdn_update(S[j].w, a, d, k4.w);
        }
    }
}

template <int TT>
__global__ __launch_bounds__(kThreads) void gdn_record_kernel(
    const float *__restrict__ S0, const float *__restrict__ q, const float *__restrict__ k,
    const float *__restrict__ v, const float *__restrict__ alpha, const float *__restrict__ beta,
    int H, int n_heads, float *__restrict__ o, float *__restrict__ delta,
    float *__restrict__ S_final) {
    constexpr int T = TT;
    __shared__ RecordShared<TT> sh;
    const HeadBlock hb = head_block(blockIdx.x);
    if (hb.bh >= n_heads)
        return;
    const int bh = hb.bh, row0 = hb.row0;
    const int b = bh / H, h = bh - b * H;
    const int t = threadIdx.x;
    const int lr = t >> 3, l8 = t & 7;       // row within the block, lane within the row
    const int row = row0 + lr;

    // the state rows first (the long HBM reads), then the step inputs
    float4 S[4];
    load_rows(S, S0 + ((size_t)bh * kD + row) * kD + 4 * l8);
    stage_record(sh, q, k, v, alpha, beta, b, h, T, H, row0, t);
    __syncthreads();
    record_steps<TT>(S, sh, H, b, h, row, lr, l8, o, delta);
    if (S_final)
        store_rows(S_final + ((size_t)bh * kD + row) * kD + 4 * l8, S);
}

__global__ __launch_bounds__(kThreads) void gdn_commit_kernel(
    float *__restrict__ S, const float *__restrict__ alpha, const float *__restrict__ k,
    const float *__restrict__ delta, const int32_t *__restrict__ n_steps, int T, int H,
    int n_heads) {
    __shared__ CommitShared sh;
    const HeadBlock hb = head_block(blockIdx.x);
    if (hb.bh >= n_heads)
        return;
    const int bh = hb.bh, row0 = hb.row0;
    const int b = bh / H, h = bh - b * H;
    const int n = min(n_steps[b], T);
    if (n <= 0)
        return;   // nothing accepted: the state stays as it is
    const int t = threadIdx.x;
    const int lr = t >> 3, l8 = t & 7;
    const int row = row0 + lr;
    float *srow = S + ((size_t)bh * kD + row) * kD + 4 * l8;
    float4 st[4];
    load_rows(st, srow);
    stage_commit(sh, alpha, k, delta, b, h, n, T, H, row0, t);
    __syncthreads();
    commit_steps(st, sh, n, lr, l8);
    store_rows(srow, st);
}

// One cycle boundary in one pass over the state: the commit of the previous
// cycle's accepted steps (tape of Tp positions), written back in place, then
// the capture of the next T verify positions from the committed rows still
// in registers.  The same staging and step functions as the two kernels
// above, in the same order, so the results are theirs bit for bit.
template <int TT>
struct CycleShared {
    CommitShared c;
    RecordShared<TT> r;
};

template <int TT>
__global__ __launch_bounds__(kThreads) void gdn_commit_record_kernel(
    float *__restrict__ S, const float *__restrict__ prev_alpha,
    const float *__restrict__ prev_k, const float *__restrict__ prev_delta,
    const int32_t *__restrict__ n_steps, int Tp, const float *__restrict__ q,
    const float *__restrict__ k, const float *__restrict__ v, const float *__restrict__ alpha,
    const float *__restrict__ beta, int H, int n_heads, float *__restrict__ o,
    float *__restrict__ delta, float *__restrict__ S_final) {
    constexpr int T = TT;
    __shared__ CycleShared<TT> sh;
    const HeadBlock hb = head_block(blockIdx.x);
    if (hb.bh >= n_heads)
        return;
    const int bh = hb.bh, row0 = hb.row0;
    const int b = bh / H, h = bh - b * H;
    const int n = Tp > 0 ? min(n_steps[b], Tp) : 0;
    const int t = threadIdx.x;
    const int lr = t >> 3, l8 = t & 7;
    const int row = row0 + lr;
    float *srow = S + ((size_t)bh * kD + row) * kD + 4 * l8;
    float4 st[4];
    load_rows(st, srow);
    if (n > 0)
        stage_commit(sh.c, prev_alpha, prev_k, prev_delta, b, h, n, Tp, H, row0, t);
    stage_record(sh.r, q, k, v, alpha, beta, b, h, T, H, row0, t);
    __syncthreads();
    if (n > 0) {
        commit_steps(st, sh.c, n, lr, l8);
        store_rows(srow, st);
    }
    record_steps<TT>(st, sh.r, H, b, h, row, lr, l8, o, delta);
    if (S_final)
        store_rows(S_final + ((size_t)bh * kD + row) * kD + 4 * l8, st);
}

// Calls f(std::integral_constant<int, T>) for 0 <= T <= kMaxT (the kernels'
// step count is a template argument), then reports the launch status.
template <int TT = 0, class F>
hipError_t with_steps(int T, F &&f) {
    if constexpr (TT > kMaxT) {
        return hipErrorInvalidValue;
    } else {
        if (T == TT) {
            f(std::integral_constant<int, TT>{});
            return hipGetLastError();
        }
        return with_steps<TT + 1>(T, f);
    }
}

} // namespace

hipError_t launch_gdn_record(const float *S0, const float *q, const float *k, const float *v,
                             const float *alpha, const float *beta, int B, int T, int H,
                             float *o, float *delta, float *S_final, hipStream_t stream) {
    if (B == 0 || H == 0 || (T == 0 && !S_final))
        return hipSuccess;
    const int groups = (B * H + 7) / 8;   // 8 heads per group of 32 workgroups
    return with_steps(T, [&](auto tt) {
        gdn_record_kernel<decltype(tt)::value><<<groups * 8 * kBlocksPerHead, kThreads, 0, stream>>>(
            S0, q, k, v, alpha, beta, H, B * H, o, delta, S_final);
    });
}

hipError_t launch_gdn_commit(float *S, const float *alpha, const float *k, const float *delta,
                             const int32_t *n_steps, int B, int T, int H, hipStream_t stream) {
    if (B == 0 || H == 0 || T == 0)
        return hipSuccess;
    const int groups = (B * H + 7) / 8;
    gdn_commit_kernel<<<groups * 8 * kBlocksPerHead, kThreads, 0, stream>>>(
        S, alpha, k, delta, n_steps, T, H, B * H);
    return hipGetLastError();
}

hipError_t launch_gdn_commit_record(float *S, const float *prev_alpha, const float *prev_k,
                                    const float *prev_delta, const int32_t *n_steps, int Tp,
                                    const float *q, const float *k, const float *v,
                                    const float *alpha, const float *beta, int B, int T, int H,
                                    float *o, float *delta, float *S_final, hipStream_t stream) {
    if (B == 0 || H == 0 || (Tp == 0 && T == 0 && !S_final))
        return hipSuccess;
    const int groups = (B * H + 7) / 8;
    return with_steps(T, [&](auto tt) {
        gdn_commit_record_kernel<decltype(tt)::value>
            <<<groups * 8 * kBlocksPerHead, kThreads, 0, stream>>>(
                S, prev_alpha, prev_k, prev_delta, n_steps, Tp, q, k, v, alpha, beta, H, B * H, o,
                delta, S_final);
    });
}

} // namespace spec
