// C ABI of libspec: host-side validation, then kernel launches.  Every
// argument check runs before anything is enqueued.  Declarations and the
// meaning of every argument: include/spec.h.
#include "../../include/spec.h"
#include "spec_internal.h"

#include <climits>
#include <cmath>
#include <mutex>

namespace {

constexpr int kMaxM = 16;
constexpr int kMaxValuM = 4;     // rows of the vector-ALU comparison variant
constexpr int kMaxD = 15;
constexpr int kMaxCand = 256;
constexpr int kMaxV = (1 << 24) - 1;
constexpr size_t kMaxRows = (size_t)1 << 23;  // grid x of 256-thread workgroups

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// A byte range of an argument; empty when the pointer is null or the size 0.
struct Span {
    const void *p;
    size_t bytes;
};
bool disjoint(const Span &a, const Span &b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0)
        return true;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 + a.bytes <= b0 || b0 + b.bytes <= a0;
}

spec_status qmv_shape_ok(int N, int K, int G) {
    if (N < 0 || K < 0 || G <= 0 || K % G != 0)
        return SPEC_ERR_INVALID;
    if (G != 64)
        return SPEC_ERR_UNSUPPORTED;
    // Buffer ranges and offsets inside the kernels are 32-bit: with K below
    // 2^24 a packed tile (K/128 pairs of up to 2 KB), sixteen interchange rows
    // (16 K bytes at W8) and x (16 rows of 2 K bytes) all stay below 2^29.
    if (K >= (1 << 24) || N > (1 << 28))
        return SPEC_ERR_UNSUPPORTED;
    return SPEC_OK;
}

spec_status pack_common(int bits, const void *w, const uint16_t *scales,
                        const uint16_t *biases, int N, int K, int G,
                        void *w_packed, void *sb_packed, hipStream_t stream) {
    const spec_status s = qmv_shape_ok(N, K, G);
    if (s != SPEC_OK)
        return s;
    if (N == 0 || K == 0)
        return SPEC_OK;
    if (!w || !scales || !biases || !w_packed || !sb_packed)
        return SPEC_ERR_INVALID;
    if (!aligned16(w) || !aligned16(w_packed) || !aligned4(sb_packed))
        return SPEC_ERR_UNSUPPORTED;
    if (spec::launch_pack(bits, w, scales, biases, nullptr, nullptr, nullptr, N, K, w_packed,
                          sb_packed, stream) != hipSuccess)
        return SPEC_ERR_DEVICE;
    return SPEC_OK;
}

spec_status qmv_common(int bits, bool interchange, const void *w, const void *sb,
                       const uint16_t *biases, const uint16_t *x, float *y, int M, int N,
                       int K, int G, hipStream_t stream) {
    if (M < 0)
        return SPEC_ERR_INVALID;
    const spec_status s = qmv_shape_ok(N, K, G);
    if (s != SPEC_OK)
        return s;
    if (M > kMaxM)
        return SPEC_ERR_UNSUPPORTED;
    if (M == 0 || N == 0)
        return SPEC_OK;
    if (!y || (K > 0 && (!w || !sb || !x || (interchange && !biases))))
        return SPEC_ERR_INVALID;
    if (K > 0 && (!aligned16(w) || !aligned16(x)))
        return SPEC_ERR_UNSUPPORTED;
    if (K > 0 && !interchange && !aligned4(sb))
        return SPEC_ERR_UNSUPPORTED;
    if (K > 0 && interchange &&
        ((reinterpret_cast<uintptr_t>(sb) | reinterpret_cast<uintptr_t>(biases)) & 1u))
        return SPEC_ERR_INVALID;
    if (!aligned4(y))
        return SPEC_ERR_INVALID;
    if (spec::launch_qmv(bits, interchange, w, sb, biases, x, y, M, N, K, stream) != hipSuccess)
        return SPEC_ERR_DEVICE;
    return SPEC_OK;
}

// Shared checks of the sampling settings.
spec_status check_sampling(int V, float temperature, int top_k, float top_p) {
    if (V < 2 || V > kMaxV)
        return V < 2 ? SPEC_ERR_INVALID : SPEC_ERR_UNSUPPORTED;
    if (!std::isfinite(temperature) || std::isnan(top_p))
        return SPEC_ERR_INVALID;
    const spec::SamplingParams sp = spec::sampling_params(temperature, top_k, top_p, V);
    if (sp.candidates && sp.k_eff > kMaxCand)
        return SPEC_ERR_UNSUPPORTED;
    return SPEC_OK;
}

bool ws_ok(const void *ws, size_t have, size_t need) {
    return need == 0 || (ws && have >= need && (reinterpret_cast<uintptr_t>(ws) & 255u) == 0);
}

// Workspace of spec_verify_accept_noalloc: a fixed array in device memory,
// one copy per GPU (each GPU that loads the library holds it until the
// process ends), shared by every such call on that GPU.  Host code never
// passes the name itself to a kernel or a copy: the per-device address from
// hipGetSymbolAddress is used instead.
static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the stream's device, looked up once per
// device (with that device current) and kept.
spec_status scratch_ptr(hipStream_t stream, void **out) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess)
        return SPEC_ERR_DEVICE;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess)
            return SPEC_ERR_DEVICE;
        if (sdev != cur)
            return SPEC_ERR_INVALID;     // the stream must belong to the current device
    }
    if (cur < 0 || cur >= kMaxDevices)
        return SPEC_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[cur]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return SPEC_ERR_DEVICE;
        g_scratch_ptr[cur] = p;
    }
    *out = g_scratch_ptr[cur];
    return SPEC_OK;
}

// spec_verify_accept with a caller workspace, or (fixed_scratch) with the
// library's scratch array.
spec_status verify_accept_common(const float *target_logits, const float *draft_logits,
                                 const int32_t *draft_tokens, const float *uniforms, int B,
                                 int D, int V, float temperature, int top_k, float top_p,
                                 int32_t *accepted_len, int32_t *next_token, float *p_draft,
                                 float *q_draft, void *workspace, size_t workspace_bytes,
                                 bool fixed_scratch, hipStream_t stream) {
    if (B < 0 || D < 0)
        return SPEC_ERR_INVALID;
    if (D > kMaxD)
        return SPEC_ERR_UNSUPPORTED;
    const spec_status s = check_sampling(V, temperature, top_k, top_p);
    if (s != SPEC_OK)
        return s;
    if (B == 0)
        return SPEC_OK;
    if (!target_logits || !uniforms || !accepted_len || !next_token)
        return SPEC_ERR_INVALID;
    if (D > 0 && (!draft_logits || !draft_tokens))
        return SPEC_ERR_INVALID;
    if (!aligned4(target_logits) || (D > 0 && !aligned4(draft_logits)))
        return SPEC_ERR_INVALID;
    if (((V & 3) == 0) && (!aligned16(target_logits) || (D > 0 && !aligned16(draft_logits))))
        return SPEC_ERR_UNSUPPORTED;
    if ((size_t)B * (2 * D + 1) > kMaxRows)
        return SPEC_ERR_UNSUPPORTED;
    const spec::SamplingParams sp = spec::sampling_params(temperature, top_k, top_p, V);
    const spec::AcceptPlan plan = spec::accept_plan(B, D, V, sp.k_eff, sp.candidates);
    if (fixed_scratch) {
        if (plan.ws_bytes > SPEC_NOALLOC_SCRATCH_BYTES)
            return SPEC_ERR_WORKSPACE;
        const spec_status ps = scratch_ptr(stream, &workspace);
        if (ps != SPEC_OK)
            return ps;
    } else if (!ws_ok(workspace, workspace_bytes, plan.ws_bytes)) {
        return SPEC_ERR_WORKSPACE;
    }
    if (spec::launch_accept(target_logits, draft_logits, draft_tokens, uniforms,
                            plan, sp, accepted_len, next_token, p_draft,
                            q_draft, workspace, stream) != hipSuccess)
        return SPEC_ERR_DEVICE;
    return SPEC_OK;
}

} // namespace

extern "C" {

const char *spec_status_str(spec_status s) {
    switch (s) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_ERR_INVALID: return "SPEC_ERR_INVALID";
    case SPEC_ERR_UNSUPPORTED: return "SPEC_ERR_UNSUPPORTED";
    case SPEC_ERR_WORKSPACE: return "SPEC_ERR_WORKSPACE";
    case SPEC_ERR_DEVICE: return "SPEC_ERR_DEVICE";
    }
    return "SPEC_ERR_UNKNOWN";
}

int spec_version(void) { return 100; }

size_t spec_qmv_packed_weight_bytes(int bits, int N, int K, int G) {
    if ((bits != 4 && bits != 8) || qmv_shape_ok(N, K, G) != SPEC_OK)
        return 0;
    return spec::qmv_packed_bytes(bits, N, K);
}

size_t spec_qmv_packed_sb_bytes(int N, int K, int G) {
    if (qmv_shape_ok(N, K, G) != SPEC_OK)
        return 0;
    return spec::qmv_packed_sb_bytes(N, K);
}

spec_status spec_pack_w4(const uint32_t *w, const uint16_t *scales,
                         const uint16_t *biases, int N, int K, int G,
                         void *w_packed, void *sb_packed, hipStream_t stream) {
    if (K % 8 != 0)
        return SPEC_ERR_INVALID;
    return pack_common(4, w, scales, biases, N, K, G, w_packed, sb_packed, stream);
}

spec_status spec_pack_w8(const uint8_t *w, const uint16_t *scales,
                         const uint16_t *biases, int N, int K, int G,
                         void *w_packed, void *sb_packed, hipStream_t stream) {
    return pack_common(8, w, scales, biases, N, K, G, w_packed, sb_packed, stream);
}

spec_status spec_qmv_w4(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                        const uint16_t *x, float *y, int M, int N, int K, int G,
                        hipStream_t stream) {
    return qmv_common(4, true, w, scales, biases, x, y, M, N, K, G, stream);
}

spec_status spec_qmv_w8(const uint8_t *w, const uint16_t *scales, const uint16_t *biases,
                        const uint16_t *x, float *y, int M, int N, int K, int G,
                        hipStream_t stream) {
    return qmv_common(8, true, w, scales, biases, x, y, M, N, K, G, stream);
}

spec_status spec_qmv_w4_packed(const void *w_packed, const void *sb_packed,
                               const uint16_t *x, float *y, int M, int N, int K, int G,
                               hipStream_t stream) {
    return qmv_common(4, false, w_packed, sb_packed, nullptr, x, y, M, N, K, G, stream);
}

spec_status spec_qmv_w8_packed(const void *w_packed, const void *sb_packed,
                               const uint16_t *x, float *y, int M, int N, int K, int G,
                               hipStream_t stream) {
    return qmv_common(8, false, w_packed, sb_packed, nullptr, x, y, M, N, K, G, stream);
}

spec_status spec_qmv_w4_packed_valu(const void *w_packed, const void *sb_packed,
                                    const uint16_t *x, float *y, int M, int N, int K, int G,
                                    hipStream_t stream) {
    if (M < 0)
        return SPEC_ERR_INVALID;
    const spec_status s = qmv_shape_ok(N, K, G);
    if (s != SPEC_OK)
        return s;
    if (M > kMaxValuM)
        return SPEC_ERR_UNSUPPORTED;
    if (M == 0 || N == 0)
        return SPEC_OK;
    if (!y || (K > 0 && (!w_packed || !sb_packed || !x)))
        return SPEC_ERR_INVALID;
    if (K > 0 && (!aligned16(w_packed) || !aligned16(x) || !aligned4(sb_packed)))
        return SPEC_ERR_UNSUPPORTED;
    if (!aligned4(y))
        return SPEC_ERR_INVALID;
    if (spec::launch_qmv_valu(w_packed, sb_packed, x, y, M, N, K, 0, stream) != hipSuccess)
        return SPEC_ERR_DEVICE;
    return SPEC_OK;
}

spec_status spec_qmv_gate_up_silu_w4_valu(const void *w_packed, const void *sb_packed,
                                          const uint16_t *x, uint16_t *h, int M, int F, int K,
                                          int G, hipStream_t stream) {
    if (M < 0 || F < 0)
        return SPEC_ERR_INVALID;
    if (F > (1 << 27))
        return SPEC_ERR_UNSUPPORTED;
    const spec_status s = qmv_shape_ok(spec::gate_up_rows(F), K, G);
    if (s != SPEC_OK)
        return s;
    if (M > kMaxValuM)
        return SPEC_ERR_UNSUPPORTED;
    if (M == 0 || F == 0)
        return SPEC_OK;
    if (!h || (K > 0 && (!w_packed || !sb_packed || !x)))
        return SPEC_ERR_INVALID;
    if (K > 0 && (!aligned16(w_packed) || !aligned16(x) || !aligned4(sb_packed)))
        return SPEC_ERR_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(h) & 1u)
        return SPEC_ERR_INVALID;
    if (spec::launch_qmv_valu(w_packed, sb_packed, x, h, M, spec::gate_up_rows(F), K, F, stream) !=
        hipSuccess)
        return SPEC_ERR_DEVICE;
    return SPEC_OK;
}

spec_status spec_requantize_w4(const uint16_t *w_bf16, int N, int K, int G, uint32_t *w4,
                               uint16_t *scales, uint16_t *biases, hipStream_t stream) {
    if (N < 0 || K < 0 || G <= 0 || K % G != 0)
        return SPEC_ERR_INVALID;
    if (G != 64)
        return SPEC_ERR_UNSUPPORTED;
    if (N == 0 || K == 0)
        return SPEC_OK;
    if (!w_bf16 || !w4 || !scales || !biases)
        return SPEC_ERR_INVALID;
    if (!aligned16(w_bf16) || !aligned16(w4))
        return SPEC_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(scales) | reinterpret_cast<uintptr_t>(biases)) & 1u)
        return SPEC_ERR_INVALID;
    if (spec::launch_requantize_w4(w_bf16, N, K, w4, scales, biases, stream) != hipSuccess)
        return SPEC_ERR_DEVICE;
    return SPEC_OK;
}

int spec_gate_up_packed_rows(int F) {
    if (F < 0 || F > (1 << 27))
        return 0;
    return spec::gate_up_rows(F);
}

spec_status spec_pack_gate_up(int bits, const void *gate_w, const uint16_t *gate_scales,
                              const uint16_t *gate_biases, const void *up_w,
                              const uint16_t *up_scales, const uint16_t *up_biases,
                              int F, int K, int G, void *w_packed, void *sb_packed,
                              hipStream_t stream) {
    if (bits != 4 && bits != 8)
        return SPEC_ERR_INVALID;
    if (bits == 4 && K % 8 != 0)
        return SPEC_ERR_INVALID;
    if (F < 0 || F > (1 << 27))
        return F < 0 ? SPEC_ERR_INVALID : SPEC_ERR_UNSUPPORTED;
    const spec_status s = qmv_shape_ok(spec::gate_up_rows(F), K, G);
    if (s != SPEC_OK)
        return s;
    if (F == 0 || K == 0)
        return SPEC_OK;
    if (!gate_w || !gate_scales || !gate_biases || !up_w || !up_scales || !up_biases ||
        !w_packed || !sb_packed)
        return SPEC_ERR_INVALID;
    if (!aligned16(gate_w) || !aligned16(up_w) || !aligned16(w_packed) || !aligned4(sb_packed))
        return SPEC_ERR_UNSUPPORTED;
    if (spec::launch_pack(bits, gate_w, gate_scales, gate_biases, up_w, up_scales, up_biases,
                          F, K, w_packed, sb_packed, stream) != hipSuccess)
        return SPEC_ERR_DEVICE;
    return SPEC_OK;
}

spec_status spec_qmv_gate_up_silu(int bits, const void *w_packed, const void *sb_packed,
                                  const uint16_t *x, uint16_t *h, int M, int F, int K,
                                  int G, hipStream_t stream) {
    if (bits != 4 && bits != 8)
        return SPEC_ERR_INVALID;
    if (M < 0 || F < 0)
        return SPEC_ERR_INVALID;
    if (F > (1 << 27))
        return SPEC_ERR_UNSUPPORTED;
    const spec_status s = qmv_shape_ok(spec::gate_up_rows(F), K, G);
    if (s != SPEC_OK)
        return s;
    if (M > kMaxM)
        return SPEC_ERR_UNSUPPORTED;
    if (M == 0 || F == 0)
        return SPEC_OK;
    if (!h || (K > 0 && (!w_packed || !sb_packed || !x)))
        return SPEC_ERR_INVALID;
    if (K > 0 && (!aligned16(w_packed) || !aligned16(x) || !aligned4(sb_packed)))
        return SPEC_ERR_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(h) & 1u)
        return SPEC_ERR_INVALID;
    if (spec::launch_qmv_gate_up_silu(bits, w_packed, sb_packed, x, h, M, F, K, stream) !=
        hipSuccess)
        return SPEC_ERR_DEVICE;
    return SPEC_OK;
}

size_t spec_verify_accept_workspace(int B, int D, int V, int top_k) {
    if (B <= 0 || D < 0 || D > kMaxD || V < 2 || V > kMaxV)
        return 0;
    // Size for the larger of the two modes, so any temperature / top_p works.
    const int k = (top_k >= 1 && top_k < V) ? top_k : 1;
    const int kc = std::min(std::max(k, 1), kMaxCand);
    const spec::AcceptPlan a = spec::accept_plan(B, D, V, kc, true);
    const spec::AcceptPlan f = spec::accept_plan(B, D, V, 0, false);
    const int kv = std::min(V, kMaxCand);  // top_p over a small full vocabulary
    const spec::AcceptPlan v = spec::accept_plan(B, D, V, kv, true);
    return std::max(a.ws_bytes, std::max(f.ws_bytes, V <= kMaxCand ? v.ws_bytes : 0));
}

spec_status spec_verify_accept(const float *target_logits,
                               const float *draft_logits,
                               const int32_t *draft_tokens,
                               const float *uniforms, int B, int D, int V,
                               float temperature, int top_k, float top_p,
                               int32_t *accepted_len, int32_t *next_token,
                               float *p_draft, float *q_draft, void *workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    return verify_accept_common(target_logits, draft_logits, draft_tokens, uniforms, B, D, V,
                                temperature, top_k, top_p, accepted_len, next_token, p_draft,
                                q_draft, workspace, workspace_bytes, false, stream);
}

spec_status spec_verify_accept_noalloc(const float *target_logits,
                                       const float *draft_logits,
                                       const int32_t *draft_tokens,
                                       const float *uniforms, int B, int D, int V,
                                       float temperature, int top_k, float top_p,
                                       int32_t *accepted_len, int32_t *next_token,
                                       float *p_draft, float *q_draft, hipStream_t stream) {
    return verify_accept_common(target_logits, draft_logits, draft_tokens, uniforms, B, D, V,
                                temperature, top_k, top_p, accepted_len, next_token, p_draft,
                                q_draft, nullptr, 0, true, stream);
}

size_t spec_sample_workspace_size(int R, int V, int top_k) {
    return spec_verify_accept_workspace(R, 0, V, top_k);
}

spec_status spec_sample_probs(const float *logits, int R, int V,
                              float temperature, int top_k, float top_p,
                              float *probs, void *workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    if (R < 0)
        return SPEC_ERR_INVALID;
    const spec_status s = check_sampling(V, temperature, top_k, top_p);
    if (s != SPEC_OK)
        return s;
    if (R == 0)
        return SPEC_OK;
    if ((size_t)R > kMaxRows)
        return SPEC_ERR_UNSUPPORTED;
    if (!logits || !probs || !aligned4(logits) || !aligned4(probs))
        return SPEC_ERR_INVALID;
    if (((V & 3) == 0) && !aligned16(logits))
        return SPEC_ERR_UNSUPPORTED;
    const spec::SamplingParams sp = spec::sampling_params(temperature, top_k, top_p, V);
    const spec::AcceptPlan plan = spec::accept_plan(R, 0, V, sp.k_eff, sp.candidates);
    if (!ws_ok(workspace, workspace_bytes, plan.ws_bytes))
        return SPEC_ERR_WORKSPACE;
    if (spec::launch_probs(logits, plan, sp, probs, workspace, stream) != hipSuccess)
        return SPEC_ERR_DEVICE;
    return SPEC_OK;
}

spec_status spec_sample_tokens(const float *logits, int R, int V,
                               float temperature, int top_k, float top_p,
                               const float *uniforms, int32_t *tokens,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    if (R < 0)
        return SPEC_ERR_INVALID;
    const spec_status s = check_sampling(V, temperature, top_k, top_p);
    if (s != SPEC_OK)
        return s;
    if (R == 0)
        return SPEC_OK;
    if ((size_t)R > kMaxRows)
        return SPEC_ERR_UNSUPPORTED;
    if (!logits || !uniforms || !tokens || !aligned4(logits))
        return SPEC_ERR_INVALID;
    if (((V & 3) == 0) && !aligned16(logits))
        return SPEC_ERR_UNSUPPORTED;
    const spec::SamplingParams sp = spec::sampling_params(temperature, top_k, top_p, V);
    const spec::AcceptPlan plan = spec::accept_plan(R, 0, V, sp.k_eff, sp.candidates);
    if (!ws_ok(workspace, workspace_bytes, plan.ws_bytes))
        return SPEC_ERR_WORKSPACE;
    // D = 0: every sequence is one target row and takes the bonus draw.
    if (spec::launch_accept(logits, nullptr, nullptr, uniforms, plan, sp,
                            nullptr, tokens, nullptr, nullptr, workspace,
                            stream) != hipSuccess)
        return SPEC_ERR_DEVICE;
    return SPEC_OK;
}

size_t spec_verify_greedy_workspace(int B, int D, int V) {
    if (B <= 0 || D < 0 || D > kMaxD || V < 2 || V > kMaxV)
        return 0;
    return spec::greedy_plan(B, D, V).ws_bytes;
}

spec_status spec_verify_greedy(const float *target_logits,
                               const int32_t *draft_tokens, int B, int D, int V,
                               int32_t *accepted_len, int32_t *next_token,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    if (B < 0 || D < 0 || V < 2)
        return SPEC_ERR_INVALID;
    if (D > kMaxD || V > kMaxV)
        return SPEC_ERR_UNSUPPORTED;
    if (B == 0)
        return SPEC_OK;
    if (!target_logits || !accepted_len || !next_token || (D > 0 && !draft_tokens))
        return SPEC_ERR_INVALID;
    if (!aligned4(target_logits))
        return SPEC_ERR_INVALID;
    if (((V & 3) == 0) && !aligned16(target_logits))
        return SPEC_ERR_UNSUPPORTED;
    if ((size_t)B * (D + 1) > kMaxRows)
        return SPEC_ERR_UNSUPPORTED;
    const spec::GreedyPlan plan = spec::greedy_plan(B, D, V);
    if (!ws_ok(workspace, workspace_bytes, plan.ws_bytes))
        return SPEC_ERR_WORKSPACE;
    if (spec::launch_greedy(target_logits, draft_tokens, plan, accepted_len,
                            next_token, workspace, stream) != hipSuccess)
        return SPEC_ERR_DEVICE;
    return SPEC_OK;
}

spec_status spec_gdn_record(const float *S0, const float *q, const float *k, const float *v,
                            const float *alpha, const float *beta, int B, int T, int H,
                            int dk, int dv, float *o, float *delta, float *S_final,
                            hipStream_t stream) {
    if (B < 0 || T < 0 || H < 0 || dk < 1 || dv < 1)
        return SPEC_ERR_INVALID;
    if (dk != 128 || dv != 128 || T > kMaxD + 1 || (int64_t)B * H >= (1 << 28))
        return SPEC_ERR_UNSUPPORTED;
    if (B == 0 || H == 0)
        return SPEC_OK;
    if (!S0 || (T > 0 && (!q || !k || !v || !alpha || !beta || !o || !delta)))
        return SPEC_ERR_INVALID;
    if (!aligned16(S0) || (S_final && !aligned16(S_final)) ||
        (T > 0 && (!aligned16(q) || !aligned16(k))))
        return SPEC_ERR_UNSUPPORTED;
    if (T > 0 && (!aligned4(v) || !aligned4(alpha) || !aligned4(beta) || !aligned4(o) ||
                  !aligned4(delta)))
        return SPEC_ERR_INVALID;
    if (spec::launch_gdn_record(S0, q, k, v, alpha, beta, B, T, H, o, delta, S_final, stream) !=
        hipSuccess)
        return SPEC_ERR_DEVICE;
    return SPEC_OK;
}

spec_status spec_gdn_commit(float *S, const float *alpha, const float *k, const float *delta,
                            const int32_t *n_steps, int B, int T, int H, int dk, int dv,
                            hipStream_t stream) {
    if (B < 0 || T < 0 || H < 0 || dk < 1 || dv < 1)
        return SPEC_ERR_INVALID;
    if (dk != 128 || dv != 128 || T > kMaxD + 1 || (int64_t)B * H >= (1 << 28))
        return SPEC_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || T == 0)
        return SPEC_OK;
    if (!S || !alpha || !k || !delta || !n_steps)
        return SPEC_ERR_INVALID;
    if (!aligned16(S) || !aligned16(k))
        return SPEC_ERR_UNSUPPORTED;
    if (!aligned4(alpha) || !aligned4(delta) || !aligned4(n_steps))
        return SPEC_ERR_INVALID;
    if (spec::launch_gdn_commit(S, alpha, k, delta, n_steps, B, T, H, stream) != hipSuccess)
        return SPEC_ERR_DEVICE;
    return SPEC_OK;
}

spec_status spec_gdn_commit_record(float *S, const float *prev_alpha, const float *prev_k,
                                   const float *prev_delta, const int32_t *n_steps, int T_prev,
                                   const float *q, const float *k, const float *v,
                                   const float *alpha, const float *beta, int B, int T, int H,
                                   int dk, int dv, float *o, float *delta, float *S_final,
                                   hipStream_t stream) {
    if (B < 0 || T_prev < 0 || T < 0 || H < 0 || dk < 1 || dv < 1)
        return SPEC_ERR_INVALID;
    if (dk != 128 || dv != 128 || T_prev > kMaxD + 1 || T > kMaxD + 1 ||
        (int64_t)B * H >= (1 << 28))
        return SPEC_ERR_UNSUPPORTED;
    if (B == 0 || H == 0)
        return SPEC_OK;
    if (!S || (T_prev > 0 && (!prev_alpha || !prev_k || !prev_delta || !n_steps)) ||
        (T > 0 && (!q || !k || !v || !alpha || !beta || !o || !delta)))
        return SPEC_ERR_INVALID;
    if (!aligned16(S) || (S_final && !aligned16(S_final)) ||
        (T_prev > 0 && !aligned16(prev_k)) || (T > 0 && (!aligned16(q) || !aligned16(k))))
        return SPEC_ERR_UNSUPPORTED;
    if ((T_prev > 0 && (!aligned4(prev_alpha) || !aligned4(prev_delta) || !aligned4(n_steps))) ||
        (T > 0 && (!aligned4(v) || !aligned4(alpha) || !aligned4(beta) || !aligned4(o) ||
                   !aligned4(delta))))
        return SPEC_ERR_INVALID;
    // Workgroups of one head write what those of another read: no output may
    // share memory with any other argument (the two tapes are separate).
    const size_t heads = (size_t)B * H, f = sizeof(float);
    const size_t state = heads * 128 * 128 * f;
    const size_t tp = T_prev > 0 ? heads * T_prev : 0, tn = T > 0 ? heads * T : 0;
    const Span outs[] = {{S, state}, {o, tn * 128 * f}, {delta, tn * 128 * f}, {S_final, state}};
    const Span ins[] = {{prev_alpha, tp * f}, {prev_k, tp * 128 * f}, {prev_delta, tp * 128 * f},
                        {T_prev > 0 ? n_steps : nullptr, (size_t)B * sizeof(int32_t)},
                        {q, tn * 128 * f}, {k, tn * 128 * f}, {v, tn * 128 * f},
                        {alpha, tn * f}, {beta, tn * f}};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
            if (!disjoint(outs[i], outs[j]))
                return SPEC_ERR_INVALID;
        for (const Span &in : ins)
            if (!disjoint(outs[i], in))
                return SPEC_ERR_INVALID;
    }
    if (spec::launch_gdn_commit_record(S, prev_alpha, prev_k, prev_delta, n_steps, T_prev, q, k,
                                       v, alpha, beta, B, T, H, o, delta, S_final,
                                       stream) != hipSuccess)
        return SPEC_ERR_DEVICE;
    return SPEC_OK;
}

spec_status spec_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream) {
    if (bytes % 16 != 0 || !sink || !aligned4(sink) || (bytes > 0 && !src))
        return SPEC_ERR_INVALID;
    if (bytes > 0 && !aligned16(src))
        return SPEC_ERR_UNSUPPORTED;
    if (spec::launch_stream_read(src, bytes, sink, SPEC_STREAM_READ_GROUPS, stream) != hipSuccess)
        return SPEC_ERR_DEVICE;
    return SPEC_OK;
}

} // extern "C"
