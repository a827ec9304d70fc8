"""Python binding of libspec, the MI355X (gfx950) speculative-decoding hot path.

Argument marshalling only: every function hands device pointers, sizes and
torch's current HIP stream to the C ABI declared in ``include/spec.h`` and
raises :class:`SpecError` on a non-OK status.  All arithmetic runs in the HIP
kernels; there is no CPU fallback, and calling any function without the
built library (``libspec.so`` next to this file) raises immediately.

Names follow the C ABI:

    spec_qmv_w4 / spec_qmv_w8        small-M group-quantized verify qmv on the
                                     weights as stored (w, scales, biases)
    spec_pack_w4 / spec_pack_w8      one-time repack of quantized weights into
                                     the order the kernel streams
    spec_qmv_w4_packed /             the same product from the repacked copy
    spec_qmv_w8_packed               (the faster form)
    spec_requantize_w4               draft-only 4-bit copy of a bf16 matrix
    spec_pack_gate_up /              gate and up projections as one launch with
    spec_qmv_gate_up_silu            the SiLU-gated activation applied (bf16 out)
    spec_qmv_w4_packed_valu /        the W4 products with the multiply-accumulate
    spec_qmv_gate_up_silu_w4_valu    on the vector ALU instead of the matrix
                                     cores (M <= 4; the comparison variant)
    spec_verify_accept               ratio acceptance + residual / bonus draw
    spec_verify_accept_noalloc       the same with the library's fixed device
                                     scratch instead of a workspace
    spec_sample_probs                filtered sampling distribution
    spec_sample_tokens               inverse-CDF draw from that distribution
    spec_verify_greedy               greedy verification (match the target argmax)
    spec_gdn_record / spec_gdn_commit  recurrent-layer state over the verify
                                     positions with an innovation tape, and
                                     the commit of the accepted steps
    spec_gdn_commit_record           both at a cycle boundary, one pass
                                     over the state
    spec_stream_read                 a plain streaming read (attainable
                                     HBM read rate, for measurement)
    spec_*_workspace_size            workspace queries
    bind_qmv / bind_verify_accept /  the same calls with arguments marshalled
    bind_verify_greedy / bind_gdn_*  once, for launch loops
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
# SPEC_LIB_PATH selects another build of the same library (the host-side
# sanitizer build of the CPU test run); the default is the in-tree build.
LIB_PATH = os.environ.get("SPEC_LIB_PATH") or os.path.join(_HERE, "libspec.so")

STATUS = {0: "SPEC_OK", 1: "SPEC_ERR_INVALID", 2: "SPEC_ERR_UNSUPPORTED",
          3: "SPEC_ERR_WORKSPACE", 4: "SPEC_ERR_DEVICE"}


class SpecError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        self.status_name = STATUS.get(status, f"status {status}")
        super().__init__(f"{fn} returned {self.status_name}")


_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library {LIB_PATH} is missing: build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'` "
                "(hipcc --offload-arch=gfx950). There is no CPU fallback.")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.spec_status_str.argtypes = [i]
        L.spec_status_str.restype = ctypes.c_char_p
        L.spec_version.restype = i
        L.spec_qmv_packed_weight_bytes.argtypes = [i, i, i, i]
        L.spec_qmv_packed_weight_bytes.restype = sz
        L.spec_qmv_packed_sb_bytes.argtypes = [i, i, i]
        L.spec_qmv_packed_sb_bytes.restype = sz
        for name in ("spec_pack_w4", "spec_pack_w8"):
            fn = getattr(L, name)
            fn.argtypes = [vp, vp, vp, i, i, i, vp, vp, vp]
            fn.restype = i
        for name in ("spec_qmv_w4", "spec_qmv_w8"):
            fn = getattr(L, name)
            fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, vp]
            fn.restype = i
        for name in ("spec_qmv_w4_packed", "spec_qmv_w8_packed", "spec_qmv_w4_packed_valu"):
            fn = getattr(L, name)
            fn.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
            fn.restype = i
        L.spec_verify_accept_workspace.argtypes = [i, i, i, i]
        L.spec_verify_accept_workspace.restype = sz
        L.spec_verify_accept.argtypes = [vp, vp, vp, vp, i, i, i, f, i, f, vp, vp,
                                         vp, vp, vp, sz, vp]
        L.spec_verify_accept.restype = i
        L.spec_verify_accept_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, f, i, f, vp, vp,
                                                 vp, vp, vp]
        L.spec_verify_accept_noalloc.restype = i
        L.spec_sample_workspace_size.argtypes = [i, i, i]
        L.spec_sample_workspace_size.restype = sz
        L.spec_sample_probs.argtypes = [vp, i, i, f, i, f, vp, vp, sz, vp]
        L.spec_sample_probs.restype = i
        L.spec_sample_tokens.argtypes = [vp, i, i, f, i, f, vp, vp, vp, sz, vp]
        L.spec_requantize_w4.argtypes = [vp, i, i, i, vp, vp, vp, vp]
        L.spec_requantize_w4.restype = i
        L.spec_gate_up_packed_rows.argtypes = [i]
        L.spec_gate_up_packed_rows.restype = i
        L.spec_pack_gate_up.argtypes = [i, vp, vp, vp, vp, vp, vp, i, i, i, vp, vp, vp]
        L.spec_pack_gate_up.restype = i
        L.spec_qmv_gate_up_silu.argtypes = [i, vp, vp, vp, vp, i, i, i, i, vp]
        L.spec_qmv_gate_up_silu.restype = i
        L.spec_qmv_gate_up_silu_w4_valu.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
        L.spec_qmv_gate_up_silu_w4_valu.restype = i
        L.spec_gdn_record.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp]
        L.spec_gdn_record.restype = i
        L.spec_gdn_commit.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp]
        L.spec_gdn_commit.restype = i
        L.spec_gdn_commit_record.argtypes = [vp, vp, vp, vp, vp, i, vp, vp, vp, vp, vp,
                                             i, i, i, i, i, vp, vp, vp, vp]
        L.spec_gdn_commit_record.restype = i
        L.spec_stream_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
        L.spec_stream_read.restype = i
        L.spec_verify_greedy_workspace.argtypes = [i, i, i]
        L.spec_verify_greedy_workspace.restype = sz
        L.spec_verify_greedy.argtypes = [vp, vp, i, i, i, vp, vp, vp, sz, vp]
        L.spec_verify_greedy.restype = i
        L.spec_sample_tokens.restype = i
        _lib = L
        return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise SpecError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t, dtype, name, device=None):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


# ---- workspaces: device buffers cached per (device, stream, purpose) ----
_ws_cache: dict = {}


def _cached_buffer(cache: dict, slot, nbytes: int, alloc):
    """The cached buffer of `slot`, replaced by alloc(n) when missing or
    smaller than nbytes (n = max(nbytes, 4096))."""
    buf = cache.get(slot)
    if buf is None or buf.numel() < nbytes:
        buf = alloc(max(nbytes, 4096))
        cache[slot] = buf
    return buf


def get_workspace(nbytes: int, device, key: str = "default", stream=None):
    """A 256-byte aligned device buffer of at least nbytes for calls issued
    on `stream` (torch's current stream of `device` when None).

    Workspaces need no initialization and hold nothing between calls, so one
    buffer serves every later call ordered on the same stream.  Buffers are
    cached per stream: calls on two streams never share one, and a buffer
    that grows is replaced only for its own stream, where the torch
    allocator orders its reuse after that stream's earlier work."""
    import torch
    if nbytes == 0:
        return None
    if stream is None:
        stream = torch.cuda.current_stream(device)
    slot = (str(device), int(stream.cuda_stream), key)
    buf = _cached_buffer(_ws_cache, slot, nbytes,
                         lambda n: torch.empty(n, dtype=torch.uint8, device=device))
    assert buf.data_ptr() % 256 == 0
    return buf


class PackedWeights:
    """Quantized weights in the layout the qmv kernels stream (see
    include/spec.h): produced once by spec_pack_w4 / spec_pack_w8."""

    def __init__(self, bits, N, K, G, w, sb):
        self.bits, self.N, self.K, self.G, self.w, self.sb = bits, N, K, G, w, sb


def spec_qmv_packed_weight_bytes(bits: int, N: int, K: int, G: int = 64) -> int:
    return int(lib().spec_qmv_packed_weight_bytes(bits, N, K, G))


def spec_qmv_packed_sb_bytes(N: int, K: int, G: int = 64) -> int:
    return int(lib().spec_qmv_packed_sb_bytes(N, K, G))


def _pack(name, bits, w, scales, biases, G):
    import torch
    dev = w.device
    wdt = torch.int32 if bits == 4 else torch.uint8
    _require(w, wdt, "w", dev)
    N = w.shape[0]
    K = w.shape[1] * 8 if bits == 4 else w.shape[1]
    _require(scales, torch.float16, "scales", dev)
    _require(biases, torch.float16, "biases", dev)
    if G <= 0 or K % G:
        raise ValueError("K must be a multiple of G")
    if tuple(scales.shape) != (N, K // G) or tuple(biases.shape) != (N, K // G):
        raise ValueError(f"scales / biases must be [{N}][{K // G}]")
    wb = spec_qmv_packed_weight_bytes(bits, N, K, G)
    sbb = spec_qmv_packed_sb_bytes(N, K, G)
    wp = torch.empty(max(wb, 16), dtype=torch.uint8, device=dev)
    sbp = torch.empty(max(sbb, 16), dtype=torch.uint8, device=dev)
    st = getattr(lib(), name)(_ptr(w), _ptr(scales), _ptr(biases), N, K, G,
                              _ptr(wp), _ptr(sbp), _stream(dev))
    _check(name, st)
    return PackedWeights(bits, N, K, G, wp, sbp)


def spec_pack_w4(w, scales, biases, G: int = 64) -> PackedWeights:
    """Pack W4 weights: w int32 [N][K/8] (element k at bits 4*(k%8) of word
    k/8), scales / biases fp16 [N][K/G]."""
    return _pack("spec_pack_w4", 4, w, scales, biases, G)


def spec_pack_w8(w, scales, biases, G: int = 64) -> PackedWeights:
    """Pack W8 weights: w uint8 [N][K], scales / biases fp16 [N][K/G]."""
    return _pack("spec_pack_w8", 8, w, scales, biases, G)


class PackedGateUp:
    """A gate/up pair packed with alternating tiles by spec_pack_gate_up."""

    def __init__(self, bits, F, K, G, w, sb):
        self.bits, self.F, self.K, self.G, self.w, self.sb = bits, F, K, G, w, sb


def spec_pack_gate_up(bits: int, gate, up, G: int = 64) -> PackedGateUp:
    """Pack the gate and up projections (each (w, scales, biases) as for
    spec_pack_w4 / spec_pack_w8, F rows) for spec_qmv_gate_up_silu."""
    import torch
    dev = gate[0].device
    wdt = torch.int32 if bits == 4 else torch.uint8
    for name, t in (("gate", gate), ("up", up)):
        _require(t[0], wdt, f"{name} w", dev)
        _require(t[1], torch.float16, f"{name} scales", dev)
        _require(t[2], torch.float16, f"{name} biases", dev)
    F = gate[0].shape[0]
    K = gate[0].shape[1] * 8 if bits == 4 else gate[0].shape[1]
    if tuple(up[0].shape) != tuple(gate[0].shape):
        raise ValueError("gate and up must have the same shape")
    if G <= 0 or K % G:
        raise ValueError("K must be a multiple of G")
    for t in (gate, up):
        if tuple(t[1].shape) != (F, K // G) or tuple(t[2].shape) != (F, K // G):
            raise ValueError(f"scales / biases must be [{F}][{K // G}]")
    R = int(lib().spec_gate_up_packed_rows(F))
    wp = torch.empty(max(spec_qmv_packed_weight_bytes(bits, R, K, G), 16), dtype=torch.uint8,
                     device=dev)
    sbp = torch.empty(max(spec_qmv_packed_sb_bytes(R, K, G), 16), dtype=torch.uint8, device=dev)
    st = lib().spec_pack_gate_up(bits, _ptr(gate[0]), _ptr(gate[1]), _ptr(gate[2]),
                                 _ptr(up[0]), _ptr(up[1]), _ptr(up[2]), F, K, G,
                                 _ptr(wp), _ptr(sbp), _stream(dev))
    _check("spec_pack_gate_up", st)
    return PackedGateUp(bits, F, K, G, wp, sbp)


def _gate_up_args(packed: PackedGateUp, x, h, valu):
    """(C function name, argument tuple) of one gated gate/up call, checked."""
    import torch
    dev = x.device
    _require(x, torch.bfloat16, "x", dev)
    M, K = x.shape
    if K != packed.K:
        raise ValueError(f"x has K={K}, weights have K={packed.K}")
    _require(h, torch.bfloat16, "h", dev)
    if tuple(h.shape) != (M, packed.F):
        raise ValueError(f"h must be [{M}][{packed.F}]")
    if valu:
        if packed.bits != 4:
            raise ValueError("the vector-ALU variant takes W4 weights")
        return "spec_qmv_gate_up_silu_w4_valu", (_ptr(packed.w), _ptr(packed.sb), _ptr(x), _ptr(h),
                                                 M, packed.F, K, packed.G, _stream(dev))
    return "spec_qmv_gate_up_silu", (packed.bits, _ptr(packed.w), _ptr(packed.sb), _ptr(x), _ptr(h),
                                     M, packed.F, K, packed.G, _stream(dev))


def spec_qmv_gate_up_silu(packed: PackedGateUp, x, h=None):
    """h[M][F] bf16 = silu(x G^T) * (x U^T) for a pair packed by spec_pack_gate_up."""
    import torch
    if h is None:
        h = torch.empty((x.shape[0], packed.F), dtype=torch.bfloat16, device=x.device)
    name, args = _gate_up_args(packed, x, h, False)
    _check(name, getattr(lib(), name)(*args))
    return h


def spec_qmv_gate_up_silu_w4_valu(packed: PackedGateUp, x, h=None):
    """spec_qmv_gate_up_silu (W4, M <= 4) with the products on the vector ALU."""
    import torch
    if h is None:
        h = torch.empty((x.shape[0], packed.F), dtype=torch.bfloat16, device=x.device)
    name, args = _gate_up_args(packed, x, h, True)
    _check(name, getattr(lib(), name)(*args))
    return h


def bind_qmv_gate_up_silu(packed: PackedGateUp, x, h, valu: bool = False) -> "_Bound":
    """spec_qmv_gate_up_silu (or, with valu, spec_qmv_gate_up_silu_w4_valu)
    on fixed tensors, marshalled once (first call checked)."""
    name, args = _gate_up_args(packed, x, h, valu)
    _check(name, getattr(lib(), name)(*args))
    return _Bound(name, getattr(lib(), name), args, (packed, x, h))


class QWeights:
    """Quantized weights in the interchange layout, as stored: w int32
    [N][K/8] (W4, element k at bits 4*(k%8) of word k/8) or uint8 [N][K]
    (W8), scales / biases fp16 [N][K/G].  Read directly by spec_qmv_w4 /
    spec_qmv_w8."""

    def __init__(self, bits, w, scales, biases, G=64):
        import torch
        dev = w.device
        _require(w, torch.int32 if bits == 4 else torch.uint8, "w", dev)
        _require(scales, torch.float16, "scales", dev)
        _require(biases, torch.float16, "biases", dev)
        N = w.shape[0]
        K = w.shape[1] * 8 if bits == 4 else w.shape[1]
        if G <= 0 or K % G:
            raise ValueError("K must be a multiple of G")
        if tuple(scales.shape) != (N, K // G) or tuple(biases.shape) != (N, K // G):
            raise ValueError(f"scales / biases must be [{N}][{K // G}]")
        self.bits, self.N, self.K, self.G = bits, N, K, G
        self.w, self.scales, self.biases = w, scales, biases


def _qmv_args(weights, x, y, valu=False):
    """(C function name, argument tuple) of one qmv call, checked."""
    import torch
    dev = x.device
    _require(x, torch.bfloat16, "x", dev)
    M, K = x.shape
    if K != weights.K:
        raise ValueError(f"x has K={K}, weights have K={weights.K}")
    _require(y, torch.float32, "y", dev)
    if tuple(y.shape) != (M, weights.N):
        raise ValueError(f"y must be [{M}][{weights.N}]")
    if valu and not (isinstance(weights, PackedWeights) and weights.bits == 4):
        raise ValueError("the vector-ALU variant takes W4 packed weights")
    if isinstance(weights, PackedWeights):
        name = f"spec_qmv_w{weights.bits}_packed" + ("_valu" if valu else "")
        args = (_ptr(weights.w), _ptr(weights.sb), _ptr(x), _ptr(y), M, weights.N, K, weights.G,
                _stream(dev))
    elif isinstance(weights, QWeights):
        name = f"spec_qmv_w{weights.bits}"
        args = (_ptr(weights.w), _ptr(weights.scales), _ptr(weights.biases), _ptr(x), _ptr(y), M,
                weights.N, K, weights.G, _stream(dev))
    else:
        raise TypeError("weights must be QWeights or PackedWeights")
    return name, args


def _qmv(weights, x, y):
    import torch
    if y is None:
        y = torch.empty((x.shape[0], weights.N), dtype=torch.float32, device=x.device)
    name, args = _qmv_args(weights, x, y)
    _check(name, getattr(lib(), name)(*args))
    return y


def spec_qmv_w4(w, scales, biases, x, y=None, G: int = 64):
    """y[M][N] fp32 = x[M][K] (bf16) times the dequantized W4 matrix given as
    stored: w int32 [N][K/8], scales / biases fp16 [N][K/G]."""
    return _qmv(QWeights(4, w, scales, biases, G), x, y)


def spec_qmv_w8(w, scales, biases, x, y=None, G: int = 64):
    """As spec_qmv_w4 for W8 weights: w uint8 [N][K]."""
    return _qmv(QWeights(8, w, scales, biases, G), x, y)


def spec_qmv_w4_packed(packed: PackedWeights, x, y=None):
    """spec_qmv_w4 from weights repacked by spec_pack_w4."""
    if packed.bits != 4:
        raise ValueError(f"spec_qmv_w4_packed needs W4 packed weights, got W{packed.bits}")
    return _qmv(packed, x, y)


def spec_qmv_w4_packed_valu(packed: PackedWeights, x, y=None):
    """spec_qmv_w4_packed (M <= 4) with the products on the vector ALU."""
    import torch
    if y is None:
        y = torch.empty((x.shape[0], packed.N), dtype=torch.float32, device=x.device)
    name, args = _qmv_args(packed, x, y, valu=True)
    _check(name, getattr(lib(), name)(*args))
    return y


def spec_qmv_w8_packed(packed: PackedWeights, x, y=None):
    """spec_qmv_w8 from weights repacked by spec_pack_w8."""
    if packed.bits != 8:
        raise ValueError(f"spec_qmv_w8_packed needs W8 packed weights, got W{packed.bits}")
    return _qmv(packed, x, y)


class _Bound:
    """A C-ABI call with its arguments marshalled once (pointers, sizes and
    the stream current at bind time).  Calling it re-issues the same call
    with no Python-side checks: for loops that launch the same shapes over
    and over.  The tensors it was bound to must stay alive and in place."""

    def __init__(self, name, fn, args, keep):
        self.name, self._fn, self._args, self._keep = name, fn, args, keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            raise SpecError(self.name, st)


def bind_qmv(weights, x, y, valu: bool = False) -> _Bound:
    """A qmv on fixed tensors, marshalled once: weights are PackedWeights
    (spec_qmv_w*_packed, or with valu spec_qmv_w4_packed_valu) or QWeights
    (spec_qmv_w*, interchange layout).  The first call is checked like the
    unbound functions."""
    name, args = _qmv_args(weights, x, y, valu)
    _check(name, getattr(lib(), name)(*args))
    return _Bound(name, getattr(lib(), name), args, (weights, x, y))


def spec_verify_accept_workspace(B: int, D: int, V: int, top_k: int) -> int:
    return int(lib().spec_verify_accept_workspace(B, D, V, top_k))


def spec_verify_accept(target_logits, draft_logits, draft_tokens, uniforms,
                       temperature: float, top_k: int = 0, top_p: float = 1.0,
                       with_probs: bool = False, out=None, workspace=None, noalloc=False):
    """Acceptance for B sequences.  target_logits fp32 [B][D+1][V],
    draft_logits fp32 [B][D][V], draft_tokens int32 [B][D], uniforms fp32
    [B][D+1].  Returns (accepted_len, next_token) int32 [B], plus
    (p_draft, q_draft) fp32 [B][D] when with_probs.  With noalloc (and `out`
    given) the call goes to spec_verify_accept_noalloc: no workspace, nothing
    allocated."""
    import torch
    dev = target_logits.device
    _require(target_logits, torch.float32, "target_logits", dev)
    B, D1, V = target_logits.shape
    D = D1 - 1
    if D > 0:
        _require(draft_logits, torch.float32, "draft_logits", dev)
        _require(draft_tokens, torch.int32, "draft_tokens", dev)
        if tuple(draft_logits.shape) != (B, D, V) or tuple(draft_tokens.shape) != (B, D):
            raise ValueError("draft_logits must be [B][D][V] and draft_tokens [B][D]")
    _require(uniforms, torch.float32, "uniforms", dev)
    if tuple(uniforms.shape) != (B, D + 1):
        raise ValueError("uniforms must be [B][D+1]")
    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        nxt = torch.empty(B, dtype=torch.int32, device=dev)
        pd = torch.empty((B, D), dtype=torch.float32, device=dev) if with_probs else None
        qd = torch.empty((B, D), dtype=torch.float32, device=dev) if with_probs else None
    else:
        acc, nxt, pd, qd = out
    if noalloc:
        st = lib().spec_verify_accept_noalloc(
            _ptr(target_logits), _ptr(draft_logits if D > 0 else None),
            _ptr(draft_tokens if D > 0 else None), _ptr(uniforms), B, D, V,
            float(temperature), int(top_k), float(top_p), _ptr(acc), _ptr(nxt),
            _ptr(pd), _ptr(qd), _stream(dev))
        _check("spec_verify_accept_noalloc", st)
        return (acc, nxt, pd, qd) if with_probs else (acc, nxt)
    need = spec_verify_accept_workspace(B, D, V, top_k)
    if workspace is None:
        workspace = get_workspace(need, dev, "accept")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().spec_verify_accept(
        _ptr(target_logits), _ptr(draft_logits if D > 0 else None),
        _ptr(draft_tokens if D > 0 else None), _ptr(uniforms), B, D, V,
        float(temperature), int(top_k), float(top_p), _ptr(acc), _ptr(nxt),
        _ptr(pd), _ptr(qd), _ptr(workspace), nbytes, _stream(dev))
    _check("spec_verify_accept", st)
    return (acc, nxt, pd, qd) if with_probs else (acc, nxt)


def bind_verify_accept(target_logits, draft_logits, draft_tokens, uniforms,
                       temperature: float, top_k: int = 0, top_p: float = 1.0,
                       out=None) -> _Bound:
    """spec_verify_accept on fixed tensors, marshalled once (first call
    checked through spec_verify_accept).  `out` = (accepted_len, next_token,
    p_draft or None, q_draft or None)."""
    import torch
    dev = target_logits.device
    B, D1, V = target_logits.shape
    D = D1 - 1
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev), None, None)
    need = spec_verify_accept_workspace(B, D, V, top_k)
    ws = torch.empty(max(need, 4096), dtype=torch.uint8, device=dev)
    spec_verify_accept(target_logits, draft_logits, draft_tokens, uniforms, temperature,
                       top_k, top_p, out=out, workspace=ws)
    acc, nxt, pd, qd = out
    args = (_ptr(target_logits), _ptr(draft_logits if D > 0 else None),
            _ptr(draft_tokens if D > 0 else None), _ptr(uniforms), B, D, V,
            ctypes.c_float(temperature), int(top_k), ctypes.c_float(top_p), _ptr(acc),
            _ptr(nxt), _ptr(pd), _ptr(qd), _ptr(ws), ws.numel(), _stream(dev))
    keep = (target_logits, draft_logits, draft_tokens, uniforms, out, ws)
    return _Bound("spec_verify_accept", lib().spec_verify_accept, args, keep)


def spec_sample_workspace_size(R: int, V: int, top_k: int) -> int:
    return int(lib().spec_sample_workspace_size(R, V, top_k))


def spec_sample_probs(logits, temperature: float, top_k: int = 0,
                      top_p: float = 1.0, probs=None, workspace=None):
    """probs fp32 [R][V] = filtered distribution of each row of logits [R][V]."""
    import torch
    dev = logits.device
    _require(logits, torch.float32, "logits", dev)
    R, V = logits.shape
    if probs is None:
        probs = torch.empty((R, V), dtype=torch.float32, device=dev)
    _require(probs, torch.float32, "probs", dev)
    need = spec_sample_workspace_size(R, V, top_k)
    if workspace is None:
        workspace = get_workspace(need, dev, "sample")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().spec_sample_probs(_ptr(logits), R, V, float(temperature), int(top_k),
                                 float(top_p), _ptr(probs), _ptr(workspace), nbytes,
                                 _stream(dev))
    _check("spec_sample_probs", st)
    return probs


def spec_sample_tokens(logits, uniforms, temperature: float, top_k: int = 0,
                       top_p: float = 1.0, tokens=None, workspace=None):
    """tokens int32 [R]: one inverse-CDF draw per row of logits [R][V]."""
    import torch
    dev = logits.device
    _require(logits, torch.float32, "logits", dev)
    R, V = logits.shape
    _require(uniforms, torch.float32, "uniforms", dev)
    if uniforms.numel() != R:
        raise ValueError("uniforms must hold one value per row")
    if tokens is None:
        tokens = torch.empty(R, dtype=torch.int32, device=dev)
    need = spec_sample_workspace_size(R, V, top_k)
    if workspace is None:
        workspace = get_workspace(need, dev, "sample")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().spec_sample_tokens(_ptr(logits), R, V, float(temperature), int(top_k),
                                  float(top_p), _ptr(uniforms), _ptr(tokens),
                                  _ptr(workspace), nbytes, _stream(dev))
    _check("spec_sample_tokens", st)
    return tokens


def spec_verify_greedy_workspace(B: int, D: int, V: int) -> int:
    return int(lib().spec_verify_greedy_workspace(B, D, V))


def spec_verify_greedy(target_logits, draft_tokens, out=None, workspace=None):
    """Greedy verification of B sequences: target_logits fp32 [B][D+1][V],
    draft_tokens int32 [B][D].  Returns (accepted_len, next_token) int32 [B]."""
    import torch
    dev = target_logits.device
    _require(target_logits, torch.float32, "target_logits", dev)
    B, D1, V = target_logits.shape
    D = D1 - 1
    if D > 0:
        _require(draft_tokens, torch.int32, "draft_tokens", dev)
        if tuple(draft_tokens.shape) != (B, D):
            raise ValueError("draft_tokens must be [B][D]")
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev))
    acc, nxt = out
    need = spec_verify_greedy_workspace(B, D, V)
    if workspace is None:
        workspace = get_workspace(need, dev, "greedy")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().spec_verify_greedy(_ptr(target_logits), _ptr(draft_tokens if D > 0 else None),
                                  B, D, V, _ptr(acc), _ptr(nxt), _ptr(workspace), nbytes,
                                  _stream(dev))
    _check("spec_verify_greedy", st)
    return acc, nxt


def bind_verify_greedy(target_logits, draft_tokens, out=None) -> _Bound:
    """spec_verify_greedy on fixed tensors, marshalled once (first call
    checked through spec_verify_greedy).  `out` = (accepted_len, next_token)."""
    import torch
    dev = target_logits.device
    B, D1, V = target_logits.shape
    D = D1 - 1
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev))
    need = spec_verify_greedy_workspace(B, D, V)
    ws = torch.empty(max(need, 4096), dtype=torch.uint8, device=dev)
    spec_verify_greedy(target_logits, draft_tokens, out=out, workspace=ws)
    acc, nxt = out
    args = (_ptr(target_logits), _ptr(draft_tokens if D > 0 else None), B, D, V,
            _ptr(acc), _ptr(nxt), _ptr(ws), ws.numel(), _stream(dev))
    keep = (target_logits, draft_tokens, out, ws)
    return _Bound("spec_verify_greedy", lib().spec_verify_greedy, args, keep)


def spec_gdn_record(S0, q, k, v, alpha, beta, o=None, delta=None, S_final=None,
                    want_final: bool = False):
    """Gated-delta-rule steps over T positions from S0 [B][H][dv][dk] (left
    untouched) with q, k [B][T][H][dk], v [B][T][H][dv], alpha, beta
    [B][T][H]; returns (o, delta, S_final or None)."""
    import torch
    dev = S0.device
    for name, t in (("S0", S0), ("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta)):
        _require(t, torch.float32, name, dev)
    B, H, dv, dk = S0.shape
    T = q.shape[1]
    if (tuple(q.shape) != (B, T, H, dk) or tuple(k.shape) != (B, T, H, dk)
            or tuple(v.shape) != (B, T, H, dv) or tuple(alpha.shape) != (B, T, H)
            or tuple(beta.shape) != (B, T, H)):
        raise ValueError("shapes must be S0 [B][H][dv][dk], q/k [B][T][H][dk], v [B][T][H][dv], "
                         "alpha/beta [B][T][H]")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    if delta is None:
        delta = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    if S_final is None and want_final:
        S_final = torch.empty_like(S0)
    st = lib().spec_gdn_record(_ptr(S0), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                               B, T, H, dk, dv, _ptr(o), _ptr(delta), _ptr(S_final), _stream(dev))
    _check("spec_gdn_record", st)
    return o, delta, S_final


def spec_gdn_commit(S, alpha, k, delta, n_steps):
    """In place: S (holding S0, [B][H][dv][dk]) becomes the state after the
    first n_steps[b] steps of the tape (alpha [B][T][H], k [B][T][H][dk],
    delta [B][T][H][dv]); n_steps int32 [B]."""
    import torch
    dev = S.device
    for name, t in (("S", S), ("alpha", alpha), ("k", k), ("delta", delta)):
        _require(t, torch.float32, name, dev)
    _require(n_steps, torch.int32, "n_steps", dev)
    B, H, dv, dk = S.shape
    T = alpha.shape[1]
    st = lib().spec_gdn_commit(_ptr(S), _ptr(alpha), _ptr(k), _ptr(delta), _ptr(n_steps),
                               B, T, H, dk, dv, _stream(dev))
    _check("spec_gdn_commit", st)
    return S


def _gdn_commit_record_args(S, prev_alpha, prev_k, prev_delta, n_steps, q, k, v, alpha, beta,
                            o, delta, S_final):
    import torch
    dev = S.device
    _require(S, torch.float32, "S", dev)
    B, H, dv, dk = S.shape
    Tp = 0 if prev_alpha is None else prev_alpha.shape[1]
    T = q.shape[1]
    if Tp > 0:
        for name, t in (("prev_alpha", prev_alpha), ("prev_k", prev_k), ("prev_delta", prev_delta)):
            _require(t, torch.float32, name, dev)
        _require(n_steps, torch.int32, "n_steps", dev)
        if (tuple(prev_alpha.shape) != (B, Tp, H) or tuple(prev_k.shape) != (B, Tp, H, dk)
                or tuple(prev_delta.shape) != (B, Tp, H, dv) or tuple(n_steps.shape) != (B,)):
            raise ValueError("previous tape must be alpha [B][Tp][H], k [B][Tp][H][dk], "
                             "delta [B][Tp][H][dv], n_steps [B]")
    for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta),
                    ("o", o), ("delta", delta)):
        _require(t, torch.float32, name, dev)
    if (tuple(q.shape) != (B, T, H, dk) or tuple(k.shape) != (B, T, H, dk)
            or tuple(v.shape) != (B, T, H, dv) or tuple(alpha.shape) != (B, T, H)
            or tuple(beta.shape) != (B, T, H) or tuple(o.shape) != (B, T, H, dv)
            or tuple(delta.shape) != (B, T, H, dv)):
        raise ValueError("shapes must be S [B][H][dv][dk], q/k [B][T][H][dk], "
                         "v/o/delta [B][T][H][dv], alpha/beta [B][T][H]")
    if S_final is not None:
        _require(S_final, torch.float32, "S_final", dev)
    if Tp == 0:
        prev_alpha = prev_k = prev_delta = n_steps = None
    return (_ptr(S), _ptr(prev_alpha), _ptr(prev_k), _ptr(prev_delta), _ptr(n_steps), Tp,
            _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), B, T, H, dk, dv,
            _ptr(o), _ptr(delta), _ptr(S_final), _stream(dev))


def spec_gdn_commit_record(S, prev_alpha, prev_k, prev_delta, n_steps, q, k, v, alpha, beta,
                           o=None, delta=None, S_final=None, want_final: bool = False):
    """At a cycle boundary, in place in S [B][H][dv][dk]: commit the first
    n_steps[b] steps of the previous tape (prev_alpha [B][Tp][H], prev_k
    [B][Tp][H][dk], prev_delta [B][Tp][H][dv]; prev_alpha None commits
    nothing), then record the next T steps from the committed state; returns
    (o, delta, S_final or None), bitwise those of spec_gdn_commit followed by
    spec_gdn_record.  The new tape must not share memory with the old one."""
    import torch
    B, H, dv, dk = S.shape
    T = q.shape[1]
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=S.device)
    if delta is None:
        delta = torch.empty((B, T, H, dv), dtype=torch.float32, device=S.device)
    if S_final is None and want_final:
        S_final = torch.empty_like(S)
    args = _gdn_commit_record_args(S, prev_alpha, prev_k, prev_delta, n_steps, q, k, v, alpha,
                                   beta, o, delta, S_final)
    _check("spec_gdn_commit_record", lib().spec_gdn_commit_record(*args))
    return o, delta, S_final


def bind_gdn_commit_record(S, prev_alpha, prev_k, prev_delta, n_steps, q, k, v, alpha, beta,
                           o, delta, S_final=None) -> _Bound:
    """spec_gdn_commit_record on fixed tensors, marshalled once (no checked
    first call: the call works in place on S)."""
    args = _gdn_commit_record_args(S, prev_alpha, prev_k, prev_delta, n_steps, q, k, v, alpha,
                                   beta, o, delta, S_final)
    return _Bound("spec_gdn_commit_record", lib().spec_gdn_commit_record, args,
                  (S, prev_alpha, prev_k, prev_delta, n_steps, q, k, v, alpha, beta, o, delta,
                   S_final))


def bind_gdn_record(S0, q, k, v, alpha, beta, o, delta, S_final=None) -> _Bound:
    """spec_gdn_record on fixed tensors, marshalled once (first call checked)."""
    spec_gdn_record(S0, q, k, v, alpha, beta, o=o, delta=delta, S_final=S_final)
    B, H, dv, dk = S0.shape
    T = q.shape[1]
    args = (_ptr(S0), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), B, T, H, dk, dv,
            _ptr(o), _ptr(delta), _ptr(S_final), _stream(S0.device))
    return _Bound("spec_gdn_record", lib().spec_gdn_record, args,
                  (S0, q, k, v, alpha, beta, o, delta, S_final))


def bind_gdn_commit(S, alpha, k, delta, n_steps, check: bool = True) -> _Bound:
    """spec_gdn_commit on fixed tensors, marshalled once.  The commit works in
    place, so the checked first call (check=True) already applies it once."""
    if check:
        spec_gdn_commit(S, alpha, k, delta, n_steps)
    B, H, dv, dk = S.shape
    T = alpha.shape[1]
    args = (_ptr(S), _ptr(alpha), _ptr(k), _ptr(delta), _ptr(n_steps), B, T, H, dk, dv,
            _stream(S.device))
    return _Bound("spec_gdn_commit", lib().spec_gdn_commit, args, (S, alpha, k, delta, n_steps))


STREAM_READ_GROUPS = 2048   # SPEC_STREAM_READ_GROUPS


def spec_stream_read(src, sink=None):
    """A plain streaming read of a device tensor's bytes (16-byte aligned, a
    multiple of 16 bytes); returns the int32 sink [2048] whose XOR is the XOR
    of src's 32-bit words."""
    import torch
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    if sink is None:
        sink = torch.empty(STREAM_READ_GROUPS, dtype=torch.int32, device=src.device)
    _require(sink, torch.int32, "sink", src.device)
    if sink.numel() < STREAM_READ_GROUPS:
        raise ValueError(f"sink must hold {STREAM_READ_GROUPS} words")
    nbytes = src.numel() * src.element_size()
    _check("spec_stream_read", lib().spec_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(src.device)))
    return sink


def bind_stream_read(src, sink) -> _Bound:
    """spec_stream_read on fixed tensors, marshalled once (first call checked)."""
    spec_stream_read(src, sink)
    args = (_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(src.device))
    return _Bound("spec_stream_read", lib().spec_stream_read, args, (src, sink))


def spec_requantize_w4(w_bf16, G: int = 64):
    """(w int32 [N][K/8], scales fp16 [N][K/G], biases fp16 [N][K/G]): the
    draft-only 4-bit copy of a bf16 [N][K] matrix, in spec_pack_w4's input
    layout."""
    import torch
    dev = w_bf16.device
    _require(w_bf16, torch.bfloat16, "w_bf16", dev)
    N, K = w_bf16.shape
    if G <= 0 or K % G or K % 8:
        raise ValueError("K must be a multiple of G and of 8")
    w4 = torch.empty((N, K // 8), dtype=torch.int32, device=dev)
    s = torch.empty((N, K // G), dtype=torch.float16, device=dev)
    b = torch.empty((N, K // G), dtype=torch.float16, device=dev)
    st = lib().spec_requantize_w4(_ptr(w_bf16), N, K, G, _ptr(w4), _ptr(s), _ptr(b), _stream(dev))
    _check("spec_requantize_w4", st)
    return w4, s, b


def bind_sample_tokens(logits, uniforms, temperature: float, top_k: int = 0, top_p: float = 1.0,
                       tokens=None) -> _Bound:
    """spec_sample_tokens on fixed tensors, marshalled once (first call
    checked), with a workspace of its own."""
    import torch
    dev = logits.device
    R, V = logits.shape
    if tokens is None:
        tokens = torch.empty(R, dtype=torch.int32, device=dev)
    need = spec_sample_workspace_size(R, V, top_k)
    ws = torch.empty(max(need, 4096), dtype=torch.uint8, device=dev)
    spec_sample_tokens(logits, uniforms, temperature, top_k, top_p, tokens=tokens, workspace=ws)
    args = (_ptr(logits), R, V, ctypes.c_float(temperature), int(top_k), ctypes.c_float(top_p),
            _ptr(uniforms), _ptr(tokens), _ptr(ws), ws.numel(), _stream(dev))
    return _Bound("spec_sample_tokens", lib().spec_sample_tokens, args,
                  (logits, uniforms, tokens, ws))
