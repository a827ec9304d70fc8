"""fp64 CPU oracle for the speculative-decoding hot path (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP
library and its Python binding never import it, and it imports nothing from
them: the two implementations share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64, no fused multiply-add);
this module only marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# Address- and undefined-behaviour-sanitized build, loaded instead when
# SPEC_ORACLE_SANITIZE=1 (the process must preload gcc's libasan).
_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")
_SANITIZE = os.environ.get("SPEC_ORACLE_SANITIZE") == "1"

_c_long_p = ctypes.POINTER(ctypes.c_long)


def build(sanitize: bool = False) -> str:
    """Compile oracle.c with gcc into liboracle.so (always recompiles); with
    sanitize, into liboracle_san.so with AddressSanitizer and
    UndefinedBehaviorSanitizer (any report aborts)."""
    out = _LIB_SAN if sanitize else _LIB
    tmp = out + ".tmp"
    extra = (["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-g"] if sanitize else [])
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", *extra, "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = _LIB_SAN if _SANITIZE else _LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build(sanitize=_SANITIZE)
        L = ctypes.CDLL(path)
        vp, lg, i, f = ctypes.c_void_p, ctypes.c_long, ctypes.c_int, ctypes.c_float
        L.oracle_qmv.argtypes = [i, vp, vp, vp, vp, lg, lg, lg, lg, lg, lg, vp, vp]
        L.oracle_qmv.restype = i
        L.oracle_qmv_points.argtypes = [i, vp, vp, vp, vp, lg, lg, lg, lg, vp, vp,
                                        lg, vp, vp]
        L.oracle_qmv_points.restype = i
        L.oracle_probs.argtypes = [vp, lg, f, i, f, vp]
        L.oracle_probs.restype = i
        L.oracle_sample.argtypes = [vp, lg, f, i, f, f]
        L.oracle_sample.restype = lg
        L.oracle_sample_rows.argtypes = [vp, lg, lg, f, i, f, vp, vp]
        L.oracle_sample_rows.restype = i
        L.oracle_accept.argtypes = [vp, vp, vp, vp, lg, lg, lg, f, i, f, vp, vp, vp,
                                    vp, vp, vp]
        L.oracle_accept.restype = i
        L.oracle_splitmix64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.oracle_splitmix64.restype = ctypes.c_uint64
        L.oracle_stream_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.oracle_stream_uniform.restype = ctypes.c_float
        L.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        L.oracle_double_to_bf16.restype = ctypes.c_uint16
        L.oracle_gate_up_silu.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, lg, lg, lg, lg,
                                          lg, lg, vp, vp]
        L.oracle_gate_up_silu.restype = i
        L.oracle_gdn_record.argtypes = [vp, vp, vp, vp, vp, vp, lg, lg, lg, lg, lg, vp, vp, vp]
        L.oracle_gdn_record.restype = i
        L.oracle_gdn_commit.argtypes = [vp, vp, vp, vp, vp, lg, lg, lg, lg, lg, vp]
        L.oracle_gdn_commit.restype = i
        L.oracle_float_to_half.argtypes = [ctypes.c_float]
        L.oracle_float_to_half.restype = ctypes.c_uint16
        L.oracle_requantize_w4.argtypes = [vp, lg, lg, lg, vp, vp, vp]
        L.oracle_requantize_w4.restype = i
        L.oracle_verify_greedy.argtypes = [vp, vp, lg, lg, lg, vp, vp]
        L.oracle_verify_greedy.restype = i
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = ctypes.c_double
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def half_to_double(h: int) -> float:
    return lib().oracle_half_to_double(h)


def bf16_to_double(b: int) -> float:
    return lib().oracle_bf16_to_double(b)


def qmv(bits: int, w: np.ndarray, scales: np.ndarray, biases: np.ndarray,
        x: np.ndarray, group: int, rows: tuple[int, int] | None = None,
        with_abs: bool = False):
    """y[m][n] for n in ``rows`` (default all), fp64 [M][n1-n0].

    ``w``: uint32 [N][K/8] (bits=4) or uint8 [N][K] (bits=8); ``scales`` and
    ``biases``: fp16 bit patterns as uint16 [N][K/G]; ``x``: bf16 bit patterns
    as uint16 [M][K].  With ``with_abs`` also returns sum_k |x * w| per output.
    """
    M, K = x.shape
    N = w.shape[0]
    n0, n1 = rows if rows is not None else (0, N)
    y = np.empty((M, n1 - n0), np.float64)
    a = np.empty_like(y) if with_abs else None
    rc = lib().oracle_qmv(bits, _ptr(w), _ptr(scales), _ptr(biases), _ptr(x),
                          M, N, K, group, n0, n1, _ptr(y), _ptr(a))
    if rc != 0:
        raise ValueError(f"oracle_qmv rejected its arguments (rc={rc})")
    return (y, a) if with_abs else y


def double_to_bf16(v: float) -> int:
    """Nearest-even bfloat16 bit pattern of a double."""
    return int(lib().oracle_double_to_bf16(float(v)))


def gate_up_silu(bits: int, gate: tuple, up: tuple, x: np.ndarray, group: int = 64,
                 rows: tuple[int, int] | None = None):
    """(h fp64 [M][n1-n0], h as bf16 bit patterns uint16 [M][n1-n0]) with
    h = silu(x G^T) * (x U^T); ``gate`` and ``up`` are (w, scales, biases)
    in the layout of :func:`qmv`."""
    gw, gs, gb = [np.ascontiguousarray(a) for a in gate]
    uw, us, ub = [np.ascontiguousarray(a) for a in up]
    x = np.ascontiguousarray(x)
    M, K = x.shape
    F = gw.shape[0]
    n0, n1 = rows if rows is not None else (0, F)
    h = np.empty((M, n1 - n0), np.float64)
    hb = np.empty((M, n1 - n0), np.uint16)
    rc = lib().oracle_gate_up_silu(bits, _ptr(gw), _ptr(gs), _ptr(gb), _ptr(uw), _ptr(us),
                                   _ptr(ub), _ptr(x), M, F, K, group, n0, n1, _ptr(h),
                                   _ptr(hb))
    if rc != 0:
        raise ValueError(f"oracle_gate_up_silu rejected its arguments (rc={rc})")
    return h, hb


def qmv_points(bits: int, w: np.ndarray, scales: np.ndarray, biases: np.ndarray,
               x: np.ndarray, group: int, m_idx, n_idx):
    """Selected outputs y[m_idx[i]][n_idx[i]] and their sum_k |x * w|."""
    M, K = x.shape
    N = w.shape[0]
    mi = np.ascontiguousarray(m_idx, dtype=np.int64)
    ni = np.ascontiguousarray(n_idx, dtype=np.int64)
    y = np.empty(mi.shape[0], np.float64)
    a = np.empty_like(y)
    rc = lib().oracle_qmv_points(bits, _ptr(w), _ptr(scales), _ptr(biases),
                                 _ptr(x), M, N, K, group, _ptr(mi), _ptr(ni),
                                 mi.shape[0], _ptr(y), _ptr(a))
    if rc != 0:
        raise ValueError(f"oracle_qmv_points rejected its arguments (rc={rc})")
    return y, a


def probs(z: np.ndarray, temperature: float, top_k: int = 0,
          top_p: float = 1.0) -> np.ndarray | None:
    """Filtered sampling distribution of one fp32 row (fp64), None if invalid."""
    z = np.ascontiguousarray(z, dtype=np.float32)
    out = np.empty(z.shape[0], np.float64)
    rc = lib().oracle_probs(_ptr(z), z.shape[0], temperature, top_k, top_p, _ptr(out))
    if rc == -1:
        return None
    if rc != 0:
        raise MemoryError("oracle_probs failed")
    return out


def probs_rows(z: np.ndarray, temperature: float, top_k: int = 0,
               top_p: float = 1.0) -> tuple[np.ndarray, np.ndarray]:
    """Row-wise probs of z [R][V]; returns (probs [R][V], valid [R] bool)."""
    z = np.ascontiguousarray(z, dtype=np.float32)
    R, V = z.shape
    out = np.zeros((R, V), np.float64)
    valid = np.zeros(R, bool)
    for r in range(R):
        p = probs(z[r], temperature, top_k, top_p)
        if p is not None:
            out[r] = p
            valid[r] = True
    return out, valid


def sample(z: np.ndarray, temperature: float, top_k: int, top_p: float,
           u: float) -> int:
    z = np.ascontiguousarray(z, dtype=np.float32)
    return int(lib().oracle_sample(_ptr(z), z.shape[0], temperature, top_k, top_p, u))


def sample_rows(z: np.ndarray, temperature: float, top_k: int, top_p: float,
                u: np.ndarray) -> np.ndarray:
    """One token per row of z [R][V] with uniforms u [R] (int32 [R])."""
    z = np.ascontiguousarray(z, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    R, V = z.shape
    tok = np.empty(R, np.int32)
    lib().oracle_sample_rows(_ptr(z), R, V, temperature, top_k, top_p, _ptr(u), _ptr(tok))
    return tok


def accept(target_logits: np.ndarray, draft_logits: np.ndarray | None,
           draft_tokens: np.ndarray | None, uniforms: np.ndarray,
           temperature: float, top_k: int = 0, top_p: float = 1.0) -> dict:
    """Acceptance for B sequences; target [B][D+1][V], draft [B][D][V]."""
    tl = np.ascontiguousarray(target_logits, dtype=np.float32)
    B, D1, V = tl.shape
    D = D1 - 1
    dl = None if D == 0 else np.ascontiguousarray(draft_logits, dtype=np.float32)
    dt = None if D == 0 else np.ascontiguousarray(draft_tokens, dtype=np.int32)
    u = np.ascontiguousarray(uniforms, dtype=np.float32)
    assert u.shape == (B, D + 1)
    acc = np.empty(B, np.int32)
    nxt = np.empty(B, np.int32)
    pd = np.empty((B, max(D, 1)), np.float64)
    qd = np.empty((B, max(D, 1)), np.float64)
    row = np.empty(B, np.int32)
    margin = np.empty(B, np.float64)
    rc = lib().oracle_accept(_ptr(tl), _ptr(dl), _ptr(dt), _ptr(u), B, D, V,
                             temperature, top_k, top_p, _ptr(acc), _ptr(nxt),
                             _ptr(pd), _ptr(qd), _ptr(row), _ptr(margin))
    if rc != 0:
        raise ValueError(f"oracle_accept failed (rc={rc})")
    return {"accepted_len": acc, "next_token": nxt, "p_draft": pd[:, :D],
            "q_draft": qd[:, :D], "draw_row": row, "draw_margin": margin}


def splitmix64(seed: int, i: int) -> int:
    """Output i of the SplitMix64 stream with the given seed."""
    return int(lib().oracle_splitmix64(seed, i))


def stream_uniform(seed: int, i: int) -> float:
    """Output i of the stream as an exact fp32 uniform on [0, 1)."""
    return float(lib().oracle_stream_uniform(seed, i))


def verify_greedy(target_logits: np.ndarray, draft_tokens: np.ndarray | None) -> dict:
    """Greedy verification (sample-and-match) of B sequences; target
    [B][D+1][V], draft_tokens [B][D]."""
    tl = np.ascontiguousarray(target_logits, dtype=np.float32)
    B, D1, V = tl.shape
    D = D1 - 1
    dt = None if D == 0 else np.ascontiguousarray(draft_tokens, dtype=np.int32)
    acc = np.empty(B, np.int32)
    nxt = np.empty(B, np.int32)
    rc = lib().oracle_verify_greedy(_ptr(tl), _ptr(dt), B, D, V, _ptr(acc), _ptr(nxt))
    if rc != 0:
        raise ValueError(f"oracle_verify_greedy failed (rc={rc})")
    return {"accepted_len": acc, "next_token": nxt}


def gdn_record(S0, q, k, v, alpha, beta) -> dict:
    """Gated-delta-rule steps over T positions with the innovation tape:
    S0 [B][H][dv][dk], q/k [B][T][H][dk], v [B][T][H][dv], alpha/beta
    [B][T][H] (fp32).  Returns o and delta [B][T][H][dv] and S_final, fp64."""
    S0, q, k, v, alpha, beta = [np.ascontiguousarray(a, dtype=np.float32)
                                for a in (S0, q, k, v, alpha, beta)]
    B, H, dv, dk = S0.shape
    T = q.shape[1]
    assert q.shape == (B, T, H, dk) and k.shape == (B, T, H, dk) and v.shape == (B, T, H, dv)
    assert alpha.shape == (B, T, H) and beta.shape == (B, T, H)
    o = np.empty((B, T, H, dv))
    d = np.empty((B, T, H, dv))
    Sf = np.empty((B, H, dv, dk))
    rc = lib().oracle_gdn_record(_ptr(S0), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                 B, T, H, dk, dv, _ptr(o), _ptr(d), _ptr(Sf))
    if rc != 0:
        raise ValueError(f"oracle_gdn_record failed (rc={rc})")
    return {"o": o, "delta": d, "S_final": Sf}


def gdn_commit(S0, alpha, k, delta, n) -> np.ndarray:
    """The state after the first n[b] steps, from S0 and the tape alone."""
    S0, alpha, k, delta = [np.ascontiguousarray(a, dtype=np.float32) for a in (S0, alpha, k, delta)]
    n = np.ascontiguousarray(n, dtype=np.int32)
    B, H, dv, dk = S0.shape
    T = alpha.shape[1]
    out = np.empty((B, H, dv, dk))
    rc = lib().oracle_gdn_commit(_ptr(S0), _ptr(alpha), _ptr(k), _ptr(delta), _ptr(n), B, T, H,
                                 dk, dv, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_gdn_commit failed (rc={rc})")
    return out


def requantize_w4(w_bf16: np.ndarray, group: int = 64):
    """(w4 uint32 [N][K/8], scales fp16 bits [N][K/G], biases fp16 bits) from
    bf16 bit patterns [N][K]: the draft-only 4-bit copy of a weight matrix."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    N, K = w.shape
    w4 = np.empty((N, K // 8), np.uint32)
    s = np.empty((N, K // group), np.uint16)
    b = np.empty((N, K // group), np.uint16)
    rc = lib().oracle_requantize_w4(_ptr(w), N, K, group, _ptr(w4), _ptr(s), _ptr(b))
    if rc != 0:
        raise ValueError(f"oracle_requantize_w4 rejected its arguments (rc={rc})")
    return w4, s, b


def float_to_half(f: float) -> int:
    """Nearest-even binary16 bit pattern of a float32 value."""
    return int(lib().oracle_float_to_half(float(f)))
