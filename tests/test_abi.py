"""The C ABI: the library loads, exports every function include/spec.h
declares, and rejects bad arguments on the host before touching a GPU.

Validation runs before any HIP call, so these checks need no device: the
pointers below are never dereferenced."""
import ctypes
import os
import re

import pytest

import speculative_decoding_spec_amd as spec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
P = ctypes.c_void_p(0x10000)      # fake, 256-byte aligned device address
P2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10004)    # 4-byte aligned, not 16-byte aligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return spec.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(L, n), f"libspec.so does not export {n}"
    out = os.popen(f"nm -D --defined-only {spec.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def test_status_strings(L):
    assert L.spec_status_str(0) == b"SPEC_OK"
    assert L.spec_status_str(3) == b"SPEC_ERR_WORKSPACE"
    assert L.spec_version() >= 100


def qmv(L, fn="spec_qmv_w4_packed", w=P, sb=P, x=P, y=P, M=4, N=64, K=128, G=64, b=P2):
    if fn.endswith("_packed") or fn.endswith("_valu"):
        return getattr(L, fn)(w, sb, x, y, M, N, K, G, None)
    return getattr(L, fn)(w, sb, b, x, y, M, N, K, G, None)


def pack(L, fn="spec_pack_w4", w=P, s=P, b=P, N=64, K=128, G=64, wp=P, sbp=P2):
    return getattr(L, fn)(w, s, b, N, K, G, wp, sbp, None)


@pytest.mark.parametrize("fn", ["spec_qmv_w4", "spec_qmv_w8", "spec_qmv_w4_packed",
                                "spec_qmv_w8_packed"])
def test_qmv_validation(L, fn):
    assert qmv(L, fn, M=-1) == INVALID
    assert qmv(L, fn, K=100) == INVALID            # K % G != 0
    assert qmv(L, fn, G=32, K=128) == UNSUPPORTED
    assert qmv(L, fn, M=17) == UNSUPPORTED
    assert qmv(L, fn, M=0) == OK
    assert qmv(L, fn, w=None) == INVALID
    assert qmv(L, fn, sb=None) == INVALID
    assert qmv(L, fn, x=None) == INVALID
    assert qmv(L, fn, y=None) == INVALID
    assert qmv(L, fn, w=MIS) == UNSUPPORTED
    assert qmv(L, fn, x=MIS) == UNSUPPORTED
    assert qmv(L, fn, M=0) == OK                   # no-op, nothing enqueued
    assert qmv(L, fn, N=0) == OK
    # 32-bit buffer ranges and offsets in the kernel: K below 2^24, N at most 2^28
    assert qmv(L, fn, K=1 << 24) == UNSUPPORTED
    assert qmv(L, fn, N=(1 << 28) + 1) == UNSUPPORTED
    if not fn.endswith("_packed"):
        assert qmv(L, fn, b=None) == INVALID
        assert qmv(L, fn, b=ctypes.c_void_p(0x20001)) == INVALID    # fp16 biases, odd address
        assert qmv(L, fn, sb=ctypes.c_void_p(0x10001)) == INVALID   # fp16 scales, odd address


def test_valu_variant_validation(L):
    fn = "spec_qmv_w4_packed_valu"
    assert qmv(L, fn, M=-1) == INVALID
    assert qmv(L, fn, K=100) == INVALID
    assert qmv(L, fn, G=32, K=128) == UNSUPPORTED
    assert qmv(L, fn, M=5) == UNSUPPORTED           # the vector-ALU variant serves M <= 4
    assert qmv(L, fn, M=0) == OK
    assert qmv(L, fn, w=None) == INVALID
    assert qmv(L, fn, x=MIS) == UNSUPPORTED
    assert qmv(L, fn, K=1 << 24) == UNSUPPORTED
    g = L.spec_qmv_gate_up_silu_w4_valu
    assert g(P, P, P, P, 5, 64, 128, 64, None) == UNSUPPORTED
    assert g(P, P, P, P, -1, 64, 128, 64, None) == INVALID
    assert g(P, P, P, ctypes.c_void_p(0x20001), 2, 64, 128, 64, None) == INVALID   # bf16 h, odd
    assert g(P, P, MIS, P, 2, 64, 128, 64, None) == UNSUPPORTED
    assert g(P, P, P, P, 0, 64, 128, 64, None) == OK


@pytest.mark.parametrize("fn", ["spec_pack_w4", "spec_pack_w8"])
def test_pack_validation(L, fn):
    assert pack(L, fn, N=-1) == INVALID
    assert pack(L, fn, K=96) == INVALID            # K % G != 0
    assert pack(L, fn, G=128, K=256) == UNSUPPORTED
    assert pack(L, fn, w=None) == INVALID
    assert pack(L, fn, s=None) == INVALID
    assert pack(L, fn, wp=None) == INVALID
    assert pack(L, fn, w=MIS) == UNSUPPORTED
    assert pack(L, fn, N=0) == OK


def test_packed_sizes(L):
    # 16-row tiles x 128-wide K steps of 1 KB (W4) / 2 KB (W8); one 32-bit
    # scale/bias word per row and group, in blocks of two K steps (256 B per
    # tile and block, the last block padded).
    assert L.spec_qmv_packed_weight_bytes(4, 5120, 17408, 64) == 320 * 136 * 1024
    assert L.spec_qmv_packed_weight_bytes(8, 151936, 5120, 64) == 9496 * 40 * 2048
    assert L.spec_qmv_packed_weight_bytes(4, 100, 192, 64) == 7 * 2 * 1024   # ragged N, odd groups
    assert L.spec_qmv_packed_sb_bytes(100, 192, 64) == 7 * 1 * 256
    assert L.spec_qmv_packed_sb_bytes(100, 320, 64) == 7 * 2 * 256        # 3 K steps -> 2 blocks
    assert L.spec_qmv_packed_weight_bytes(4, 64, 100, 64) == 0           # invalid shape


def accept(L, t=P, d=P, tok=P, u=P, B=2, D=3, V=1024, T=0.6, k=0, p=1.0,
           acc=P, nxt=P, ws=None, nbytes=None):
    if nbytes is None:
        nbytes = L.spec_verify_accept_workspace(B, D, V, k)
        ws = ws or P2
    return L.spec_verify_accept(t, d, tok, u, B, D, V, ctypes.c_float(T), k,
                                ctypes.c_float(p), acc, nxt, None, None, ws,
                                nbytes, None)


def test_accept_validation(L):
    assert accept(L, B=-1) == INVALID
    assert accept(L, D=16) == UNSUPPORTED
    assert accept(L, V=1) == INVALID
    assert accept(L, T=float("nan")) == INVALID
    assert accept(L, T=float("inf")) == INVALID
    assert accept(L, p=float("nan")) == INVALID
    assert accept(L, k=0, p=0.9) == UNSUPPORTED    # top-p over 1024 tokens
    assert accept(L, k=300, p=1.0) == UNSUPPORTED  # top-k above 256
    assert accept(L, t=None) == INVALID
    assert accept(L, d=None) == INVALID
    assert accept(L, tok=None) == INVALID
    assert accept(L, u=None) == INVALID
    assert accept(L, acc=None) == INVALID
    assert accept(L, t=MIS) == UNSUPPORTED         # V % 4 == 0 needs 16 B rows
    assert accept(L, ws=None, nbytes=0) == WORKSPACE
    assert accept(L, B=0) == OK
    need = L.spec_verify_accept_workspace(4, 5, 151936, 20)
    assert accept(L, B=4, D=5, V=151936, k=20, p=0.95, ws=P2, nbytes=need - 1) == WORKSPACE
    # D = 0 needs no draft arrays
    assert accept(L, d=None, tok=None, D=0, B=0) == OK


def test_sample_validation(L):
    f = ctypes.c_float
    need = L.spec_sample_workspace_size(4, 1000, 20)
    assert L.spec_sample_probs(P, 4, 1000, f(0.6), 20, f(0.9), P, None, 0, None) == WORKSPACE
    assert L.spec_sample_probs(None, 4, 1000, f(0.6), 20, f(0.9), P, P2, need, None) == INVALID
    assert L.spec_sample_probs(P, 4, 1, f(0.6), 20, f(0.9), P, P2, need, None) == INVALID
    assert L.spec_sample_tokens(P, 4, 1000, f(0.6), 0, f(0.5), P, P, P2, need, None) == UNSUPPORTED
    assert L.spec_sample_tokens(P, 0, 1000, f(0.6), 20, f(0.9), P, P, P2, need, None) == OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(spec, "_lib", None)
    monkeypatch.setattr(spec, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        spec.lib()


def greedy(L, t=P, tok=P, B=4, D=3, V=1000, acc=P, nxt=P, ws=None, nbytes=None):
    if nbytes is None:
        nbytes = L.spec_verify_greedy_workspace(B, D, V)
        ws = ws or P2
    return L.spec_verify_greedy(t, tok, B, D, V, acc, nxt, ws, nbytes, None)


def test_greedy_validation(L):
    assert greedy(L, B=-1) == INVALID
    assert greedy(L, D=-1) == INVALID
    assert greedy(L, V=1) == INVALID
    assert greedy(L, D=16) == UNSUPPORTED
    assert greedy(L, V=1 << 24) == UNSUPPORTED
    assert greedy(L, t=None) == INVALID
    assert greedy(L, tok=None) == INVALID
    assert greedy(L, acc=None) == INVALID
    assert greedy(L, nxt=None) == INVALID
    assert greedy(L, t=MIS) == UNSUPPORTED          # V % 4 == 0 needs 16 B rows
    assert greedy(L, t=ctypes.c_void_p(0x10002), V=999) == INVALID   # not 4-byte aligned
    assert greedy(L, ws=None, nbytes=0) == WORKSPACE
    need = L.spec_verify_greedy_workspace(256, 5, 151936)
    assert need == 256 * 6 * 16                     # one record per row: one chunk each
    assert greedy(L, B=256, D=5, V=151936, nbytes=need - 1, ws=P2) == WORKSPACE
    assert greedy(L, B=0) == OK
    assert greedy(L, tok=None, D=0, B=0) == OK
    # a single row splits into chunks of whole 1024-logit multiples
    assert L.spec_verify_greedy_workspace(1, 0, 151936) == 75 * 16
    assert L.spec_verify_greedy_workspace(0, 0, 1000) == 0


def test_gdn_validation(L):
    def rec(S0=P, q=P, k=P, v=P, a=P, b=P, B=2, T=6, H=4, dk=128, dv=128, o=P, d=P, sf=None):
        return L.spec_gdn_record(S0, q, k, v, a, b, B, T, H, dk, dv, o, d, sf, None)

    def com(S=P, a=P, k=P, d=P, n=P, B=2, T=6, H=4, dk=128, dv=128):
        return L.spec_gdn_commit(S, a, k, d, n, B, T, H, dk, dv, None)

    assert rec(B=-1) == INVALID and rec(T=-1) == INVALID and rec(dk=0) == INVALID
    assert rec(dk=64) == UNSUPPORTED and rec(dv=256) == UNSUPPORTED
    assert rec(T=17) == UNSUPPORTED
    assert rec(B=1 << 15, H=1 << 15) == UNSUPPORTED
    assert rec(S0=None) == INVALID and rec(q=None) == INVALID and rec(d=None) == INVALID
    assert rec(S0=MIS) == UNSUPPORTED and rec(k=MIS) == UNSUPPORTED
    assert rec(B=0) == OK and rec(H=0) == OK
    assert com(B=-1) == INVALID and com(dk=64) == UNSUPPORTED and com(T=17) == UNSUPPORTED
    assert com(S=None) == INVALID and com(n=None) == INVALID
    assert com(S=MIS) == UNSUPPORTED
    assert com(T=0) == OK and com(B=0) == OK


def test_gdn_commit_record_validation(L):
    # separate fake buffers 16 MB apart, so only the cases named overlap
    buf = {n: ctypes.c_void_p((i + 1) << 24) for i, n in enumerate(
        ["S", "pa", "pk", "pd", "n", "q", "k", "v", "a", "b", "o", "d", "sf"])}

    def cr(B=2, Tp=6, T=6, H=4, dk=128, dv=128, **kw):
        a = dict(buf, **kw)
        return L.spec_gdn_commit_record(a["S"], a["pa"], a["pk"], a["pd"], a["n"], Tp, a["q"],
                                        a["k"], a["v"], a["a"], a["b"], B, T, H, dk, dv,
                                        a["o"], a["d"], a["sf"], None)

    assert cr(B=-1) == INVALID and cr(Tp=-1) == INVALID and cr(T=-1) == INVALID
    assert cr(dk=64) == UNSUPPORTED and cr(Tp=17) == UNSUPPORTED and cr(T=17) == UNSUPPORTED
    assert cr(B=1 << 15, H=1 << 15) == UNSUPPORTED
    assert cr(S=None) == INVALID and cr(n=None) == INVALID and cr(pd=None) == INVALID
    assert cr(q=None) == INVALID and cr(o=None) == INVALID
    assert cr(S=MIS) == UNSUPPORTED and cr(pk=MIS) == UNSUPPORTED and cr(k=MIS) == UNSUPPORTED
    assert cr(pa=ctypes.c_void_p(0x10002)) == INVALID
    assert cr(B=0) == OK and cr(H=0) == OK
    # outputs sharing memory with any other argument are refused
    assert cr(d=buf["pd"]) == INVALID                   # one tape buffer for both cycles
    assert cr(o=buf["d"]) == INVALID
    assert cr(sf=buf["S"]) == INVALID
    assert cr(S=buf["k"]) == INVALID
    assert cr(o=ctypes.c_void_p(buf["q"].value + 4096)) == INVALID   # partial overlap
    # with nothing to commit (or record) those arguments may be NULL: the
    # first error met is then the misaligned state
    none_prev = dict(pa=None, pk=None, pd=None, n=None)
    none_next = dict(q=None, k=None, v=None, a=None, b=None, o=None, d=None)
    assert cr(Tp=0, S=MIS, **none_prev) == UNSUPPORTED
    assert cr(T=0, S=MIS, **none_next) == UNSUPPORTED
    assert cr(Tp=0, T=0, S=MIS, sf=None, **none_prev, **none_next) == UNSUPPORTED


def test_stream_read_validation(L):
    L.spec_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    f = L.spec_stream_read
    assert f(P, 100, P2, None) == INVALID                      # not a multiple of 16
    assert f(None, 64, P2, None) == INVALID
    assert f(P, 64, None, None) == INVALID
    assert f(P, 64, ctypes.c_void_p(0x20002), None) == INVALID  # sink not 4-byte aligned
    assert f(MIS, 64, P2, None) == UNSUPPORTED                 # src not 16-byte aligned


def test_requantize_validation(L):
    f = L.spec_requantize_w4
    assert f(P, -1, 128, 64, P, P, P, None) == INVALID
    assert f(P, 4, 100, 64, P, P, P, None) == INVALID      # K % G
    assert f(P, 4, 128, 32, P, P, P, None) == UNSUPPORTED
    assert f(None, 4, 128, 64, P, P, P, None) == INVALID
    assert f(MIS, 4, 128, 64, P, P, P, None) == UNSUPPORTED
    assert f(P, 4, 128, 64, P, ctypes.c_void_p(0x10001), P, None) == INVALID
    assert f(P, 0, 128, 64, P, P, P, None) == OK


def test_noalloc_rejects_workspace_beyond_its_scratch(L):
    """spec_verify_accept_noalloc refuses, before touching a device, a call
    whose workspace exceeds its fixed scratch (8192 sequences of D = 5 over
    151936 tokens need about 39 MB of block sums), and validates like
    spec_verify_accept otherwise."""
    f = L.spec_verify_accept_noalloc
    args = lambda B, D, V, T=0.6, k=0, p=1.0: (P, P2, P, P, B, D, V, T, k, p, P, P2, None, None, None)
    assert f(*args(8192, 5, 151936)) == WORKSPACE
    assert f(*args(-1, 5, 1000)) == INVALID
    assert f(*args(4, 16, 1000)) == UNSUPPORTED
    assert f(*args(4, 5, 1)) == INVALID
    assert f(*args(0, 5, 1000)) == OK
    assert f(P, None, P, P, 4, 3, 1000, 0.6, 0, 1.0, P, P2, None, None, None) == INVALID
