"""GPU parity of the verify qmv against the fp64 oracle, through the C ABI.

Shapes: the 4096 x 1024 M=4 case; the verify-MLP projections (gate/up
5120 -> 17408, down 17408 -> 5120) at M = 1..8 and, in the wide form for
16-wide drafter blocks, M = 9, 12, 16; the attention projections
of the 64-layer 5120-hidden decoder (q 5120 -> 6144, k/v 5120 -> 1024, o
6144 -> 5120) at M = 3..6; the 151936-row LM head (W4 at M = 6, W8 at M = 8)
on sampled outputs; ragged and degenerate shapes.  Plus row independence
(row m of an M-row call equals the one-row call bitwise) and determinism.
"""
import numpy as np
import pytest

import oracle
from speculative_decoding_spec_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def run(bits, w, s, b, x, dev, G=64, layout="packed"):
    """y from the weights as stored (spec_qmv_w*, layout="interchange") or
    from the repacked copy (spec_qmv_w*_packed)."""
    import speculative_decoding_spec_amd as spec
    wt, st, bt = parity.dev_qweights(w, s, b, dev)
    xt = parity.dev_x(x, dev)
    if layout == "interchange":
        fn = spec.spec_qmv_w4 if bits == 4 else spec.spec_qmv_w8
        y = fn(wt, st, bt, xt, G=G)
    else:
        pack = spec.spec_pack_w4 if bits == 4 else spec.spec_pack_w8
        fn = spec.spec_qmv_w4_packed if bits == 4 else spec.spec_qmv_w8_packed
        y = fn(pack(wt, st, bt, G=G), xt)
    return y.cpu().numpy()


def full_check(bits, M, N, K, dev, cfg, salt=0):
    """Every output against the oracle; both layouts, bitwise equal."""
    w, s, b = synth.qweights(cfg, bits, N, K, 64, salt=salt)
    x = synth.activations(cfg, M, K, salt=salt)
    got = run(bits, w, s, b, x, dev)
    inter = run(bits, w, s, b, x, dev, layout="interchange")
    assert np.array_equal(got.view(np.uint32), inter.view(np.uint32)), "layouts differ"
    ref, mag = parity.oracle_qmv_threaded(bits, w, s, b, x, 64)
    nf, nabs, worst = parity.check_qmv(got, ref, mag)
    print(f"W{bits} M={M} N={N} K={K}: fail={nf} abs-only={nabs} worst_rel={worst:.2e}", flush=True)
    assert nf == 0
    assert nabs <= parity.abs_only_limit(got.size), nabs
    return got


def test_pr1_reference_shape(dev):
    full_check(4, 4, 4096, 1024, dev, cfg=0)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 16])
@pytest.mark.parametrize("shape", [(17408, 5120), (5120, 17408)], ids=["gate_up", "down"])
def test_verify_mlp_shapes(dev, M, shape):
    N, K = shape
    full_check(4, M, N, K, dev, cfg=1, salt=N)


@pytest.mark.parametrize("M", [3, 4, 5, 6])
@pytest.mark.parametrize("shape", [(6144, 5120), (1024, 5120), (5120, 6144)], ids=["q", "kv", "o"])
def test_attention_projection_shapes(dev, M, shape):
    N, K = shape
    full_check(4, M, N, K, dev, cfg=3, salt=N + 7 * K)


@pytest.mark.parametrize("bits,M", [(4, 6), (8, 8)])
def test_lm_head_sampled(dev, bits, M):
    N, K = 151936, 5120
    w, s, b = synth.qweights(2 if bits == 4 else 4, bits, N, K, 64)
    x = synth.activations(2 if bits == 4 else 4, M, K)
    got = run(bits, w, s, b, x, dev)
    inter = run(bits, w, s, b, x, dev, layout="interchange")
    assert np.array_equal(got.view(np.uint32), inter.view(np.uint32)), "layouts differ"
    rng = np.random.default_rng(17)
    n_idx = np.concatenate([np.arange(64), np.arange(N - 64, N), rng.integers(0, N, 1500)])
    m_idx = rng.integers(0, M, n_idx.shape[0])
    ref, mag = oracle.qmv_points(bits, w, s, b, x, 64, m_idx, n_idx)
    nf, nabs, worst = parity.check_qmv(got[m_idx, n_idx], ref, mag)
    print(f"LM head W{bits} M={M}: fail={nf} abs-only={nabs} worst_rel={worst:.2e}", flush=True)
    assert nf == 0
    assert nabs <= parity.abs_only_limit(n_idx.shape[0]), nabs
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("bits,M", [(4, 1), (4, 2), (4, 6), (8, 1), (8, 8)])
def test_lm_head_launch_shape_full(dev, bits, M):
    """The launch shapes of heads of 4096 tiles or more (W4: 4 tiles x 4 waves,
    2 tiles at M <= 2; W8: 2 tiles x 8 waves, 1 tile at M <= 2) on every
    output, at a K the oracle finishes fast: 65621 rows (4102 tiles, the last
    one of 5 rows; a ragged last workgroup of 4 tiles) x 256."""
    full_check(bits, M, 65621, 256, dev, cfg=2, salt=65600 + M)


@pytest.mark.parametrize("bits", [4, 8])
def test_lm_head_rows_do_not_depend_on_tiles_per_workgroup(dev, bits):
    """At M <= 2 a head launch takes half the tiles per workgroup; the waves
    and so every output's arithmetic are unchanged: rows of a 6-row call
    equal the one- and two-row calls bitwise."""
    w, s, b = synth.qweights(8, bits, 65621, 256, 64)
    x = synth.activations(8, 6, 256)
    full = run(bits, w, s, b, x, dev)
    for m in range(6):
        one = run(bits, w, s, b, np.ascontiguousarray(x[m:m + 1]), dev)
        assert np.array_equal(one[0].view(np.uint32), full[m].view(np.uint32)), m
    two = run(bits, w, s, b, np.ascontiguousarray(x[2:4]), dev)
    assert np.array_equal(two.view(np.uint32), full[2:4].view(np.uint32))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (3, 100, 192), (8, 77, 320), (5, 1000, 64 * 13),
                                   (2, 4095, 1024), (7, 129, 17408), (9, 77, 320),
                                   (13, 1000, 64 * 13), (16, 4095, 1024), (11, 129, 17408)])
def test_ragged_shapes(dev, bits, M, N, K):
    full_check(bits, M, N, K, dev, cfg=5, salt=M * 100000 + N + K)


@pytest.mark.parametrize("bits", [4, 8])
def test_w8_full_small(dev, bits):
    full_check(bits, 8, 2048, 5120, dev, cfg=4, salt=3)


def test_degenerate_shapes(dev):
    import torch
    import speculative_decoding_spec_amd as spec
    # K = 0: every output is an empty sum.
    pk = spec.spec_pack_w4(torch.zeros((16, 0), dtype=torch.int32, device=dev),
                           torch.zeros((16, 0), dtype=torch.float16, device=dev),
                           torch.zeros((16, 0), dtype=torch.float16, device=dev))
    y = torch.full((3, 16), 7.0, device=dev)
    spec.spec_qmv_w4_packed(pk, torch.zeros((3, 0), dtype=torch.bfloat16, device=dev), y=y)
    assert torch.all(y == 0)
    # M = 0 is a no-op.
    pk = spec.spec_pack_w4(torch.zeros((16, 8), dtype=torch.int32, device=dev),
                           torch.zeros((16, 1), dtype=torch.float16, device=dev),
                           torch.zeros((16, 1), dtype=torch.float16, device=dev))
    spec.spec_qmv_w4_packed(pk, torch.zeros((0, 64), dtype=torch.bfloat16, device=dev))
    torch.cuda.synchronize()


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("N,K", [(5120, 17408), (4096, 1024)])
def test_row_independence_and_determinism(dev, bits, N, K):
    """Row m of any call equals the one-row call bitwise, across the 8-row
    boundary between the pair form and the wide form as well."""
    w, s, b = synth.qweights(6, bits, N, K, 64)
    x = synth.activations(6, 16, K)
    full = run(bits, w, s, b, x, dev)
    again = run(bits, w, s, b, x, dev)
    assert np.array_equal(full.view(np.uint32), again.view(np.uint32))
    for m in range(16):
        one = run(bits, w, s, b, np.ascontiguousarray(x[m:m + 1]), dev)
        assert np.array_equal(one[0].view(np.uint32), full[m].view(np.uint32)), m
    for M in (3, 5, 8, 9, 12):
        part = run(bits, w, s, b, np.ascontiguousarray(x[:M]), dev)
        assert np.array_equal(part.view(np.uint32), full[:M].view(np.uint32)), M


def test_bound_call_matches_plain_call(dev):
    import torch
    import speculative_decoding_spec_amd as spec
    w, s, b = synth.qweights(7, 4, 4096, 1024, 64)
    x = synth.activations(7, 5, 1024)
    wt, st, bt = parity.dev_qweights(w, s, b, dev)
    pk = spec.spec_pack_w4(wt, st, bt)
    xt = parity.dev_x(x, dev)
    y = torch.empty((5, 4096), dtype=torch.float32, device=dev)
    call = spec.bind_qmv(pk, xt, y)
    first = y.clone()
    y.fill_(float("nan"))
    call()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), first.view(torch.int32))
    assert torch.equal(spec.spec_qmv_w4_packed(pk, xt).view(torch.int32), y.view(torch.int32))


def test_fused_gate_up_matches_separate_launches(dev):
    """Packing the gate and up projections as one 5120 -> 34816 matrix (one
    launch) gives bitwise the outputs of the two separate launches."""
    import torch
    import speculative_decoding_spec_amd as spec
    K, N = 5120, 17408
    gate = synth.qweights(8, 4, N, K, 64, salt=1)
    up = synth.qweights(8, 4, N, K, 64, salt=2)
    x = parity.dev_x(synth.activations(8, 6, K), dev)
    g = spec.spec_pack_w4(*parity.dev_qweights(*gate, dev))
    u = spec.spec_pack_w4(*parity.dev_qweights(*up, dev))
    cat = [np.concatenate([a, b], axis=0) for a, b in zip(gate, up)]
    gu = spec.spec_pack_w4(*parity.dev_qweights(*cat, dev))
    y = spec.spec_qmv_w4_packed(gu, x)
    assert torch.equal(y[:, :N].view(torch.int32), spec.spec_qmv_w4_packed(g, x).view(torch.int32))
    assert torch.equal(y[:, N:].view(torch.int32), spec.spec_qmv_w4_packed(u, x).view(torch.int32))


@pytest.mark.parametrize("M", [3, 6])
def test_fused_qkv_matches_separate_launches(dev, M):
    """q (5120 -> 6144), k and v (5120 -> 1024 each) share their input: packed
    as one 5120 -> 8192 matrix they give bitwise the three separate outputs,
    which match the oracle on sampled outputs."""
    import torch
    import speculative_decoding_spec_amd as spec
    K = 5120
    parts = [synth.qweights(9, 4, n, K, 64, salt=s) for n, s in ((6144, 1), (1024, 2), (1024, 3))]
    xa = synth.activations(9, M, K)
    x = parity.dev_x(xa, dev)
    cat = [np.concatenate(list(t), axis=0) for t in zip(*parts)]
    y = spec.spec_qmv_w4_packed(spec.spec_pack_w4(*parity.dev_qweights(*cat, dev)), x)
    lo = 0
    for p in parts:
        n = p[0].shape[0]
        ys = spec.spec_qmv_w4_packed(spec.spec_pack_w4(*parity.dev_qweights(*p, dev)), x)
        assert torch.equal(y[:, lo:lo + n].view(torch.int32), ys.view(torch.int32))
        lo += n
    rng = np.random.default_rng(M)
    m_idx, n_idx = rng.integers(0, M, 256), rng.integers(0, 8192, 256)
    ref, mag = oracle.qmv_points(4, *cat, xa, 64, m_idx, n_idx)
    nf, _, _ = parity.check_qmv(y.cpu().numpy()[m_idx, n_idx], ref, mag)
    assert nf == 0


@pytest.mark.parametrize("bits", [4, 8])
def test_long_k(dev, bits):
    """K = 131072 (1024 pairs per row, 64-128 per wave) on two ragged tiles."""
    full_check(bits, 8, 30, 131072, dev, cfg=10, salt=bits)


@pytest.mark.parametrize("bits", [4, 8])
def test_interchange_scales_not_8_byte_aligned(dev, bits):
    """Scales and biases on odd 2-byte offsets (rows of 80 groups, a multiple
    of 4, so only the alignment rules out the 8-byte scale/bias loads): the
    2-byte-load form, bitwise equal to the packed copy."""
    import torch
    import speculative_decoding_spec_amd as spec
    N, K, M = 1000, 5120, 5
    w, s, b = synth.qweights(11, bits, N, K, 64)
    x = parity.dev_x(synth.activations(11, M, K), dev)
    wt, st, bt = parity.dev_qweights(w, s, b, dev)

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=torch.float16, device=dev)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        assert v.data_ptr() % 8 != 0
        return v
    fn = spec.spec_qmv_w4 if bits == 4 else spec.spec_qmv_w8
    pack = spec.spec_pack_w4 if bits == 4 else spec.spec_pack_w8
    yi = fn(wt, shifted(st), shifted(bt), x).cpu().numpy()
    yp = (spec.spec_qmv_w4_packed if bits == 4 else spec.spec_qmv_w8_packed)(pack(wt, st, bt), x).cpu().numpy()
    assert np.array_equal(yi.view(np.uint32), yp.view(np.uint32))
