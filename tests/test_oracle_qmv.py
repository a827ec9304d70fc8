"""Pins of the oracle's qmv against facts fixed outside the oracle itself.

Each check is chosen so that a plausible slip in the oracle (a wrong nibble
order, a swapped scale/bias, a dropped group term, a transposed operand, a
wrong fp16/bf16 decode) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
from speculative_decoding_spec_amd import synth


def _np_dequant(bits, w, s16, b16, K, G):
    """Independent decode with numpy primitives (bit ops, numpy's float16)."""
    if bits == 4:
        shifts = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
        q = ((w[:, :, None] >> shifts) & 0xF).reshape(w.shape[0], K)
    else:
        q = w.astype(np.int64)
    s = s16.view(np.float16).astype(np.float64)
    b = b16.view(np.float16).astype(np.float64)
    return q * np.repeat(s, G, axis=1) + np.repeat(b, G, axis=1)


def _np_x(x16):
    return synth.bf16_bits_to_f32(x16).astype(np.float64)


def test_format_decoders_against_known_bit_patterns():
    # IEEE binary16: 1.0, smallest subnormal, largest normal, -2, 1/3 rounded.
    assert oracle.half_to_double(0x3C00) == 1.0
    assert oracle.half_to_double(0x0001) == 2.0**-24
    assert oracle.half_to_double(0x7BFF) == 65504.0
    assert oracle.half_to_double(0xC000) == -2.0
    assert oracle.half_to_double(0x3555) == 0.333251953125
    assert oracle.half_to_double(0x8000) == 0.0
    # bfloat16 is the top half of a binary32.
    assert oracle.bf16_to_double(0x3F80) == 1.0
    assert oracle.bf16_to_double(0xC2F7) == -123.5
    # Every fp16 pattern agrees with numpy's decoder.
    pats = np.arange(0, 65536, 7, dtype=np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(p)) for p in pats])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])


def test_bf16_rounding_matches_torch():
    import torch
    a = np.random.default_rng(5).normal(0, 3, size=4096).astype(np.float32)
    a[:4] = [1.00390625, 1.01171875, -2.0, 0.0]  # exact halfway cases included
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(a), ref)


@pytest.mark.parametrize("bits", [4, 8])
def test_matches_numpy_matmul(bits):
    M, N, K, G = 3, 37, 256, 64
    w, s, b = synth.qweights(11, bits, N, K, G)
    x = synth.activations(11, M, K)
    y = oracle.qmv(bits, w, s, b, x, G)
    ref = _np_x(x) @ _np_dequant(bits, w, s, b, K, G).T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_hand_computed_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "qmv_hand_m1_k64_n2.json")))
    w = np.array(g["w_words"], dtype=np.uint32)
    s = np.array(g["scales_fp16"], dtype=np.uint16)
    b = np.array(g["biases_fp16"], dtype=np.uint16)
    x = np.array([[g["x_bf16_first32"]] * 32 + [g["x_bf16_last32"]] * 32], dtype=np.uint16)
    y = oracle.qmv(4, w, s, b, x, g["G"])
    assert y[0].tolist() == g["y"]


def test_nibble_order_little_endian():
    # Word 0x76543210 holds codes 0..7 at elements 0..7; with s = 1, b = 0 and
    # x = e_k, the output is the code of element k.
    K, G = 64, 64
    w = np.full((1, K // 8), 0x76543210, dtype=np.uint32)
    s = np.full((1, 1), 0x3C00, dtype=np.uint16)
    b = np.zeros((1, 1), dtype=np.uint16)
    x = np.zeros((K, K), dtype=np.uint16)
    x[np.arange(K), np.arange(K)] = 0x3F80
    y = oracle.qmv(4, w, s, b, x, G)
    assert y[:, 0].tolist() == [float(k % 8) for k in range(K)]


@pytest.mark.parametrize("bits", [4, 8])
def test_zero_codes_give_bias_times_group_sums(bits):
    M, N, K, G = 2, 5, 192, 64
    _, s, b = synth.qweights(3, bits, N, K, G)
    w = np.zeros((N, K // 8), np.uint32) if bits == 4 else np.zeros((N, K), np.uint8)
    x = synth.activations(3, M, K)
    y = oracle.qmv(bits, w, s, b, x, G)
    xs = _np_x(x).reshape(M, K // G, G).sum(axis=2)           # [M][groups]
    ref = xs @ b.view(np.float16).astype(np.float64).T        # sum_g b_g X_g
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_one_hot_codes_select_one_activation():
    # s = 1, b = 0 and a single code 1 at column c_n: y[m][n] = x[m][c_n] exactly.
    M, N, K, G = 4, 16, 128, 64
    rng = np.random.default_rng(9)
    cols = rng.integers(0, K, size=N)
    w = np.zeros((N, K // 8), np.uint32)
    for n, c in enumerate(cols):
        w[n, c // 8] = np.uint32(1) << np.uint32(4 * (c % 8))
    s = np.full((N, K // G), 0x3C00, np.uint16)
    b = np.zeros((N, K // G), np.uint16)
    x = synth.activations(4, M, K)
    y = oracle.qmv(4, w, s, b, x, G)
    assert np.array_equal(y, _np_x(x)[:, cols])


def test_unit_activations_give_scaled_code_sums():
    M, N, K, G = 1, 9, 256, 64
    w, s, _ = synth.qweights(5, 4, N, K, G)
    b = np.zeros_like(s)
    x = np.full((M, K), 0x3F80, np.uint16)
    y = oracle.qmv(4, w, s, b, x, G)
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
    q = ((w[:, :, None] >> shifts) & 0xF).reshape(N, K).astype(np.float64)
    qs = q.reshape(N, K // G, G).sum(axis=2)
    ref = (qs * s.view(np.float16).astype(np.float64)).sum(axis=1)
    np.testing.assert_allclose(y[0], ref, rtol=1e-14)


def test_w4_reencoded_as_w8_is_bitwise_identical():
    M, N, K, G = 2, 11, 320, 64
    w4, s, b = synth.qweights(6, 4, N, K, G)
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
    w8 = ((w4[:, :, None] >> shifts) & 0xF).reshape(N, K).astype(np.uint8)
    x = synth.activations(6, M, K)
    assert np.array_equal(oracle.qmv(4, w4, s, b, x, G), oracle.qmv(8, w8, s, b, x, G))


def test_row_window_and_points_agree_with_full():
    M, N, K, G = 3, 40, 128, 64
    w, s, b = synth.qweights(7, 4, N, K, G)
    x = synth.activations(7, M, K)
    full, mag = oracle.qmv(4, w, s, b, x, G, with_abs=True)
    part = oracle.qmv(4, w, s, b, x, G, rows=(10, 25))
    assert np.array_equal(part, full[:, 10:25])
    mi = np.array([0, 2, 1, 2]); ni = np.array([0, 39, 17, 3])
    y, a = oracle.qmv_points(4, w, s, b, x, G, mi, ni)
    assert np.array_equal(y, full[mi, ni]) and np.array_equal(a, mag[mi, ni])
    assert np.all(mag >= np.abs(full))


def test_rejects_bad_arguments():
    w, s, b = synth.qweights(8, 4, 4, 128, 64)
    x = synth.activations(8, 1, 128)
    with pytest.raises(ValueError):
        oracle.qmv(4, w, s, b, x, 48)     # K % G != 0
    with pytest.raises(ValueError):
        oracle.qmv(5, w, s, b, x, 64)     # unsupported width


# ------------------------------------------- SiLU-gated MLP activation ----

def test_double_to_bf16_known_patterns_and_ties():
    r = oracle.double_to_bf16
    assert r(1.0) == 0x3F80 and r(-2.0) == 0xC000 and r(0.0) == 0x0000
    assert r(-0.0) == 0x8000
    assert r(1 + 2**-8) == 0x3F80            # halfway: to the even neighbour 1.0
    assert r(1 + 3 * 2**-8) == 0x3F82        # halfway: to the even neighbour above
    assert r(1 + 2**-8 + 2**-40) == 0x3F81   # just above halfway (a double-only case)
    assert r(-123.5) == 0xC2F7
    assert r(2.0**-133) == 0x0001            # smallest subnormal
    assert r(2.0**-134) == 0x0000            # halfway to zero: even
    assert r(3 * 2.0**-134) == 0x0002        # halfway between 1 and 2 subnormal ulps
    assert r(2.0**128) == 0x7F80             # overflow
    assert r(float.fromhex("0x1.fffp127")) == 0x7F80   # rounds up past the largest finite


def test_double_to_bf16_matches_torch_on_float32_values():
    # Every float32 is a double, and torch's float32 -> bfloat16 conversion is
    # nearest-even: the two must agree on all of them (subnormals included).
    import torch
    rng = np.random.default_rng(6)
    a = np.concatenate([rng.normal(0, 3, 3000), rng.normal(0, 1e-39, 500),
                        rng.normal(0, 1e30, 500)]).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.double_to_bf16(float(v)) for v in a], np.uint16)
    assert np.array_equal(got, ref)


def test_double_to_bf16_is_the_nearest():
    rng = np.random.default_rng(7)
    for v in rng.normal(0, 10, 2000):
        b = oracle.double_to_bf16(v)
        d = abs(oracle.bf16_to_double(b) - v)
        assert d <= abs(oracle.bf16_to_double(b + 1) - v)
        assert d <= abs(oracle.bf16_to_double(b - 1) - v)


def test_gate_up_silu_matches_numpy():
    import scipy.special
    M, F, K, G = 3, 40, 256, 64
    gate = synth.qweights(12, 4, F, K, G, salt=1)
    up = synth.qweights(12, 4, F, K, G, salt=2)
    x = synth.activations(12, M, K)
    h, hb = oracle.gate_up_silu(4, gate, up, x, G)
    g = _np_x(x) @ _np_dequant(4, *gate, K, G).T
    u = _np_x(x) @ _np_dequant(4, *up, K, G).T
    ref = g * scipy.special.expit(g) * u
    np.testing.assert_allclose(h, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(hb, np.vectorize(oracle.double_to_bf16)(h).astype(np.uint16))
    h2, hb2 = oracle.gate_up_silu(4, gate, up, x, G, rows=(7, 19))
    assert np.array_equal(h2, h[:, 7:19]) and np.array_equal(hb2, hb[:, 7:19])


def test_gate_up_silu_closed_forms():
    # Zero gate codes and biases: g = 0, silu(0) = 0, h = 0 for any up.
    M, F, K, G = 2, 16, 128, 64
    up = synth.qweights(13, 8, F, K, G)
    x = synth.activations(13, M, K)
    z = (np.zeros((F, K), np.uint8), up[1], np.zeros_like(up[2]))
    h, hb = oracle.gate_up_silu(8, z, up, x, G)
    assert np.all(h == 0.0) and np.all((hb & 0x7FFF) == 0)
    # Opposite gates: silu(g) - silu(-g) = g, so h(g) - h(-g) = g * u.
    b = np.full((F, K // G), 0x3C00, np.uint16)          # bias +1.0
    gp = (np.zeros((F, K), np.uint8), up[1], b)
    gm = (np.zeros((F, K), np.uint8), up[1], b | 0x8000)  # bias -1.0
    hp, _ = oracle.gate_up_silu(8, gp, up, x, G)
    hm, _ = oracle.gate_up_silu(8, gm, up, x, G)
    g = oracle.qmv(8, *gp, x, G)
    u = oracle.qmv(8, *up, x, G)
    np.testing.assert_allclose(hp - hm, g * u, rtol=1e-12, atol=1e-12)


# ------------------------------------------ draft-only 4-bit requantization ----

def test_float_to_half_matches_numpy():
    # numpy's float32 -> float16 conversion is nearest-even: agree on normal,
    # subnormal, overflowing and halfway values
    rng = np.random.default_rng(8)
    a = np.concatenate([rng.normal(0, 3, 4000), rng.normal(0, 1e-5, 2000),
                        rng.normal(0, 3e4, 1000),
                        [65504, 65519.99, 65520, 2.0**-25, 3 * 2.0**-26, 1 + 2.0**-11]]).astype(np.float32)
    with np.errstate(over="ignore"):
        ref = a.astype(np.float16).view(np.uint16)
    got = np.array([oracle.float_to_half(float(v)) for v in a], np.uint16)
    assert np.array_equal(got, ref)


def _bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_requantize_recovers_grid_values_exactly():
    # weights on the affine grid b + s q with s, b exact in fp16 and the
    # group's min and max present: codes, scales and biases come back exactly
    rng = np.random.default_rng(9)
    N, K, G = 6, 128, 64
    q = rng.integers(0, 16, size=(N, K))
    q[:, ::G] = 0
    q[:, 1::G] = 15
    # power-of-two steps and biases on a 1/32 grid: every b + s q is an
    # integer over 32 below 2^7, exact in bf16 (8 significant bits) and fp16
    s = (2.0 ** -rng.integers(3, 6, size=(N, K // G))).astype(np.float32)
    b = (rng.integers(-32, 33, size=(N, K // G)) / 32.0).astype(np.float32)
    w = q * np.repeat(s, G, axis=1) + np.repeat(b, G, axis=1)
    wb = _bf16(w)
    assert np.array_equal(synth.bf16_bits_to_f32(wb), w.astype(np.float32))  # exact in bf16
    w4, s16, b16 = oracle.requantize_w4(wb, G)
    assert np.array_equal(s16.view(np.float16).astype(np.float32), s)
    assert np.array_equal(b16.view(np.float16).astype(np.float32), b)
    shifts = 4 * np.arange(8, dtype=np.uint32)
    codes = ((w4[:, :, None] >> shifts) & 0xF).reshape(N, K)
    assert np.array_equal(codes, q)


def test_requantize_error_is_at_most_half_a_step():
    rng = np.random.default_rng(10)
    N, K, G = 8, 256, 64
    wb = _bf16(rng.normal(0, 0.05, size=(N, K)))
    w = synth.bf16_bits_to_f32(wb).astype(np.float64)
    w4, s16, b16 = oracle.requantize_w4(wb, G)
    s = np.repeat(s16.view(np.float16).astype(np.float64), G, axis=1)
    b = np.repeat(b16.view(np.float16).astype(np.float64), G, axis=1)
    shifts = 4 * np.arange(8, dtype=np.uint32)
    q = ((w4[:, :, None] >> shifts) & 0xF).reshape(N, K)
    err = np.abs(q * s + b - w)
    # half a step, plus what the fp16 rounding of s and b can add at the ends
    slack = 15 * np.abs(s) * 2.0**-11 + np.abs(b) * 2.0**-11 + 1e-12
    assert np.all(err <= s / 2 + slack)
    # and the codes use the whole range in every group
    assert np.all(q.reshape(N, K // G, G).min(axis=2) == 0)
    assert np.all(q.reshape(N, K // G, G).max(axis=2) == 15)


def test_requantize_ties_and_constant_groups():
    G = 64
    # a constant group: scale 0, codes 0, the bias carries the value
    w = np.full((1, G), 0.375, np.float32)
    w4, s16, b16 = oracle.requantize_w4(_bf16(w), G)
    assert s16[0, 0] == 0 and b16.view(np.float16)[0, 0] == 0.375 and np.all(w4 == 0)
    # min 0, max 15 (step 1): a value 2.5 lies halfway, nearest even is 2;
    # 3.5 rounds to 4
    w = np.zeros((1, G), np.float32)
    w[0, 1] = 15.0
    w[0, 2] = 2.5
    w[0, 3] = 3.5
    w4, s16, b16 = oracle.requantize_w4(_bf16(w), G)
    q = [(int(w4[0, 0]) >> (4 * i)) & 0xF for i in range(4)]
    assert q == [0, 15, 2, 4]
    # requantized codes feed the qmv oracle like any other W4 matrix
    x = synth.activations(11, 2, G)
    y = oracle.qmv(4, w4, s16, b16, x, G)
    assert y.shape == (2, 1) and np.all(np.isfinite(y))
