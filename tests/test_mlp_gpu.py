"""GPU parity of the gated MLP activation (spec_qmv_gate_up_silu: gate and up
as one launch, h = bf16(silu(g) * u)) and of the whole MLP block chained on
the GPU (h feeds the down projection), against the fp64 oracle.

Tolerance of h, derived from the qmv rule: the kernel's g and u each obey
|err| <= 1e-3 |v| + 2^-20 sum|x w| (the qmv parity bound), silu has slope
below 1.1, and the result is rounded to bf16 (at most one ulp, 2^-8 |h|, from
the exact value once the input errors are counted).  So
    |h_gpu - h| <= 1.1 e_g |u| + |silu(g)| e_u + e_g e_u + 2^-8 |h|.
Outside that, the bf16 bits must equal the oracle's nearest-even rounding of
the exact h, except where the exact h lies within the input-error part of the
bound (the first three terms) of a rounding boundary (the midpoint between two
bf16 neighbours): there either neighbour is correct, and such ties are
counted.  The down projection of the chained block is held to the plain qmv
rule against the oracle's own chain (bf16 h from the oracle)."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import scipy.special

import oracle
from speculative_decoding_spec_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def oracle_h_threaded(bits, gate, up, x, G=64):
    F = gate[0].shape[0]
    edges = np.linspace(0, F, parity.THREADS * 4 + 1).astype(int)
    spans = [(int(a), int(c)) for a, c in zip(edges[:-1], edges[1:]) if c > a]
    with ThreadPoolExecutor(parity.THREADS) as ex:
        parts = list(ex.map(lambda r: oracle.gate_up_silu(bits, gate, up, x, G, rows=r), spans))
    return (np.concatenate([p[0] for p in parts], axis=1),
            np.concatenate([p[1] for p in parts], axis=1))


def gpu_h(bits, gate, up, x, dev, G=64, valu=False):
    import speculative_decoding_spec_amd as spec
    pk = spec.spec_pack_gate_up(bits, parity.dev_qweights(*gate, dev),
                                parity.dev_qweights(*up, dev), G=G)
    fn = spec.spec_qmv_gate_up_silu_w4_valu if valu else spec.spec_qmv_gate_up_silu
    return fn(pk, parity.dev_x(x, dev))


def bf16_midpoints(h):
    """The rounding boundaries below and above each value: midpoints between
    the bf16 values that bracket it."""
    import torch
    t = torch.from_numpy(np.asarray(h, np.float64).astype(np.float32))
    lo = t.to(torch.bfloat16).to(torch.float64).numpy()       # one neighbour
    bits = torch.from_numpy(lo.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    up = (bits.astype(np.int32) + 1).astype(np.int16)
    dn = (bits.astype(np.int32) - 1).astype(np.int16)
    f = lambda b: synth.bf16_bits_to_f32(b.view(np.uint16)).astype(np.float64)
    return (lo + f(dn)) / 2, (lo + f(up)) / 2


def check_h(bits, M, F, K, dev, cfg, valu=False):
    import torch
    gate = synth.qweights(cfg, bits, F, K, 64, salt=1)
    up = synth.qweights(cfg, bits, F, K, 64, salt=2)
    x = synth.activations(cfg, M, K)
    hg = gpu_h(bits, gate, up, x, dev, valu=valu)
    got_bits = hg.view(torch.int16).cpu().numpy().view(np.uint16)
    got = synth.bf16_bits_to_f32(got_bits).astype(np.float64)
    h, hb = oracle_h_threaded(bits, gate, up, x)
    g, ag = parity.oracle_qmv_threaded(bits, *gate, x, 64)
    u, au = parity.oracle_qmv_threaded(bits, *up, x, 64)
    eg = 1e-3 * np.abs(g) + 2.0**-20 * ag
    eu = 1e-3 * np.abs(u) + 2.0**-20 * au
    silu = g * scipy.special.expit(g)
    tol_in = 1.1 * eg * np.abs(u) + np.abs(silu) * eu + eg * eu
    tol = tol_in + 2.0**-8 * np.abs(h)
    m_lo, m_hi = bf16_midpoints(h)
    tie = (np.abs(h - m_lo) <= tol_in) | (np.abs(h - m_hi) <= tol_in)
    far = int((np.abs(got - h) > tol).sum())
    wrong_bits = int(((got_bits != hb) & ~tie).sum())
    print(f"W{bits}{' valu' if valu else ''} M={M} F={F} K={K}: outside_bound={far} wrong_bits={wrong_bits} "
          f"ties={int(tie.sum())} bits_differ={int((got_bits != hb).sum())} of {h.size}",
          flush=True)
    assert far == 0
    assert wrong_bits == 0
    return gate, up, x, hg, hb


@pytest.mark.parametrize("M", [1, 3, 4, 5, 8, 12, 16])
def test_gate_up_silu_verify_mlp(dev, M):
    """Gate and up 5120 -> 17408 (one launch of 34816 rows), every M."""
    check_h(4, M, 17408, 5120, dev, cfg=20 + M)


@pytest.mark.parametrize("bits,M,F,K", [
    (4, 3, 100, 192),            # ragged tile pair, odd group count
    (8, 3, 100, 192),
    (4, 7, 1000, 64 * 13),
    (8, 8, 2048, 5120),          # W8 launch shape
    (4, 5, 33000, 256),          # four tiles per workgroup, last pair past the end
    (4, 16, 77, 320),            # wide form, ragged
])
def test_gate_up_silu_shapes(dev, bits, M, F, K):
    check_h(bits, M, F, K, dev, cfg=30 + M + F)


def test_mlp_block_chain(dev):
    """x -> gate/up with the gated activation -> down, all on the GPU,
    against the oracle's chain (its own bf16 h into its own down qmv)."""
    import speculative_decoding_spec_amd as spec
    M, F, H = 6, 17408, 5120
    gate, up, x, hg, hb = check_h(4, M, F, H, dev, cfg=40)
    down = synth.qweights(40, 4, H, F, 64, salt=3)
    pk = spec.spec_pack_w4(*parity.dev_qweights(*down, dev))
    y = spec.spec_qmv_w4_packed(pk, hg).cpu().numpy()
    ref, mag = parity.oracle_qmv_threaded(4, *down, hb, 64)
    nf, nabs, worst = parity.check_qmv(y, ref, mag)
    print(f"MLP block M={M}: fail={nf} abs-only={nabs} worst_rel={worst:.2e}", flush=True)
    assert nf == 0
    assert nabs <= parity.abs_only_limit(y.size), nabs


def test_degenerate_shapes(dev):
    import torch
    import speculative_decoding_spec_amd as spec
    # K = 0: g = u = 0, so h = +0 everywhere.
    z = (torch.zeros((20, 0), dtype=torch.int32, device=dev),
         torch.zeros((20, 0), dtype=torch.float16, device=dev),
         torch.zeros((20, 0), dtype=torch.float16, device=dev))
    pk = spec.spec_pack_gate_up(4, z, z)
    h = torch.full((3, 20), 7.0, dtype=torch.bfloat16, device=dev)
    spec.spec_qmv_gate_up_silu(pk, torch.zeros((3, 0), dtype=torch.bfloat16, device=dev), h=h)
    torch.cuda.synchronize()
    assert torch.all(h.view(torch.int16) == 0)
    # M = 0 is a no-op.
    g = synth.qweights(41, 4, 16, 64, 64)
    pk = spec.spec_pack_gate_up(4, parity.dev_qweights(*g, dev), parity.dev_qweights(*g, dev))
    spec.spec_qmv_gate_up_silu(pk, torch.zeros((0, 64), dtype=torch.bfloat16, device=dev))
    torch.cuda.synchronize()


def test_bound_call_matches_plain_call(dev):
    import torch
    import speculative_decoding_spec_amd as spec
    gate = synth.qweights(42, 4, 1000, 1024, 64, salt=1)
    up = synth.qweights(42, 4, 1000, 1024, 64, salt=2)
    x = parity.dev_x(synth.activations(42, 5, 1024), dev)
    pk = spec.spec_pack_gate_up(4, parity.dev_qweights(*gate, dev), parity.dev_qweights(*up, dev))
    h = torch.empty((5, 1000), dtype=torch.bfloat16, device=dev)
    call = spec.bind_qmv_gate_up_silu(pk, x, h)
    first = h.clone()
    h.fill_(float("nan"))
    call()
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), first.view(torch.int16))
    assert torch.equal(spec.spec_qmv_gate_up_silu(pk, x).view(torch.int16), h.view(torch.int16))
