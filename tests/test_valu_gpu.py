"""GPU parity of the vector-ALU comparison variants (spec_qmv_w4_packed_valu,
spec_qmv_gate_up_silu_w4_valu: the W4 small-M products with v_dot2c_f32_bf16
instead of MFMA) against the fp64 oracle, through the C ABI, under the same
bounds as the MFMA path: every output of the verify-MLP shapes at M = 1..4,
ragged shapes, the launch shape of 4096-tile heads, the gated activation,
and the degenerate cases.  The two paths sum the same products in different
orders, so they are compared with the oracle, not with each other."""
import numpy as np
import pytest

from speculative_decoding_spec_amd import synth
from tests import parity
from tests.test_mlp_gpu import check_h

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def valu_check(M, N, K, dev, cfg, salt=0):
    import speculative_decoding_spec_amd as spec
    w, s, b = synth.qweights(cfg, 4, N, K, 64, salt=salt)
    x = synth.activations(cfg, M, K, salt=salt)
    pk = spec.spec_pack_w4(*parity.dev_qweights(w, s, b, dev))
    got = spec.spec_qmv_w4_packed_valu(pk, parity.dev_x(x, dev)).cpu().numpy()
    ref, mag = parity.oracle_qmv_threaded(4, w, s, b, x, 64)
    nf, nabs, worst = parity.check_qmv(got, ref, mag)
    print(f"W4 valu M={M} N={N} K={K}: fail={nf} abs-only={nabs} worst_rel={worst:.2e}", flush=True)
    assert nf == 0
    assert nabs <= parity.abs_only_limit(got.size), nabs


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("shape", [(17408, 5120), (5120, 17408)], ids=["gate_up", "down"])
def test_valu_verify_mlp_shapes(dev, M, shape):
    N, K = shape
    valu_check(M, N, K, dev, cfg=1, salt=N)


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (3, 100, 192), (2, 4095, 1024), (4, 129, 17408),
                                   (1, 65600, 256), (4, 65600, 256)])
def test_valu_ragged_and_head_shapes(dev, M, N, K):
    valu_check(M, N, K, dev, cfg=5, salt=M * 100000 + N + K)


@pytest.mark.parametrize("M", [1, 2, 4])
def test_valu_gate_up_silu(dev, M):
    check_h(4, M, 17408, 5120, dev, cfg=20 + M, valu=True)


def test_valu_gate_up_silu_ragged(dev):
    check_h(4, 3, 100, 192, dev, cfg=33, valu=True)


def test_valu_degenerate_shapes(dev):
    import torch
    import speculative_decoding_spec_amd as spec
    z = torch.zeros((20, 0), dtype=torch.int32, device=dev)
    zs = torch.zeros((20, 0), dtype=torch.float16, device=dev)
    pk = spec.spec_pack_w4(z, zs, zs)
    y = torch.full((3, 20), 7.0, device=dev)
    spec.spec_qmv_w4_packed_valu(pk, torch.zeros((3, 0), dtype=torch.bfloat16, device=dev), y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)
    g = synth.qweights(41, 4, 16, 64, 64)
    pk = spec.spec_pack_w4(*parity.dev_qweights(*g, dev))
    spec.spec_qmv_w4_packed_valu(pk, torch.zeros((0, 64), dtype=torch.bfloat16, device=dev))
    torch.cuda.synchronize()
    with pytest.raises(spec.SpecError):
        spec.spec_qmv_w4_packed_valu(pk, torch.zeros((5, 64), dtype=torch.bfloat16, device=dev))
