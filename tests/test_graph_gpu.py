"""The library's calls captured into a HIP graph (through torch.cuda.graph)
replay to the eager results: none of them records a memset, allocates, or
synchronizes.  Each replay is checked, with eager work and synchronizations
between the replays."""
import pytest

from speculative_decoding_spec_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu


def test_qmv_and_acceptance_replay_from_a_graph():
    import torch
    import speculative_decoding_spec_amd as spec
    dev = torch.device("cuda:0")
    K, N, M = 5120, 4096, 6
    pk = spec.spec_pack_w4(*parity.dev_qweights(*synth.qweights(9, 4, N, K, 64), dev))
    x = parity.dev_x(synth.activations(9, M, K), dev)
    B, D, V, T = 16, 5, 32768, 0.6
    t, d = synth.logits_pair(9, B, D, V)
    import oracle
    dt = oracle.sample_rows(d.reshape(B * D, V), T, 0, 1.0,
                            synth.uniforms(9, synth.U_DRAFT, B * D)).reshape(B, D)
    u = synth.uniforms(9, synth.U_ACCEPT, (B, D + 1))
    tt, dd = torch.from_numpy(t).to(dev), torch.from_numpy(d).to(dev)
    tk, uu = torch.from_numpy(dt).to(dev), torch.from_numpy(u).to(dev)
    y_ref = spec.spec_qmv_w4_packed(pk, x)
    a_ref, n_ref = spec.spec_verify_accept(tt, dd, tk, uu, T)
    torch.cuda.synchronize()

    y = torch.empty_like(y_ref)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm up allocations outside the capture
        spec.spec_qmv_w4_packed(pk, x, y=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        qmv = spec.bind_qmv(pk, x, y)
        accept = spec.bind_verify_accept(tt, dd, tk, uu, T, out=(acc, nxt, None, None))
    for rep in range(4):
        y.fill_(float("nan"))
        acc.fill_(-9)
        nxt.fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), rep
        assert torch.equal(acc, a_ref) and torch.equal(nxt, n_ref), rep
        # eager work between replays, on other data
        spec.spec_qmv_w4_packed(pk, torch.flip(x, [0]).contiguous())
        spec.spec_verify_accept(tt[:4].contiguous(), dd[:4].contiguous(), tk[:4].contiguous(),
                                uu[:4].contiguous(), 1.0)
        torch.cuda.synchronize()
    del qmv, accept
