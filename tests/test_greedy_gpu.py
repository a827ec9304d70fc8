"""GPU parity of greedy verification (spec_verify_greedy) against the fp64
oracle's sample-and-match loop, through the C ABI.

Results are integers, so every comparison is bit-exact.  Draft tokens are the
greedy draft's own choice (argmax of the draft row) with some replaced by
random tokens, so both outcomes occur at every position.  Workloads: the
batched B=256 D=5 V=151936 block (full size), single sequences whose rows span
many vocabulary chunks, odd vocabularies (scalar loads), D = 0 and D = 15,
and rows built with repeated maxima to pin the lowest-index rule across
threads and chunks."""
import numpy as np
import pytest

import oracle
from speculative_decoding_spec_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def T_(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def greedy_tokens(t, d, cfg, miss=0.25):
    """The greedy draft's tokens (argmax of each draft row), a fraction of
    them replaced by random tokens."""
    B, D, V = d.shape
    tok = np.argmax(d, axis=2).astype(np.int32)
    r = synth.rng(cfg, synth.U_DRAFT)
    m = r.random((B, D)) < miss
    tok[m] = r.integers(0, V, size=int(m.sum()))
    return tok


def gpu_greedy(t, tok, dev):
    import torch
    import speculative_decoding_spec_amd as spec
    D = t.shape[1] - 1
    acc, nxt = spec.spec_verify_greedy(T_(t, dev), T_(tok, dev) if D else None)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), nxt.cpu().numpy()


def check(t, tok, dev):
    acc, nxt = gpu_greedy(t, tok, dev)
    ref = oracle.verify_greedy(t, tok)
    B, D1, V = t.shape
    bad = np.nonzero((acc != ref["accepted_len"]) | (nxt != ref["next_token"]))[0]
    print(f"B={B} D={D1 - 1} V={V}: mismatches={len(bad)} "
          f"accepted_mean={ref['accepted_len'].mean():.3f}", flush=True)
    assert len(bad) == 0, [(int(b), int(acc[b]), int(nxt[b]), int(ref["accepted_len"][b]),
                            int(ref["next_token"][b])) for b in bad[:5]]
    return acc, nxt, ref


@pytest.mark.parametrize("B,D,V", [
    (1, 3, 32768),          # one sequence, rows split into chunks
    (64, 15, 4096),         # deepest block
    (4096, 2, 256),         # many sequences, small vocabulary
    (3, 2, 999),            # odd vocabulary: scalar loads
    (5, 4, 2),              # two-token vocabulary
    (1, 5, 151936),         # LM-head vocabulary, 75 chunks per row
])
def test_parity(dev, B, D, V):
    t, d = synth.logits_pair(800 + D, B, D, V)
    tok = greedy_tokens(t, d, 800 + D)
    check(t, tok, dev)


def test_parity_batched_full_size(dev):
    """B = 256, D = 5, V = 151936: the batched block the benchmark times (one
    vocabulary chunk per row)."""
    B, D, V = 256, 5, 151936
    t, d = synth.logits_pair(4, B, D, V)
    tok = greedy_tokens(t, d, 4, miss=0.0)
    acc, nxt, ref = check(t, tok, dev)
    assert len(set(ref["accepted_len"].tolist())) >= 3     # several outcomes occur


def test_depth_zero_is_argmax(dev):
    B, V = 37, 50000
    t, _ = synth.logits_pair(810, B, 0, V)
    acc, nxt = gpu_greedy(t, None, dev)
    assert np.all(acc == 0)
    assert np.array_equal(nxt, np.argmax(t[:, 0], axis=1))


@pytest.mark.parametrize("V", [151936, 32768, 1001])
def test_repeated_maxima_take_the_lowest_index(dev, V):
    """Each row holds its maximum at several random positions (spread over
    threads, unrolled loads and vocabulary chunks): the first one wins."""
    B, D = 16, 3
    r = np.random.default_rng(V)
    t = r.normal(0, 1, size=(B, D + 1, V)).astype(np.float32)
    for b in range(B):
        for i in range(D + 1):
            pos = r.choice(V, size=int(r.integers(2, 9)), replace=False)
            t[b, i, pos] = 7.5
    am = np.argmax(t, axis=2)
    tok = am[:, :D].astype(np.int32).copy()
    tok[::3, 1] = (tok[::3, 1] + 1) % V
    acc, nxt, ref = check(t, tok, dev)
    assert np.array_equal(nxt, am[np.arange(B), ref["accepted_len"]])


def test_all_equal_rows(dev):
    B, D, V = 4, 2, 70000
    t = np.full((B, D + 1, V), -2.5, np.float32)
    tok = np.zeros((B, D), np.int32)
    tok[1, 0] = 5
    acc, nxt, _ = check(t, tok, dev)
    assert acc.tolist() == [2, 0, 2, 2] and nxt.tolist() == [0, 0, 0, 0]


def test_invalid_sequences(dev):
    B, D, V = 6, 2, 5000
    t, d = synth.logits_pair(811, B, D, V)
    tok = np.argmax(d, axis=2).astype(np.int32)
    t[1, 2, 4999] = np.nan         # NaN in the bonus row, last element
    t[2, 0, 17] = np.inf           # +inf
    t[3, 1, :] = -np.inf           # no finite logit
    tok[4, 1] = V                  # draft token out of range
    t[5, 1, :100] = -np.inf        # -inf entries alone are allowed
    acc, nxt, ref = check(t, tok, dev)
    assert acc[1:5].tolist() == [-1] * 4 and nxt[1:5].tolist() == [-1] * 4
    assert acc[0] >= 0 and acc[5] >= 0


def test_equals_ratio_rule_at_top_k_one(dev):
    """The sampling path with top_k = 1 returns the same as the greedy path
    whenever the draft rows are valid (GPU against GPU, bit-exact)."""
    import torch
    import speculative_decoding_spec_amd as spec
    B, D, V = 64, 5, 151936
    t, d = synth.logits_pair(812, B, D, V)
    tok = greedy_tokens(t, d, 812)
    u = synth.uniforms(812, synth.U_ACCEPT, (B, D + 1))
    acc_g, nxt_g = gpu_greedy(t, tok, dev)
    acc_s, nxt_s = spec.spec_verify_accept(T_(t, dev), T_(d, dev), T_(tok, dev), T_(u, dev),
                                           0.6, top_k=1)
    torch.cuda.synchronize()
    assert np.array_equal(acc_g, acc_s.cpu().numpy())
    assert np.array_equal(nxt_g, nxt_s.cpu().numpy())


def test_workspace_contents_do_not_matter(dev):
    import torch
    import speculative_decoding_spec_amd as spec
    B, D, V = 8, 3, 151936          # several chunks per row
    t, d = synth.logits_pair(813, B, D, V)
    tok = greedy_tokens(t, d, 813)
    ref = oracle.verify_greedy(t, tok)
    need = spec.spec_verify_greedy_workspace(B, D, V)
    for fill in (0, 255, 127):
        ws = torch.full((need,), fill, dtype=torch.uint8, device=dev)
        acc, nxt = spec.spec_verify_greedy(T_(t, dev), T_(tok, dev), workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy(), ref["accepted_len"])
        assert np.array_equal(nxt.cpu().numpy(), ref["next_token"])


def test_bound_call_matches_plain_call(dev):
    import torch
    import speculative_decoding_spec_amd as spec
    B, D, V = 32, 5, 32768
    t, d = synth.logits_pair(814, B, D, V)
    tok = greedy_tokens(t, d, 814)
    tt, tk = T_(t, dev), T_(tok, dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    call = spec.bind_verify_greedy(tt, tk, out=(acc, nxt))
    acc.fill_(-7)
    nxt.fill_(-7)
    call()
    torch.cuda.synchronize()
    ref = oracle.verify_greedy(t, tok)
    assert np.array_equal(acc.cpu().numpy(), ref["accepted_len"])
    assert np.array_equal(nxt.cpu().numpy(), ref["next_token"])
