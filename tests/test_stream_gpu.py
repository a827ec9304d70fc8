"""The streaming-read probe reads every byte once: the XOR of its per-
workgroup sink words equals the XOR of the buffer's 32-bit words, computed
on the host, for sizes that fill whole rounds of 8 loads per lane, ragged
ones, one 16-byte word, and none."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

ROUND = 2048 * 256 * 8 * 16   # bytes of one round of every workgroup


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 48, ROUND - 16, ROUND, 3 * ROUND + 16 * 12345])
def test_stream_read_touches_every_word(dev, nbytes):
    import torch
    import speculative_decoding_spec_amd as spec
    words = np.random.default_rng(nbytes % 1000 + 7).integers(
        0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).to(dev)
    if nbytes == 0:
        src = torch.empty(0, dtype=torch.int32, device=dev)
    sink = torch.full((spec.STREAM_READ_GROUPS,), -1, dtype=torch.int32, device=dev)
    spec.spec_stream_read(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(words) if nbytes else np.uint32(0)
    assert got == want, (nbytes, hex(int(got)), hex(int(want)))
