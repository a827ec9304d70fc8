"""Host logic of the binding's workspace cache: one buffer per (device,
stream, purpose), so calls on two streams never share a workspace, and a
buffer that grows is replaced for its own stream only."""
import speculative_decoding_spec_amd as spec


class FakeBuf:
    def __init__(self, n):
        self.n = n

    def numel(self):
        return self.n


def test_streams_get_distinct_buffers():
    cache = {}
    a = spec._cached_buffer(cache, ("cuda:0", 11, "accept"), 10000, FakeBuf)
    b = spec._cached_buffer(cache, ("cuda:0", 22, "accept"), 10000, FakeBuf)
    assert a is not b
    assert spec._cached_buffer(cache, ("cuda:0", 11, "accept"), 9000, FakeBuf) is a
    assert spec._cached_buffer(cache, ("cuda:0", 22, "accept"), 10000, FakeBuf) is b


def test_growth_replaces_only_its_own_slot():
    cache = {}
    a = spec._cached_buffer(cache, ("cuda:0", 11, "accept"), 10000, FakeBuf)
    b = spec._cached_buffer(cache, ("cuda:0", 22, "accept"), 10000, FakeBuf)
    a2 = spec._cached_buffer(cache, ("cuda:0", 11, "accept"), 50000, FakeBuf)
    assert a2 is not a and a2.numel() >= 50000
    assert cache[("cuda:0", 22, "accept")] is b
    # purposes and devices are separate slots too
    c = spec._cached_buffer(cache, ("cuda:0", 11, "sample"), 100, FakeBuf)
    d = spec._cached_buffer(cache, ("cuda:1", 11, "accept"), 100, FakeBuf)
    assert len({id(x) for x in (a2, b, c, d)}) == 4
    assert c.numel() == 4096          # small requests get a 4 KB minimum
