"""The bandwidth probe on the GPU: every destination holds the bytewise XOR of
the sources, for one to many streams and sizes that span several tiles, a
ragged last tile and a single vector.  Expected values are numpy XORs of the
host copies of the sources."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_owned_amd as zs  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    zs.lib()
    yield


@pytest.mark.parametrize("n_src,n_dst,n_vec", [(1, 1, 1), (1, 1, 64 * 4 * 3 + 5), (3, 2, 100_003),
                                               (10, 7, 70_001), (33, 1, 9_999), (64, 64, 517)])
@pytest.mark.parametrize("order", [0, 1])
def test_probe_writes_xor_of_sources(n_src, n_dst, n_vec, order):
    rng = np.random.default_rng(n_src * 1000 + n_vec)
    host = [rng.integers(0, 2 ** 32, size=4 * n_vec, dtype=np.uint32) for _ in range(n_src)]
    srcs = [torch.from_numpy(h.view(np.int32)).to("cuda") for h in host]
    dsts = [torch.full((4 * n_vec + 8,), -7, dtype=torch.int32, device="cuda") for _ in range(n_dst)]
    views = [d[:4 * n_vec] for d in dsts]
    zs.zero_stream_probe(srcs, views, order)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(np.stack(host), axis=0) if n_src > 1 else host[0]
    for d in dsts:
        got = d.cpu().numpy().view(np.uint32)
        assert np.array_equal(got[:4 * n_vec], want)
        assert np.all(got[4 * n_vec:].view(np.int32) == -7)  # nothing past the streams


def test_probe_write_only_and_read_only():
    n_vec = 64 * 256 + 3
    dsts = [torch.full((4 * n_vec + 8,), -7, dtype=torch.int32, device="cuda") for _ in range(2)]
    zs.zero_stream_probe([], [d[:4 * n_vec] for d in dsts])  # no sources: zeros
    src = torch.arange(4 * n_vec, dtype=torch.int32, device="cuda")
    keep = src.clone()
    zs.zero_stream_probe([src], [])  # reads only
    torch.cuda.synchronize()
    for d in dsts:
        got = d.cpu().numpy()
        assert np.all(got[:4 * n_vec] == 0) and np.all(got[4 * n_vec:] == -7)
    assert torch.equal(src, keep)
    with pytest.raises(ValueError):
        zs.zero_stream_probe([], [])


def test_probe_rejects_mismatched_sizes():
    a = torch.zeros(64, dtype=torch.int32, device="cuda")
    b = torch.zeros(68, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        zs.zero_stream_probe([a], [b])
    c = torch.zeros(68, dtype=torch.int32, device="cuda")
    with pytest.raises(zs.ZeroShardError):
        zs.zero_stream_probe([b[1:65]], [c[1:65]])  # 16-byte alignment


@pytest.mark.parametrize("src_w,dst_w,n_vec", [([1, 2], [2], 70_001), ([1] * 8 + [2] * 3, [2, 2, 2, 1], 9_999),
                                               ([2] * 4, [2, 2, 2, 1], 256 * 3 + 7), ([1] * 64, [2], 517)])
def test_probe_with_stream_widths(src_w, dst_w, n_vec):
    """Streams of width 2 hand each thread two consecutive 16-byte vectors: thread i
    XORs vectors [w i, w i + w) of every source (both vectors of a wide source
    into the same lanes) and writes the result to both vectors of a wide
    destination.  Expected values are built with numpy from the host copies."""
    rng = np.random.default_rng(len(src_w) * 100 + n_vec)
    host = [rng.integers(0, 2 ** 32, size=(n_vec, w, 4), dtype=np.uint32) for w in src_w]
    srcs = [torch.from_numpy(h.reshape(-1).view(np.int32)).to("cuda") for h in host]
    acc = np.zeros((n_vec, 4), dtype=np.uint32)
    for h in host:
        acc ^= np.bitwise_xor.reduce(h, axis=1)
    dsts = [torch.full((4 * n_vec * w + 8,), -7, dtype=torch.int32, device="cuda") for w in dst_w]
    zs.zero_stream_probe(srcs, [d[:4 * n_vec * w] for d, w in zip(dsts, dst_w)], 1, src_widths=src_w,
                         dst_widths=dst_w)
    torch.cuda.synchronize()
    for d, w in zip(dsts, dst_w):
        got = d.cpu().numpy().view(np.uint32)
        want = np.repeat(acc[:, None, :], w, axis=1).reshape(-1)
        assert np.array_equal(got[:4 * n_vec * w], want)
        assert np.all(got[4 * n_vec * w:].view(np.int32) == -7)
    with pytest.raises(ValueError):
        zs.zero_stream_probe(srcs[:1], [dsts[0][:4 * n_vec * dst_w[0]]], src_widths=[3], dst_widths=dst_w[:1])
