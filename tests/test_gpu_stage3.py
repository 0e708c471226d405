"""ZeRO-3 per-tensor partition and the gathered working set on the GPU, bit-exact
against the oracle (the data moves unchanged, so every element must match)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import BF16, F32, assert_bits_equal, from_dev, gen, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bench  # noqa: E402
import zero_sharded_optimizer_owned_amd as zs  # noqa: E402

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    zs.lib()
    yield


def _groups(spans, code):
    g = zs.zero_span_groups(spans, 2 if code == BF16 else 4)
    return dict(groups_dev=torch.from_numpy(g.astype(np.int64)).to(DEV), n_groups=g.size - 1)


@pytest.mark.parametrize("code", [BF16, F32])
@pytest.mark.parametrize("R", [1, 3, 8])
@pytest.mark.parametrize("max_span", [7, 4096])
@pytest.mark.parametrize("grouped", [False, True])
def test_partition_then_gather_matches_oracle(code, R, max_span, grouped):
    sizes = [5, 9, 2, 1000, 4096, 13, 77_777, 64] + [1 + (31 * k) % 90 for k in range(40)]
    dense = gen(R, synth.STREAM_MASTER, sum(sizes), synth.DIST_NORMAL, 0.02, code)
    dense_dev = to_dev(dense, code)
    shard_numel, resident, _ = zs.zero3_storage(sizes, R)
    want_shards = oracle.stage3_shards(sizes, R, dense)
    shard_devs = []
    for r in range(R):
        spans = zs.zero3_partition_spans(sizes, R, r, max_span=max_span)
        buf = torch.zeros(resident, dtype=dense_dev.dtype, device=DEV)
        gk = _groups(spans, code) if grouped and spans.size else {}
        zs.zero_copy_spans(zs.spans_to_device(spans) if spans.size else None, spans.size, [dense_dev], buf, **gk)
        assert_bits_equal(from_dev(buf), want_shards[r], f"shard of rank {r}")
        shard_devs.append(buf)
    for live in ([1], [0, 1], [6, 3, 0], list(range(len(sizes))), list(range(8, len(sizes)))):
        _, _, gathered = zs.zero3_storage(sizes, R, live)
        spans = zs.zero3_gather_spans(sizes, R, live, max_span=max_span)
        out = torch.full((gathered,), 7, dtype=dense_dev.dtype, device=DEV)
        gk = _groups(spans, code) if grouped else {}
        zs.zero_copy_spans(zs.spans_to_device(spans), spans.size, shard_devs, out, **gk)
        want = oracle.stage3_gather(sizes, R, want_shards, live)
        assert_bits_equal(from_dev(out), want, f"gather of {live}")


def test_gather_working_set_full_size():
    """Four Llama-style layers gathered from 8 ranks' shard buffers (bench configuration)."""
    g = bench.Stage3Gather()
    print(f"stage 3: {g.resident} resident per rank, {g.gathered} gathered, {g.spans.size} spans", flush=True)
    g.run()
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    pos = np.unique(np.concatenate([rng.integers(0, g.gathered, 50_000), [0, g.gathered - 1]]))
    want = g.expected(pos)
    got = g.out[torch.from_numpy(pos.astype(np.int64)).to(DEV)].cpu().view(torch.int16).numpy().view(np.uint16)
    assert_bits_equal(got, want, "gathered working set")
