"""The library's device calls inside a HIP graph (captured with
torch.cuda.graph): the fused step, and a reduce with the fused check whose
fold takes two stages.  The calls allocate nothing and record no memset, so a
captured step can be replayed.  Each replay is preceded by eager work (inputs
restored, unrelated kernels) and followed by a synchronisation, and must
reproduce the eager results bit for bit."""
import numpy as np
import pytest

import synth
from helpers import F16, F32, gen, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_owned_amd as zs  # noqa: E402

DEV = "cuda"
HP = dict(lr=1e-3, beta1=0.8, beta2=0.999, eps=1e-8, weight_decay=3e-7, adamw=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    zs.lib()
    yield
    torch.cuda.synchronize()


def _bits(t):
    return t.detach().view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy().copy()


def test_fused_step_in_a_graph_replays_like_eager():
    sh = zs.OwnerShard([1000, 37, 5003, 64, 20_000], 4, 1, align=64, max_chunk=512, device=DEV)
    sh.alloc_state()
    L = sh.master.numel()
    sh.master.copy_(to_dev(gen(1, synth.STREAM_MASTER, L, synth.DIST_NORMAL, 0.02, F32), F32))
    sh.exp_avg.copy_(to_dev(gen(1, synth.STREAM_EXP_AVG, L, synth.DIST_NORMAL, 5e-4, F32), F32))
    sh.exp_avg_sq.copy_(to_dev(gen(1, synth.STREAM_EXP_AVG_SQ, L, synth.DIST_SQUARE, 1e-4, F32), F32))
    grads = [to_dev(gen(2, synth.STREAM_GRAD, sh.padded_total, synth.DIST_NORMAL, 1e-3, F16, rank=r), F16)
             for r in range(4)]
    p16 = torch.zeros(sh.padded_total, dtype=torch.float16, device=DEV)
    saved = [x.clone() for x in (sh.master, sh.exp_avg, sh.exp_avg_sq)]

    def step():
        sh.adam_step(step=7, hyper=HP, rank_grads=grads, divisor=4.0, param16=p16)

    def restore():
        for x, s in zip((sh.master, sh.exp_avg, sh.exp_avg_sq), saved):
            x.copy_(s)
        p16.zero_()

    step()  # eager reference
    torch.cuda.synchronize()
    want = [_bits(x) for x in (sh.master, sh.exp_avg, sh.exp_avg_sq, p16)]
    restore()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for replay in range(3):
        restore()
        torch.randn(4096, device=DEV).sum()  # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        got = [_bits(x) for x in (sh.master, sh.exp_avg, sh.exp_avg_sq, p16)]
        for g, w, name in zip(got, want, ("master", "exp_avg", "exp_avg_sq", "param16")):
            assert np.array_equal(g, w), f"replay {replay}: {name} differs from the eager step"


def test_checked_reduce_in_a_graph_replays_like_eager():
    R, begin, n = 3, 5, 9_000_003  # more first-stage blocks than one fold block takes
    grads = [to_dev(gen(3, synth.STREAM_GRAD, begin + n, synth.DIST_NORMAL, 65.536, F16, rank=r), F16)
             for r in range(R)]
    out = torch.empty(begin + n, dtype=torch.float32, device=DEV)
    ov = torch.zeros(1, dtype=torch.int32, device=DEV)
    ss = torch.zeros(1, dtype=torch.float64, device=DEV)
    ws = zs.check_workspace(n, DEV)

    def reduce():
        zs.zero_reduce_owned(grads, begin, n, float(R) * 65536, out, check=(ov, ss, ws))

    reduce()
    torch.cuda.synchronize()
    want = (_bits(out[begin:]), int(ov.item()), float(ss.item()))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        reduce()
    for replay in range(3):
        out.fill_(-1.0)
        ov.fill_(7)
        ss.fill_(-1.0)
        torch.randn(4096, device=DEV).sum()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out[begin:]), want[0]), f"replay {replay}: reduced gradient differs"
        assert torch.all(out[:begin] == -1.0), f"replay {replay}: wrote below begin"
        assert (int(ov.item()), float(ss.item())) == want[1:], f"replay {replay}: flag or norm differs"


def test_allocation_free_checked_reduce_in_a_graph_replays_like_eager():
    """The allocation-free checked reduce, for callers under graph capture: captured
    after a first eager call on the device (which looks up its scratch array) and
    replayed three times with eager work, and a workspace-form reduce over other
    data, between the replays; every replay gives the eager result."""
    R, begin, n = 5, 3, 9_000_011
    grads = [to_dev(gen(8, synth.STREAM_GRAD, begin + n, synth.DIST_NORMAL, 65.536, F16, rank=r), F16)
             for r in range(R)]
    out = torch.empty(begin + n, dtype=torch.float32, device=DEV)
    ov = torch.zeros(1, dtype=torch.int32, device=DEV)
    ss = torch.zeros(1, dtype=torch.float64, device=DEV)

    def reduce():
        zs.zero_reduce_owned_noalloc(grads, begin, n, float(R) * 65536, out, check=(ov, ss))

    reduce()
    torch.cuda.synchronize()
    want = (_bits(out[begin:]), int(ov.item()), float(ss.item()))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        reduce()
    other = torch.ones(1 << 20, dtype=torch.float16, device=DEV)
    o_out = torch.empty(1 << 20, dtype=torch.float32, device=DEV)
    o_ov = torch.zeros(1, dtype=torch.int32, device=DEV)
    o_ss = torch.zeros(1, dtype=torch.float64, device=DEV)
    for replay in range(3):
        out.fill_(-1.0)
        ov.fill_(7)
        ss.fill_(-1.0)
        torch.randn(4096, device=DEV).sum()
        # an eager allocation-free call on other data in between: it shares the scratch array
        zs.zero_reduce_owned_noalloc([other], 0, other.numel(), 1.0, o_out, check=(o_ov, o_ss))
        graph.replay()
        torch.cuda.synchronize()
        assert float(o_ss.item()) == other.numel() and int(o_ov.item()) == 0
        assert np.array_equal(_bits(out[begin:]), want[0]), f"replay {replay}: reduced gradient differs"
        assert (int(ov.item()), float(ss.item())) == want[1:], f"replay {replay}: flag or norm differs"
