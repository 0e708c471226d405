"""The allocation-free checked reduce (zero_reduce_owned_noalloc) through the C ABI
against the workspace form (zero_reduce_owned), which the other GPU tests hold
to the oracle: two calls in a row, the second over a smaller range, each with
identical reduced gradients, flags and squared norms (same kernels, same fold
tree), and the gradients bit-exact against the oracle too."""
import numpy as np
import pytest

import oracle
import synth
from helpers import BF16, F16, F32, assert_bits_equal, from_dev, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_owned_amd as zs  # noqa: E402

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    zs.lib()
    yield
    torch.cuda.synchronize()


def test_noalloc_checked_reduce_equals_the_workspace_form_twice():
    # the second call is smaller, so stale partials of the first would show
    # the first call folds its partials in two stages (more than 4096 blocks)
    cases = [(64, F16, 9_000_011, 5, 64.0 * 65536.0), (8, BF16, 100_003, 3, 8.0)]
    for i, (R, code, n, begin, D) in enumerate(cases):
        print(f"call {i}: R={R} dtype={code} begin={begin} n={n}", flush=True)
        total = begin + n + 8
        grads = [synth.host_values(synth.stream_key(40 + i, synth.STREAM_GRAD, r), 0, total, synth.DIST_NORMAL,
                                   65.536 if code == F16 else 1e-3, code) for r in range(R)]
        if i == 1:
            grads[3][begin + n // 2] = 0x7F80 if code == BF16 else 0x7C00  # +inf: the flag must be set
        dgr = [to_dev(g, code) for g in grads]
        out_ws = torch.full((total,), 7.0, dtype=torch.float32, device=DEV)
        out_na = torch.full((total,), 7.0, dtype=torch.float32, device=DEV)
        ov_ws = torch.full((1,), 5, dtype=torch.int32, device=DEV)
        ss_ws = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
        ov_na = torch.full((1,), 5, dtype=torch.int32, device=DEV)
        ss_na = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
        ws = zs.check_workspace(n, DEV)
        zs.zero_reduce_owned(dgr, begin, n, D, out_ws, check=(ov_ws, ss_ws, ws))
        zs.zero_reduce_owned_noalloc(dgr, begin, n, D, out_na, check=(ov_na, ss_na))
        torch.cuda.synchronize()
        assert_bits_equal(from_dev(out_na), from_dev(out_ws), f"call {i} gradient")
        assert int(ov_na.item()) == int(ov_ws.item()) == (1 if i == 1 else 0)
        if i == 0:
            assert ss_na.item() == ss_ws.item() and ss_ws.item() > 0
        want = oracle.reduce([g[begin:begin + n] for g in grads], code, D)
        assert_bits_equal(from_dev(out_na)[begin:begin + n], want, f"call {i} against the oracle")
        assert np.all(from_dev(out_na)[:begin] == 7.0) and np.all(from_dev(out_na)[begin + n:] == 7.0)
        # without the check it is the plain reduce
        out_plain = torch.full((total,), 7.0, dtype=torch.float32, device=DEV)
        zs.zero_reduce_owned_noalloc(dgr, begin, n, D, out_plain)
        assert_bits_equal(from_dev(out_plain), from_dev(out_ws), f"call {i} unchecked")
        del dgr, ws


def test_noalloc_accumulate_modes_equal_the_workspace_form():
    # accumulate 1 (out = (out + sum) / D) and 2 (out = out + sum / D) start from the
    # same fp32 contents on both sides; the second call is again the smaller one
    R, code, D = 16, BF16, 16.0
    for i, (mode, n, begin) in enumerate([(1, 600_001, 3), (2, 70_007, 11)]):
        print(f"accumulate {mode}: R={R} begin={begin} n={n}", flush=True)
        total = begin + n + 8
        grads = [synth.host_values(synth.stream_key(50 + i, synth.STREAM_GRAD, r), 0, total, synth.DIST_NORMAL,
                                   1e-3, code) for r in range(R)]
        start = synth.host_values(synth.stream_key(50 + i, synth.STREAM_MASTER, 0), 0, total, synth.DIST_NORMAL,
                                  1e-2, F32)
        dgr = [to_dev(g, code) for g in grads]
        out_ws, out_na = to_dev(start, F32), to_dev(start, F32)
        ov_ws = torch.full((1,), 5, dtype=torch.int32, device=DEV)
        ss_ws = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
        ov_na = torch.full((1,), 5, dtype=torch.int32, device=DEV)
        ss_na = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
        ws = zs.check_workspace(n, DEV)
        zs.zero_reduce_owned(dgr, begin, n, D, out_ws, accumulate=mode, check=(ov_ws, ss_ws, ws))
        zs.zero_reduce_owned_noalloc(dgr, begin, n, D, out_na, accumulate=mode, check=(ov_na, ss_na))
        torch.cuda.synchronize()
        assert_bits_equal(from_dev(out_na), from_dev(out_ws), f"accumulate {mode}")
        assert int(ov_na.item()) == int(ov_ws.item()) == 0
        assert ss_na.item() == ss_ws.item() and ss_ws.item() > 0
        part = [g[begin:begin + n] for g in grads]
        acc = start.view(np.float32)[begin:begin + n].copy()
        want = oracle.reduce(part, code, D, out=acc, accumulate=True) if mode == 1 else \
            oracle.reduce_add(part, code, D, acc)
        assert_bits_equal(from_dev(out_na)[begin:begin + n], want, f"accumulate {mode} against the oracle")
        del dgr, ws


def test_noalloc_at_the_largest_check_its_scratch_array_holds():
    # the largest n whose check partials fit the 16 MiB array (one element more is
    # ERANGE, checked on the CPU): accepted, with the same bits, flag and norm as the
    # workspace form
    scratch = 16 << 20
    lo, hi = 1, 1 << 40
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if zs.check_workspace_bytes(mid) <= scratch:
            lo = mid
        else:
            hi = mid
    n = lo
    assert zs.check_workspace_bytes(n) <= scratch < zs.check_workspace_bytes(n + 1)
    print(f"largest checked reduce without a workspace: n={n}", flush=True)
    g = torch.empty(n, dtype=torch.float16, device=DEV)
    synth.device_fill(g, synth.stream_key(61, synth.STREAM_GRAD, 0), 0, synth.DIST_NORMAL, 1.0)
    out_ws = torch.empty(n, dtype=torch.float32, device=DEV)
    out_na = torch.empty(n, dtype=torch.float32, device=DEV)
    ov_ws = torch.full((1,), 5, dtype=torch.int32, device=DEV)
    ss_ws = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
    ov_na = torch.full((1,), 5, dtype=torch.int32, device=DEV)
    ss_na = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
    ws = zs.check_workspace(n, DEV)
    zs.zero_reduce_owned([g], 0, n, 1.0, out_ws, check=(ov_ws, ss_ws, ws))
    zs.zero_reduce_owned_noalloc([g], 0, n, 1.0, out_na, check=(ov_na, ss_na))
    torch.cuda.synchronize()
    assert torch.equal(out_na.view(torch.int32), out_ws.view(torch.int32))
    assert int(ov_na.item()) == int(ov_ws.item()) == 0
    assert ss_na.item() == ss_ws.item() and ss_ws.item() > 0
    del g, out_ws, out_na, ws
    torch.cuda.empty_cache()
