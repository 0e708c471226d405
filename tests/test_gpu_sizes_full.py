"""Full-size parity: each benchmark workload, built exactly as bench.py builds
it (same sizes, seeds, chunk size and launch configuration), runs one step on
the GPU; sampled outputs are compared with the oracle evaluated on inputs that
the host regenerates at those indices (the generator is counter-based), and
whole-buffer properties are checked at full size.

Sampled: owner ends, chunk ends, tensor ends, and random interior elements.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_bits_equal, assert_p16_within_ulp, assert_state_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bench  # noqa: E402
import zero_sharded_optimizer_owned_amd as zs  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    zs.lib()
    yield
    torch.cuda.empty_cache()


def _sample(w, n_random=20_000, seed=0):
    sh = w.sh
    ch = sh.chunks
    rng = np.random.default_rng(seed)
    picks = [ch["flat"], ch["flat"] + ch["len"] - 1]  # every chunk's first and last element
    lens = ch["len"].astype(np.int64)
    cum = np.cumsum(lens)
    r = rng.integers(0, int(cum[-1]), size=n_random)
    k = np.searchsorted(cum, r, side="right")
    start = cum - lens
    picks.append(ch["flat"][k] + (r - start[k]).astype(np.uint64))
    idx = np.unique(np.concatenate([p.astype(np.uint64) for p in picks]))
    return idx


def _grad_code(cfg):
    return {2: synth.F16, 3: synth.BF16, 4: synth.F16, 5: synth.F32}[cfg]


def _oracle_grads(w, idx):
    seed, R = w.cfg, w.R
    if w.cfg == 5:
        out = []
        for r in range(R):
            acc = np.zeros(idx.size, dtype=np.float32)
            for k in range(8):
                g = synth.values(synth.stream_key(seed, synth.STREAM_MICRO, r, k), idx, synth.DIST_NORMAL,
                                 1e-3, synth.BF16)
                oracle.accumulate(g, synth.BF16, acc, first=(k == 0))
            out.append(acc)
        return out
    return [synth.values(synth.stream_key(seed, synth.STREAM_GRAD, r), idx, synth.DIST_NORMAL,
                         w.grad_scale, _grad_code(w.cfg)) for r in range(R)]


def _state0(w, idx):
    seed = w.cfg
    mk = lambda st, dist, s: synth.values_f32(synth.stream_key(seed, st, 0), idx, dist, s)
    return (mk(synth.STREAM_MASTER, synth.DIST_NORMAL, 0.02), mk(synth.STREAM_EXP_AVG, synth.DIST_NORMAL, 5e-4),
            mk(synth.STREAM_EXP_AVG_SQ, synth.DIST_SQUARE, 1e-4))


def _gather(t, idx_local):
    it = torch.from_numpy(idx_local.astype(np.int64)).to(t.device)
    return t[it].cpu()


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def _check_owner(w, idx, step, coef=1.0, reduced_g=None):
    sh = w.sh
    pcode = synth.F16 if w.p16.dtype == torch.float16 else synth.BF16
    w0, m0, v0 = _state0(w, idx)
    p_or = np.zeros(idx.size, dtype=np.uint16)
    h = oracle.hyper(step=step, clip_coef=coef, **bench.HP)
    if reduced_g is not None:
        oracle.owner_step([(0, idx.size)], h, w0, m0, v0, 0, reduced_g=reduced_g, p16=p_or, pdtype=pcode)
    else:
        oracle.owner_step([(0, idx.size)], h, w0, m0, v0, 0, grads=_oracle_grads(w, idx),
                          gdtype=_grad_code(w.cfg), divisor=w.divisor, p16=p_or, pdtype=pcode)
    loc = idx - np.uint64(sh.local_base)
    assert_state_close(_gather(sh.master, loc).numpy(), w0, f"config {w.cfg} w")
    assert_state_close(_gather(sh.exp_avg, loc).numpy(), m0, f"config {w.cfg} m")
    assert_state_close(_gather(sh.exp_avg_sq, loc).numpy(), v0, f"config {w.cfg} v")
    ploc = idx - np.uint64(w.param_base)
    assert_p16_within_ulp(_bits(_gather(w.p16, ploc)), p_or, f"config {w.cfg} p16")


def _pow2(k):
    """2.0**k (int64 tensor k, normal fp64 range) built from its IEEE bit pattern: exact."""
    return ((k + 1023) << 52).view(torch.float64)


def _decode16(bits, is_f16):
    """Exact fp64 values of fp16/bf16 bit patterns and their ulp, from integer fields."""
    b = bits.view(torch.int16).to(torch.int64) & 0xFFFF
    mbits, bias = (10, 15) if is_f16 else (7, 127)
    sign = torch.where((b >> 15) == 1, -1.0, 1.0).double()
    e = (b >> mbits) & ((1 << (15 - mbits)) - 1)
    m = (b & ((1 << mbits) - 1)).double()
    mant = torch.where(e == 0, m, m + float(1 << mbits))
    ulp = _pow2(torch.clamp(e, min=1) - bias - mbits)
    return sign * mant * ulp, ulp


def _check_coverage(w):
    """Every real element's 16-bit copy lies within half an ulp of its master weight
    (a rounding to nearest); padding and everything outside the owner stay zero."""
    sh = w.sh
    lb, pb = sh.local_base, w.param_base
    is_f16 = w.p16.dtype == torch.float16
    p = w.p16.view(torch.int16)
    segs = []
    for k, (n, off) in enumerate(zip(w.numels, sh.offsets)):
        b, e = max(sh.begin, int(off)), min(sh.end, int(off) + n)
        if b >= e:
            continue
        segs.append((b, e))
        for s0 in range(b, e, 1 << 27):  # bounded temporaries
            s1 = min(e, s0 + (1 << 27))
            val, ulp = _decode16(p[s0 - pb:s1 - pb], is_f16)
            master = sh.master[s0 - lb:s1 - lb].double()
            bad = (val - master).abs() > ulp / 2
            nbad = int(bad.sum())
            if nbad:
                i = torch.nonzero(bad)[:5, 0]
                raise AssertionError(
                    f"config {w.cfg}: tensor {k}: {nbad} 16-bit values not a nearest rounding of the master; "
                    f"flat {(i + s0).tolist()}: p16 bits {p[i + s0 - pb].tolist()} master "
                    f"{sh.master[i + s0 - lb].tolist()}")
    gaps, cur = [], pb
    for b, e in segs:
        gaps.append((cur, b))
        cur = e
    gaps.append((cur, pb + w.p16.numel()))
    for b, e in gaps:
        if b < e:
            assert int(torch.count_nonzero(p[b - pb:e - pb])) == 0, \
                f"config {w.cfg}: 16-bit elements in [{b}, {e}) were written"


@pytest.mark.parametrize("cfg", [2, 3])
def test_fused_step_full_size(cfg):
    w = bench.Workload(cfg, bench.DEFAULT_CHUNK, 0)
    idx = _sample(w)
    print(f"config {cfg}: {w.sh.n_real} owned, {w.sh.chunks.size} chunks, {idx.size} sampled", flush=True)
    w.step()
    torch.cuda.synchronize()
    _check_owner(w, idx, bench.FIRST_STEP)
    _check_coverage(w)
    del w
    torch.cuda.empty_cache()


def test_loss_scaled_two_pass_full_size():
    """70e9 / R=64 owner: fused reduce + check, then AdamW from the stored gradient."""
    w = bench.Workload(4, bench.DEFAULT_CHUNK, 0)
    sh = w.sh
    idx = _sample(w, n_random=10_000)
    print(f"config 4: {sh.n_real} owned, {idx.size} sampled", flush=True)
    zs.zero_reduce_owned(w.grads, sh.begin, sh.end - sh.begin, w.divisor, w.g32, grad_base=sh.local_base,
                         out_base=sh.local_base, check=(w.ov, w.ss, w.ws))
    torch.cuda.synchronize()
    grads = _oracle_grads(w, idx)
    g_or = oracle.reduce(grads, synth.F16, w.divisor)
    loc = idx - np.uint64(sh.local_base)
    assert_bits_equal(_gather(w.g32, loc).numpy(), g_or, "config 4 reduced gradient")
    # all inputs are finite by construction (|x| <= 2*sqrt(3)*sigma*2^16 << 65504)
    assert int(w.ov.item()) == 0
    g64 = w.g32[sh.begin - sh.local_base:].double()
    assert abs(w.ss.item() - float(torch.dot(g64, g64))) <= 1e-9 * w.ss.item()
    # one injected +inf and one NaN: flagged
    saved = (w.grads[5][12345].clone(), w.grads[17][777_777].clone())
    w.grads[5][12345] = float("inf")
    w.grads[17][777_777] = float("nan")
    zs.zero_reduce_owned(w.grads, sh.begin, sh.end - sh.begin, w.divisor, w.g32, grad_base=sh.local_base,
                         out_base=sh.local_base, check=(w.ov, w.ss, w.ws))
    assert int(w.ov.item()) == 1
    w.grads[5][12345] = saved[0]
    w.grads[17][777_777] = saved[1]
    zs.zero_reduce_owned(w.grads, sh.begin, sh.end - sh.begin, w.divisor, w.g32, grad_base=sh.local_base,
                         out_base=sh.local_base, check=(w.ov, w.ss, w.ws))
    # second pass with a clip factor chosen here (the data-derived factor is checked at small sizes)
    coef = 0.37
    sh.adam_step(step=bench.FIRST_STEP, hyper=bench.HP, reduced_g=w.g32, param16=w.p16,
                 param_base=w.param_base, clip_coef=coef)
    torch.cuda.synchronize()
    g_or = oracle.reduce(_oracle_grads(w, idx), synth.F16, w.divisor)  # inputs restored
    _check_owner(w, idx, bench.FIRST_STEP, coef=coef, reduced_g=g_or)
    del w
    torch.cuda.empty_cache()


def test_accumulation_and_owner_step_full_size():
    """10,000 tensors, R=16: eight bf16 microsteps into fp32, then the fused owner step."""
    w = bench.Workload(5, bench.DEFAULT_CHUNK, 0)
    sh = w.sh
    idx = _sample(w, n_random=5_000)
    print(f"config 5: {sh.n_real} owned, {sh.chunks.size} chunks, {idx.size} sampled", flush=True)
    w.step()
    torch.cuda.synchronize()
    # the local rank's accumulator over the whole flat buffer, sampled everywhere
    rng = np.random.default_rng(1)
    aidx = np.unique(np.concatenate([rng.integers(0, sh.padded_total, 4000).astype(np.uint64),
                                     np.array([0, sh.padded_total - 1], dtype=np.uint64)]))
    acc = np.zeros(aidx.size, dtype=np.float32)
    for k in range(8):
        g = synth.values(synth.stream_key(5, synth.STREAM_MICRO, sh.owner, k), aidx, synth.DIST_NORMAL, 1e-3,
                         synth.BF16)
        oracle.accumulate(g, synth.BF16, acc, first=(k == 0))
    assert_bits_equal(_gather(w.acc, aidx).numpy(), acc, "config 5 accumulator")
    _check_owner(w, idx, bench.FIRST_STEP)
    _check_coverage(w)
    assert sum(1 for n in w.numels if n < 64) == 0 and min(w.numels) == 64
    del w
    torch.cuda.empty_cache()


def test_per_backward_schedule_full_size():
    """Config 5 sizes under the per-backward schedule: every microstep reduces the 16 ranks'
    owned bf16 slices and adds the mean to the owner's fp32 accumulator; AdamW at the end."""
    w = bench.Workload(5, bench.DEFAULT_CHUNK, 0, "per-backward")
    sh = w.sh
    idx = _sample(w, n_random=5_000)
    print(f"config 5 per-backward: {sh.n_real} owned, {idx.size} sampled", flush=True)
    w.step()
    torch.cuda.synchronize()
    acc = np.zeros(idx.size, dtype=np.float32)
    for k in range(8):
        row = [synth.values(synth.stream_key(5, synth.STREAM_MICRO, r, k), idx, synth.DIST_NORMAL, 1e-3,
                            synth.BF16) for r in range(w.R)]
        if k == 0:
            acc[:] = oracle.reduce(row, synth.BF16, float(w.R))
        else:
            oracle.reduce_add(row, synth.BF16, float(w.R), acc)
    loc = idx - np.uint64(sh.local_base)
    assert_bits_equal(_gather(w.acc_owned, loc).numpy(), acc, "per-backward accumulator")
    _check_owner(w, idx, bench.FIRST_STEP, reduced_g=acc)
    _check_coverage(w)
    del w
    torch.cuda.empty_cache()


def test_flat_reduce_past_the_grid_cap():
    """A flat range of more than 2^23 pieces (the launch's block cap): blocks take
    the pieces past the grid with a grid stride, and the check folds 2^23
    per-block partials in two stages.  One bf16 source and divisor 1, so each
    output is the widened input; the inputs are dyadic, so the squared norm is
    exact in fp64 whatever the summation order (closed form)."""
    cap_elems = (1 << 23) * 2048
    n = cap_elems + 12_345
    c = 0.0625
    g = torch.full((n,), c, dtype=torch.bfloat16, device="cuda")
    special = {3: 0.5, cap_elems + 5: -0.25, n - 1: 0.125}
    for i, x in special.items():
        g[i] = x
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    ov = torch.zeros(1, dtype=torch.int32, device="cuda")
    ss = torch.zeros(1, dtype=torch.float64, device="cuda")
    ws = zs.check_workspace(n, "cuda")
    zs.zero_reduce_owned([g], 0, n, 1.0, out, check=(ov, ss, ws))
    torch.cuda.synchronize()
    want_sumsq = (n - len(special)) * c * c + sum(x * x for x in special.values())
    assert int(ov.item()) == 0
    assert ss.item() == want_sumsq
    for i, x in special.items():
        assert float(out[i]) == x
    # every other element equals c: count them slice by slice on the device
    step = 1 << 30
    equal = 0
    for lo in range(0, n, step):
        equal += int(torch.count_nonzero(out[lo:lo + step] == c))
    assert equal == n - len(special)
    # a non-finite value in a piece past the grid cap sets the flag
    g[cap_elems + 7] = float("inf")
    zs.zero_reduce_owned([g], 0, n, 1.0, out, check=(ov, ss, ws))
    assert int(ov.item()) == 1
    del g, out, ws
    torch.cuda.empty_cache()
