"""Full-size parity: each benchmark workload, built exactly as bench.py builds
it (same sizes, seeds, chunk size and launch configuration), runs on the GPU
and is compared with the oracle over every owned element: the host
regenerates the inputs slice by slice with the multi-threaded generator and
runs the oracle on them (tests/fullsize.py).  Config 4 also checks its whole
reduced gradient, overflow flag and squared norm, and runs the bench's
checked step over a four-step cycle (one of them skipped); config 5 checks the
local accumulator over the whole flat buffer and every one of its 16 owners
(owner 1 in full, the others sampled).  Whole-buffer properties (every 16-bit
value a rounding of its master weight, padding untouched) are checked on the
device.
"""
import time

import numpy as np
import pytest

import fullsize as FS
import oracle
import synth
from helpers import assert_bits_equal, assert_state_close, assert_write_back, shard_ranges

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
    """Configs 2 and 3: one fused step, every owned w/m/v/p16 element against the oracle."""
    w = bench.Workload(cfg, bench.DEFAULT_CHUNK, 0)
    print(f"config {cfg}: {w.sh.n_real} owned, {w.sh.chunks.size} chunks", flush=True)
    w.step()
    torch.cuda.synchronize()
    FS.check_fused_step_full(w, bench.FIRST_STEP)
    _check_coverage(w)
    del w
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- config 4
_C4 = {}


def _config4():
    if "w" not in _C4:
        _C4["w"] = bench.Workload(4, bench.DEFAULT_CHUNK, 0)
    return _C4["w"]


def test_config4_whole_reduced_gradient_flag_and_norm():
    """70e9 / R=64 owner: the reduce with the fused check, as the checked step runs
    it; the whole fp32 gradient bit-exact, the flag exact and the squared norm
    within 1e-9 of the oracle's; then an injected +inf and NaN are flagged."""
    w = _config4()
    sh = w.sh
    flag, sumsq = sh.reduce_and_check(rank_grads=w.grads, grad_base=sh.local_base, divisor=w.divisor)
    g_or = FS.reduced_gradient_full(w, w.g32)
    t0 = time.time()
    oflag, osumsq = oracle.grad_check(g_or)
    print(f"config 4: oracle check of {g_or.size} elements in {time.time() - t0:.1f} s; sumsq {osumsq}", flush=True)
    # all inputs are finite by construction (|x| <= 2*sqrt(3)*sigma*2^16 << 65504)
    assert flag == oflag == 0
    assert abs(sumsq - osumsq) <= 1e-9 * osumsq
    _C4["g_or"], _C4["sumsq"] = g_or, osumsq
    saved = (w.grads[5][12345].clone(), w.grads[17][777_777].clone())
    w.grads[5][12345] = float("inf")
    w.grads[17][777_777] = float("nan")
    assert sh.reduce_and_check(rank_grads=w.grads, grad_base=sh.local_base, divisor=w.divisor)[0] == 1
    w.grads[5][12345], w.grads[17][777_777] = saved


def test_config4_checked_step_cycle_full_size():
    """The bench's checked step (reduce + check, host decision, AdamW from the
    stored gradient) over its four-step cycle at full size: an update with the
    bench's clip threshold 1.0 (the gradient norm is about 4.1, so the clip
    applies, with the factor from the oracle's norm), an update with a
    threshold of 8 (factor 1: no clip), a third update, and the step with the
    injected inf and NaN, which is skipped and leaves w/m/v/p16 bit-identical.
    Every owned element is compared with the oracle after the first two
    updates."""
    w = _config4()
    sh = w.sh
    if "g_or" not in _C4:  # run on its own: the oracle's gradient, as the test before computes it
        sh.reduce_and_check(rank_grads=w.grads, grad_base=sh.local_base, divisor=w.divisor)
        g_or = FS.reduced_gradient_full(w, w.g32)
        _C4["g_or"], _C4["sumsq"] = g_or, oracle.grad_check(g_or)[1]
    g_or, osumsq = _C4["g_or"], _C4["sumsq"]
    ow, om, ov, p_or = FS.owner_state_full(w)
    b = sh.begin
    for i, max_norm in enumerate((1.0, 8.0)):
        t = w.t
        w.max_norm = max_norm
        assert w.step() is False and w.t == t + 1, "an updating step"
        torch.cuda.synchronize()
        coef = oracle.clip_coef(osumsq, max_norm)
        assert (coef < 0.5) if i == 0 else (coef == 1.0)
        t0 = time.time()
        oracle.owner_step([(b, sh.end)], oracle.hyper(step=t, clip_coef=coef, **bench.HP), ow, om, ov, b,
                          reduced_g=g_or, p16=p_or, pdtype=synth.F16, param_base=b)
        FS.compare_owner_full(w, ow, om, ov, p_or, f"config 4 step {t} (clip {coef:.6f})")
        print(f"config 4: step {t} compared over {sh.end - b} elements in {time.time() - t0:.1f} s", flush=True)
    w.max_norm = 1.0
    t = w.t
    assert w.step() is False and w.t == t + 1
    before = [x.clone() for x in (sh.master, sh.exp_avg, sh.exp_avg_sq, w.p16)]
    assert w.calls % 4 == 3
    assert w.step() is True and w.t == t + 1, "the injected step is skipped and the count stays"
    torch.cuda.synchronize()
    for a, x in zip(before, (sh.master, sh.exp_avg, sh.exp_avg_sq, w.p16)):
        assert torch.equal(a.view(torch.int16) if a.dtype != torch.float32 else a.view(torch.int32),
                           x.view(torch.int16) if x.dtype != torch.float32 else x.view(torch.int32))
    del before
    _C4.clear()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- config 5
def test_config5_accumulation_and_owner_step_full_size():
    """10,000 tensors, R=16: eight bf16 microsteps into fp32 (the whole flat
    buffer bit-exact), then the fused owner step over every owned element."""
    w = bench.Workload(5, bench.DEFAULT_CHUNK, 0)
    sh = w.sh
    print(f"config 5: {sh.n_real} owned, {sh.chunks.size} chunks", flush=True)
    w.step()
    torch.cuda.synchronize()
    FS.check_local_accumulator_full(w)
    FS.check_fused_step_full(w, bench.FIRST_STEP)
    _check_coverage(w)
    assert sum(1 for n in w.numels if n < 64) == 0 and min(w.numels) == 64
    del w
    torch.cuda.empty_cache()


def _sampled_real(ranges, n, seed):
    """Each range's first and last element plus n random real elements."""
    rng = np.random.default_rng(seed)
    b = np.array([r[0] for r in ranges], dtype=np.int64)
    e = np.array([r[1] for r in ranges], dtype=np.int64)
    cum = np.cumsum(e - b)
    pick = rng.integers(0, int(cum[-1]), size=n)
    k = np.searchsorted(cum, pick, side="right")
    rand = b[k] + (pick - (cum[k] - (e[k] - b[k])))
    return np.unique(np.concatenate([b, e - 1, rand])).astype(np.uint64)


def test_config5_every_owner_sampled():
    """All 16 owners of config 5 at full size, each built like the bench's owner
    (16 fp32 rank slices, each the eight-microstep accumulation of its rank;
    generated state): one fused step, compared with the oracle at every real
    range's ends and 4,000 random real elements per owner."""
    numels, R = bench.config5_numels(), 16
    dev = torch.device("cuda")
    p16 = None
    for owner in range(R):
        sh = zs.OwnerShard(numels, R, owner, align=64, max_chunk=bench.DEFAULT_CHUNK, device=dev)
        ranges = shard_ranges(sh)
        lb, end = sh.local_base, sh.end
        if p16 is None:
            p16 = torch.zeros(sh.padded_total, dtype=torch.bfloat16, device=dev)
        tmp = torch.empty(end - lb, dtype=torch.bfloat16, device=dev)
        grads = []
        for r in range(R):
            acc = torch.empty(end - lb, dtype=torch.float32, device=dev)
            for k in range(8):
                bench.fill(tmp, 5, synth.STREAM_MICRO, r, lb, synth.DIST_NORMAL, 1e-3, step=k)
                zs.zero_reduce_owned([tmp], lb, end - lb, 1.0, acc, grad_base=lb, out_base=lb, accumulate=k > 0)
            grads.append(acc)
        sh.alloc_state()
        bench.fill(sh.master, 5, synth.STREAM_MASTER, 0, lb, synth.DIST_NORMAL, 0.02)
        bench.fill(sh.exp_avg, 5, synth.STREAM_EXP_AVG, 0, lb, synth.DIST_NORMAL, 5e-4)
        bench.fill(sh.exp_avg_sq, 5, synth.STREAM_EXP_AVG_SQ, 0, lb, synth.DIST_SQUARE, 1e-4)
        sh.adam_step(step=bench.FIRST_STEP, hyper=bench.HP, rank_grads=grads, grad_base=lb, divisor=float(R),
                     param16=p16)
        torch.cuda.synchronize()
        idx = _sampled_real(ranges, 4000, owner)
        gr = []
        for r in range(R):
            acc = np.zeros(idx.size, dtype=np.float32)
            for k in range(8):
                g = synth.values(synth.stream_key(5, synth.STREAM_MICRO, r, k), idx, synth.DIST_NORMAL, 1e-3,
                                 synth.BF16)
                oracle.accumulate(g, synth.BF16, acc, first=(k == 0))
            gr.append(acc)
        mk = lambda st, dist, s: synth.values_f32(synth.stream_key(5, st, 0), idx, dist, s)
        w0 = mk(synth.STREAM_MASTER, synth.DIST_NORMAL, 0.02)
        m0 = mk(synth.STREAM_EXP_AVG, synth.DIST_NORMAL, 5e-4)
        v0 = mk(synth.STREAM_EXP_AVG_SQ, synth.DIST_SQUARE, 1e-4)
        p_or = np.zeros(idx.size, dtype=np.uint16)
        oracle.owner_step([(0, idx.size)], oracle.hyper(step=bench.FIRST_STEP, **bench.HP), w0, m0, v0, 0,
                          grads=gr, gdtype=synth.F32, divisor=float(R), p16=p_or, pdtype=synth.BF16)
        loc = torch.from_numpy((idx - np.uint64(lb)).astype(np.int64)).to(dev)
        what = f"config 5 owner {owner}"
        assert_state_close(sh.master[loc].cpu().numpy(), w0, what + " w")
        assert_state_close(sh.exp_avg[loc].cpu().numpy(), m0, what + " m")
        assert_state_close(sh.exp_avg_sq[loc].cpu().numpy(), v0, what + " v")
        pg = p16[torch.from_numpy(idx.astype(np.int64)).to(dev)].cpu().view(torch.int16).numpy().view(np.uint16)
        assert_write_back(pg, sh.master[loc].cpu().numpy(), w0, synth.BF16, what + " p16")
        print(f"{what}: {sh.n_real} owned, {idx.size} compared", flush=True)
        del grads, tmp, sh
    # every owner wrote every one of its real elements (no master weight rounds to
    # zero in bf16) and nothing else: exactly the real elements are non-zero
    assert int(torch.count_nonzero(p16.view(torch.int16))) == sum(numels)
    del p16
    torch.cuda.empty_cache()


def test_per_backward_schedule_full_size():
    """Config 5 sizes under the per-backward schedule: every microstep reduces the
    16 ranks' owned bf16 slices and adds the mean to the owner's fp32
    accumulator (every owned element bit-exact); AdamW from it at the end (every
    owned element against the oracle)."""
    w = bench.Workload(5, bench.DEFAULT_CHUNK, 0, "per-backward")
    sh = w.sh
    print(f"config 5 per-backward: {sh.n_real} owned", flush=True)
    w.step()
    torch.cuda.synchronize()
    t0 = time.time()
    h = oracle.hyper(step=bench.FIRST_STEP, **bench.HP)
    lb = sh.local_base
    for lo, hi, parts in FS.slices(shard_ranges(sh)):
        n = hi - lo
        acc = np.empty(n, dtype=np.float32)
        for k in range(8):
            row = [synth.host_values(synth.stream_key(5, synth.STREAM_MICRO, r, k), lo, n, synth.DIST_NORMAL, 1e-3,
                                     synth.BF16) for r in range(w.R)]
            if k == 0:
                oracle.reduce(row, synth.BF16, float(w.R), out=acc)
            else:
                oracle.reduce_add(row, synth.BF16, float(w.R), acc)
        got = w.acc_owned[lo - lb:hi - lb].cpu().numpy()
        for b, e in parts:  # the accumulator is defined on real elements
            assert_bits_equal(got[b - lo:e - lo], acc[b - lo:e - lo], f"per-backward accumulator [{b}, {e})")
        ow, om, ov = FS.state0(5, lo, hi)
        p_or = np.zeros(n, dtype=np.uint16)
        oracle.owner_step(parts, h, ow, om, ov, lo, reduced_g=acc, p16=p_or, pdtype=synth.BF16, param_base=lo)
        FS.compare_owner_state(w, lo, hi, ow, om, ov, p_or, f"per-backward [{lo}, {hi})", parts)
    print(f"config 5 per-backward: compared in {time.time() - t0:.1f} s", flush=True)
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
