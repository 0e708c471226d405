"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by
element, on seeded inputs that span many vectors, chunks and ragged ends.

Reduced gradients, overflow flags and the input generator: bit-exact.
Master weights and moments: |gpu - oracle| <= 1e-7 + 1e-6 |oracle| after each
step.  16-bit copies: within 1 ulp of the oracle's rounding of its own master
weight.  Squared norms: 1e-9 relative.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from helpers import (BF16, F16, F32, assert_bits_equal, assert_chunks_cover, assert_copy_of_master, assert_state_close,
                     checked_layout, shard_ranges,
                     from_dev, gen, to_dev)

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


# ---------------------------------------------------------------- generator
@pytest.mark.parametrize("code", [F16, BF16, F32])
@pytest.mark.parametrize("dist,scale", [(synth.DIST_NORMAL, 1e-3), (synth.DIST_NORMAL, 65.536),
                                        (synth.DIST_UNIFORM, 0.3), (synth.DIST_SQUARE, 1e-4)])
def test_device_generator_matches_host(code, dist, scale):
    n, i0 = 100_003, 12_345
    key = synth.stream_key(7, synth.STREAM_GRAD, 3, 2)
    t = torch.empty(n, dtype={F16: torch.float16, BF16: torch.bfloat16, F32: torch.float32}[code],
                    device=DEV)
    synth.device_fill(t, key, i0, dist, scale)
    torch.cuda.synchronize()
    want = synth.values(key, synth.arange(i0, i0 + n), dist, scale, code)
    assert_bits_equal(from_dev(t), want, "device generator")


# ---------------------------------------------------------------- reduce
def _rank_inputs(code, R, total, seed=1, scale=1e-3):
    return [gen(seed, synth.STREAM_GRAD, total, synth.DIST_NORMAL, scale, code, rank=r) for r in range(R)]


@pytest.mark.parametrize("code", [F16, BF16, F32])
@pytest.mark.parametrize("R", [1, 3, 4, 8, 13, 16, 24, 64])
def test_reduce_bitexact(code, R):
    total = 70_001
    begin, n = 13, 50_005          # ragged on both ends
    grads = _rank_inputs(code, R, total, seed=R)
    dgr = [to_dev(g, code) for g in grads]
    for divisor in (float(R), float(R) * 65536.0, 3.0):
        out_base = begin & ~7
        out = torch.full((begin + n - out_base + 16,), 7.0, dtype=torch.float32, device=DEV)
        zs.zero_reduce_owned(dgr, begin, n, divisor, out, out_base=out_base)
        got = from_dev(out)
        want = oracle.reduce([g[begin:begin + n] for g in grads], code, divisor)
        assert_bits_equal(got[begin - out_base:begin - out_base + n], want, f"R={R} D={divisor}")
        assert np.all(got[:begin - out_base] == 7.0) and np.all(got[begin - out_base + n:] == 7.0)


@pytest.mark.parametrize("code", [F16, BF16, F32])
def test_reduce_accumulate_and_slices(code):
    """Owner-local rank slices (grad_base = local_base) and accumulation into out."""
    R, total = 5, 40_000
    begin, end = 1234 + 3, 33_333
    lb = begin & ~7
    grads = _rank_inputs(code, R, total, seed=11)
    slices = [to_dev(g[lb:end], code) for g in grads]
    start = gen(2, synth.STREAM_EXP_AVG, end - lb, synth.DIST_NORMAL, 1e-2, F32)
    out = to_dev(start.copy(), F32)
    zs.zero_reduce_owned(slices, begin, end - begin, 1.0, out, grad_base=lb, out_base=lb,
                         accumulate=True)
    want = start.copy()
    oracle.reduce([g[begin:end] for g in grads], code, 1.0, out=want[begin - lb:], accumulate=True)
    assert_bits_equal(from_dev(out), want, "accumulate")


def test_negative_zero_and_specials():
    n = 64
    neg0 = np.full(n, 0x8000, dtype=np.uint16)
    out = torch.empty(n, dtype=torch.float32, device=DEV)
    zs.zero_reduce_owned([to_dev(neg0, F16)] * 3, 0, n, 4.0, out)
    got = from_dev(out)
    assert np.all(got == 0) and not np.any(np.signbit(got))
    big = np.array([3e38] * 8 + [1e8, 1.0, -1e8] + [0.0] * 5, dtype=np.float32)
    rows = [big, big, -big]
    out = torch.empty(16, dtype=torch.float32, device=DEV)
    zs.zero_reduce_owned([to_dev(r, F32) for r in rows], 0, 16, 1.0, out)
    assert_bits_equal(from_dev(out), oracle.reduce(rows, F32, 1.0), "specials")


def _check_bufs(n=1 << 24):
    return (torch.zeros(1, dtype=torch.int32, device=DEV), torch.zeros(1, dtype=torch.float64, device=DEV),
            zs.check_workspace(n, DEV))


@pytest.mark.parametrize("code", [F16, BF16])
def test_reduce_fused_check(code):
    R, total = 8, 300_007
    begin, n = 5, 300_000
    grads = _rank_inputs(code, R, total, seed=3, scale=65.536)
    dgr = [to_dev(g, code) for g in grads]
    D = float(R) * 65536.0
    ov, ss, ws = _check_bufs()
    out = torch.empty(begin + n, dtype=torch.float32, device=DEV)
    zs.zero_reduce_owned(dgr, begin, n, D, out, check=(ov, ss, ws))
    want = oracle.reduce([g[begin:begin + n] for g in grads], code, D)
    assert_bits_equal(from_dev(out)[begin:], want, "fused reduce")
    flag, sumsq = oracle.grad_check(want)
    assert int(ov.item()) == flag == 0
    assert math.isclose(ss.item(), sumsq, rel_tol=1e-9)
    first = ss.item()
    zs.zero_reduce_owned(dgr, begin, n, D, out, check=(ov, ss, ws))
    assert ss.item() == first  # run to run identical


@pytest.mark.parametrize("pos", [0, 3, 7, 8, 100_003, 299_999])
@pytest.mark.parametrize("kind", ["inf", "nan", "pm_inf"])
def test_overflow_flag_positions(pos, kind):
    R, n, begin = 4, 300_000, 5
    grads = _rank_inputs(F16, R, begin + n, seed=4, scale=65.536)
    f = begin + pos
    if kind == "inf":
        grads[2][f] = 0x7C00
    elif kind == "nan":
        grads[R - 1][f] = 0x7E00
    else:  # +inf in one rank and -inf in another: their sum is NaN
        grads[0][f], grads[1][f] = 0x7C00, 0xFC00
    dgr = [to_dev(g, F16) for g in grads]
    ov, ss, ws = _check_bufs()
    out = torch.empty(begin + n, dtype=torch.float32, device=DEV)
    zs.zero_reduce_owned(dgr, begin, n, float(R) * 65536, out, check=(ov, ss, ws))
    want = oracle.reduce([g[begin:] for g in grads], F16, float(R) * 65536)
    assert_bits_equal(from_dev(out)[begin:], want, "reduce with non-finite input")
    assert int(ov.item()) == oracle.grad_check(want)[0] == 1


def test_reduce_fused_check_two_stage_fold():
    """A reduce with the fused check over more first-stage blocks than one fold
    block takes (9,000,003 elements from a misaligned begin)."""
    R, begin, n = 2, 3, 9_000_003
    grads = _rank_inputs(F16, R, begin + n, seed=8, scale=65.536)
    dgr = [to_dev(g, F16) for g in grads]
    ov, ss, ws = _check_bufs(n)
    out = torch.empty(begin + n, dtype=torch.float32, device=DEV)
    zs.zero_reduce_owned(dgr, begin, n, float(R) * 65536, out, check=(ov, ss, ws))
    want = oracle.reduce([g[begin:] for g in grads], F16, float(R) * 65536)
    assert_bits_equal(from_dev(out)[begin:], want, "reduce, two-stage check")
    flag, sumsq = oracle.grad_check(want)
    assert int(ov.item()) == flag == 0
    assert math.isclose(ss.item(), sumsq, rel_tol=1e-9, abs_tol=0.0)


# 8,390,660 and 20,000,001 elements give more than 4096 first-stage blocks,
# which are folded in two stages.
@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 1000, 65_537, 1_000_003, 8_390_660, 20_000_001])
def test_grad_check_standalone(n):
    g = gen(5, synth.STREAM_GRAD, max(n, 1), synth.DIST_NORMAL, 1e-3, F32)[:n]
    ov, ss, ws = _check_bufs(max(n, 1))
    ov.fill_(9)
    ss.fill_(-1)
    zs.zero_grad_check(to_dev(g, F32) if n else torch.empty(0, dtype=torch.float32, device=DEV),
                       ov, ss, ws)
    flag, sumsq = oracle.grad_check(g)
    assert int(ov.item()) == flag
    assert math.isclose(ss.item(), sumsq, rel_tol=1e-9, abs_tol=0.0)
    if n:
        g2 = g.copy()
        g2[n // 2] = np.inf
        zs.zero_grad_check(to_dev(g2, F32), ov, ss, ws)
        assert int(ov.item()) == 1


# ---------------------------------------------------------------- fused step
LAYOUTS = {
    "ragged": ([1000, 37, 5003, 1, 64, 777, 4096, 9, 20_000], 3, 64),
    "tiny_tensors": ([1, 2, 3, 5, 7, 8, 9, 15, 16, 17, 31, 33, 63, 64, 65, 100] * 6, 5, 8),
    "empty_owners": ([3, 2], 9, 1),
    "one_big": ([123_457], 4, 64),
    # padding after almost every tensor: short chunks that the group table packs
    "padded_tiny": ([1 + (37 * k) % 150 for k in range(300)], 3, 64),
}


def _owner_inputs(numels, R, A, owner, gcode, seed):
    off, total, b, e = checked_layout(numels, R, A)
    begin, end = int(b[owner]), int(e[owner])
    lb = begin & ~7
    grads = _rank_inputs(gcode, R, total, seed=seed)
    size = max(8, end - lb)
    w = gen(seed, synth.STREAM_MASTER, size, synth.DIST_NORMAL, 0.02, F32)
    m = gen(seed, synth.STREAM_EXP_AVG, size, synth.DIST_NORMAL, 5e-4, F32)
    v = gen(seed, synth.STREAM_EXP_AVG_SQ, size, synth.DIST_SQUARE, 1e-4, F32)
    return off, total, begin, end, lb, grads, w, m, v


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("gcode,pcode", [(F16, F16), (BF16, BF16), (F32, BF16), (F32, 0), (F16, BF16)])
@pytest.mark.parametrize("max_chunk", [64, 2048])
@pytest.mark.parametrize("grouped", [False, True])
def test_adam_step_matches_oracle(layout, gcode, pcode, max_chunk, grouped):
    numels, R, A = LAYOUTS[layout]
    for owner in range(R):
        off, total, begin, end, lb, grads, w, m, v = _owner_inputs(numels, R, A, owner, gcode, owner + 1)
        chunks = zs.zero_chunk_table(numels, off, begin, end, max_chunk)
        dchunks = zs.chunks_to_device(chunks) if chunks.size else None
        gkw = {}
        if grouped and chunks.size:
            groups = zs.zero_chunk_groups(chunks, max_chunk)
            gkw = dict(groups_dev=torch.from_numpy(groups.astype(np.int64)).to(DEV), n_groups=groups.size - 1)
        dgr = [to_dev(g, gcode) for g in grads]
        dw, dm, dv = to_dev(w, F32), to_dev(m, F32), to_dev(v, F32)
        sentinel = 0x7BFF if pcode == F16 else 0x3F80
        p16_host = np.full(total + 8, sentinel, dtype=np.uint16)
        dp = to_dev(p16_host, pcode) if pcode else None
        ow, om, ov_ = w.copy(), m.copy(), v.copy()
        ranges = oracle.real_ranges(numels, list(off), begin, end)
        assert_chunks_cover(chunks, ranges, f"{layout} owner {owner}")
        for t in (11, 12, 13):  # independent trajectories, three steps
            zs.zero_adam_step(chunks_dev=dchunks, n_chunks=chunks.size, begin=begin, end=end,
                              master=dw, exp_avg=dm, exp_avg_sq=dv, local_base=lb, step=t,
                              rank_grads=dgr, divisor=float(R), param16=dp, **gkw, **HP)
            oracle.owner_step(ranges, oracle.hyper(step=t, **HP), ow, om, ov_, lb, grads=grads,
                              gdtype=gcode, divisor=float(R), p16=p16_host if pcode else None,
                              pdtype=pcode)
            what = f"{layout} owner {owner} step {t}"
            assert_state_close(from_dev(dw), ow, what + " w")
            assert_state_close(from_dev(dm), om, what + " m")
            assert_state_close(from_dev(dv), ov_, what + " v")
            if pcode:
                got = from_dev(dp)
                real = np.zeros(total + 8, dtype=bool)
                for s, e_ in ranges:
                    real[s:e_] = True
                assert np.all(got[~real] == sentinel), what + ": padding or foreign elements written"
                assert_copy_of_master(got, p16_host, from_dev(dw), ow, lb, ranges, pcode, what + " p16")


def test_group_tables_give_the_same_bits():
    """One block per chunk, the packed group table, a hand-made group of 300
    chunks (more chunks and more work units than one block has threads) and a
    small grid that strides over the groups: identical bits every way."""
    numels, R, A = [1 + (53 * k) % 120 for k in range(700)], 2, 64
    off, total, b, e = checked_layout(numels, R, A)
    begin, end = int(b[1]), int(e[1])
    lb = begin & ~7
    grads = [to_dev(g, F16) for g in _rank_inputs(F16, R, total, seed=12)]
    w0 = gen(12, synth.STREAM_MASTER, end - lb, synth.DIST_NORMAL, 0.02, F32)
    chunks = zs.zero_chunk_table(numels, off, begin, end, 2048)
    dch = zs.chunks_to_device(chunks)
    packed = zs.zero_chunk_groups(chunks, 2048)
    assert packed.size - 1 < chunks.size // 4
    n = chunks.size
    handmade = np.array([0, 1, 301] + ([n] if n > 301 else []), dtype=np.uint64)
    handmade = np.unique(np.minimum(handmade, n))
    variants = [dict(), dict(groups=packed), dict(groups=handmade), dict(groups=packed, grid_blocks=3)]
    results = []
    for v in variants:
        dw = to_dev(w0, F32)
        dm, dv = torch.zeros_like(dw), torch.zeros_like(dw)
        p16 = torch.zeros(total, dtype=torch.float16, device=DEV)
        kw = {}
        if "groups" in v:
            g = v["groups"]
            kw = dict(groups_dev=torch.from_numpy(g.astype(np.int64)).to(DEV), n_groups=g.size - 1)
        zs.zero_adam_step(chunks_dev=dch, n_chunks=n, begin=begin, end=end, master=dw, exp_avg=dm, exp_avg_sq=dv,
                          local_base=lb, step=2, rank_grads=grads, divisor=2.0, param16=p16,
                          grid_blocks=v.get("grid_blocks", 0), **kw, **HP)
        results.append([from_dev(x).view(np.uint32) for x in (dw, dm, dv)] + [from_dev(p16)])
    for r in results[1:]:
        for x, y in zip(r, results[0]):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("adamw,wd", [(False, 0.05), (False, 0.0), (True, 0.01)])
def test_adam_variants(adamw, wd):
    numels, R, A = [4099, 17, 333], 2, 8
    hp = dict(HP, adamw=adamw, weight_decay=wd)
    off, total, begin, end, lb, grads, w, m, v = _owner_inputs(numels, R, A, 1, F16, 9)
    chunks = zs.zero_chunk_table(numels, off, begin, end, 512)
    dw, dm, dv = to_dev(w, F32), to_dev(m, F32), to_dev(v, F32)
    zs.zero_adam_step(chunks_dev=zs.chunks_to_device(chunks), n_chunks=chunks.size, begin=begin,
                      end=end, master=dw, exp_avg=dm, exp_avg_sq=dv, local_base=lb, step=3,
                      rank_grads=[to_dev(g, F16) for g in grads], divisor=2.0, **hp)
    ranges = oracle.real_ranges(numels, list(off), begin, end)
    oracle.owner_step(ranges, oracle.hyper(step=3, **hp), w, m, v, lb, grads=grads, gdtype=F16,
                      divisor=2.0)
    assert_state_close(from_dev(dw), w, "w")
    assert_state_close(from_dev(dm), m, "m")
    assert_state_close(from_dev(dv), v, "v")


def test_two_pass_with_clip_matches_oracle_and_fused():
    """reduce (+check) -> adam from the reduced gradient with a clip factor."""
    numels, R, A = [50_000, 1234, 77_777], 4, 64
    off, total, begin, end, lb, grads, w, m, v = _owner_inputs(numels, R, A, 2, F16, 21)
    dgr = [to_dev(g, F16) for g in grads]
    chunks = zs.zero_chunk_table(numels, off, begin, end, 4096)
    dch = zs.chunks_to_device(chunks)
    g_dev = torch.zeros(end - lb, dtype=torch.float32, device=DEV)
    ov, ss, ws = _check_bufs()
    zs.zero_reduce_owned(dgr, begin, end - begin, float(R), g_dev, out_base=lb, check=(ov, ss, ws))
    coef = 0.37
    dw, dm, dv = to_dev(w, F32), to_dev(m, F32), to_dev(v, F32)
    dp = torch.zeros(total, dtype=torch.float16, device=DEV)
    zs.zero_adam_step(chunks_dev=dch, n_chunks=chunks.size, begin=begin, end=end, master=dw,
                      exp_avg=dm, exp_avg_sq=dv, local_base=lb, step=5, reduced_g=g_dev,
                      param16=dp, clip_coef=coef, **HP)
    g_or = np.zeros(end - lb, dtype=np.float32)
    g_or[begin - lb:] = oracle.reduce([g[begin:end] for g in grads], F16, float(R))
    assert_bits_equal(from_dev(g_dev)[begin - lb:], g_or[begin - lb:], "two-pass reduce")
    ranges = oracle.real_ranges(numels, list(off), begin, end)
    ow, om, ovv = w.copy(), m.copy(), v.copy()
    p_or = np.zeros(total, dtype=np.uint16)
    oracle.owner_step(ranges, oracle.hyper(step=5, clip_coef=coef, **HP), ow, om, ovv, lb,
                      reduced_g=g_or, p16=p_or, pdtype=F16)
    assert_state_close(from_dev(dw), ow, "w")
    assert_state_close(from_dev(dm), om, "m")
    assert_state_close(from_dev(dv), ovv, "v")
    assert_copy_of_master(from_dev(dp), p_or, from_dev(dw), ow, lb, ranges, F16, "p16")
    # the fused single pass gives the same bits as reduce-then-step with coef 1
    fw, fm, fv = to_dev(w, F32), to_dev(m, F32), to_dev(v, F32)
    tw, tm, tv = to_dev(w, F32), to_dev(m, F32), to_dev(v, F32)
    zs.zero_adam_step(chunks_dev=dch, n_chunks=chunks.size, begin=begin, end=end, master=fw,
                      exp_avg=fm, exp_avg_sq=fv, local_base=lb, step=5, rank_grads=dgr,
                      divisor=float(R), **HP)
    zs.zero_adam_step(chunks_dev=dch, n_chunks=chunks.size, begin=begin, end=end, master=tw,
                      exp_avg=tm, exp_avg_sq=tv, local_base=lb, step=5, reduced_g=g_dev, **HP)
    for a, b in ((fw, tw), (fm, tm), (fv, tv)):
        assert_bits_equal(from_dev(a), from_dev(b), "fused vs two-pass")


@pytest.mark.parametrize("code", [F16, BF16, F32])
@pytest.mark.parametrize("R", [1, 2, 6, 8, 16, 17, 24, 37, 256])
def test_fused_step_every_rank_path(code, R):
    """The fused step's rank reduce at every code path: fully unrolled counts
    (1, 2, 8, 16), a batched count with a remainder (6), one full batch plus a
    remainder (17), several double-buffered batches (24, 37) and the maximum
    (256).  Against the oracle, and bit-identical to reduce-then-step.  The
    layout has two owners; the rank count only sets how many buffers are
    summed."""
    numels, A = [1000, 37, 5003, 1, 64, 777], 64
    off, total, b, e = checked_layout(numels, 2, A)
    begin, end = int(b[1]), int(e[1])
    lb = begin & ~7
    grads = _rank_inputs(code, R, total, seed=50 + R)
    dgr = [to_dev(g, code) for g in grads]
    size = end - lb
    w = gen(R, synth.STREAM_MASTER, size, synth.DIST_NORMAL, 0.02, F32)
    m = gen(R, synth.STREAM_EXP_AVG, size, synth.DIST_NORMAL, 5e-4, F32)
    v = gen(R, synth.STREAM_EXP_AVG_SQ, size, synth.DIST_SQUARE, 1e-4, F32)
    chunks = zs.zero_chunk_table(numels, off, begin, end, 512)
    dch = zs.chunks_to_device(chunks)
    pcode = BF16 if code == F32 else code
    dw, dm, dv = to_dev(w, F32), to_dev(m, F32), to_dev(v, F32)
    dp = torch.zeros(total, dtype=torch.float16 if pcode == F16 else torch.bfloat16, device=DEV)
    zs.zero_adam_step(chunks_dev=dch, n_chunks=chunks.size, begin=begin, end=end, master=dw, exp_avg=dm,
                      exp_avg_sq=dv, local_base=lb, step=4, rank_grads=dgr, divisor=float(R), param16=dp, **HP)
    ranges = oracle.real_ranges(numels, list(off), begin, end)
    ow, om, ovv = w.copy(), m.copy(), v.copy()
    p_or = np.zeros(total, dtype=np.uint16)
    oracle.owner_step(ranges, oracle.hyper(step=4, **HP), ow, om, ovv, lb, grads=grads, gdtype=code,
                      divisor=float(R), p16=p_or, pdtype=pcode)
    what = f"R={R}"
    assert_state_close(from_dev(dw), ow, what + " w")
    assert_state_close(from_dev(dm), om, what + " m")
    assert_state_close(from_dev(dv), ovv, what + " v")
    assert_copy_of_master(from_dev(dp), p_or, from_dev(dw), ow, lb, ranges, pcode, what + " p16")
    # reduce-then-step: the flat reduce over the owner range, then AdamW from it
    g_dev = torch.zeros(size, dtype=torch.float32, device=DEV)
    zs.zero_reduce_owned(dgr, begin, end - begin, float(R), g_dev, out_base=lb)
    tw, tm, tv = to_dev(w, F32), to_dev(m, F32), to_dev(v, F32)
    zs.zero_adam_step(chunks_dev=dch, n_chunks=chunks.size, begin=begin, end=end, master=tw, exp_avg=tm,
                      exp_avg_sq=tv, local_base=lb, step=4, reduced_g=g_dev, **HP)
    for a, c in ((dw, tw), (dm, tm), (dv, tv)):
        assert_bits_equal(from_dev(a), from_dev(c), what + " fused vs two-pass")
    # both again over the packed group table: the same bits
    groups = zs.zero_chunk_groups(chunks, 2048)
    gkw = dict(groups_dev=torch.from_numpy(groups.astype(np.int64)).to(DEV), n_groups=groups.size - 1)
    gw, gm, gv = to_dev(w, F32), to_dev(m, F32), to_dev(v, F32)
    gp = torch.zeros_like(dp)
    zs.zero_adam_step(chunks_dev=dch, n_chunks=chunks.size, begin=begin, end=end, master=gw, exp_avg=gm,
                      exp_avg_sq=gv, local_base=lb, step=4, rank_grads=dgr, divisor=float(R), param16=gp,
                      **gkw, **HP)
    rw, rm, rv = to_dev(w, F32), to_dev(m, F32), to_dev(v, F32)
    zs.zero_adam_step(chunks_dev=dch, n_chunks=chunks.size, begin=begin, end=end, master=rw, exp_avg=rm,
                      exp_avg_sq=rv, local_base=lb, step=4, reduced_g=g_dev, **gkw, **HP)
    for a, c, x in ((dw, gw, rw), (dm, gm, rm), (dv, gv, rv)):
        assert_bits_equal(from_dev(c), from_dev(a), what + " grouped fused")
        assert_bits_equal(from_dev(x), from_dev(a), what + " grouped two-pass")
    assert np.array_equal(from_dev(gp), from_dev(dp)), what + " grouped p16"


def test_checked_step_skips_clips_and_updates():
    """OwnerShard.checked_step: reduce + check, the host decision, AdamW from the
    reduced gradient with the clip factor; an overflowed step writes no state;
    an empty owner launches nothing."""
    numels, R, A = [3000, 77, 20_001, 5], 4, 64
    sh = zs.OwnerShard(numels, R, 1, align=A, max_chunk=512, device=DEV)
    sh.alloc_state()
    lb, begin, end, total = sh.local_base, sh.begin, sh.end, sh.padded_total
    grads = _rank_inputs(F16, R, total, seed=23, scale=0.5)  # a norm far above 1: the clip applies
    dgr = [to_dev(g, F16) for g in grads]
    w = gen(23, synth.STREAM_MASTER, sh.local_size, synth.DIST_NORMAL, 0.02, F32)
    m = gen(23, synth.STREAM_EXP_AVG, sh.local_size, synth.DIST_NORMAL, 5e-4, F32)
    v = gen(23, synth.STREAM_EXP_AVG_SQ, sh.local_size, synth.DIST_SQUARE, 1e-4, F32)
    for dst, src in ((sh.master, w), (sh.exp_avg, m), (sh.exp_avg_sq, v)):
        dst[:src.size].copy_(to_dev(src, F32))
    dp = torch.zeros(total, dtype=torch.float16, device=DEV)
    updated, coef = sh.checked_step(step=3, hyper=HP, rank_grads=dgr, divisor=float(R), param16=dp)
    assert updated
    g_or = oracle.reduce([g[begin:end] for g in grads], F16, float(R))
    flag, sumsq = oracle.grad_check(g_or)
    assert flag == 0
    want_coef = oracle.clip_coef(sumsq)
    assert want_coef < 0.5 and abs(coef - want_coef) <= 1e-6 * want_coef
    g_loc = np.zeros(sh.local_size, dtype=np.float32)
    g_loc[begin - lb:] = g_or
    ranges = shard_ranges(sh)
    ow, om, ov_ = w.copy(), m.copy(), v.copy()
    p_or = np.zeros(total, dtype=np.uint16)
    oracle.owner_step(ranges, oracle.hyper(step=3, clip_coef=coef, **HP), ow, om, ov_, lb, reduced_g=g_loc,
                      p16=p_or, pdtype=F16)
    assert_state_close(from_dev(sh.master)[:sh.local_size], ow, "w")
    assert_state_close(from_dev(sh.exp_avg)[:sh.local_size], om, "m")
    assert_state_close(from_dev(sh.exp_avg_sq)[:sh.local_size], ov_, "v")
    assert_copy_of_master(from_dev(dp), p_or, from_dev(sh.master), ow, lb, ranges, F16, "p16")
    # an inf in one rank: the step is skipped and no state or 16-bit value changes
    before = [from_dev(x).copy() for x in (sh.master, sh.exp_avg, sh.exp_avg_sq, dp)]
    dgr[2][begin + 5] = float("inf")
    assert sh.checked_step(step=4, hyper=HP, rank_grads=dgr, divisor=float(R), param16=dp) == (False, None)
    for a, b in zip(before, (sh.master, sh.exp_avg, sh.exp_avg_sq, dp)):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              from_dev(b).view(np.uint32) if a.dtype == np.float32 else from_dev(b))
    # an empty owner: nothing to do
    empty = zs.OwnerShard([3, 2], 9, 0, align=1, device=DEV)
    assert empty.begin == empty.end
    empty.alloc_state()
    assert empty.checked_step(step=1, hyper=HP, rank_grads=[to_dev(np.zeros(8, np.float32), F32)]) == (True, 1.0)


@pytest.mark.parametrize("numels,R,A,scale", [([3000, 77, 20_001, 5, 9000], 5, 64, 0.5), ([3, 2], 9, 1, 40.0),
                                               ([40, 7, 1000], 4, 8, 2.0)])
def test_checked_step_over_every_owner_is_the_unsharded_clip_and_skip(numels, R, A, scale):
    """Every owner of a layout (empty owners included) reduces and checks its own
    slice; the host combines the flags and partial norms (zero_step_decision)
    and every owner applies the same decision.  The result is the oracle's
    unsharded step: one overflow flag and one clip factor from the whole
    gradient.  Then an inf in one owner's slice skips every owner's step."""
    off, total, owners = oracle.layout(numels, R, A)
    shards = [zs.OwnerShard(numels, R, r, align=A, max_chunk=256, device=DEV) for r in range(R)]
    ranges = [shard_ranges(sh) for sh in shards]
    grads = _rank_inputs(F16, R, total, seed=31, scale=scale)  # the whole norm is far above 1
    # the rank buffers hold zeros in the padding (no parameter lives there): the
    # checked reduce runs over each owner's flat range, padding included
    pad = np.ones(total, dtype=bool)
    for rr in ranges:
        for b, e in rr:
            pad[b:e] = False
    for g in grads:
        g[pad] = 0
    dgr = [to_dev(g, F16) for g in grads]
    w = gen(31, synth.STREAM_MASTER, total + 8, synth.DIST_NORMAL, 0.02, F32)
    m = gen(31, synth.STREAM_EXP_AVG, total + 8, synth.DIST_NORMAL, 5e-4, F32)
    v = gen(31, synth.STREAM_EXP_AVG_SQ, total + 8, synth.DIST_SQUARE, 1e-4, F32)
    for sh in shards:
        sh.alloc_state()
        for dst, src in ((sh.master, w), (sh.exp_avg, m), (sh.exp_avg_sq, v)):
            dst[:sh.local_size].copy_(to_dev(src[sh.local_base:sh.end], F32))
    dp = torch.zeros(total, dtype=torch.float16, device=DEV)

    def run(step):
        parts = [sh.reduce_and_check(rank_grads=dgr, divisor=float(R)) for sh in shards]
        updated, coef = zs.zero_step_decision([f for f, _ in parts], [s for _, s in parts], 1.0)
        if updated:
            for sh in shards:
                sh.apply_update(step=step, hyper=HP, coef=coef, param16=dp)
        return updated, coef

    updated, coef = run(3)
    # the oracle's unsharded step: the whole gradient's flag and norm
    real = [rg for rr in ranges for rg in rr]
    g_all = np.zeros(total, dtype=np.float32)
    for b, e in real:
        g_all[b:e] = oracle.reduce([g[b:e] for g in grads], F16, float(R))
    flag, sumsq = oracle.grad_check(np.concatenate([g_all[b:e] for b, e in real]))
    assert flag == 0 and updated
    want_coef = oracle.clip_coef(sumsq)
    assert want_coef < 0.5 and abs(coef - want_coef) <= 1e-6 * want_coef
    ow, om, ov_ = w.copy(), m.copy(), v.copy()
    p_or = np.zeros(total, dtype=np.uint16)
    oracle.owner_step(real, oracle.hyper(step=3, clip_coef=coef, **HP), ow, om, ov_, 0, reduced_g=g_all,
                      p16=p_or, pdtype=F16)
    for r, sh in enumerate(shards):
        b, e, lb = sh.begin, sh.end, sh.local_base
        for got, want, nm in ((sh.master, ow, "w"), (sh.exp_avg, om, "m"), (sh.exp_avg_sq, ov_, "v")):
            assert_state_close(from_dev(got)[b - lb:e - lb], want[b:e], f"owner {r} {nm}")
    gw = w.copy()  # the kernels' master weights, flat-indexed
    for sh in shards:
        gw[sh.begin:sh.end] = from_dev(sh.master)[sh.begin - sh.local_base:sh.end - sh.local_base]
    assert_copy_of_master(from_dev(dp), p_or, gw, ow, 0, real, F16, "p16")
    # one owner's slice holds an inf: every owner skips, nothing changes anywhere
    r_bad = max(range(R), key=lambda r: shards[r].end - shards[r].begin)
    before = [[from_dev(x).copy() for x in (sh.master, sh.exp_avg, sh.exp_avg_sq)] for sh in shards]
    p_before = from_dev(dp).copy()
    dgr[1][ranges[r_bad][0][0]] = float("inf")  # the owner's first real element
    assert run(4) == (False, None)
    for sh, old in zip(shards, before):
        for a, x in zip(old, (sh.master, sh.exp_avg, sh.exp_avg_sq)):
            assert np.array_equal(a.view(np.uint32), from_dev(x).view(np.uint32))
    assert np.array_equal(p_before, from_dev(dp))
    # the owners without the inf saw no overflow of their own: the decision is global
    own_flags = [sh.reduce_and_check(rank_grads=dgr, divisor=float(R))[0] for sh in shards]
    assert own_flags[r_bad] == 1 and sum(own_flags) == 1


def test_no_op_cases_leave_memory_untouched():
    dw = torch.full((16,), 3.0, device=DEV)
    dm, dv = torch.zeros(16, device=DEV), torch.zeros(16, device=DEV)
    g = torch.ones(16, dtype=torch.float16, device=DEV)
    zs.zero_adam_step(chunks_dev=None, n_chunks=0, begin=8, end=8, master=dw, exp_avg=dm,
                      exp_avg_sq=dv, local_base=8, step=1, rank_grads=[g], divisor=1.0, **HP)
    out = torch.full((16,), 5.0, device=DEV)
    zs.zero_reduce_owned([g], 3, 0, 1.0, out)
    torch.cuda.synchronize()
    assert torch.all(dw == 3.0) and torch.all(out == 5.0)


def test_max_ranks():
    R, n = zs.ZERO_MAX_RANKS, 1000
    grads = [gen(8, synth.STREAM_GRAD, n, synth.DIST_NORMAL, 1.0, BF16, rank=r) for r in range(R)]
    out = torch.empty(n, dtype=torch.float32, device=DEV)
    zs.zero_reduce_owned([to_dev(g, BF16) for g in grads], 0, n, float(R), out)
    assert_bits_equal(from_dev(out), oracle.reduce(grads, BF16, float(R)), "R=256")
    with pytest.raises(zs.ZeroShardError):
        zs.zero_reduce_owned([to_dev(grads[0], BF16)] * (R + 1), 0, n, 1.0, out)


# ---------------------------------------------------------------- the pages' tiny case
def _tiny_run(owners, grads_fn, steps=5):
    P, R = 11, 4
    hp = dict(lr=0.01, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, adamw=False)
    w = torch.tensor([0.1 * i for i in range(P)] + [0.0] * 5, dtype=torch.float32, device=DEV)
    m, v = torch.zeros(16, device=DEV), torch.zeros(16, device=DEV)
    for t in range(1, steps + 1):
        rows = [to_dev(np.array([grads_fn(i, r, t) for i in range(P)] + [0.0] * 5, dtype=np.float32), F32)
                for r in range(R)]
        for b, e in owners:
            if b == e:
                continue
            lb = b & ~7
            ch = zs.zero_chunk_table([P], [0], b, e, 8)
            zs.zero_adam_step(chunks_dev=zs.chunks_to_device(ch), n_chunks=ch.size, begin=b, end=e,
                              master=w[lb:], exp_avg=m[lb:], exp_avg_sq=v[lb:], local_base=lb,
                              step=t, rank_grads=rows, divisor=float(R), **hp)
    return from_dev(w)[:P], from_dev(m)[:P], from_dev(v)[:P]


def _uniform_grad(i, r, t):
    key = synth.stream_key(1, synth.STREAM_GRAD, r, t)
    return float(synth.values_f32(key, [i], synth.DIST_UNIFORM, 0.3)[0])


@pytest.mark.parametrize("grad_fn", [oracle.pages_gradient, _uniform_grad])
def test_tiny_sharded_equals_unsharded_on_gpu(grad_fn):
    owners = [(o.start, o.stop) for o in oracle.owner_ranges(11, 4)]
    sharded = _tiny_run(owners, grad_fn)
    unsharded = _tiny_run([(0, 11)], grad_fn)
    for a, b in zip(sharded, unsharded):
        assert_bits_equal(a, b, "sharded vs unsharded")
    reference, _ = oracle.compare_owned_updates(11, 4, 5, grad=grad_fn)
    ref = np.array(reference)
    for k in range(3):
        assert_state_close(sharded[k], ref[:, k].astype(np.float32), f"vs the pages' lab, field {k}")


def test_first_step_closed_form_on_gpu():
    # w = 1, gradient 2, lr 0.01, t = 1: w = 1 - 0.01 * 2 / (2 + 1e-8), m = 0.2, v = 0.004
    w = torch.ones(8, device=DEV)
    m, v = torch.zeros(8, device=DEV), torch.zeros(8, device=DEV)
    g = torch.full((8,), 2.0, device=DEV)
    ch = zs.zero_chunk_table([8], [0], 0, 8, 8)
    zs.zero_adam_step(chunks_dev=zs.chunks_to_device(ch), n_chunks=1, begin=0, end=8, master=w,
                      exp_avg=m, exp_avg_sq=v, local_base=0, step=1, rank_grads=[g], divisor=1.0,
                      lr=0.01, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, adamw=False)
    assert_state_close(from_dev(w), np.full(8, 1.0 - 0.01 * 2.0 / (2.0 + 1e-8)), "w")
    assert_state_close(from_dev(m), np.full(8, 0.2), "m")
    assert_state_close(from_dev(v), np.full(8, 0.004), "v")


# ---------------------------------------------------------------- per-backward reduce + accumulate
@pytest.mark.parametrize("code", [F16, BF16, F32])
@pytest.mark.parametrize("R", [1, 6, 16])
def test_reduce_add_mean_bitexact(code, R):
    total, begin, n = 40_011, 3, 40_000
    grads = _rank_inputs(code, R, total, seed=31 + R)
    start = gen(3, synth.STREAM_EXP_AVG, begin + n, synth.DIST_NORMAL, 1e-2, F32)
    out = to_dev(start.copy(), F32)
    zs.zero_reduce_owned([to_dev(g, code) for g in grads], begin, n, float(R), out, accumulate=2)
    want = start.copy()
    oracle.reduce_add([g[begin:begin + n] for g in grads], code, float(R), want[begin:])
    assert_bits_equal(from_dev(out), want, f"add-mean R={R}")


def test_per_backward_schedule_matches_oracle():
    """Four microsteps: each reduces the ranks' owned slices and adds the mean to the
    owner's fp32 accumulator; AdamW runs once from it at the boundary."""
    numels, R, A, K = [3000, 77, 20_001, 5], 4, 64, 4
    off, total, b, e = checked_layout(numels, R, A)
    owner = 2
    begin, end = int(b[owner]), int(e[owner])
    lb = begin & ~7
    micro = [[gen(40 + k, synth.STREAM_MICRO, total, synth.DIST_NORMAL, 1e-3, BF16, rank=r) for r in range(R)]
             for k in range(K)]
    acc_dev = torch.zeros(end - lb, dtype=torch.float32, device=DEV)
    for k in range(K):
        slices = [to_dev(m[lb:end], BF16) for m in micro[k]]
        zs.zero_reduce_owned(slices, begin, end - begin, float(R), acc_dev, grad_base=lb, out_base=lb,
                             accumulate=0 if k == 0 else 2)
    acc = np.zeros(end - lb, dtype=np.float32)
    for k in range(K):
        if k == 0:
            acc[begin - lb:] = oracle.reduce([m[begin:end] for m in micro[k]], BF16, float(R))
        else:
            oracle.reduce_add([m[begin:end] for m in micro[k]], BF16, float(R), acc[begin - lb:])
    assert_bits_equal(from_dev(acc_dev)[begin - lb:], acc[begin - lb:], "per-backward accumulator")
    _, _, _, _, _, _, w, m, v = _owner_inputs(numels, R, A, owner, BF16, 5)
    chunks = zs.zero_chunk_table(numels, off, begin, end, 512)
    dw, dm, dv = to_dev(w, F32), to_dev(m, F32), to_dev(v, F32)
    dp = torch.zeros(total, dtype=torch.bfloat16, device=DEV)
    zs.zero_adam_step(chunks_dev=zs.chunks_to_device(chunks), n_chunks=chunks.size, begin=begin, end=end,
                      master=dw, exp_avg=dm, exp_avg_sq=dv, local_base=lb, step=7, reduced_g=acc_dev,
                      param16=dp, **HP)
    p_or = np.zeros(total, dtype=np.uint16)
    ranges = oracle.real_ranges(numels, list(off), begin, end)
    oracle.owner_step(ranges, oracle.hyper(step=7, **HP), w, m, v, lb, reduced_g=acc, p16=p_or, pdtype=BF16)
    assert_state_close(from_dev(dw), w, "w")
    assert_state_close(from_dev(dm), m, "m")
    assert_state_close(from_dev(dv), v, "v")
    assert_copy_of_master(from_dev(dp), p_or, from_dev(dw), w, lb, ranges, BF16, "p16")


# ---------------------------------------------------------------- launch-shape independence
def _fused_once(numels, R, A, owner, max_chunk, grid_blocks, chunks_override=None):
    off, total, begin, end, lb, grads, w, m, v = _owner_inputs(numels, R, A, owner, F16, 77)
    chunks = chunks_override if chunks_override is not None else zs.zero_chunk_table(numels, off, begin, end, max_chunk)
    dw, dm, dv = to_dev(w, F32), to_dev(m, F32), to_dev(v, F32)
    dp = torch.zeros(total + 8, dtype=torch.float16, device=DEV)
    zs.zero_adam_step(chunks_dev=zs.chunks_to_device(chunks), n_chunks=chunks.size, begin=begin, end=end,
                      master=dw, exp_avg=dm, exp_avg_sq=dv, local_base=lb, step=4,
                      rank_grads=[to_dev(g, F16) for g in grads], divisor=float(R), param16=dp,
                      grid_blocks=grid_blocks, **HP)
    return [from_dev(x) for x in (dw, dm, dv, dp)]


def test_fused_step_is_deterministic_and_independent_of_grid_and_chunking():
    numels, R, A, owner = [10_000, 37, 70_001, 5], 4, 64, 1
    ref = _fused_once(numels, R, A, owner, 2048, 0)
    again = _fused_once(numels, R, A, owner, 2048, 0)
    for a, b in zip(ref, again):
        assert_bits_equal(a, b, "run to run")
    for chunk, grid in ((8, 0), (64, 1), (2048, 1), (2048, 3), (16384, 7), (1 << 20, 0)):
        got = _fused_once(numels, R, A, owner, chunk, grid)
        for a, b in zip(ref, got):
            assert_bits_equal(a, b, f"chunk {chunk} grid {grid}")


def test_chunks_outside_the_owner_range_are_ignored():
    numels, R, A, owner = [5000, 3000], 3, 8, 1
    off, total, b, e = checked_layout(numels, R, A)
    begin, end = int(b[owner]), int(e[owner])
    good = zs.zero_chunk_table(numels, off, begin, end, 512)
    ref = _fused_once(numels, R, A, owner, 512, 0)
    # a table that also names elements of the neighbouring owners: clamped to [begin, end)
    wide = zs.zero_chunk_table(numels, off, 0, total, 512)
    got = _fused_once(numels, R, A, owner, 512, 0, chunks_override=wide)
    for a, b_ in zip(ref, got):
        assert_bits_equal(a, b_, "wide chunk table")
    assert good.size < wide.size
