"""GPU parity at the edges of the number formats, through the C ABI.

* The 16-bit write-back: with lr = 0, zero gradients and zero moments, AdamW
  leaves every fp32 master weight unchanged, so the written fp16/bf16 copy
  must be the round-to-nearest-even encoding of the given weight itself --
  bit-exact against the oracle's own encoder (which the CPU tests pin to
  numpy's fp16 cast and torch's bf16 cast).  The weights cover the overflow
  threshold (fp16 65504 / 65520, bf16 and fp32 maxima), ties at every scale,
  the subnormal ranges of both formats, signed zeros, infinities, NaNs, and
  random fp32 bit patterns.
* The rank reduce over subnormal inputs of each dtype: bit-exact against the
  oracle, with an IEEE (non-power-of-two) divisor too, and a fused check
  whose squared norm matches the oracle's.  This holds only if the kernels
  keep subnormals (no flush to zero) and divide with IEEE rounding.
* The fused step at extreme step counts and betas, against the oracle to its
  tolerance: bias corrections tiny, near one or exactly one, and zero betas.
"""
import math

import numpy as np
import pytest

import oracle
from helpers import BF16, F16, F32, assert_bits_equal, checked_layout, from_dev, to_dev

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


def _f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def _edge_weights(pcode: int, seed: int) -> np.ndarray:
    """fp32 weights at the edges of the 16-bit format, then random bit patterns."""
    rng = np.random.default_rng(seed)
    vals = [0.0, -0.0, np.inf, -np.inf, np.nan, 1.0, -1.0]
    if pcode == F16:
        half_ulp_max = 16.0  # ulp of the top fp16 binade is 32
        vals += [65504.0, -65504.0, 65504.0 + half_ulp_max, -(65504.0 + half_ulp_max),  # ties: to inf
                 np.nextafter(np.float32(65520.0), np.float32(0.0)), 65536.0, 1e5, -3e38]
        # subnormal fp16 range: k * 2^-25, i.e. every half-way point between subnormals
        vals += [k * 2.0 ** -25 for k in range(-70, 71)]
        vals += [2.0 ** -14, -(2.0 ** -14), 2.0 ** -14 - 2.0 ** -25, 2.0 ** -26, 3 * 2.0 ** -26]
        # ties at every binade: 1 + (2j+1) 2^-11 scaled, and one fp32 ulp either side
        for e in range(-14, 16):
            for j in range(4):
                t = np.float32((1.0 + (2 * j + 1) * 2.0 ** -11) * 2.0 ** e)
                vals += [t, np.nextafter(t, np.float32(0.0)), np.nextafter(t, np.float32(np.inf))]
    else:
        vals += [float(_f32(0x7F7F0000)), float(_f32(0x7F7F8000)), float(_f32(0x7F7F7FFF)),
                 float(_f32(0x7F7FFFFF)), float(_f32(0xFF7FFFFF)), float(_f32(0x7F7E8000))]
        # fp32 subnormals around bf16 ties (low 16 bits 0x8000 with even and odd upper halves)
        vals += [float(x) for x in _f32([0x00000001, 0x00008000, 0x00018000, 0x00007FFF, 0x80008000,
                                         0x007F8000, 0x007FFFFF, 0x00800000, 0x80018001])]
        for e in range(-126, 128, 7):
            for j in range(4):
                t = np.float32((1.0 + (2 * j + 1) * 2.0 ** -8) * 2.0 ** e)
                vals += [t, np.nextafter(t, np.float32(0.0)), np.nextafter(t, np.float32(np.inf))]
    fixed = np.array(vals, dtype=np.float32)
    # NaN payloads, and random bit patterns over the whole fp32 range
    nans = _f32([0x7F800001, 0xFFC00001, 0x7FBFFFFF, 0x7FC12345])
    rand = rng.integers(0, 2 ** 32, size=3000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    return np.concatenate([fixed, nans, rand])


@pytest.mark.parametrize("grouped", [False, True])
@pytest.mark.parametrize("pcode", [F16, BF16])
def test_write_back_encodes_the_master_weight_exactly(pcode, grouped):
    w = _edge_weights(pcode, seed=pcode)
    n = w.size + 5  # a ragged end: the last elements take the scalar path
    w = np.concatenate([w, np.array([65504.0, -0.0, 2.0 ** -24, np.nan, 1e-40], dtype=np.float32)])
    print(f"write-back {pcode} grouped={grouped} n={n}", flush=True)
    # two tensors, the second short and padded, so that chunks, vectors and scalar ends all occur
    numels = [n - 13, 13]
    off, total, b, e = checked_layout(numels, 1, 8)
    begin, end = int(b[0]), int(e[0])
    flat_w = np.zeros(end, dtype=np.float32)
    flat_w[:n - 13] = w[:n - 13]
    flat_w[int(off[1]):int(off[1]) + 13] = w[n - 13:]
    chunks = zs.zero_chunk_table(numels, off, begin, end, 64)
    kw = {}
    if grouped:
        groups = zs.zero_chunk_groups(chunks, 2048)
        kw = dict(groups_dev=torch.from_numpy(groups.astype(np.int64)).to(DEV), n_groups=groups.size - 1)
    dw = to_dev(flat_w, F32)
    zeros = lambda: torch.zeros(end, dtype=torch.float32, device=DEV)  # noqa: E731
    dm, dv = zeros(), zeros()
    grads = [torch.zeros(end, dtype=torch.float16, device=DEV)]
    sentinel = 0x1234
    dp = to_dev(np.full(end, sentinel, dtype=np.uint16), pcode)
    zs.zero_adam_step(chunks_dev=zs.chunks_to_device(chunks), n_chunks=chunks.size, begin=begin, end=end,
                      master=dw, exp_avg=dm, exp_avg_sq=dv, local_base=0, step=1, rank_grads=grads,
                      divisor=1.0, param16=dp, lr=0.0, beta1=0.9, beta2=0.999, eps=1e-8,
                      weight_decay=0.0, adamw=True, **kw)
    got_w = from_dev(dw)
    assert_bits_equal(got_w, flat_w, "master weights unchanged at lr = 0")
    real = np.zeros(end, dtype=bool)
    for s, t in oracle.real_ranges(numels, list(off), begin, end):
        real[s:t] = True
    got = from_dev(dp)
    assert np.all(got[~real] == sentinel), "padding written"
    want = oracle.encode16(flat_w[real], pcode)
    got_r = got[real]
    gnan = np.isnan(oracle.decode16(got_r, pcode))
    wnan = np.isnan(oracle.decode16(want, pcode))
    assert np.array_equal(gnan, wnan), "NaN positions differ"
    assert_bits_equal(got_r[~gnan], want[~wnan], f"16-bit write-back ({'fp16' if pcode == F16 else 'bf16'})")
    # and the bf16 quiet-NaN rule: a NaN keeps its sign and is quiet
    if pcode == BF16:
        assert np.all((got_r[gnan] & 0x0040) != 0)


def _subnormal_ranks(code: int, R: int, n: int, seed: int):
    """R rank buffers of subnormal (and a few tiny normal) values of the dtype."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(R):
        if code == F16:
            mant = rng.integers(0, 0x400, size=n, dtype=np.uint32)  # exponent field 0
            bits = (mant | (rng.integers(0, 2, size=n, dtype=np.uint32) << 15)).astype(np.uint16)
            bits[::17] = 0x0400  # smallest normal
            out.append(bits)
        elif code == BF16:
            mant = rng.integers(0, 0x80, size=n, dtype=np.uint32)
            bits = (mant | (rng.integers(0, 2, size=n, dtype=np.uint32) << 15)).astype(np.uint16)
            bits[::17] = 0x0080
            out.append(bits)
        else:
            mant = rng.integers(0, 0x800000, size=n, dtype=np.uint64).astype(np.uint32)
            bits = mant | (rng.integers(0, 2, size=n, dtype=np.uint32) << 31).astype(np.uint32)
            bits[::17] = 0x00800000
            out.append(bits.view(np.float32))
    return out


@pytest.mark.parametrize("divisor", [1.0, 3.0, 4.0])
@pytest.mark.parametrize("code", [F16, BF16, F32])
def test_reduce_of_subnormals_is_bitexact(code, divisor):
    R, n, begin = 5, 20_011, 3
    print(f"subnormal reduce code={code} divisor={divisor}", flush=True)
    grads = _subnormal_ranks(code, R, begin + n, seed=10 * code + int(divisor))
    dgr = [to_dev(g, code) for g in grads]
    out = torch.empty(begin + n, dtype=torch.float32, device=DEV)
    ov = torch.zeros(1, dtype=torch.int32, device=DEV)
    ss = torch.zeros(1, dtype=torch.float64, device=DEV)
    ws = zs.check_workspace(n, DEV)
    zs.zero_reduce_owned(dgr, begin, n, divisor, out, check=(ov, ss, ws))
    want = oracle.reduce([g[begin:] for g in grads], code, divisor)
    got = from_dev(out)[begin:]
    assert_bits_equal(got, want, "reduce of subnormal inputs")
    if code != F16:  # bf16 and fp32 subnormal inputs give subnormal fp32 sums: they must survive
        assert np.count_nonzero((want.view(np.uint32) & 0x7F800000) == 0) > n // 4
    flag, sumsq = oracle.grad_check(want)
    assert int(ov.item()) == flag == 0
    assert math.isclose(ss.item(), sumsq, rel_tol=1e-9, abs_tol=0.0)


# (step, beta1, beta2): bias corrections near 0 (betas near 1 early on), near 1
# (late steps), exactly 1 (beta^t underflows), and betas of 0 (no averaging).
HYPER_EDGES = [(1, 0.9, 0.999), (3, 0.999, 0.999999), (1_000_000, 0.9, 0.99999), (2 ** 40, 0.8, 0.999),
               (7, 0.0, 0.0), (2, 0.0, 0.999)]


@pytest.mark.parametrize("step,beta1,beta2", HYPER_EDGES)
def test_fused_step_at_extreme_steps_and_betas(step, beta1, beta2):
    """The fused step against the oracle (common pre-state, tolerance 1e-6 rel /
    1e-7 abs, 16-bit copy within 1 ulp), where the host's fp64 bias corrections
    are tiny, exactly one, or the betas are zero."""
    import synth
    from helpers import assert_copy_of_master, assert_state_close, gen

    print(f"hyper edges step={step} beta1={beta1} beta2={beta2}", flush=True)
    numels, R, A, owner = [1000, 37, 5003, 1, 777], 3, 64, 1
    off, total, b, e = checked_layout(numels, R, A)
    begin, end = int(b[owner]), int(e[owner])
    lb = begin & ~7
    size = end - lb
    grads = [gen(9, synth.STREAM_GRAD, total, synth.DIST_NORMAL, 1e-3, F16, rank=r) for r in range(R)]
    w = gen(9, synth.STREAM_MASTER, size, synth.DIST_NORMAL, 0.02, F32)
    m = gen(9, synth.STREAM_EXP_AVG, size, synth.DIST_NORMAL, 5e-4, F32)
    v = gen(9, synth.STREAM_EXP_AVG_SQ, size, synth.DIST_SQUARE, 1e-4, F32)
    hp = dict(lr=1e-3, beta1=beta1, beta2=beta2, eps=1e-8, weight_decay=3e-7, adamw=True)
    chunks = zs.zero_chunk_table(numels, off, begin, end, 256)
    dw, dm, dv = to_dev(w, F32), to_dev(m, F32), to_dev(v, F32)
    p_host = np.zeros(total, dtype=np.uint16)
    dp = to_dev(p_host, F16)
    zs.zero_adam_step(chunks_dev=zs.chunks_to_device(chunks), n_chunks=chunks.size, begin=begin, end=end,
                      master=dw, exp_avg=dm, exp_avg_sq=dv, local_base=lb, step=step,
                      rank_grads=[to_dev(g, F16) for g in grads], divisor=float(R), param16=dp, **hp)
    ranges = oracle.real_ranges(numels, list(off), begin, end)
    oracle.owner_step(ranges, oracle.hyper(step=step, **hp), w, m, v, lb, grads=grads, gdtype=F16,
                      divisor=float(R), p16=p_host, pdtype=F16)
    assert_state_close(from_dev(dw), w, "w")
    assert_state_close(from_dev(dm), m, "m")
    assert_state_close(from_dev(dv), v, "v")
    assert_copy_of_master(from_dev(dp), p_host, from_dev(dw), w, lb, ranges, F16, "p16")
