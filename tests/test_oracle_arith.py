"""Oracle pins for the arithmetic: 16-bit encoders, fp32 rank reduce, accumulation,
overflow flag and squared norm, Adam/AdamW, and the composed owner step.

Pins come from library routines (numpy fp16 casts, torch bf16 casts,
torch.optim.Adam/AdamW in float64, math.fsum), exact rational arithmetic and
closed forms -- never from the oracle's own formula retyped.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

F16, BF16, F32 = oracle.F16, oracle.BF16, oracle.F32


# ---------------------------------------------------------------- encoders
def _edge_f32():
    h = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)].astype(np.float32)
    up = np.nextafter(h, np.float32(np.inf))
    down = np.nextafter(h, np.float32(-np.inf))
    mids = ((h.astype(np.float64)[:-1] + h.astype(np.float64)[1:]) / 2).astype(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 65504, 65519.99, 65520, 65536, 1e-8, 6e-8,
                        5.96e-8, 2.98e-8, 2.9802322e-8, 3.4e38, 1e-45, -1e-45], dtype=np.float32)
    return np.concatenate([h, up, down, mids, special])


def test_f16_encoder_matches_numpy():
    rng = np.random.default_rng(0)
    x = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([x[np.isfinite(x)], _edge_f32()])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.encode16(x, F16), want)


def test_bf16_encoder_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([x[np.isfinite(x)], _edge_f32(),
                        np.array([3.3895314e38, 3.3961775e38, 3.4028235e38], dtype=np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.encode16(x, BF16), want)


def test_nan_encodes_to_nan():
    out = oracle.encode16(np.array([np.nan, -np.nan], dtype=np.float32), F16)
    assert all(np.isnan(np.array(out, dtype=np.uint16).view(np.float16)))
    out = oracle.encode16(np.array([np.nan], dtype=np.float32), BF16)
    assert (out[0] & 0x7F80) == 0x7F80 and (out[0] & 0x7F) != 0


def test_decoders_are_exact():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    d16 = oracle.decode16(bits, F16)
    want = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(d16[fin], want[fin]) and np.array_equal(np.isnan(d16), np.isnan(want))
    db = oracle.decode16(bits, BF16)
    wantb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(wantb)
    assert np.array_equal(db[fin], wantb[fin]) and np.array_equal(np.isnan(db), np.isnan(wantb))


# ---------------------------------------------------------------- reduce
def _exact_round_f32(q: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32 value, ties to even (normal range)."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (e - 23)
    k = a / quantum
    fl = math.floor(k)
    rem = k - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return np.float32(sign * float(fl * quantum))


def test_single_rank_divisor_one_is_widening():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(10_000).astype(np.float32) * 100
    h = x.astype(np.float16)
    assert np.array_equal(oracle.reduce([h.view(np.uint16)], F16, 1.0), h.astype(np.float32))
    b = torch.from_numpy(x).to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().view(np.uint16).copy()
    assert np.array_equal(oracle.reduce([bits], BF16, 1.0), b.to(torch.float32).numpy())
    assert np.array_equal(oracle.reduce([x], F32, 1.0), x)


@pytest.mark.parametrize("R", [1, 2, 3, 4, 8, 16, 64])
def test_dyadic_inputs_are_exact(R):
    """Multiples of 2^-10 with |k| <= 1024: every partial sum is exact in fp32."""
    rng = np.random.default_rng(R)
    n = 4096
    ks = rng.integers(-1024, 1025, size=(R, n))
    grads = [(k * 2.0 ** -10).astype(np.float16).view(np.uint16) for k in ks]
    D = float(R)
    out = oracle.reduce(grads, F16, D)
    for i in range(0, n, 37):
        exact = Fraction(int(ks[:, i].sum()), 1024) / R
        assert out[i] == _exact_round_f32(exact)


def test_sum_order_is_rank_order_in_fp32():
    # Closed forms that any other order or width gets wrong: ulp(1e8) in fp32 is 8.
    big = np.float32(1e8)
    cases = [([big, 1.0, -big], 0.0), ([big, -big, 1.0], 1.0), ([1.0, big, -big], 0.0),
             ([1.0, 1.0, big, -big], 0.0), ([big, 4.0, 4.0, -big], 0.0),
             ([big, 12.0, -big], 16.0), ([4.0, 4.0, big, -big], 8.0), ([big, -big, 4.0, 4.0], 8.0)]
    for vals, want in cases:
        grads = [np.array([v], dtype=np.float32) for v in vals]
        assert oracle.reduce(grads, F32, 1.0)[0] == want


def test_negative_zero_sum_starts_at_plus_zero():
    grads = [np.array([-0.0, -0.0], dtype=np.float32) for _ in range(3)]
    out = oracle.reduce(grads, F32, 4.0)
    assert out[0] == 0.0 and not np.signbit(out[0])
    hz = np.array([0x8000, 0x8000], dtype=np.uint16)
    out = oracle.reduce([hz, hz], F16, 2.0)
    assert not np.signbit(out[0])


def test_division_is_correctly_rounded_for_any_divisor():
    rng = np.random.default_rng(5)
    for D in (3.0, 5.0, 7.0, 12.0, 6.0 * 65536):
        ks = rng.integers(-1024, 1025, size=(3, 500))
        grads = [(k * 2.0 ** -10).astype(np.float32) for k in ks]
        out = oracle.reduce(grads, F32, D)
        for i in range(500):
            exact = Fraction(int(ks[:, i].sum()), 1024) / Fraction(D)
            assert out[i] == _exact_round_f32(exact)


def test_random_sum_within_recursive_summation_bound():
    rng = np.random.default_rng(6)
    R, n = 64, 20_000
    x = (rng.standard_normal((R, n)) * 50).astype(np.float16)
    out = oracle.reduce([r.view(np.uint16) for r in x], F16, 1.0)
    xs = x.astype(np.float64)
    exact = xs.sum(axis=0)  # every term and partial sum is exact in fp64 here
    bound = (R - 1) * 2.0 ** -24 * np.abs(xs).sum(axis=0) * 1.0001
    assert np.all(np.abs(out.astype(np.float64) - exact) <= bound)


def test_overflow_and_nan_propagate():
    big = np.array([3e38, 1.0], dtype=np.float32)
    out = oracle.reduce([big, big], F32, 2.0)
    assert np.isinf(out[0]) and out[1] == 1.0
    nan_rank = np.array([np.nan, 2.0], dtype=np.float32)
    out = oracle.reduce([big, nan_rank], F32, 1.0)
    assert np.isnan(out[0])
    pinf = np.array([np.inf], dtype=np.float32)
    out = oracle.reduce([pinf, -pinf], F32, 1.0)
    assert np.isnan(out[0])


def test_accumulate_starts_from_out():
    a = np.array([0.5, -2.0, 1e8], dtype=np.float32)
    g = [np.array([0.25, 0.5, 1.0], dtype=np.float32)]
    out = oracle.reduce(g, F32, 1.0, out=a.copy(), accumulate=True)
    assert np.array_equal(out, np.array([0.75, -1.5, 1e8], dtype=np.float32))


def test_gradient_accumulation_is_rank_reduce_with_divisor_one():
    rng = np.random.default_rng(8)
    micro = [torch.from_numpy(rng.standard_normal(3000).astype(np.float32) * 1e-3).to(torch.bfloat16)
             .view(torch.int16).numpy().view(np.uint16).copy() for _ in range(8)]
    acc = np.full(3000, 123.0, dtype=np.float32)  # stale contents must be ignored on the first
    for k, g in enumerate(micro):
        oracle.accumulate(g, BF16, acc, first=(k == 0))
    assert np.array_equal(acc, oracle.reduce(micro, BF16, 1.0))
    # dyadic microsteps: exact
    ks = rng.integers(-512, 513, size=(8, 100))
    gs = [(k * 2.0 ** -8).astype(np.float32) for k in ks]
    acc = np.zeros(100, dtype=np.float32)
    for k, g in enumerate(gs):
        oracle.accumulate(g, F32, acc, first=(k == 0))
    assert np.array_equal(acc, (ks.sum(axis=0) * 2.0 ** -8).astype(np.float32))


# ---------------------------------------------------------------- grad check
def test_grad_check_closed_forms():
    assert oracle.grad_check(np.ones(100_000, dtype=np.float32)) == (0, 100_000.0)
    ints = np.arange(-500, 500, dtype=np.float32)
    assert oracle.grad_check(ints) == (0, float(sum(i * i for i in range(-500, 500))))
    c = np.float32(0.003)
    flag, s = oracle.grad_check(np.full(4096, c, dtype=np.float32))
    assert flag == 0 and math.isclose(math.sqrt(s), 64 * float(c), rel_tol=1e-15)
    assert oracle.clip_coef(s) == oracle.lib().oracle_clip_coef(s, 1.0, 1e-6)
    assert oracle.clip_coef(0.25) == 1.0
    assert math.isclose(oracle.clip_coef(16.0), 1.0 / (4.0 + 1e-6))


def test_grad_check_sum_matches_fsum():
    rng = np.random.default_rng(9)
    g = (rng.standard_normal(200_000) * 1e-3).astype(np.float32)
    flag, s = oracle.grad_check(g)
    exact = math.fsum(float(x) * float(x) for x in g)
    assert flag == 0 and abs(s - exact) <= 1e-15 * exact


@pytest.mark.parametrize("pos", [0, 1, 7, 8, 1000, 4095])
@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
def test_grad_check_flags_non_finite(pos, bad):
    g = np.full(4096, 0.5, dtype=np.float32)
    g[pos] = bad
    assert oracle.grad_check(g)[0] == 1


# ---------------------------------------------------------------- Adam / AdamW
def _torch_traj(opt_cls, w0, grads, **kw):
    p = torch.nn.Parameter(torch.tensor(w0, dtype=torch.float64))
    opt = opt_cls([p], **kw)
    for g in grads:
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("adamw,wd", [(True, 3e-7), (True, 0.01), (False, 0.0), (False, 0.05)])
def test_adam_matches_torch_float64(adamw, wd):
    rng = np.random.default_rng(10)
    n, steps = 257, 6
    w0 = rng.standard_normal(n) * 0.02
    grads = [rng.standard_normal(n) * 1e-3 for _ in range(steps)]
    cls = torch.optim.AdamW if adamw else torch.optim.Adam
    tw, tm, tv = _torch_traj(cls, w0, grads, lr=1e-3, betas=(0.8, 0.999), eps=1e-8, weight_decay=wd)
    w, m, v = w0.copy(), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        oracle.adam_f64(g.copy(), w, m, v, oracle.hyper(lr=1e-3, beta1=0.8, beta2=0.999, eps=1e-8,
                                                        weight_decay=wd, adamw=adamw, step=t))
    np.testing.assert_allclose(w, tw, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(m, tm, rtol=1e-12, atol=1e-18)
    np.testing.assert_allclose(v, tv, rtol=1e-12, atol=1e-20)


def test_first_step_closed_form_any_betas():
    """At t=1 the bias-corrected moments are g and g^2: w1 = w0(1 - lr wd) - lr g/(|g| + eps)."""
    rng = np.random.default_rng(12)
    n = 1000
    g = rng.standard_normal(n) * 1e-3
    w0 = rng.standard_normal(n) * 0.02
    for b1, b2, lr, wd in [(0.8, 0.999, 1e-3, 3e-7), (0.9, 0.95, 2e-5, 0.01), (0.5, 0.5, 0.1, 0.0)]:
        w, m, v = w0.copy(), np.zeros(n), np.zeros(n)
        oracle.adam_f64(g.copy(), w, m, v, oracle.hyper(lr=lr, beta1=b1, beta2=b2, eps=1e-8,
                                                        weight_decay=wd, adamw=True, step=1))
        np.testing.assert_allclose(w, w0 * (1 - lr * wd) - lr * g / (np.abs(g) + 1e-8), rtol=1e-13)
        np.testing.assert_allclose(m, (1 - b1) * g, rtol=1e-15)
        np.testing.assert_allclose(v, (1 - b2) * g * g, rtol=1e-15)


def test_zero_betas_any_step_and_pure_decay():
    g = np.array([0.5, -2.0, 1e-3])
    w0 = np.array([1.0, -3.0, 0.25])
    for t in (1, 5, 1000):
        w, m, v = w0.copy(), np.full(3, 7.0), np.full(3, 9.0)
        oracle.adam_f64(g.copy(), w, m, v, oracle.hyper(lr=0.1, beta1=0.0, beta2=0.0, eps=1e-8,
                                                        weight_decay=0.0, adamw=True, step=t))
        np.testing.assert_allclose(w, w0 - 0.1 * g / (np.abs(g) + 1e-8), rtol=1e-15)
    # zero gradient and zero moments: only the decoupled decay acts
    w, m, v = w0.copy(), np.zeros(3), np.zeros(3)
    oracle.adam_f64(np.zeros(3), w, m, v, oracle.hyper(lr=1e-3, weight_decay=0.01, adamw=True, step=4))
    assert np.array_equal(w, w0 * (1 - 1e-3 * 0.01))


def test_clip_coefficient_scales_the_gradient():
    rng = np.random.default_rng(13)
    g = rng.standard_normal(100) * 1e-3
    base = dict(lr=1e-3, beta1=0.8, beta2=0.999, eps=1e-8, weight_decay=3e-7, adamw=True, step=3)
    m0 = rng.standard_normal(100) * 1e-4
    v0 = (rng.standard_normal(100) * 1e-4) ** 2
    w0 = rng.standard_normal(100) * 0.02
    a = [w0.copy(), m0.copy(), v0.copy()]
    oracle.adam_f64(g.copy(), *a, oracle.hyper(clip_coef=0.37, **base))
    b = [w0.copy(), m0.copy(), v0.copy()]
    oracle.adam_f64(g * 0.37, *b, oracle.hyper(clip_coef=1.0, **base))
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-15, atol=0)


def test_adam_f32_is_f64_rounded_once():
    rng = np.random.default_rng(14)
    n = 5000
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = ((rng.standard_normal(n) * 1e-4) ** 2).astype(np.float32)
    h = oracle.hyper(lr=1e-3, beta1=0.8, beta2=0.999, eps=1e-8, weight_decay=3e-7, step=11)
    w64, m64, v64 = w.astype(np.float64), m.astype(np.float64), v.astype(np.float64)
    oracle.adam_f64(g.astype(np.float64), w64, m64, v64, h)
    oracle.adam_f32(g, w, m, v, h)
    assert np.array_equal(w, w64.astype(np.float32))
    assert np.array_equal(m, m64.astype(np.float32))
    assert np.array_equal(v, v64.astype(np.float32))


# ---------------------------------------------------------------- composed step
def test_owner_step_is_reduce_then_adam_then_cast_over_real_elements():
    rng = np.random.default_rng(15)
    numels = [37, 5, 130, 64, 1]
    R, A = 3, 8
    offsets, total, owners = oracle.layout(numels, R, A)
    grads = [(rng.standard_normal(total) * 1e-3).astype(np.float16).view(np.uint16) for _ in range(R)]
    h = oracle.hyper(lr=1e-3, beta1=0.8, beta2=0.999, eps=1e-8, weight_decay=3e-7, step=2)
    for (b, e), pdtype in zip(owners, (BF16, F16, BF16)):
        lb = b & ~7
        size = e - lb
        w = (rng.standard_normal(size) * 0.02).astype(np.float32)
        m = np.zeros(size, dtype=np.float32)
        v = np.zeros(size, dtype=np.float32)
        p16 = np.full(total, 0xABCD, dtype=np.uint16)
        w1, m1, v1 = w.copy(), m.copy(), v.copy()
        ranges = oracle.real_ranges(numels, offsets, b, e)
        oracle.owner_step(ranges, h, w1, m1, v1, lb, grads=grads, gdtype=F16, divisor=float(R),
                          p16=p16, pdtype=pdtype)
        g = oracle.reduce(grads, F16, float(R))
        real = np.zeros(total, dtype=bool)
        for rb, re_ in ranges:
            real[rb:re_] = True
        w2, m2, v2 = w.copy(), m.copy(), v.copy()
        idx = np.nonzero(real)[0]
        loc = idx - lb
        ww, mm, vv = w2[loc].copy(), m2[loc].copy(), v2[loc].copy()
        oracle.adam_f32(g[idx].copy(), ww, mm, vv, h)
        w2[loc], m2[loc], v2[loc] = ww, mm, vv
        assert np.array_equal(w1, w2) and np.array_equal(m1, m2) and np.array_equal(v1, v2)
        want = np.full(total, 0xABCD, dtype=np.uint16)
        want[idx] = oracle.encode16(ww, pdtype)
        assert np.array_equal(p16, want)  # padding and other owners untouched


# ---------------------------------------------------------------- per-backward reduce + accumulate
def test_reduce_add_dyadic_microsteps_are_exact():
    rng = np.random.default_rng(16)
    R, K, n = 8, 6, 3000
    ks = rng.integers(-1024, 1025, size=(K, R, n))
    acc = np.zeros(n, dtype=np.float32)
    for k in range(K):
        grads = [(ks[k, r] * 2.0 ** -10).astype(np.float16).view(np.uint16) for r in range(R)]
        oracle.reduce_add(grads, F16, float(R), acc)
    for i in range(0, n, 29):
        exact = Fraction(int(ks[:, :, i].sum()), 1024 * R)
        assert acc[i] == _exact_round_f32(exact)


def test_reduce_add_rounds_the_mean_before_adding():
    # Closed forms: the reduced value is rounded to fp32 first, then added.
    big = np.float32(1e8)
    acc = np.array([big], dtype=np.float32)
    g = [np.array([4.0], dtype=np.float32), np.array([4.0], dtype=np.float32)]
    oracle.reduce_add(g, F32, 1.0, acc)
    assert acc[0] == big + np.float32(8.0)            # 1e8 + (4 + 4)
    acc2 = oracle.reduce(g, F32, 1.0, out=np.array([big], dtype=np.float32), accumulate=True)
    assert acc2[0] == big                               # (1e8 + 4) + 4, ties to even twice
    # division happens on the fresh sum only: acc + (3 + 5) / 4 = 10 + 2
    acc = np.array([10.0], dtype=np.float32)
    oracle.reduce_add([np.array([3.0], dtype=np.float32), np.array([5.0], dtype=np.float32)], F32, 4.0, acc)
    assert acc[0] == 12.0


def test_reduce_add_is_reduce_then_fp32_add():
    rng = np.random.default_rng(17)
    grads = [torch.from_numpy(rng.standard_normal(5000).astype(np.float32) * 1e-3).to(torch.bfloat16)
             .view(torch.int16).numpy().view(np.uint16).copy() for _ in range(5)]
    acc0 = (rng.standard_normal(5000) * 1e-2).astype(np.float32)
    got = oracle.reduce_add(grads, BF16, 5.0, acc0.copy())
    want = (acc0 + oracle.reduce(grads, BF16, 5.0)).astype(np.float32)
    assert np.array_equal(got, want)
