"""Oracle pins: values and statements the pages fix for the owner update.

Every expected value comes from tests/golden/ (printed by the pages) or from a
closed form; nothing comes from the HIP path.
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def _lab_hyper(step, **kw):
    return oracle.hyper(lr=0.01, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, adamw=False,
                        step=step, **kw)


def test_first_step_python_and_c():
    row = _rows("first_adam_step.txt")[0]
    w0, m0, v0, g, t = map(float, row[:5])
    ew, em, ev = map(float, row[6:9])
    w, m, v = oracle.adam_step(w0, m0, v0, g, int(t))
    assert math.isclose(w, ew, rel_tol=1e-15) and math.isclose(w, 1.0 - 0.01 * 2.0 / (2.0 + 1e-8))
    assert math.isclose(m, em, rel_tol=1e-15) and math.isclose(v, ev, rel_tol=1e-15)
    # the C core gives the same numbers
    a = [np.array([x], dtype=np.float64) for x in (g, w0, m0, v0)]
    oracle.adam_f64(*a, _lab_hyper(int(t)))
    assert math.isclose(a[1][0], ew, rel_tol=1e-15)
    assert math.isclose(a[2][0], em, rel_tol=1e-15)
    assert math.isclose(a[3][0], ev, rel_tol=1e-15)


def test_sharded_equals_unsharded_lab():
    reference, reconstructed = oracle.compare_owned_updates(11, 4, 5)
    assert len(reference) == 11
    for exp, act in zip(reference, reconstructed):
        for a, b in zip(exp, act):
            assert math.isclose(a, b, rel_tol=1e-12, abs_tol=1e-12)


@pytest.mark.parametrize("bad", [(0, 4, 5), (11, 0, 5), (11, 4, 0), (11.0, 4, 5), (-1, 4, 5)])
def test_compare_rejects_non_positive(bad):
    with pytest.raises(ValueError):
        oracle.compare_owned_updates(*bad)


def _c_lab_trajectory(parameters, ranks, steps, owners):
    """The lab run through the C core, owner by owner (fp64 state)."""
    w = np.array([0.1 * i for i in range(parameters)])
    m = np.zeros(parameters)
    v = np.zeros(parameters)
    for t in range(1, steps + 1):
        for own in owners:
            idx = list(own)
            if not idx:
                continue
            g = np.array([sum(oracle.pages_gradient(i, r, t) for r in range(ranks)) / ranks
                          for i in idx])
            ws, ms, vs = w[idx].copy(), m[idx].copy(), v[idx].copy()
            oracle.adam_f64(g, ws, ms, vs, _lab_hyper(t))
            w[idx], m[idx], v[idx] = ws, ms, vs
    return w, m, v


def test_c_core_matches_lab_sharded_and_unsharded():
    reference, _ = oracle.compare_owned_updates(11, 4, 5)
    for owners in (oracle.owner_ranges(11, 4), [range(0, 11)]):
        w, m, v = _c_lab_trajectory(11, 4, 5, owners)
        for i, (ew, em, ev) in enumerate(reference):
            assert math.isclose(w[i], ew, rel_tol=1e-12, abs_tol=1e-12)
            assert math.isclose(m[i], em, rel_tol=1e-12, abs_tol=1e-12)
            assert math.isclose(v[i], ev, rel_tol=1e-12, abs_tol=1e-12)


def test_resume_lab_printed_values():
    gold = {k: float(v) for k, v in _rows("resume_lab.txt")}
    reference, _ = oracle.compare_owned_updates(11, 4, 5)
    w, m, v = reference[0]
    full = oracle.adam_step(w, m, v, 0.4, 6)
    weights_only = oracle.adam_step(w, 0.0, 0.0, 0.4, 6)
    assert f"{full[0]:.8f}" == f"{gold['full_state_next_weight']:.8f}"
    assert f"{weights_only[0]:.8f}" == f"{gold['weights_only_next_weight']:.8f}"
    assert f"{abs(weights_only[0] - full[0]):.8f}" == f"{gold['next_update_gap']:.8f}"
    # the C core reaches the same printed values
    a = [np.array([x]) for x in (0.4, w, m, v)]
    oracle.adam_f64(*a, _lab_hyper(6))
    assert f"{a[1][0]:.8f}" == f"{gold['full_state_next_weight']:.8f}"
    b = [np.array([x]) for x in (0.4, w, 0.0, 0.0)]
    oracle.adam_f64(*b, _lab_hyper(6))
    assert f"{b[1][0]:.8f}" == f"{gold['weights_only_next_weight']:.8f}"


def test_mean_of_squares_is_not_square_of_mean():
    # Two ranks with gradients 1 and 3 for one parameter: mean of squares 5, square of mean 4.
    assert (1 ** 2 + 3 ** 2) / 2 == 5 and ((1 + 3) / 2) ** 2 == 4
    # Reduce-then-update (what the owner does) vs update-per-rank-then-average.
    _, _, v_reduce_first = oracle.adam_step(0.0, 0.0, 0.0, (1.0 + 3.0) / 2, 1)
    per_rank = [oracle.adam_step(0.0, 0.0, 0.0, g, 1) for g in (1.0, 3.0)]
    v_avg = sum(s[2] for s in per_rank) / 2
    assert math.isclose(v_reduce_first, 0.001 * 4)
    assert math.isclose(v_avg, 0.001 * 5)
    assert not math.isclose(v_reduce_first, v_avg, rel_tol=1e-12, abs_tol=1e-12)


def test_uniform_seeded_lab_sharded_equals_unsharded():
    """The tiny case with per-rank grads seeded uniform in [-0.3, 0.3]."""
    import synth

    def grad(i, r, t):
        key = synth.stream_key(1, synth.STREAM_GRAD, r, t)
        return float(synth.values_f32(key, [i], synth.DIST_UNIFORM, 0.3)[0])

    reference, reconstructed = oracle.compare_owned_updates(11, 4, 5, grad=grad)
    for exp, act in zip(reference, reconstructed):
        for a, b in zip(exp, act):
            assert math.isclose(a, b, rel_tol=1e-12, abs_tol=1e-12)
    assert any(abs(a[0] - 0.1 * i) > 1e-3 for i, a in enumerate(reference))
