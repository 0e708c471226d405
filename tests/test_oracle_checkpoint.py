"""Oracle pins for consolidation (export) and the resume lab of the pages."""
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_consolidate_round_trip_and_drops_padding():
    rng = np.random.default_rng(3)
    numels, R, A = [5, 17, 1, 64, 9], 3, 8
    offsets, total, owners = oracle.layout(numels, R, A)
    flat = np.full(total, np.nan, dtype=np.float32)  # padding slots hold NaN
    for n, off in zip(numels, offsets):
        flat[off:off + n] = rng.standard_normal(n).astype(np.float32)
    bases = [b & ~7 for b, _ in owners]
    arrays = [flat[lb:e].copy() for lb, (_, e) in zip(bases, owners)]
    dense = oracle.consolidate(numels, offsets, owners, arrays, bases)
    assert dense.size == sum(numels) and not np.isnan(dense).any()
    want = np.concatenate([flat[off:off + n] for n, off in zip(numels, offsets)])
    assert np.array_equal(dense, want)
    for r, (b, e) in enumerate(owners):
        back = np.full(e - bases[r], -1.0, dtype=np.float32)
        oracle.distribute(numels, offsets, b, e, dense, back, bases[r])
        real = ~np.isnan(flat[bases[r]:e])
        inside = np.zeros(e - bases[r], dtype=bool)
        inside[b - bases[r]:] = True
        assert np.array_equal(back[real & inside], flat[bases[r]:e][real & inside])
        assert np.all(back[~(real & inside)] == -1.0)


def test_resume_lab_through_consolidation():
    """Full-state resume reproduces the uninterrupted next update; a weights-only
    restore (consolidated weights, zero moments) does not: the pages' printed numbers."""
    gold = {}
    for ln in open(os.path.join(GOLDEN, "resume_lab.txt")):
        if ln.strip() and not ln.startswith("#"):
            k, v = ln.split()
            gold[k] = float(v)
    P, R = 11, 4
    owners = [(o.start, o.stop) for o in oracle.owner_ranges(P, R)]
    w, m, v = np.array([0.1 * i for i in range(P)]), np.zeros(P), np.zeros(P)
    for t in range(1, 6):
        g = np.array([sum(oracle.pages_gradient(i, r, t) for r in range(R)) / R for i in range(P)])
        oracle.adam_f64(g, w, m, v, oracle.hyper(lr=0.01, beta1=0.9, beta2=0.999, eps=1e-8,
                                                  weight_decay=0.0, adamw=False, step=t))
    arrays = [w[b:e].astype(np.float32) for b, e in owners]
    dense = oracle.consolidate([P], [0], owners, arrays, [b for b, _ in owners])
    assert np.array_equal(dense, w.astype(np.float32))
    h6 = oracle.hyper(lr=0.01, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, adamw=False, step=6)
    full = [np.array([x]) for x in (0.4, w[0], m[0], v[0])]
    oracle.adam_f64(*full, h6)
    weights_only = [np.array([x]) for x in (0.4, float(dense[0]), 0.0, 0.0)]
    oracle.adam_f64(*weights_only, h6)
    assert f"{full[1][0]:.8f}" == f"{gold['full_state_next_weight']:.8f}"
    assert f"{weights_only[1][0]:.8f}" == f"{gold['weights_only_next_weight']:.8f}"
    assert not math.isclose(full[1][0], weights_only[1][0], rel_tol=1e-12, abs_tol=1e-12)
