"""Host half of the seeded input generator: determinism, index addressing, value recipes."""
import math

import numpy as np

import synth


def test_index_addressable_and_deterministic():
    key = synth.stream_key(2, synth.STREAM_GRAD, rank=3, step=1)
    full = synth.values_f32(key, synth.arange(0, 10_000), synth.DIST_NORMAL, 1e-3)
    idx = np.array([0, 1, 17, 4095, 9999], dtype=np.uint64)
    assert np.array_equal(synth.values_f32(key, idx, synth.DIST_NORMAL, 1e-3), full[idx])
    assert np.array_equal(full, synth.values_f32(key, synth.arange(0, 10_000), synth.DIST_NORMAL, 1e-3))


def test_keys_differ_by_every_id():
    keys = {synth.stream_key(s, st, r, t) for s in range(3) for st in range(3) for r in range(3)
            for t in range(3)}
    assert len(keys) == 81


def test_normal_recipe_moments_and_bound():
    key = synth.stream_key(5, synth.STREAM_MASTER)
    x = synth.values_f32(key, synth.arange(0, 1_000_000), synth.DIST_NORMAL, 0.02).astype(np.float64)
    assert abs(x.mean()) < 3 * 0.02 / math.sqrt(1e6) * 1.5
    assert abs(x.std() / 0.02 - 1) < 0.005
    assert np.abs(x).max() <= 2 * math.sqrt(3) * 0.02 * (1 + 1e-6)


def test_uniform_and_square_recipes():
    key = synth.stream_key(1, synth.STREAM_GRAD)
    u = synth.values_f32(key, synth.arange(0, 200_000), synth.DIST_UNIFORM, 0.3)
    assert u.min() >= -0.3 and u.max() < 0.3
    assert abs(u.astype(np.float64).std() - 0.3 / math.sqrt(3)) < 0.003
    s = synth.values_f32(key, synth.arange(0, 1000), synth.DIST_SQUARE, 1e-2)
    n = synth.values_f32(key, synth.arange(0, 1000), synth.DIST_NORMAL, 1e-2)
    assert np.array_equal(s, n * n) and (s >= 0).all()


def test_sixteen_bit_storage():
    key = synth.stream_key(3, synth.STREAM_GRAD)
    x = synth.values_f32(key, synth.arange(0, 1000), synth.DIST_NORMAL, 65.536)
    h = synth.values(key, synth.arange(0, 1000), synth.DIST_NORMAL, 65.536, synth.F16)
    assert h.dtype == np.uint16 and np.array_equal(h.view(np.float16), x.astype(np.float16))
    b = synth.values(key, synth.arange(0, 1000), synth.DIST_NORMAL, 65.536, synth.BF16)
    assert b.dtype == np.uint16
    assert np.allclose((b.astype(np.uint32) << 16).view(np.float32), x, rtol=2 ** -8)


def test_log_uniform_sizes():
    s = synth.log_uniform_sizes(5, 10_000, 64, 1 << 24)
    assert s.min() >= 64 and s.max() <= 1 << 24
    logs = np.log(s.astype(np.float64))
    assert abs(logs.mean() - (math.log(64) + math.log(1 << 24)) / 2) < 0.1


def test_threaded_host_generator_matches_numpy():
    """The C host generator (all host cores) gives the numpy generator's bits for
    every dtype and recipe, including fp16 overflow to infinity (scale 3e4) and
    fp16 / bf16 subnormals (scale 1e-6, 1e-40)."""
    cases = [(synth.DIST_NORMAL, 1e-3), (synth.DIST_NORMAL, 65.536), (synth.DIST_UNIFORM, 0.3),
             (synth.DIST_SQUARE, 1e-4), (synth.DIST_NORMAL, 3e4), (synth.DIST_UNIFORM, 7e4),
             (synth.DIST_NORMAL, 1e-6), (synth.DIST_NORMAL, 1e-40)]
    with np.errstate(over="ignore"):
        for dist, scale in cases:
            for dt in (synth.F16, synth.BF16, synth.F32):
                key = synth.stream_key(3, synth.STREAM_GRAD, 5, 2)
                want = synth.values(key, synth.arange(1000, 101_000), dist, scale, dt)
                got = synth.host_values(key, 1000, 100_000, dist, scale, dt)
                if dt == synth.F32:
                    want, got = want.view(np.uint32), got.view(np.uint32)
                assert np.array_equal(got, want), (dist, scale, dt)
