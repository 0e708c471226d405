"""Host logic of the full-size comparisons (tests/fullsize.py): slicing of the
owner's real ranges."""
import random

import fullsize as FS


def test_slices_cover_every_real_element_once_within_the_limit():
    rnd = random.Random(8)
    for _ in range(300):
        ranges, pos = [], rnd.randrange(0, 50)
        for _ in range(rnd.randrange(1, 30)):
            b = pos + rnd.choice([0, 0, rnd.randrange(1, 40)])
            e = b + rnd.randrange(1, 200)
            ranges.append((b, e))
            pos = e
        limit = rnd.choice([1, 7, 64, 500, 10_000])
        out = FS.slices(ranges, limit)
        covered = []
        last_hi = -1
        for lo, hi, parts in out:
            assert 0 < hi - lo <= limit and lo >= last_hi
            assert parts[0][0] == lo and parts[-1][1] == hi
            for b, e in parts:
                assert lo <= b < e <= hi
                covered.extend(range(b, e))
            last_hi = hi
        want = [i for b, e in ranges for i in range(b, e)]
        assert covered == want


def test_write_back_check_accepts_exact_roundings_and_rejects_others():
    """helpers.assert_write_back: the copy must be the exact rounding of the
    kernel's master, and within 1 ulp of the oracle's rounding where the master
    weights' tolerance is below half a 16-bit ulp."""
    import numpy as np
    import pytest

    import oracle
    from helpers import F16, BF16, assert_write_back

    for code in (F16, BF16):
        w_or = np.array([0.02, -0.013, 1e-9, 3e-3], dtype=np.float32)
        w_gpu = w_or.copy()
        w_gpu[2] = -4e-8  # near zero: far from the oracle in 16-bit ulps, inside the state tolerance
        bits = oracle.encode16(w_gpu, code)
        assert_write_back(bits, w_gpu, w_or, code, "exact")
        with pytest.raises(AssertionError):  # not the rounding of the kernel's master
            bad = bits.copy()
            bad[0] += 1
            assert_write_back(bad, w_gpu, w_or, code, "off by one")
        with pytest.raises(AssertionError):  # a master two ulps away at a normal magnitude
            w2 = w_gpu.copy()
            w2[1] = np.float32(w_or[1] * (1 + (2.5 * 2.0 ** -10 if code == F16 else 2.5 * 2.0 ** -7)))
            assert_write_back(oracle.encode16(w2, code), w2, w_or, code, "two ulps")
