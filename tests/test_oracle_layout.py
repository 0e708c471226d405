"""Oracle pins for contiguous ownership and the padded flat layout.

The floor formula is checked against an element-by-element characterisation
found by search (not the formula retyped), and the padded layout against a
slot-by-slot construction of the flat buffer.
"""
import random

import pytest

import oracle


def _owner_by_search(P, R, i):
    # The owner of element i is the first rank whose share of the first i+1
    # elements is reached: smallest r with P*(r+1) >= R*(i+1).
    for r in range(R):
        if P * (r + 1) >= R * (i + 1):
            return r
    raise AssertionError


def test_tiny_brute_force_all_P_R():
    for P in range(1, 65):
        for R in range(1, 65):
            owners = oracle.owner_ranges(P, R)
            assert len(owners) == R
            seen = []
            for r, own in enumerate(owners):
                assert own.step == 1 and own.start <= own.stop
                for i in own:
                    seen.append(i)
                    assert _owner_by_search(P, R, i) == r
            assert seen == list(range(P))  # ordered, disjoint, covering
            sizes = [len(o) for o in owners]
            assert max(sizes) - min(sizes) <= 1
            assert (min(sizes) == 0) == (R > P)  # empty owners exactly when ranks > params


def test_eleven_over_four():
    assert [(o.start, o.stop) for o in oracle.owner_ranges(11, 4)] == [(0, 2), (2, 5), (5, 8), (8, 11)]


def _slots(numels, align):
    """Build the flat buffer one slot at a time: ('real', k, j) or ('pad', k)."""
    slots = []
    for k, n in enumerate(numels):
        for j in range(n):
            slots.append(("real", k, j))
        while len(slots) % align:
            slots.append(("pad", k))
    return slots


def test_padded_layout_against_slots():
    rnd = random.Random(11)
    for _ in range(300):
        T = rnd.randrange(1, 7)
        numels = [rnd.randrange(1, 40) for _ in range(T)]
        align = rnd.choice([1, 2, 4, 8, 16, 64])
        R = rnd.randrange(1, 20)
        offsets, total, owners = oracle.layout(numels, R, align)
        slots = _slots(numels, align)
        assert total == len(slots) and total % align == 0
        for k, off in enumerate(offsets):
            assert slots[off] == ("real", k, 0)
            assert off % align == 0
        assert [(o.start, o.stop) for o in oracle.owner_ranges(total, R)] == owners
        for b, e in owners:
            real = oracle.real_ranges(numels, offsets, b, e)
            got = [f for rb, re_ in real for f in range(rb, re_)]
            want = [f for f in range(b, e) if slots[f][0] == "real"]
            assert got == want


def test_layout_with_one_tensor_and_align_one_is_the_page_formula():
    for P in range(1, 30):
        for R in range(1, 12):
            _, total, owners = oracle.layout([P], R, 1)
            assert total == P
            assert owners == [(o.start, o.stop) for o in oracle.owner_ranges(P, R)]


@pytest.mark.parametrize("args", [([], 4, 1), ([3, 0], 4, 1), ([3], 0, 1), ([3], 4, 0)])
def test_layout_rejects(args):
    with pytest.raises(ValueError):
        oracle.layout(*args)


def test_dense_offsets_against_a_labelled_concatenation():
    """The dense layout is the tensors laid end to end: build that buffer element by
    element with each element labelled (tensor, index) and find where every
    tensor's first element landed."""
    rnd = random.Random(17)
    for _ in range(300):
        numels = [rnd.randrange(1, 50) for _ in range(rnd.randrange(1, 9))]
        dense = [(k, j) for k, n in enumerate(numels) for j in range(n)]
        want = [dense.index((k, 0)) for k in range(len(numels))]
        assert oracle.dense_offsets(numels) == want
        # and every element sits at its tensor's start plus its index
        off = oracle.dense_offsets(numels)
        assert all(dense[off[k] + j] == (k, j) for k, n in enumerate(numels) for j in range(n))
