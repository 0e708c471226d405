"""Oracle pins for the per-rank state accounting (printed tables and the memory matrix)."""
import os
import random
from fractions import Fraction

import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_printed_table_1p5e9_4_ranks():
    sb = oracle.state_bytes(1_500_000_000, 4)
    for stage, gb, gib in _rows("state_bytes_1p5e9_4ranks.txt"):
        assert f"{float(sb[stage] / 10 ** 9):.2f}" == gb
        assert f"{float(sb[stage] / 2 ** 30):.2f}" == gib


def test_printed_intro_and_seventy_b_totals():
    """M1: 3 GB of two-byte weights inside 24 GB of state (21 GB more); M5: 1.12 TB for 70e9 in DP."""
    for params, ranks, what, want in _rows("state_bytes_intro.txt"):
        sb = oracle.state_bytes(int(params), int(ranks))
        weights = int(params) * 2  # the estimator's two-byte compute weights
        got = {"weights_2byte": weights, "DP": sb["DP"], "DP_minus_weights": sb["DP"] - weights}[what]
        assert got == int(want)


def test_printed_asserts():
    for p, r, pa, gr, op, stage, expected in _rows("state_bytes_asserts.txt"):
        sb = oracle.state_bytes(int(p), int(r), int(pa), int(gr), int(op))
        assert sb[stage] == int(expected)


def test_memory_matrix_identity():
    """ZeRO Q&A matrix: 16P, 4P + 12P/N, 2P + 14P/N, 16P/N for 2/2/12-byte widths."""
    rnd = random.Random(7)
    for _ in range(200):
        P, N = rnd.randrange(1, 10 ** 12), rnd.randrange(1, 1025)
        sb = oracle.state_bytes(P, N)
        assert sb["DP"] == 16 * P
        assert sb["ZeRO-1"] == 4 * P + Fraction(12 * P, N)
        assert sb["ZeRO-2"] == 2 * P + Fraction(14 * P, N)
        assert sb["ZeRO-3"] == Fraction(16 * P, N)


def test_seventy_b_at_64_way_is_17p5_gb_not_14():
    # The Q&A's "~14 GB per GPU" contradicts its own matrix: 16 * 70e9 / 64 = 17.5e9.
    assert oracle.state_bytes(70_000_000_000, 64)["ZeRO-3"] == 17_500_000_000


def test_one_rank_all_stages_equal():
    rnd = random.Random(3)
    for _ in range(50):
        P = rnd.randrange(1, 10 ** 9)
        widths = [rnd.randrange(1, 17) for _ in range(3)]
        assert len(set(oracle.state_bytes(P, 1, *widths).values())) == 1


@pytest.mark.parametrize("args", [(0, 4), (10, 0), (10, 4, 0), (10, 4, 2, -2), (10.0, 4), (10, 4, 2, 2, 1.5)])
def test_rejects_non_positive_or_non_int(args):
    with pytest.raises(ValueError):
        oracle.state_bytes(*args)


def test_parameter_storage_printed():
    for row in _rows("parameter_storage.txt"):
        sizes = [int(x) for x in row[0].split(",")]
        live = [] if row[2] == "-" else [int(x) for x in row[2].split(",")]
        assert oracle.parameter_storage(sizes, 4, live) == tuple(int(x) for x in row[4:7])


@pytest.mark.parametrize("args", [([], 4, []), ([8], 0, []), ([8, 0], 4, []), ([8], 4, [1]),
                                  ([8, 8], 4, [0, 0])])
def test_parameter_storage_rejects(args):
    with pytest.raises(ValueError):
        oracle.parameter_storage(*args)


def test_stage3_gather_sizes_match_parameter_storage_and_rebuild_tensors():
    """The gathered buffers of the live tensors have the storage counts of the
    pages' example, and their first n elements are the tensors themselves."""
    import numpy as np

    rng = np.random.default_rng(4)
    for sizes, R, live in ([[8, 8, 8, 8], 4, [0]], [[8, 8, 8, 8], 4, [0, 1]], [[5, 9, 2], 4, [1]],
                           [[13, 1, 64, 7], 3, [3, 0, 2]]):
        dense = rng.standard_normal(sum(sizes)).astype(np.float32)
        bufs = oracle.stage3_shards(sizes, R, dense)
        resident, gathered, total = oracle.parameter_storage(sizes, R, live)
        assert all(b.size == resident for b in bufs)
        g = oracle.stage3_gather(sizes, R, bufs, live)
        assert g.size == gathered
        dstart = [sum(sizes[:k]) for k in range(len(sizes))]
        pos = 0
        for k in live:
            s = -(-sizes[k] // R)
            assert np.array_equal(g[pos:pos + sizes[k]], dense[dstart[k]:dstart[k] + sizes[k]])
            assert np.all(g[pos + sizes[k]:pos + R * s] == 0)  # padding of the last shards
            pos += R * s
