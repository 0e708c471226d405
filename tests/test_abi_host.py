"""The C ABI on the CPU: the library loads, exports every declared symbol, and its
host calls (layout, chunk table, state accounting, clip scalar, argument
validation) agree with the oracle.  No device compute runs here.
"""
import ctypes as ct
import functools
import os
import random
import re
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import zero_sharded_optimizer_owned_amd as zs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "zero_shard.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(zero\d*_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert "zero_adam_step" in names and "zero_shard_layout" in names and len(names) >= 8
    L = ct.CDLL(zs.LIB_PATH)
    for name in names:
        assert hasattr(L, name), f"{name} is declared in zero_shard.h but not exported"
    assert set(names) == set(zs.EXPORTED)


def test_layout_matches_oracle():
    rnd = random.Random(1)
    for _ in range(400):
        numels = [rnd.randrange(1, 5000) for _ in range(rnd.randrange(1, 12))]
        R = rnd.randrange(1, 70)
        A = rnd.choice([1, 2, 8, 64, 128])
        off, total, b, e = zs.zero_shard_layout(numels, R, A)
        ooff, ototal, owners = oracle.layout(numels, R, A)
        assert list(off) == ooff and total == ototal
        assert list(zip(b.tolist(), e.tolist())) == owners


def test_dense_offsets_match_oracle():
    rnd = random.Random(5)
    for _ in range(300):
        numels = [rnd.randrange(1, 1 << 40) for _ in range(rnd.randrange(1, 40))]
        off, total = zs.zero_dense_offsets(numels)
        assert [int(x) for x in off] == oracle.dense_offsets(numels)
        assert total == sum(numels)
    with pytest.raises(zs.ZeroShardError):
        zs.zero_dense_offsets([4, 0, 3])
    with pytest.raises(zs.ZeroShardError):
        zs.zero_dense_offsets([2 ** 63, 2 ** 63])


def test_layout_large_counts_use_wide_products():
    # 7e10 elements over 64 owners: P * r exceeds 2^64 only for huge P; check the
    # formula against Python integers near the top of the range too.
    for P in (70_000_000_000, 2 ** 63 + 12345):
        off, total, b, e = zs.zero_shard_layout([P], 64, 1)
        assert total == P
        assert [int(x) for x in b] == [P * r // 64 for r in range(64)]
        assert [int(x) for x in e] == [P * (r + 1) // 64 for r in range(64)]


def test_layout_errors():
    with pytest.raises(zs.ZeroShardError) as ei:
        zs.zero_shard_layout([3, 0], 4, 1)
    assert ei.value.code == zs.ZERO_EINVAL
    with pytest.raises(zs.ZeroShardError):
        zs.zero_shard_layout([3], 0, 1)
    with pytest.raises(zs.ZeroShardError):
        zs.zero_shard_layout([3], 4, 0)
    with pytest.raises(zs.ZeroShardError) as ei:
        zs.zero_shard_layout([2 ** 63, 2 ** 63], 4, 1)
    assert ei.value.code == zs.ZERO_ERANGE


def test_chunk_table_covers_real_elements_exactly_once():
    rnd = random.Random(2)
    for _ in range(300):
        numels = [rnd.randrange(1, 3000) for _ in range(rnd.randrange(1, 9))]
        R = rnd.randrange(1, 40)
        A = rnd.choice([1, 8, 64])
        C = rnd.choice([8, 64, 512, 4096])
        off, total, b, e = zs.zero_shard_layout(numels, R, A)
        for r in range(R):
            ch = zs.zero_chunk_table(numels, off, int(b[r]), int(e[r]), C)
            got = [(int(c["flat"]), int(c["flat"]) + int(c["len"])) for c in ch]
            want = oracle.real_ranges(numels, list(off), int(b[r]), int(e[r]))
            elems = [f for s, t in got for f in range(s, t)]
            assert elems == [f for s, t in want for f in range(s, t)]
            for i, c in enumerate(ch):
                k = int(c["tensor"])
                assert off[k] <= c["flat"] < off[k] + numels[k]  # the tensor of its first element
                assert 1 <= c["len"] <= C
                # a chunk never crosses a multiple of C ...
                assert int(c["flat"]) // C == (int(c["flat"]) + int(c["len"]) - 1) // C
                # ... and is cut nowhere else: flat-contiguous neighbours meet at a multiple of C
                if i > 0 and int(ch[i - 1]["flat"]) + int(ch[i - 1]["len"]) == int(c["flat"]):
                    assert int(c["flat"]) % C == 0


def test_chunk_table_merges_tensors_without_padding():
    """Many small tensors whose sizes are multiples of the alignment have no
    padding between them, so they share full-size chunks."""
    numels = [64] * 1000 + [100] + [64] * 10
    off, total, b, e = zs.zero_shard_layout(numels, 1, 64)
    ch = zs.zero_chunk_table(numels, off, int(b[0]), int(e[0]), 2048)
    lens = [int(x) for x in ch["len"]]
    # 64,000 contiguous elements = 31 full chunks + 512, then 100 + 28 padding, then 640 more
    assert lens[:31] == [2048] * 31 and lens[31] == 512 + 100
    assert lens[32:] == [640]
    assert [int(x) for x in ch["tensor"][:3]] == [0, 32, 64]


def test_chunk_table_capacity_and_errors():
    numels = [100, 50]
    off, total, b, e = zs.zero_shard_layout(numels, 1, 8)
    L = zs.lib()
    n = np.array(numels, dtype=np.uint64)
    count = np.zeros(1, dtype=np.uint64)
    out = np.zeros(2, dtype=zs.CHUNK_DTYPE)
    rc = L.zero_chunk_table(n.ctypes.data, off.ctypes.data, 2, 0, total, 16, out.ctypes.data, 2,
                            count.ctypes.data)
    assert rc == zs.ZERO_ERANGE and int(count[0]) == 7 + 4
    assert int(out[0]["flat"]) == 0 and int(out[0]["len"]) == 16
    for C in (0, 7, 12):
        rc = L.zero_chunk_table(n.ctypes.data, off.ctypes.data, 2, 0, total, C, None, 0,
                                count.ctypes.data)
        assert rc == zs.ZERO_EINVAL
    bad = np.array([0, 90], dtype=np.uint64)  # second tensor overlaps the first
    assert L.zero_chunk_table(n.ctypes.data, bad.ctypes.data, 2, 0, total, 16, None, 0,
                              count.ctypes.data) == zs.ZERO_EINVAL
    assert L.zero_chunk_table(n.ctypes.data, off.ctypes.data, 2, 10, 5, 16, None, 0,
                              count.ctypes.data) == zs.ZERO_EINVAL
    assert zs.zero_chunk_table(numels, off, 50, 50, 16).size == 0  # empty owner


def test_state_bytes_matches_oracle():
    rnd = random.Random(3)
    for _ in range(300):
        P, R = rnd.randrange(1, 10 ** 13), rnd.randrange(1, 5000)
        w = [rnd.randrange(1, 20) for _ in range(3)]
        assert zs.zero_state_bytes(P, R, *w) == oracle.state_bytes(P, R, *w)
    assert zs.zero_state_bytes(1_500_000_000, 4) == oracle.state_bytes(1_500_000_000, 4)


def test_state_bytes_errors():
    for args in [(0, 4), (5, 0), (5, 4, 0), (5, 4, 2, 0), (5, 4, 2, 2, 0)]:
        with pytest.raises(zs.ZeroShardError) as ei:
            zs.zero_state_bytes(*args)
        assert ei.value.code == zs.ZERO_EINVAL
    with pytest.raises(zs.ZeroShardError) as ei:
        zs.zero_state_bytes(2 ** 62, 1, 16, 16, 16)
    assert ei.value.code == zs.ZERO_ERANGE


def test_clip_coef_matches_oracle():
    for s in (0.0, 0.25, 0.999998, 1.0, 2.0, 1e6, 123.456):
        assert zs.zero_clip_coef(s) == np.float32(oracle.clip_coef(s))
    for bad in (-1.0, float("nan"), float("inf")):
        with pytest.raises(zs.ZeroShardError):
            zs.zero_clip_coef(bad)


def test_device_calls_reject_bad_arguments_before_any_launch():
    """Validation happens on the host first; these never reach the HIP runtime."""
    L = zs.lib()
    a = zs.AdamArgs()
    a.step = 0
    assert L.zero_adam_step(ct.byref(a), None) == zs.ZERO_EINVAL
    assert b"step" in L.zero_last_error()
    assert L.zero_adam_step(None, None) == zs.ZERO_EINVAL
    g = zs.AdamArgs()
    g.step, g.n_groups = 1, 3  # a group count without a group table
    assert L.zero_adam_step(ct.byref(g), None) == zs.ZERO_EINVAL
    assert b"group" in L.zero_last_error()
    a.step, a.begin, a.end = 1, 10, 5
    assert L.zero_adam_step(ct.byref(a), None) == zs.ZERO_EINVAL
    a.begin, a.end = 0, 8
    a.R = 0
    assert L.zero_adam_step(ct.byref(a), None) == zs.ZERO_EINVAL
    ptrs = (ct.c_void_p * 1)(0x1000)
    out = ct.c_void_p(0x2000)
    # R out of range, unknown dtype, unaligned pointer, bad divisor, half-given check outputs
    assert L.zero_reduce_owned(ptrs, 0, zs.ZERO_F16, 0, 0, 8, 1.0, 0, out, 0, None, None, None, 0,
                               None) == zs.ZERO_EINVAL
    assert L.zero_reduce_owned(ptrs, 1, 9, 0, 0, 8, 1.0, 0, out, 0, None, None, None, 0,
                               None) == zs.ZERO_EINVAL
    bad = (ct.c_void_p * 1)(0x1002)
    assert L.zero_reduce_owned(bad, 1, zs.ZERO_F16, 0, 0, 8, 1.0, 0, out, 0, None, None, None, 0,
                               None) == zs.ZERO_EINVAL
    assert L.zero_reduce_owned(ptrs, 1, zs.ZERO_F16, 0, 0, 8, 0.0, 0, out, 0, None, None, None, 0,
                               None) == zs.ZERO_EINVAL
    assert L.zero_reduce_owned(ptrs, 1, zs.ZERO_F16, 4, 4, 8, 1.0, 0, out, 0, None, None, None, 0,
                               None) == zs.ZERO_EINVAL  # base not a multiple of 8
    assert L.zero_reduce_owned(ptrs, 1, zs.ZERO_F16, 0, 0, 8, 1.0, 0, out, 0, ct.c_void_p(0x3000),
                               None, None, 0, None) == zs.ZERO_EINVAL
    assert L.zero_reduce_owned(ptrs, 1, zs.ZERO_F16, 0, 0, 8, 1.0, 0, out, 0, ct.c_void_p(0x3000),
                               ct.c_void_p(0x4000), ct.c_void_p(0x10000), 100,
                               None) == zs.ZERO_EINVAL  # workspace too small
    assert L.zero_grad_check(None, 0, None, None, None, 0, None) == zs.ZERO_EINVAL
    # a workspace one byte short of what the query reports is rejected
    ov, ss, ws = ct.c_void_p(0x3000), ct.c_void_p(0x4000), ct.c_void_p(0x10000)
    for n in (1, 5000, 9_000_003):
        need = zs.check_workspace_bytes(n)
        assert L.zero_grad_check(ct.c_void_p(0x20000), n, ov, ss, ws, need - 1, None) == zs.ZERO_EINVAL
        assert b"workspace" in L.zero_last_error()
    # bandwidth probe: stream counts, byte size, widths, NULL and misaligned pointers
    two = (ct.c_void_p * 2)(0x1000, 0x2000)
    P = L.zero_stream_probe
    assert P(two, None, 0, two, None, 0, 64, 0, None) == zs.ZERO_EINVAL
    assert P(two, None, 65, two, None, 1, 64, 0, None) == zs.ZERO_EINVAL
    assert P(two, None, 1, two, None, 65, 64, 0, None) == zs.ZERO_EINVAL
    assert P(two, None, 1, two, None, 1, 24, 0, None) == zs.ZERO_EINVAL
    assert P(None, None, 1, two, None, 1, 64, 0, None) == zs.ZERO_EINVAL
    assert P(two, None, 1, None, None, 1, 64, 0, None) == zs.ZERO_EINVAL
    assert P(bad, None, 1, two, None, 1, 64, 0, None) == zs.ZERO_EINVAL
    assert P((ct.c_void_p * 1)(0), None, 1, two, None, 1, 64, 0, None) == zs.ZERO_EINVAL
    assert P(two, None, 1, two, None, 1, 0, 0, None) == zs.ZERO_OK  # nothing to move
    assert P(two, None, 1, two, None, 1, 64, 2, None) == zs.ZERO_EINVAL  # order 0 or 1
    w3, w0 = (ct.c_uint8 * 2)(3, 1), (ct.c_uint8 * 2)(1, 0)
    assert P(two, w3, 1, two, None, 1, 64, 0, None) == zs.ZERO_EINVAL  # widths 1 or 2
    assert P(two, None, 1, two, w0, 2, 64, 0, None) == zs.ZERO_EINVAL
    assert b"width" in L.zero_last_error()


def test_check_workspace_grows_with_the_block_count():
    """One first-stage (sum, flag) pair per 2048 elements plus the fold's pairs,
    rounded to 256 bytes; monotone in n."""
    prev = 0
    for n in (0, 1, 2047, 2048, 2049, 16_383, 16_384, 8_388_608, 8_390_660, 1_093_750_000):
        b = zs.check_workspace_bytes(n)
        parts = n // 8 // 256 + 1
        assert b == -(-parts * 12 // 256) * 256 + 256 * 12
        assert b >= prev
        prev = b
    assert zs.lib().zero_check_workspace_bytes(5, None) == zs.ZERO_EINVAL


def test_stage3_storage_matches_oracle_and_printed_example():
    import os

    gold = os.path.join(os.path.dirname(__file__), "golden", "parameter_storage.txt")
    for ln in open(gold):
        if not ln.strip() or ln.startswith("#"):
            continue
        sizes_s, live_s, counts = [x.strip() for x in ln.split("|")]
        sizes = [int(x) for x in sizes_s.split(",")]
        live = [] if live_s == "-" else [int(x) for x in live_s.split(",")]
        _, res, gat = zs.zero3_storage(sizes, 4, live)
        assert (res, gat, res + gat) == tuple(int(x) for x in counts.split())
    rnd = random.Random(5)
    for _ in range(200):
        sizes = [rnd.randrange(1, 10_000) for _ in range(rnd.randrange(1, 9))]
        R = rnd.randrange(1, 70)
        live = rnd.sample(range(len(sizes)), rnd.randrange(0, len(sizes) + 1))
        shard, res, gat = zs.zero3_storage(sizes, R, live)
        assert (res, gat, res + gat) == oracle.parameter_storage(sizes, R, live)
        assert list(shard) == [-(-n // R) for n in sizes]
    for bad in (([8, 8], 0, []), ([8, 0], 4, []), ([8], 4, [1]), ([8, 8], 4, [0, 0])):
        with pytest.raises(zs.ZeroShardError):
            zs.zero3_storage(*bad)


def test_stage3_counts_beyond_64_bits_are_erange():
    """Two tensors of 2^63 elements: every stage-3 total (dense, shard buffer,
    gathered buffer) is 2^64 at R = 1, one past the largest offset."""
    big = [1 << 63, 1 << 63]
    calls = (lambda: zs.zero3_storage(big, 1, [0, 1]),
             lambda: zs.zero3_gather_spans(big, 1, [1]),
             lambda: zs.zero3_partition_spans(big, 1, 0))
    for call in calls:
        with pytest.raises(zs.ZeroShardError) as ei:
            call()
        assert ei.value.code == zs.ZERO_ERANGE
    # totals just below 2^64 fit, with offsets beyond 2^63
    fit = [(1 << 63) - 1, 8]
    spans = zs.zero3_gather_spans(fit, 1, [1])
    assert [(int(sp["src"]), int(sp["dst"]), int(sp["len"])) for sp in spans] == [((1 << 63) - 1, 0, 8)]


def _apply_spans(spans, srcs, dst):
    for sp in spans:
        s, d, n, b = int(sp["src"]), int(sp["dst"]), int(sp["len"]), int(sp["buf"])
        dst[d:d + n] = srcs[b][s:s + n]


def test_stage3_span_tables_reproduce_the_oracle():
    rnd = random.Random(6)
    rng = np.random.default_rng(6)
    for _ in range(60):
        sizes = [rnd.randrange(1, 300) for _ in range(rnd.randrange(1, 7))]
        R = rnd.randrange(1, 9)
        dense = rng.standard_normal(sum(sizes)).astype(np.float32)
        shards = oracle.stage3_shards(sizes, R, dense)
        for r in range(R):
            out = np.zeros_like(shards[r])
            _apply_spans(zs.zero3_partition_spans(sizes, R, r, max_span=rnd.choice([1, 7, 64, 1 << 16])),
                         [dense], out)
            assert np.array_equal(out, shards[r])
        live = rnd.sample(range(len(sizes)), rnd.randrange(0, len(sizes) + 1))
        want = oracle.stage3_gather(sizes, R, shards, live)
        got = np.full(want.size, np.nan, dtype=np.float32)
        spans = zs.zero3_gather_spans(sizes, R, live, max_span=rnd.choice([3, 64, 1 << 16]))
        assert all(int(s["len"]) >= 1 for s in spans)
        _apply_spans(spans, shards, got)
        assert np.array_equal(got, want)


def _units(flat, ln):
    a0 = min(flat + ln, (flat + 7) // 8 * 8)
    a1 = max(a0, (flat + ln) // 8 * 8)
    return (a0 - flat) + (a1 - a0) // 8 + (flat + ln - a1)


def test_chunk_groups_partition_the_table():
    """Groups cover the chunks in order; a group of several chunks holds at most
    256 work units and at most max_group elements; greedy, so no group could
    have taken its successor's first chunk."""
    rnd = random.Random(11)
    for _ in range(200):
        numels = [rnd.randrange(1, rnd.choice([20, 200, 5000])) for _ in range(rnd.randrange(1, 60))]
        A = rnd.choice([1, 8, 64])
        off, total, b, e = zs.zero_shard_layout(numels, 1, A)
        C = rnd.choice([64, 512, 2048])
        ch = zs.zero_chunk_table(numels, off, int(b[0]), int(e[0]), C)
        g = zs.zero_chunk_groups(ch, C)
        assert g[0] == 0 and g[-1] == ch.size and np.all(np.diff(g.astype(np.int64)) > 0)
        for i in range(g.size - 1):
            part = ch[int(g[i]):int(g[i + 1])]
            u = sum(_units(int(c["flat"]), int(c["len"])) for c in part)
            if part.size > 1:
                assert u <= 256 and int(part["len"].sum()) <= C
            if i + 2 < g.size and _units(int(part[0]["flat"]), int(part[0]["len"])) <= 256:
                nxt = ch[int(g[i + 1])]
                grown_u = u + _units(int(nxt["flat"]), int(nxt["len"]))
                assert grown_u > 256 or int(part["len"].sum()) + int(nxt["len"]) > C
    L = zs.lib()
    ch = zs.zero_chunk_table([10] * 8, zs.zero_shard_layout([10] * 8, 1, 16)[0], 0, 128, 64)
    cnt = np.zeros(1, dtype=np.uint64)
    out = np.zeros(1, dtype=np.uint64)
    assert L.zero_chunk_groups(ch.ctypes.data, ch.size, 64, out.ctypes.data, 1, cnt.ctypes.data) == zs.ZERO_ERANGE
    assert int(cnt[0]) == 2  # 8 chunks of 10 elements (3 units each): 6 + 2 under the 64-element bound
    assert L.zero_chunk_groups(ch.ctypes.data, ch.size, 0, None, 0, cnt.ctypes.data) == zs.ZERO_EINVAL
    assert L.zero_chunk_groups(None, 3, 64, None, 0, cnt.ctypes.data) == zs.ZERO_EINVAL


def test_span_groups_partition_the_table():
    """Span groups cover the spans in order; several spans share a group only
    within 2048 work units (vectors of 16 bytes when the phases agree, else
    single elements) and max_group elements."""
    rnd = random.Random(12)
    for _ in range(100):
        sizes = [rnd.randrange(1, rnd.choice([50, 600, 9000])) for _ in range(rnd.randrange(1, 40))]
        R = rnd.randrange(1, 9)
        live = sorted(rnd.sample(range(len(sizes)), rnd.randrange(1, len(sizes) + 1)))
        sp = zs.zero3_gather_spans(sizes, R, live, max_span=rnd.choice([7, 512, 4096]))
        eb = rnd.choice([2, 4])
        V = 16 // eb
        mg = rnd.choice([64, 4096])
        g = zs.zero_span_groups(sp, eb, mg)
        assert g[0] == 0 and g[-1] == sp.size and np.all(np.diff(g.astype(np.int64)) > 0)

        def units(s):
            ln, src, dst = int(s["len"]), int(s["src"]), int(s["dst"])
            if (src - dst) % V:
                return ln
            head = min(ln, (V - dst % V) % V)
            return ln - (ln - head) // V * (V - 1)

        for i in range(g.size - 1):
            part = sp[int(g[i]):int(g[i + 1])]
            if part.size > 1:
                assert sum(units(s) for s in part) <= 2048 and int(part["len"].sum()) <= mg
    cnt = np.zeros(1, dtype=np.uint64)
    assert zs.lib().zero_span_groups(None, 2, 2, 64, None, 0, cnt.ctypes.data) == zs.ZERO_EINVAL
    assert zs.lib().zero_span_groups(sp.ctypes.data, sp.size, 3, 64, None, 0, cnt.ctypes.data) == zs.ZERO_EINVAL


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not found")
def test_piece_orders_are_bijections(tmp_path):
    """The block-to-piece remappings of launch.h, compiled for the host: bijections
    of the grid for any size, one contiguous run per XCD, runs of K consecutive
    pieces, and the identity for K = 1."""
    exe = str(tmp_path / "piece_orders")
    csrc = os.path.join(ROOT, "zero_sharded_optimizer_owned_amd", "csrc")
    res = subprocess.run(["hipcc", "--cuda-host-only", "-x", "hip", "-std=c++17", "-I", csrc,
                          os.path.join(ROOT, "tests", "host", "piece_orders.cpp"), "-o", exe],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and "clean" in run.stdout, run.stdout[-2000:]


def test_noalloc_reduce_rejects_a_check_beyond_its_scratch_before_any_device_call():
    """zero_reduce_owned_noalloc refuses a check whose partials would not fit its
    16 MiB scratch array (about 2.8e9 elements) with ERANGE, before touching a
    device (this runs on the CPU)."""
    L = zs.lib()
    buf = (ct.c_void_p * 1)(ct.c_void_p(16))
    flag, ss = ct.c_void_p(16), ct.c_void_p(32)
    rc = L.zero_reduce_owned_noalloc(buf, 1, zs.ZERO_F16, 0, 0, 3_000_000_000, 1.0, 0, ct.c_void_p(64), 0,
                                     flag, ss, None)
    assert rc == zs.ZERO_ERANGE
    assert "scratch" in L.zero_last_error().decode()


@functools.lru_cache(maxsize=None)
def _device_asm(source: str) -> str:
    """gfx950 assembly of one of the library's HIP sources, built with its flags."""
    from zero_sharded_optimizer_owned_amd.build import CSRC, HIPCC_FLAGS, INCLUDE

    if shutil.which("hipcc") is None:
        pytest.skip("no hipcc")
    flags = [f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    res = subprocess.run(["hipcc", *flags, "-I", INCLUDE, "--cuda-device-only", "-S",
                          os.path.join(CSRC, source), "-o", "-"], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    return res.stdout


def test_device_code_has_no_mixed_precision_fma():
    """The library's build flags keep the fp16 write-back a rounding of the stored
    fp32 master weight: without them the compiler folds the fp16 conversion of
    an fma result into v_fma_mix (one rounding of the exact a*b+c to fp16).
    The gfx950 assembly of the step kernels, built with those flags, holds no
    such instruction (and does hold the plain conversions)."""
    asm = _device_asm("step.hip")
    assert "v_fma_mix" not in asm and "v_mad_mix" not in asm
    assert "v_cvt_f16_f32" in asm


@pytest.mark.parametrize("source", ["step.hip", "copy.hip", "probe.hip"])
def test_no_kernel_uses_scratch_memory(source):
    """Every kernel keeps its working set in registers and LDS: the assembler's
    per-kernel scratch figure is 0 for all of them (a streaming kernel that
    spills to scratch adds memory traffic of its own)."""
    asm = _device_asm(source)
    sizes = [int(x) for x in re.findall(r"; ScratchSize: (\d+)", asm)]
    assert sizes, "no kernel found"
    assert max(sizes) == 0, sizes


def test_step_decision_is_the_unsharded_clip_and_skip():
    """zero_step_decision: any owner's flag skips the step; otherwise the clip factor
    is the oracle's clip of the owners' partial norms summed in owner order (the
    whole gradient's squared norm), rounded once to fp32."""
    rnd = random.Random(9)
    for _ in range(300):
        n = rnd.randrange(1, 70)
        parts = [rnd.choice([0.0, rnd.random() * 10 ** rnd.randrange(-8, 4)]) for _ in range(n)]
        max_norm = rnd.choice([1.0, 0.5, 8.0, 1e-3])
        updated, coef = zs.zero_step_decision([0] * n, parts, max_norm)
        total = 0.0
        for p in parts:  # owner order
            total += p
        assert updated and coef == np.float32(oracle.clip_coef(total, max_norm))
        flags = [0] * n
        flags[rnd.randrange(n)] = rnd.choice([1, 7, -1])
        assert zs.zero_step_decision(flags, parts, max_norm) == (False, None)
    # a skipped step does not look at the partials (they are meaningless after an overflow)
    assert zs.zero_step_decision([0, 1], [float("nan"), 1.0]) == (False, None)
    for bad in (([0], [float("nan")]), ([0], [-1.0]), ([0], [float("inf")])):
        with pytest.raises(zs.ZeroShardError):
            zs.zero_step_decision(*bad)
    with pytest.raises(zs.ZeroShardError):
        zs.zero_step_decision([], [])
    with pytest.raises(zs.ZeroShardError):
        zs.zero_step_decision([0], [1.0], max_norm=0.0)
