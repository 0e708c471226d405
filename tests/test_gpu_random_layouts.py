"""Seeded random cases against the oracle: the fused step, the flat reduce, the
fp32 export/import and the ZeRO-3 partition and gather copies.

Fused step:

Each case draws a tensor list (sizes from 1 to a few thousand, some of them
multiples of the alignment so that runs merge across tensors), a rank count,
an alignment, a chunk size, an owner, gradient and write-back dtypes,
Adam or AdamW, a clip factor, and whether the packed group table is used.
Master weights and moments: |gpu - oracle| <= 1e-7 + 1e-6 |oracle|; the
16-bit copy within 1 ulp of the oracle's rounding, with padding and other
owners' elements untouched.
"""
import random

import numpy as np
import pytest

import oracle
import synth
from helpers import (BF16, F16, F32, assert_chunks_cover, assert_copy_of_master, assert_state_close,
                     checked_layout, from_dev, gen, shard_ranges, to_dev)

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


def _case(seed):
    rnd = random.Random(seed)
    A = rnd.choice([1, 8, 64])
    sizes = []
    for _ in range(rnd.randrange(1, 40)):
        kind = rnd.random()
        if kind < 0.3:
            sizes.append(A * rnd.randrange(1, 40))      # no padding: merges with its neighbours
        elif kind < 0.6:
            sizes.append(rnd.randrange(1, 20))          # shorter than a vector
        else:
            sizes.append(rnd.randrange(1, 3000))
    R = rnd.choice([1, 2, 3, 4, 5, 8, 11, 16, 19])
    gcode = rnd.choice([F16, BF16, F32])
    pcode = rnd.choice([F16, BF16, 0])
    return dict(sizes=sizes, A=A, R=R, owner=rnd.randrange(R), C=rnd.choice([8, 64, 256, 2048]),
                gcode=gcode, pcode=pcode, adamw=rnd.random() < 0.7, wd=rnd.choice([0.0, 1e-2]),
                clip=rnd.choice([1.0, 0.25]), grouped=rnd.random() < 0.5, step=rnd.randrange(1, 50))


@pytest.mark.parametrize("seed", range(40))
def test_random_layout_step_matches_oracle(seed):
    c = _case(seed)
    print(f"case {seed}: {c}", flush=True)
    numels, R = c["sizes"], c["R"]
    off, total, b, e = checked_layout(numels, R, c["A"])
    begin, end = int(b[c["owner"]]), int(e[c["owner"]])
    lb = begin & ~7
    size = max(8, end - lb)
    grads = [gen(seed, synth.STREAM_GRAD, total, synth.DIST_NORMAL, 1e-3, c["gcode"], rank=r) for r in range(R)]
    w = gen(seed, synth.STREAM_MASTER, size, synth.DIST_NORMAL, 0.02, F32)
    m = gen(seed, synth.STREAM_EXP_AVG, size, synth.DIST_NORMAL, 5e-4, F32)
    v = gen(seed, synth.STREAM_EXP_AVG_SQ, size, synth.DIST_SQUARE, 1e-4, F32)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=c["wd"], adamw=c["adamw"])
    chunks = zs.zero_chunk_table(numels, off, begin, end, c["C"])
    kw = {}
    if c["grouped"] and chunks.size:
        groups = zs.zero_chunk_groups(chunks, c["C"])
        kw = dict(groups_dev=torch.from_numpy(groups.astype(np.int64)).to(DEV), n_groups=groups.size - 1)
    dw, dm, dv = to_dev(w, F32), to_dev(m, F32), to_dev(v, F32)
    sentinel = 0x7BFF if c["pcode"] == F16 else 0x3F80
    p_host = np.full(total + 8, sentinel, dtype=np.uint16)
    dp = to_dev(p_host, c["pcode"]) if c["pcode"] else None
    zs.zero_adam_step(chunks_dev=zs.chunks_to_device(chunks) if chunks.size else None, n_chunks=chunks.size,
                      begin=begin, end=end, master=dw, exp_avg=dm, exp_avg_sq=dv, local_base=lb,
                      step=c["step"], rank_grads=[to_dev(g, c["gcode"]) for g in grads], divisor=float(R),
                      param16=dp, clip_coef=c["clip"], **kw, **hp)
    ranges = oracle.real_ranges(numels, list(off), begin, end)
    assert_chunks_cover(chunks, ranges, f"case {seed}")
    oracle.owner_step(ranges, oracle.hyper(step=c["step"], clip_coef=c["clip"], **hp), w, m, v, lb,
                      grads=grads, gdtype=c["gcode"], divisor=float(R),
                      p16=p_host if c["pcode"] else None, pdtype=c["pcode"])
    assert_state_close(from_dev(dw), w, f"case {seed} w")
    assert_state_close(from_dev(dm), m, f"case {seed} m")
    assert_state_close(from_dev(dv), v, f"case {seed} v")
    if c["pcode"]:
        got = from_dev(dp)
        real = np.zeros(total + 8, dtype=bool)
        for s, t in ranges:
            real[s:t] = True
        assert np.all(got[~real] == sentinel), f"case {seed}: padding or foreign elements written"
        assert_copy_of_master(got, p_host, from_dev(dw), w, lb, ranges, c["pcode"], f"case {seed} p16")


@pytest.mark.parametrize("seed", range(30))
def test_random_flat_reduce_matches_oracle(seed):
    """The flat rank reduce with random rank count, dtype, range ends, buffer
    bases, divisor, accumulation mode and fused check: bit-exact, flag exact,
    squared norm 1e-9 relative.  Elements outside the range stay untouched."""
    from helpers import assert_bits_equal

    rnd = random.Random(1000 + seed)
    R = rnd.choice([1, 2, 3, 4, 7, 8, 9, 16, 17, 31, 32, 33, 64])
    code = rnd.choice([F16, BF16, F32])
    begin = rnd.randrange(0, 80)
    n = rnd.choice([0, 1, 7, 9, rnd.randrange(10, 3000), rnd.randrange(3000, 70_000)])
    end = begin + n
    grad_base = rnd.choice([0, begin & ~7])
    out_base = rnd.choice([0, begin & ~7])
    divisor = rnd.choice([float(R), float(R) * 65536.0, 3.0, 0.75])
    mode = rnd.choice([0, 1, 2])
    check = rnd.random() < 0.5
    print(f"case {seed}: R={R} code={code} begin={begin} n={n} grad_base={grad_base} out_base={out_base} "
          f"divisor={divisor} mode={mode} check={check}", flush=True)
    total = end + 8
    grads = [gen(2000 + seed, synth.STREAM_GRAD, total, synth.DIST_NORMAL, 1e-2, code, rank=r) for r in range(R)]
    start = gen(2000 + seed, synth.STREAM_EXP_AVG, total - out_base, synth.DIST_NORMAL, 1e-2, F32)
    out = to_dev(start.copy(), F32)
    kw = {}
    if check:
        ws = zs.check_workspace(max(n, 1), DEV)
        ov = torch.full((1,), 7, dtype=torch.int32, device=DEV)
        ss = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
        kw = dict(check=(ov, ss, ws))
    zs.zero_reduce_owned([to_dev(g[grad_base:], code) for g in grads], begin, n, divisor, out,
                         grad_base=grad_base, out_base=out_base, accumulate=mode, **kw)
    want = start.copy()
    if n:
        seg = [g[begin:end] for g in grads]
        dst = want[begin - out_base:end - out_base]
        if mode == 2:
            oracle.reduce_add(seg, code, divisor, dst)
        else:
            dst[:] = oracle.reduce(seg, code, divisor, out=dst.copy(), accumulate=mode == 1)
    assert_bits_equal(from_dev(out), want, f"case {seed}")
    if check and n:
        flag, sumsq = oracle.grad_check(want[begin - out_base:end - out_base])
        assert int(ov.item()) == flag
        if not flag:
            assert abs(ss.item() - sumsq) <= 1e-9 * sumsq


def _random_sizes(rnd, A):
    out = []
    for _ in range(rnd.randrange(1, 60)):
        k = rnd.random()
        out.append(A * rnd.randrange(1, 30) if k < 0.3 else rnd.randrange(1, 40) if k < 0.6
                   else rnd.randrange(1, 5000))
    return out


@pytest.mark.parametrize("seed", range(20))
def test_random_export_import_matches_oracle(seed):
    """Owner shards to dense per-tensor fp32 and back, every owner, with and
    without chunk groups: bit-exact against the oracle's consolidation."""
    from helpers import assert_bits_equal

    rnd = random.Random(3000 + seed)
    A = rnd.choice([1, 8, 64])
    numels = _random_sizes(rnd, A)
    R = rnd.choice([1, 2, 3, 5, 8, 13])
    C = rnd.choice([8, 64, 512, 2048])
    grouped = rnd.random() < 0.5
    print(f"case {seed}: {len(numels)} tensors R={R} A={A} C={C} grouped={grouped}", flush=True)
    shards = [zs.OwnerShard(numels, R, r, align=A, max_chunk=C, device=DEV) for r in range(R)]
    if not grouped:
        for sh in shards:
            sh.groups_dev = None
    arrays = [gen(3000 + seed, synth.STREAM_MASTER, max(8, sh.local_size), synth.DIST_NORMAL, 0.02, F32, rank=r)
              for r, sh in enumerate(shards)]
    dense = torch.full((sum(numels),), float("nan"), device=DEV)
    for sh, a in zip(shards, arrays):
        sh.to_dense(to_dev(a, F32), dense)
    off, _, owners = oracle.layout(numels, R, A)  # expected layout; the shards must agree with it
    for sh in shards:
        shard_ranges(sh)
        assert [int(x) for x in sh.dense_offsets] == oracle.dense_offsets(numels)
    want = oracle.consolidate(numels, off, owners, arrays, [b & ~7 for b, _ in owners])
    assert_bits_equal(from_dev(dense), want, f"case {seed} export")
    for sh in shards:
        back = torch.full((max(8, sh.local_size),), -1.0, device=DEV)
        sh.from_dense(dense, back)
        ref = oracle.distribute(numels, off, sh.begin, sh.end, want,
                                np.full(max(8, sh.local_size), -1.0, dtype=np.float32), sh.local_base)
        assert_bits_equal(from_dev(back), ref, f"case {seed} import")


@pytest.mark.parametrize("seed", range(20))
def test_random_stage3_partition_and_gather_match_oracle(seed):
    """ZeRO-3 per-tensor shards and gathers of random live sets, with random span
    limits and with and without span groups: bit-exact against the oracle."""
    from helpers import assert_bits_equal

    rnd = random.Random(4000 + seed)
    code = rnd.choice([BF16, F32])
    sizes = _random_sizes(rnd, 8)
    R = rnd.choice([1, 2, 3, 4, 8, 16])
    max_span = rnd.choice([1, 7, 64, 4096])
    grouped = rnd.random() < 0.5
    print(f"case {seed}: {len(sizes)} tensors R={R} code={code} max_span={max_span} grouped={grouped}",
          flush=True)
    dense = gen(4000 + seed, synth.STREAM_MASTER, sum(sizes), synth.DIST_NORMAL, 0.02, code)
    dense_dev = to_dev(dense, code)
    _, resident, _ = zs.zero3_storage(sizes, R)
    want_shards = oracle.stage3_shards(sizes, R, dense)
    eb = 2 if code == BF16 else 4

    def gk(spans):
        if not grouped or not spans.size:
            return {}
        g = zs.zero_span_groups(spans, eb)
        return dict(groups_dev=torch.from_numpy(g.astype(np.int64)).to(DEV), n_groups=g.size - 1)

    shard_devs = []
    for r in range(R):
        spans = zs.zero3_partition_spans(sizes, R, r, max_span=max_span)
        buf = torch.zeros(resident, dtype=dense_dev.dtype, device=DEV)
        zs.zero_copy_spans(zs.spans_to_device(spans) if spans.size else None, spans.size, [dense_dev], buf,
                           **gk(spans))
        assert_bits_equal(from_dev(buf), want_shards[r], f"case {seed} shard {r}")
        shard_devs.append(buf)
    for _ in range(3):
        live = rnd.sample(range(len(sizes)), rnd.randrange(1, len(sizes) + 1))
        _, _, gathered = zs.zero3_storage(sizes, R, live)
        spans = zs.zero3_gather_spans(sizes, R, live, max_span=max_span)
        out = torch.full((gathered,), 7, dtype=dense_dev.dtype, device=DEV)
        zs.zero_copy_spans(zs.spans_to_device(spans), spans.size, shard_devs, out, **gk(spans))
        assert_bits_equal(from_dev(out), oracle.stage3_gather(sizes, R, want_shards, live),
                          f"case {seed} gather {live}")
