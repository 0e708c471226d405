"""The C ABI from a plain C program: tests/c_abi/step_driver.c allocates device
memory with hipMalloc, creates its own stream and runs the fused owner step, a
checked rank reduce (with and without a workspace), the step decision and the
dense offsets through libzero_shard.so alone (no torch, no Python in the
process).  Its outputs are checked against the oracle to the same bar as the
parity tests: reduced gradient and flag bit-exact, master and moments within
1e-7 + 1e-6 |x|, 16-bit copy within 1 ulp, squared norm 1e-9 relative, the
clip factor to fp32 rounding of the oracle's, the dense offsets exactly.
"""
import math
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import synth
from helpers import BF16, F16, F32, assert_bits_equal, assert_copy_of_master, assert_state_close, gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
import __graft_entry__  # noqa: E402

DRIVER = __graft_entry__.C_DRIVER
HP = dict(lr=1e-3, beta1=0.8, beta2=0.999, eps=1e-8, weight_decay=3e-7, adamw=True)


def _driver():
    if not os.path.exists(DRIVER):
        pytest.fail(f"{DRIVER} is not built: run __graft_entry__.build()")
    return DRIVER


def test_c_driver_is_built_and_checks_its_arguments():
    """Runs on the CPU: the program links against the library and rejects a bad
    command line before any HIP call."""
    res = subprocess.run([_driver()], capture_output=True, text=True, timeout=60)
    assert res.returncode == 1
    assert "usage" in res.stderr


@pytest.mark.gpu
@pytest.mark.parametrize("gcode,pcode,R,owner", [(F16, F16, 4, 1), (BF16, BF16, 8, 5), (F32, BF16, 3, 2)])
def test_c_driver_step_matches_oracle(tmp_path, gcode, pcode, R, owner):
    numels, align, step = [1000, 37, 5003, 1, 64, 777, 20_000], 64, 3
    off, total, owners = oracle.layout(numels, R, align)  # sizes the files; the C program asks the library
    begin, end = owners[owner]
    assert end > begin
    lb = begin & ~7
    nloc = end - lb
    seed = 60 + R
    grads = [gen(seed, synth.STREAM_GRAD, total, synth.DIST_NORMAL, 1e-3, gcode, rank=r) for r in range(R)]
    w = gen(seed, synth.STREAM_MASTER, nloc, synth.DIST_NORMAL, 0.02, F32)
    m = gen(seed, synth.STREAM_EXP_AVG, nloc, synth.DIST_NORMAL, 5e-4, F32)
    v = gen(seed, synth.STREAM_EXP_AVG_SQ, nloc, synth.DIST_SQUARE, 1e-4, F32)

    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(b"ZSTEPIN1")
        np.array([len(numels), R, align, owner, gcode, pcode, step, int(HP["adamw"])], dtype="<u8").tofile(f)
        np.array([HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"]], dtype="<f8").tofile(f)
        np.array(numels, dtype="<u8").tofile(f)
        for g in grads:
            np.ascontiguousarray(g).tofile(f)
        for a in (w, m, v):
            a.astype("<f4").tofile(f)
    print(f"step_driver {gcode=} {pcode=} {R=} {owner=}", flush=True)
    res = subprocess.run([_driver(), str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    raw = out.read_bytes()
    tail = 16 * nloc + 2 * total + 4 + 8
    assert len(raw) == tail + 4 + 4 + 8 + 8 * len(numels)
    fl = np.frombuffer(raw, dtype="<f4", count=3 * nloc)
    gw, gm, gv = fl[:nloc], fl[nloc:2 * nloc], fl[2 * nloc:]
    p16 = np.frombuffer(raw, dtype="<u2", count=total, offset=12 * nloc)
    g_red = np.frombuffer(raw, dtype="<f4", count=nloc, offset=12 * nloc + 2 * total)
    flag = int(np.frombuffer(raw, dtype="<i4", count=1, offset=16 * nloc + 2 * total)[0])
    sumsq = float(np.frombuffer(raw, dtype="<f8", count=1, offset=16 * nloc + 2 * total + 4)[0])

    ranges = oracle.real_ranges(numels, list(off), begin, end)
    ow, om, ov = w.copy(), m.copy(), v.copy()
    p_or = np.zeros(total, dtype=np.uint16)
    oracle.owner_step(ranges, oracle.hyper(step=step, **HP), ow, om, ov, lb, grads=grads, gdtype=gcode,
                      divisor=float(R), p16=p_or, pdtype=pcode)
    assert_state_close(gw, ow, "w")
    assert_state_close(gm, om, "m")
    assert_state_close(gv, ov, "v")
    assert_copy_of_master(p16, p_or, gw, ow, lb, ranges, pcode, "p16")
    # the checked reduce covers the whole owner range, padding included
    g_or = oracle.reduce([g[begin:end] for g in grads], gcode, float(R))
    assert_bits_equal(g_red[begin - lb:], g_or, "reduced gradient")
    assert np.all(g_red[:begin - lb] == 0)
    want_flag, want_sumsq = oracle.grad_check(g_or)
    assert flag == want_flag == 0
    assert math.isclose(sumsq, want_sumsq, rel_tol=1e-9)
    # the decision for this owner alone, and the dense layout
    update = int(np.frombuffer(raw, dtype="<i4", count=1, offset=tail)[0])
    coef = float(np.frombuffer(raw, dtype="<f4", count=1, offset=tail + 4)[0])
    assert update == 1
    assert coef == pytest.approx(oracle.clip_coef(want_sumsq, 1.0), rel=2 ** -23)
    dense_total = int(np.frombuffer(raw, dtype="<u8", count=1, offset=tail + 8)[0])
    dense = np.frombuffer(raw, dtype="<u8", count=len(numels), offset=tail + 16)
    assert dense_total == sum(numels)
    assert [int(x) for x in dense] == oracle.dense_offsets(numels)
