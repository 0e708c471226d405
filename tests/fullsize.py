"""Full-size comparisons with the oracle, slice by slice (test infrastructure,
used by tests/test_gpu_sizes_full.py).

The workloads are built on the GPU exactly as bench.py builds them.  For each
slice of the owner's real elements the host regenerates every input of that
slice with the multi-threaded C generator (the generator is counter-based, so
any slice can be produced on its own), runs the oracle on it, copies the GPU's
outputs for the slice back and compares.  The expected ranges come from the
oracle's layout (``helpers.shard_ranges`` asserts that the workload's own
layout and chunk table agree with it).
"""
from __future__ import annotations

import time

import numpy as np

import oracle
import synth
from helpers import assert_bits_equal, assert_state_close, assert_write_back, shard_ranges

SLICE = 1 << 25  # flat elements per slice: a few GB of host memory at 64 ranks


def slices(ranges, limit=SLICE):
    """Consecutive slices of an ordered list of real ranges: ``(lo, hi, parts)``
    where ``parts`` are the real ranges inside the flat span ``[lo, hi)`` and
    ``hi - lo <= limit`` (a slice may span padding between ranges)."""
    out, lo, cur = [], None, []
    for b, e in ranges:
        while b < e:
            if lo is None:
                lo = b
            if b >= lo + limit:
                out.append((lo, cur[-1][1], cur))
                lo, cur = b, []
            t = min(e, lo + limit)
            cur.append((b, t))
            b = t
    if cur:
        out.append((lo, cur[-1][1], cur))
    return out


def key(seed, stream, rank=0, step=0):
    return synth.stream_key(seed, stream, rank, step)


def host16(t, lo, hi):
    """Elements [lo, hi) of a 16-bit device tensor as uint16 bit patterns."""
    import torch

    return t[lo:hi].cpu().view(torch.int16).numpy().view(np.uint16)


def state0(seed, lo, hi):
    """The workload's initial master weights and moments at flat indices [lo, hi)."""
    n = hi - lo
    return (synth.host_values(key(seed, synth.STREAM_MASTER), lo, n, synth.DIST_NORMAL, 0.02, synth.F32),
            synth.host_values(key(seed, synth.STREAM_EXP_AVG), lo, n, synth.DIST_NORMAL, 5e-4, synth.F32),
            synth.host_values(key(seed, synth.STREAM_EXP_AVG_SQ), lo, n, synth.DIST_SQUARE, 1e-4, synth.F32))


def rank_inputs(w, lo, hi):
    """Every rank's gradient at flat indices [lo, hi) in storage form (configs 2-4:
    the generated 16-bit slices; config 5: each rank's eight-microstep fp32
    accumulation, run through the oracle)."""
    n = hi - lo
    if w.cfg == 5:
        out = []
        for r in range(w.R):
            acc = np.empty(n, dtype=np.float32)
            for k in range(8):
                g = synth.host_values(key(5, synth.STREAM_MICRO, r, k), lo, n, synth.DIST_NORMAL, 1e-3, synth.BF16)
                oracle.accumulate(g, synth.BF16, acc, first=(k == 0))
            out.append(acc)
        return out
    code = {2: synth.F16, 3: synth.BF16, 4: synth.F16}[w.cfg]
    return [synth.host_values(key(w.cfg, synth.STREAM_GRAD, r), lo, n, synth.DIST_NORMAL, w.grad_scale, code)
            for r in range(w.R)]


def grad_code(w):
    return {2: synth.F16, 3: synth.BF16, 4: synth.F16, 5: synth.F32}[w.cfg]


def param_code(w):
    import torch

    return synth.F16 if w.p16.dtype == torch.float16 else synth.BF16


def compare_owner_state(w, lo, hi, ow, om, ov, p_or, what, parts=None):
    """The GPU's master, moments and 16-bit copy on flat [lo, hi) against the
    oracle's arrays for the same span (padding included: it must be untouched).
    ``parts``: the real ranges inside the span (default: all of it)."""
    sh, lb, pb = w.sh, w.sh.local_base, w.param_base
    gw = sh.master[lo - lb:hi - lb].cpu().numpy()
    assert_state_close(gw, ow, what + " w")
    assert_state_close(sh.exp_avg[lo - lb:hi - lb].cpu().numpy(), om, what + " m")
    assert_state_close(sh.exp_avg_sq[lo - lb:hi - lb].cpu().numpy(), ov, what + " v")
    got = host16(w.p16, lo - pb, hi - pb)
    real = np.zeros(hi - lo, dtype=bool)
    for b, e in (parts if parts is not None else [(lo, hi)]):
        real[b - lo:e - lo] = True
    assert np.all(got[~real] == p_or[~real]), what + ": 16-bit padding written"
    assert_write_back(got[real], gw[real], ow[real], param_code(w), what + " p16", oracle_bits=p_or[real])


def check_fused_step_full(w, step):
    """Configs 2, 3 and 5 (owner): one fused step at ``step`` from the generated
    state, compared over every owned element."""
    t0 = time.time()
    ranges = shard_ranges(w.sh)
    n_el = 0
    h = oracle.hyper(step=step, **_hp())
    for lo, hi, parts in slices(ranges):
        grads = rank_inputs(w, lo, hi)
        ow, om, ov = state0(w.cfg, lo, hi)
        p_or = np.zeros(hi - lo, dtype=np.uint16)
        oracle.owner_step(parts, h, ow, om, ov, lo, grads=grads, gdtype=grad_code(w), grad_base=lo,
                          divisor=w.divisor, p16=p_or, pdtype=param_code(w), param_base=lo)
        compare_owner_state(w, lo, hi, ow, om, ov, p_or, f"config {w.cfg} [{lo}, {hi})", parts)
        n_el += sum(e - b for b, e in parts)
    assert n_el == w.sh.n_real
    print(f"config {w.cfg}: {n_el} owned elements compared in {time.time() - t0:.1f} s", flush=True)


def _hp():
    import bench

    return bench.HP


def check_local_accumulator_full(w):
    """Config 5's local fp32 accumulator over the whole flat buffer: eight bf16
    microsteps, bit-exact."""
    t0 = time.time()
    P = w.sh.padded_total
    for lo in range(0, P, SLICE):
        hi = min(P, lo + SLICE)
        acc = np.empty(hi - lo, dtype=np.float32)
        for k in range(8):
            g = synth.host_values(key(5, synth.STREAM_MICRO, w.sh.owner, k), lo, hi - lo, synth.DIST_NORMAL, 1e-3,
                                  synth.BF16)
            oracle.accumulate(g, synth.BF16, acc, first=(k == 0))
        assert_bits_equal(w.acc[lo:hi].cpu().numpy(), acc, f"config 5 accumulator [{lo}, {hi})")
    print(f"config 5: local accumulator ({P} elements) compared in {time.time() - t0:.1f} s", flush=True)


def reduced_gradient_full(w, g_dev):
    """Config 4: the oracle's reduced gradient of the owner's whole range, slice by
    slice, compared bit for bit with the GPU's fp32 gradient ``g_dev``
    (owner-local).  Returns the oracle's gradient over [begin, end)."""
    t0 = time.time()
    sh = w.sh
    ranges = shard_ranges(sh)
    assert ranges == [(sh.begin, sh.end)], "the flat 7e10 buffer has no padding inside the owner"
    b0, lb = sh.begin, sh.local_base
    g_or = np.empty(sh.end - b0, dtype=np.float32)
    for lo, hi, _ in slices(ranges):
        dst = g_or[lo - b0:hi - b0]
        oracle.reduce(rank_inputs(w, lo, hi), grad_code(w), w.divisor, out=dst)
        assert_bits_equal(g_dev[lo - lb:hi - lb].cpu().numpy(), dst, f"config 4 reduced gradient [{lo}, {hi})")
    print(f"config 4: reduced gradient ({g_or.size} elements x {w.R} ranks) compared in {time.time() - t0:.1f} s",
          flush=True)
    return g_or


def owner_state_full(w):
    """Generated initial master, moments and a zero 16-bit copy over the owner's
    flat range [begin, end) (config 4: one range, no padding)."""
    b, e = w.sh.begin, w.sh.end
    ow, om, ov = state0(w.cfg, b, e)
    return ow, om, ov, np.zeros(e - b, dtype=np.uint16)


def compare_owner_full(w, ow, om, ov, p_or, what):
    """The GPU state over the owner's range [begin, end) against whole oracle arrays."""
    b, e = w.sh.begin, w.sh.end
    for lo in range(b, e, SLICE):
        hi = min(e, lo + SLICE)
        compare_owner_state(w, lo, hi, ow[lo - b:hi - b], om[lo - b:hi - b], ov[lo - b:hi - b],
                            p_or[lo - b:hi - b], f"{what} [{lo}, {hi})")
