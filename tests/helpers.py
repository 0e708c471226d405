"""Shared helpers for the GPU parity tests (marshalling and comparisons only)."""
import numpy as np

import oracle
import synth

F16, BF16, F32 = 1, 2, 3


def torch_dtype(code):
    import torch

    return {F16: torch.float16, BF16: torch.bfloat16, F32: torch.float32}[code]


def to_dev(a: np.ndarray, code: int, device="cuda"):
    """Host storage (fp32 array or uint16 bits) -> device tensor of the given dtype."""
    import torch

    if code == F32:
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
    return t.view(torch_dtype(code))


def from_dev(t) -> np.ndarray:
    """Device tensor -> host storage (fp32 array or uint16 bits)."""
    import torch

    if t.dtype == torch.float32:
        return t.detach().cpu().numpy()
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def gen(seed, stream, n, dist, scale, code, rank=0, step=0, index0=0):
    key = synth.stream_key(seed, stream, rank, step)
    return synth.values(key, synth.arange(index0, index0 + n), dist, scale, code)


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what=""):
    """Identical bits, except that any NaN matches any NaN."""
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, what
    if got.dtype == np.float32:
        gn, wn = np.isnan(got), np.isnan(want)
        assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
        gb, wb = got.view(np.uint32)[~gn], want.view(np.uint32)[~wn]
    else:
        gb, wb = got, want
    bad = np.nonzero(gb != wb)[0]
    assert bad.size == 0, f"{what}: {bad.size} elements differ, first at {bad[:5]}: {gb[bad[:5]]} vs {wb[bad[:5]]}"


def assert_state_close(got: np.ndarray, want: np.ndarray, what=""):
    """|got - want| <= 1e-7 + 1e-6 |want| elementwise (in fp64; large arrays are
    compared with torch's multi-threaded CPU ops, the same arithmetic)."""
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, what
    if got.size > (1 << 20):
        import torch

        g = torch.from_numpy(np.ascontiguousarray(got)).double()
        w = torch.from_numpy(np.ascontiguousarray(want)).double()
        ok = (g - w).abs() <= 1e-7 + 1e-6 * w.abs()
        if bool(ok.all()):
            return
        bad = torch.nonzero(~ok)[:, 0].numpy()
    else:
        g = got.astype(np.float64)
        w = want.astype(np.float64)
        bad = np.nonzero(~(np.abs(g - w) <= 1e-7 + 1e-6 * np.abs(w)))[0]
        if bad.size == 0:
            return
    raise AssertionError(f"{what}: {bad.size} elements outside tolerance, first {bad[:5]}: "
                         f"{np.asarray(got)[bad[:5]]} vs {np.asarray(want)[bad[:5]]}")


def ordered16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def assert_write_back(got_bits, gpu_w, oracle_w, code, what="", oracle_bits=None):
    """The 16-bit copy of the updated master weights.

    (1) Every value is the round-to-nearest-even of the kernel's own fp32
        master weight, bit for bit (the oracle's encoder).
    (2) It is within 1 ulp of the oracle's rounding of the oracle's master
        weight wherever the master weights' own tolerance
        (1e-7 + 1e-6 |w|) is below half a 16-bit ulp of w.  Closer to zero
        (a weight that the update nearly cancels, |w| below about 2e-4 for
        fp16 and 3e-5 for bf16) an fp32 kernel may differ from the fp64
        oracle by more than a 16-bit ulp of so small a value while its
        master weight stays within the state tolerance; there (1) and the
        state check bound the copy.
    ``oracle_bits``: the oracle's rounding of ``oracle_w``, when already at hand.
    """
    got_bits = np.asarray(got_bits)
    gpu_w = np.ascontiguousarray(gpu_w, dtype=np.float32)
    assert_bits_equal(got_bits, oracle.encode16(gpu_w, code), what + " (rounding of the kernel's master)")
    want = (np.asarray(oracle_bits) if oracle_bits is not None
            else oracle.encode16(np.ascontiguousarray(oracle_w, dtype=np.float32), code))
    w64 = np.abs(np.asarray(oracle_w, dtype=np.float64))
    mbits = 10 if code == F16 else 7
    # half a 16-bit ulp of w is above |w| * 2^-(mbits + 2)
    close = 1e-7 + 1e-6 * w64 <= w64 * 2.0 ** -(mbits + 2)
    d = np.abs(ordered16(got_bits) - ordered16(want))
    bad = np.nonzero(close & (d > 1))[0]
    assert bad.size == 0, (f"{what}: {bad.size} 16-bit values more than 1 ulp from the oracle's rounding, first "
                           f"{bad[:5]}: {got_bits[bad[:5]]} vs {want[bad[:5]]} (w {np.asarray(oracle_w)[bad[:5]]})")


def assert_copy_of_master(p16_bits, p_or_bits, gpu_w, oracle_w, w_base, ranges, code, what="", param_base=0):
    """The 16-bit buffer after an owner step: outside the owner's real ranges it
    holds what the oracle's buffer holds (nothing else was written); on them,
    ``assert_write_back`` against the kernel's and the oracle's master weights.
    Master arrays are indexed [f - w_base], 16-bit buffers [f - param_base]."""
    p16_bits, p_or_bits = np.asarray(p16_bits), np.asarray(p_or_bits)
    idx = (np.concatenate([np.arange(b, e, dtype=np.int64) for b, e in ranges]) if len(ranges)
           else np.zeros(0, dtype=np.int64))
    mask = np.zeros(p16_bits.size, dtype=bool)
    mask[idx - param_base] = True
    assert np.array_equal(p16_bits[~mask], p_or_bits[~mask]), what + ": elements outside the real ranges written"
    assert_write_back(p16_bits[idx - param_base], np.asarray(gpu_w)[idx - w_base], np.asarray(oracle_w)[idx - w_base],
                      code, what)


def oracle_hyper(step, hp):
    return oracle.hyper(step=step, **hp)


# ---------------------------------------------------------------- layouts from the oracle
def checked_layout(numels, R, A):
    """(tensor offsets, padded total, owner begins, owner ends) as the oracle
    defines them, after asserting that the library's zero_shard_layout gives
    the same; the GPU tests take their expected ranges from here."""
    import zero_sharded_optimizer_owned_amd as zs

    off, total, owners = oracle.layout(list(numels), R, A)
    loff, ltotal, lb, le = zs.zero_shard_layout(numels, R, A)
    assert [int(x) for x in loff] == off and ltotal == total, "library layout differs from the oracle's"
    assert [(int(b), int(e)) for b, e in zip(lb, le)] == owners, "library owner ranges differ from the oracle's"
    return off, total, [b for b, _ in owners], [e for _, e in owners]


def assert_chunks_cover(chunks, ranges, what=""):
    """The library's chunk table covers exactly the oracle's real ranges, in order, once."""
    pieces = [(int(c["flat"]), int(c["flat"]) + int(c["len"])) for c in chunks]
    merged = []
    for b, e in pieces:
        assert e > b, f"{what}: empty chunk"
        if merged and merged[-1][1] == b:
            merged[-1] = (merged[-1][0], e)
        else:
            assert not merged or merged[-1][1] < b, f"{what}: chunks overlap or go backwards"
            merged.append((b, e))
    want = []
    for b, e in ranges:
        if want and want[-1][1] == b:
            want[-1] = (want[-1][0], e)
        else:
            want.append((b, e))
    assert merged == want, f"{what}: chunk table does not cover the real elements exactly"


def shard_ranges(sh):
    """The oracle's real ranges of an OwnerShard's owner, after asserting that the
    shard's layout and chunk table agree with the oracle."""
    off, total, owners = oracle.layout(list(sh.numels), sh.ranks, sh.align)
    assert [int(x) for x in sh.offsets] == off and sh.padded_total == total
    assert (sh.begin, sh.end) == owners[sh.owner]
    ranges = oracle.real_ranges(sh.numels, off, sh.begin, sh.end)
    assert_chunks_cover(sh.chunks, ranges, f"owner {sh.owner}")
    return ranges
