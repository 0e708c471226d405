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
    """|got - want| <= 1e-7 + 1e-6 |want| elementwise."""
    g = got.astype(np.float64)
    w = want.astype(np.float64)
    err = np.abs(g - w)
    tol = 1e-7 + 1e-6 * np.abs(w)
    bad = np.nonzero(~(err <= tol))[0]
    assert bad.size == 0, f"{what}: {bad.size} elements outside tolerance, first {bad[:5]}: {g[bad[:5]]} vs {w[bad[:5]]}"


def ordered16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def assert_p16_within_ulp(got_bits: np.ndarray, want_bits: np.ndarray, what=""):
    d = np.abs(ordered16(got_bits) - ordered16(want_bits))
    bad = np.nonzero(d > 1)[0]
    assert bad.size == 0, f"{what}: {bad.size} 16-bit values more than 1 ulp off, first {bad[:5]}"


def oracle_hyper(step, hp):
    return oracle.hyper(step=step, **hp)
