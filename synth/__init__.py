"""Seeded synthetic inputs for tests and benchmarks (input generation only).

Every value is a pure function of integers: (seed, stream, rank, step) pick a
stream key, and element ``i`` of that stream is output ``i`` of a splitmix64
generator started at that key (Steele, Lea and Flood's SplitMix64, as published
by Vigna).  Any element can therefore be produced on its own, on the host
(this module, numpy) or on the device (``synth/csrc/synth_device.hip``), with
identical bits, so full-size device inputs can be checked on the host at
sampled indices without copying them back.

Value recipes (each ends in exactly one IEEE fp32 rounding, so host and device
agree bit for bit):

* ``normal``  : Irwin-Hall sum of the four 16-bit fields of the hash,
  ``S in [0, 262140]``, centred and scaled: ``fl32(float(S - 131070) * c)``
  with ``c = fl32(sigma * sqrt(3) / 65536)``; mean 0, standard deviation
  ``sigma``, bounded by ``2*sqrt(3)*sigma``.
* ``uniform`` : ``fl32(float((h >> 40) - 2**23) * fl32(a / 2**23))`` on
  ``[-a, a)``.
* ``square``  : ``fl32(x * x)`` of a ``normal`` draw (non-negative values).

16-bit outputs are the round-to-nearest-even conversion of the fp32 value,
done here by numpy (fp16) and torch (bf16) and on the device by the HIP
conversion routines.

This module holds no part of the optimizer arithmetic.
"""
from __future__ import annotations

import math

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Stream numbers: which quantity a key draws.
STREAM_MASTER = 0
STREAM_GRAD = 1
STREAM_MICRO = 2
STREAM_INJECT = 3
STREAM_SIZES = 4
STREAM_EXP_AVG = 5
STREAM_EXP_AVG_SQ = 6

DIST_NORMAL = 0
DIST_UNIFORM = 1
DIST_SQUARE = 2

F16 = 1
BF16 = 2
F32 = 3

_MASK64 = (1 << 64) - 1


def mix64(z):
    """SplitMix64 output function on uint64 (numpy arrays or scalars)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _mix_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int, rank: int = 0, step: int = 0) -> int:
    """Key of one value stream: four chained SplitMix64 steps over the ids."""
    k = _mix_int(seed + 0x9E3779B97F4A7C15)
    k = _mix_int(k ^ ((stream + 1) * 0x9E3779B97F4A7C15 & _MASK64))
    k = _mix_int(k ^ ((rank + 1) * 0xD1B54A32D192ED03 & _MASK64))
    k = _mix_int(k ^ ((step + 1) * 0xDB4F0B9175AE2165 & _MASK64))
    return k


def hash_at(key: int, idx) -> np.ndarray:
    """Output ``idx`` (uint64 array) of the SplitMix64 sequence started at ``key``."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = np.uint64(key) + (idx + np.uint64(1)) * GOLDEN
    return mix64(state)


def normal_scale(sigma: float) -> np.float32:
    return np.float32(sigma * math.sqrt(3.0) / 65536.0)


def uniform_scale(a: float) -> np.float32:
    return np.float32(a / 8388608.0)


def values_f32(key: int, idx, dist: int, scale: float) -> np.ndarray:
    """fp32 values at the given indices of a stream (see module docstring)."""
    h = hash_at(key, idx)
    if dist in (DIST_NORMAL, DIST_SQUARE):
        m = np.uint64(0xFFFF)
        s = (h & m) + ((h >> np.uint64(16)) & m) + ((h >> np.uint64(32)) & m) + (h >> np.uint64(48))
        centred = s.astype(np.int64) - 131070
        x = centred.astype(np.float32) * normal_scale(scale)
        if dist == DIST_SQUARE:
            x = x * x
        return x.astype(np.float32)
    if dist == DIST_UNIFORM:
        centred = (h >> np.uint64(40)).astype(np.int64) - 8388608
        return (centred.astype(np.float32) * uniform_scale(scale)).astype(np.float32)
    raise ValueError(f"unknown distribution {dist}")


def to_bits16(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round fp32 values to fp16 or bf16 (nearest, ties to even); uint16 bit patterns."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        import torch

        t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(f"not a 16-bit dtype: {dtype}")


def values(key: int, idx, dist: int, scale: float, dtype: int) -> np.ndarray:
    """Stream values in storage form: fp32 array, or uint16 bit patterns for fp16/bf16."""
    x = values_f32(key, idx, dist, scale)
    if dtype == F32:
        return x
    return to_bits16(x, dtype)


def arange(start: int, stop: int) -> np.ndarray:
    return np.arange(start, stop, dtype=np.uint64)


def log_uniform_sizes(seed: int, count: int, lo: int, hi: int) -> np.ndarray:
    """``count`` integer sizes, log-uniform on [lo, hi] (before any rescaling)."""
    key = stream_key(seed, STREAM_SIZES)
    u = (hash_at(key, arange(0, count)) >> np.uint64(11)).astype(np.float64) / float(1 << 53)
    return np.floor(np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))).astype(np.int64)


# ---------------------------------------------------------------------------
# Device twin (synth/csrc/synth_device.hip), for inputs too large to copy in.
# ---------------------------------------------------------------------------
import ctypes as _ct
import os as _os

_HERE = _os.path.dirname(_os.path.abspath(__file__))
LIB_PATH = _os.path.join(_HERE, "libzero_synth.so")
_lib = None


HOST_LIB_PATH = _os.path.join(_HERE, "libsynth_host.so")
_host_lib = None


def build_host() -> str:
    """Compile the multi-threaded host generator (gcc, OpenMP) into synth/libsynth_host.so."""
    import subprocess

    src = _os.path.join(_HERE, "csrc", "synth_host.c")
    tmp = HOST_LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-Wall", src, "-o", tmp, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building the host generator failed:\n" + res.stderr)
    _os.replace(tmp, HOST_LIB_PATH)
    return HOST_LIB_PATH


def _load_host():
    global _host_lib
    if _host_lib is None:
        if not _os.path.exists(HOST_LIB_PATH):
            build_host()
        lib = _ct.CDLL(HOST_LIB_PATH)
        lib.synth_host_fill.restype = _ct.c_int
        lib.synth_host_fill.argtypes = [_ct.c_void_p, _ct.c_int, _ct.c_uint64, _ct.c_uint64, _ct.c_uint64,
                                        _ct.c_int, _ct.c_float]
        _host_lib = lib
    return _host_lib


def host_values(key: int, start: int, count: int, dist: int, scale: float, dtype: int,
                out: np.ndarray = None) -> np.ndarray:
    """Elements [start, start + count) of a stream in storage form, on all host
    cores: the same bits as ``values(key, arange(start, start + count), ...)``."""
    want = np.float32 if dtype == F32 else np.uint16
    if out is None:
        out = np.empty(count, dtype=want)
    if out.dtype != want or out.size != count or not out.flags["C_CONTIGUOUS"]:
        raise ValueError("out must be a contiguous array of the storage dtype and length count")
    c = float(_SCALE[dist](scale))
    rc = _load_host().synth_host_fill(_ct.c_void_p(out.ctypes.data), dtype, count, key, start, dist, c)
    if rc != 0:
        raise ValueError(f"synth_host_fill rejected its arguments ({rc})")
    return out


def build(verbose: bool = False) -> str:
    """Compile the device generator for gfx950 into synth/libzero_synth.so (and the host twin)."""
    import subprocess

    build_host()

    src = _os.path.join(_HERE, "csrc", "synth_device.hip")
    tmp = LIB_PATH + ".tmp"
    cmd = [
        "hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Xclang", "-target-feature", "-Xclang", "-fma-mix-insts",
        src, "-o", tmp,
    ]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building the synthetic-input library failed:\n" + res.stderr)
    _os.replace(tmp, LIB_PATH)
    if verbose and res.stderr:
        print(res.stderr)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not _os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; run __graft_entry__.build() first")
        lib = _ct.CDLL(LIB_PATH)
        lib.synth_fill.restype = _ct.c_int
        lib.synth_fill.argtypes = [_ct.c_void_p, _ct.c_int, _ct.c_uint64, _ct.c_uint64, _ct.c_uint64,
                                   _ct.c_int, _ct.c_float, _ct.c_void_p]
        _lib = lib
    return _lib


_SCALE = {DIST_NORMAL: normal_scale, DIST_SQUARE: normal_scale, DIST_UNIFORM: uniform_scale}


def device_fill(t, key: int, index0: int, dist: int, scale: float) -> None:
    """Fill a contiguous CUDA tensor (float32, float16 or bfloat16) on the current stream."""
    import torch

    code = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}[t.dtype]
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("device_fill needs a contiguous device tensor")
    c = float(_SCALE[dist](scale))
    rc = _load().synth_fill(_ct.c_void_p(t.data_ptr()), code, t.numel(), key, index0, dist, c,
                            _ct.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill failed with code {rc}")
