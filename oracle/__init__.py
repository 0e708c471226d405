"""ORACLE -- test infrastructure, not a product path.

Plain, slow, obviously-correct CPU definitions of what the ZeRO owner-shard
optimizer step computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``zero_sharded_optimizer_owned_amd``) and imports
nothing from it.

Two halves:

* pure Python (this file), following the pages in their own notation:
  ``adam_step``, ``owner_ranges``, ``compare_owned_updates``, ``state_bytes``,
  ``parameter_storage``, the flattened-buffer layout and the clip factor;
* scalar C (``zero_oracle.c`` -> ``liboracle.so``) for the same arithmetic at
  sizes Python loops cannot reach: fp32 rank reduce, accumulation, overflow
  flag and squared norm, fp64 Adam/AdamW on fp32 state, fp16/bf16 encoders.

Sources ("the pages"), cited by title and section:

* [ZeRO-3 docs]  DeepSpeed ZeRO API documentation (zero3.rst): the list of
  ZeRO stages and the JSON configuration examples (AdamW, fp16).
* [ZeRO Q&A]     "How does DeepSpeed ZeRO stage 1, 2, and 3 partition optimizer
  states, gradients, and parameters?": "Memory Footprint Reduction Matrix".
* [Deep dive]    "Deep dive: DeepSpeed" (leetllm): sections "Count state before
  choosing a stage", "Reduce first, then update the owned slice", "Let the
  engine own the microstep", "Stage 3 needs a live working set", "Resume
  training and export weights separately".

Readings where the pages are silent are listed with each function.  Every
function is pinned by the ``-m "not gpu"`` tests.
"""
from __future__ import annotations

import ctypes as ct
import math
import os
import subprocess
from fractions import Fraction
from typing import Dict, List, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

F16, BF16, F32 = 1, 2, 3


# ---------------------------------------------------------------------------
# Pure-Python functions that follow the pages.
# ---------------------------------------------------------------------------
def adam_step(weight: float, first: float, second: float, gradient: float, step: int,
              lr: float = 0.01, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8):
    """One scalar Adam update in Python floats (fp64).

    [Deep dive] "Reduce first, then update the owned slice": moments are
    exponential averages of the gradient and of its square (uncentred), each
    divided by ``1 - beta**step``; the step is ``lr * mhat / (sqrt(vhat) + eps)``
    (eps outside the square root); steps count from 1.
    """
    first = beta1 * first + (1.0 - beta1) * gradient
    second = beta2 * second + (1.0 - beta2) * gradient * gradient
    mhat = first / (1.0 - beta1 ** step)
    vhat = second / (1.0 - beta2 ** step)
    return weight - lr * mhat / (math.sqrt(vhat) + eps), first, second


def owner_ranges(parameters: int, ranks: int) -> List[range]:
    """Contiguous ownership: owner r holds ``[floor(P*r/R), floor(P*(r+1)/R))``.

    [Deep dive] "Reduce first, then update the owned slice": owners are
    contiguous and may be empty when there are more ranks than parameters.
    """
    return [range(parameters * r // ranks, parameters * (r + 1) // ranks) for r in range(ranks)]


def pages_gradient(i: int, r: int, step: int) -> float:
    """The lab's deterministic per-rank gradient for parameter i, rank r, step t."""
    return ((i + 2 * r + step) % 7 - 3) / 10


def compare_owned_updates(parameters: int, ranks: int, steps: int, grad=pages_gradient):
    """Adam on the rank-mean gradient, run once unsharded and once owner by owner.

    [Deep dive] "Reduce first, then update the owned slice": weight i starts at
    ``0.1*i`` with both moments zero; at every step each rank supplies a
    gradient for every parameter.  The unsharded run updates every parameter
    from the mean over ranks.  In the sharded run each owner keeps the state of
    its contiguous index range only, forms the same mean for those indices
    (its share of a reduce-scatter) and updates them once.  Returns
    ``(unsharded, sharded)``: the ``(w, m, v)`` of every parameter, the sharded
    list read owner after owner.
    """
    for label, x in (("parameters", parameters), ("ranks", ranks), ("steps", steps)):
        if type(x) is not int or x <= 0:
            raise ValueError(f"{label}: expected an int above zero, got {x!r}")

    def initial(i):
        return 0.1 * i, 0.0, 0.0

    def rank_mean(g, i):
        total = 0.0
        for r in range(ranks):
            total += g[r][i]
        return total / ranks

    unsharded = [initial(i) for i in range(parameters)]
    # owner r: (its index range, the states of those indices in range order)
    owned = [(span, [initial(i) for i in span]) for span in owner_ranges(parameters, ranks)]
    for t in range(1, steps + 1):
        g = [[grad(i, r, t) for i in range(parameters)] for r in range(ranks)]  # g[r][i]
        for i in range(parameters):
            unsharded[i] = adam_step(*unsharded[i], rank_mean(g, i), t)
        for span, states in owned:
            for k, i in enumerate(span):
                states[k] = adam_step(*states[k], rank_mean(g, i), t)
    sharded = [state for _, states in owned for state in states]
    return unsharded, sharded


def state_bytes(parameters: int, ranks: int, param: int = 2, grad: int = 2,
                optimizer: int = 12) -> Dict[str, Fraction]:
    """Idealised per-rank persistent bytes for DP and ZeRO-1/2/3, as exact fractions.

    [Deep dive] "Count state before choosing a stage" and [ZeRO Q&A] "Memory
    Footprint Reduction Matrix": a parameter carries three parts -- the 16-bit
    compute copy (``param`` bytes), its gradient (``grad``) and the optimizer
    state with the fp32 master (``optimizer``).  Stage k divides a part among
    the ranks once k reaches the stage that first shards it (optimizer state
    from stage 1, gradients from stage 2, parameters at stage 3); DP (stage 0)
    replicates all three.  Every input must be an int above zero.
    """
    widths = {"param": param, "grad": grad, "optimizer": optimizer}
    for label, x in (("parameters", parameters), ("ranks", ranks), *widths.items()):
        if type(x) is not int or x <= 0:
            raise ValueError(f"{label}: expected an int above zero, got {x!r}")
    first_sharded = {"optimizer": 1, "grad": 2, "param": 3}
    out = {}
    for stage, name in enumerate(("DP", "ZeRO-1", "ZeRO-2", "ZeRO-3")):
        total = Fraction(0)
        for part, width in widths.items():
            copies = Fraction(1, ranks) if stage >= first_sharded[part] else Fraction(1)
            total += parameters * width * copies
        out[name] = total
    return out


def parameter_storage(layer_sizes: Sequence[int], ranks: int, live_layers: Sequence[int]):
    """ZeRO-3 parameter elements: resident shards + separate full gather buffers.

    [Deep dive] "Stage 3 needs a live working set": each tensor's shard holds
    ``ceil(n/R)`` whole elements; a live (gathered) tensor also needs its own
    padded buffer of ``R * ceil(n/R)`` elements, which does not alias the
    shard.  Returns ``(resident, gathered, total)`` element counts.
    """
    if type(ranks) is not int or ranks < 1:
        raise ValueError(f"ranks: expected an int of at least 1, got {ranks!r}")
    sizes = list(layer_sizes)
    if not sizes or not all(type(n) is int and n >= 1 for n in sizes):
        raise ValueError("layer_sizes: every tensor needs an int element count of at least 1")
    live = list(live_layers)
    if len(set(live)) != len(live) or not all(type(k) is int and 0 <= k < len(sizes) for k in live):
        raise ValueError("live_layers: expected distinct indices into layer_sizes")
    resident = gathered = 0
    for k, n in enumerate(sizes):
        shard = n // ranks + (1 if n % ranks else 0)  # rounded up to whole elements
        resident += shard
        if k in live:
            gathered += ranks * shard
    return resident, gathered, resident + gathered


def stage3_shards(layer_sizes: Sequence[int], ranks: int, dense: np.ndarray) -> List[np.ndarray]:
    """Every rank's shard buffer under per-tensor ZeRO-3 partitioning.

    [Deep dive] "Stage 3 needs a live working set": tensor k is cut into
    ranks shards of ceil(n_k / ranks) elements; rank r holds elements
    [r*s_k, (r+1)*s_k) of it, zero past the tensor's end.  A rank's buffer
    holds its shards of all tensors in tensor order.  ``dense`` is the
    tensors' elements concatenated.  Plain loops.
    """
    shards = [-(-n // ranks) for n in layer_sizes]
    out = [np.zeros(sum(shards), dtype=dense.dtype) for _ in range(ranks)]
    for r in range(ranks):
        pos, dpos = 0, 0
        for n, s in zip(layer_sizes, shards):
            for j in range(s):
                e = r * s + j
                if e < n:
                    out[r][pos + j] = dense[dpos + e]
            pos += s
            dpos += n
    return out


def stage3_gather(layer_sizes: Sequence[int], ranks: int, shard_buffers: Sequence[np.ndarray],
                  live: Sequence[int]) -> np.ndarray:
    """The gathered working set: for each live tensor, in the order given, a
    separate full buffer of ranks * ceil(n / ranks) elements holding the
    ranks' shards in rank order (the tensor is its first n elements)."""
    shards = [-(-n // ranks) for n in layer_sizes]
    starts = [sum(shards[:k]) for k in range(len(shards))]
    parts = []
    for k in live:
        for r in range(ranks):
            parts.append(shard_buffers[r][starts[k]:starts[k] + shards[k]])
    return np.concatenate(parts) if parts else np.zeros(0, dtype=shard_buffers[0].dtype)


# ---------------------------------------------------------------------------
# Flattened, padded parameter buffer (reading: the pages leave padding open).
# ---------------------------------------------------------------------------
def layout(numels: Sequence[int], ranks: int, align: int):
    """Tensor offsets, padded total and owner ranges of the flat buffer.

    Reading of the pages (which apply the floor ownership formula to an
    unpadded count and say the lab does not simulate padding): every tensor,
    the last included, is padded up to a multiple of ``align`` elements;
    tensor k starts at the sum of the padded sizes before it; ownership is the
    floor formula applied to the padded total.  Returns
    ``(offsets, padded_total, [(begin, end) per owner])``.
    """
    if ranks <= 0 or align <= 0 or not numels or any(n <= 0 for n in numels):
        raise ValueError("sizes, ranks and alignment must be positive")
    offsets, total = [], 0
    for n in numels:
        offsets.append(total)
        total += -(-n // align) * align
    owners = [(r.start, r.stop) for r in owner_ranges(total, ranks)] if total else []
    return offsets, total, owners


def real_ranges(numels: Sequence[int], offsets: Sequence[int], begin: int, end: int):
    """The owner's real (non-padding) elements: ``[off_k, off_k+n_k) ∩ [begin, end)``."""
    out = []
    for n, off in zip(numels, offsets):
        b, e = max(begin, off), min(end, off + n)
        if b < e:
            out.append((b, e))
    return out


def dense_offsets(numels: Sequence[int]) -> List[int]:
    """Start of each tensor in the dense (unpadded) concatenation of all tensors:
    the layout an exported fp32 checkpoint uses ([Deep dive] "Resume training
    and export weights separately": export consolidates the weights, padding
    dropped)."""
    out, pos = [], 0
    for n in numels:
        out.append(pos)
        pos += n
    return out


def consolidate(numels: Sequence[int], offsets: Sequence[int], owners, arrays, bases) -> np.ndarray:
    """Dense fp32 weights from the owners' shards (export of a sharded checkpoint).

    [Deep dive] "Resume training and export weights separately": exporting a
    model consolidates the fp32 weights.  Tensor k's element j is flat index
    ``offsets[k] + j``; it is read from the one owner whose range holds it,
    at ``arrays[r][f - bases[r]]``.  Padding is dropped.  Plain loops.
    """
    out = np.empty(sum(numels), dtype=np.float32)
    pos = 0
    for n, off in zip(numels, offsets):
        for j in range(n):
            f = off + j
            r = next(r for r, (b, e) in enumerate(owners) if b <= f < e)
            out[pos] = arrays[r][f - bases[r]]
            pos += 1
    return out


def distribute(numels: Sequence[int], offsets: Sequence[int], begin: int, end: int, dense: np.ndarray,
               out: np.ndarray, base: int) -> np.ndarray:
    """The inverse for one owner: write its real elements from dense weights into
    ``out[f - base]``; padding and other elements of ``out`` are left as they are."""
    dpos = 0
    for n, off in zip(numels, offsets):
        for j in range(n):
            f = off + j
            if begin <= f < end:
                out[f - base] = dense[dpos + j]
        dpos += n
    return out


def clip_coef(sumsq: float, max_norm: float = 1.0, eps: float = 1e-6) -> float:
    """Global-norm clip factor ``min(1, max_norm / (sqrt(sumsq) + eps))``.

    Reading: the pages name no clipping rule; this is the common
    ``clip_grad_norm_`` convention (eps 1e-6, clamp at 1).
    """
    return min(1.0, max_norm / (math.sqrt(sumsq) + eps))


# ---------------------------------------------------------------------------
# Scalar C half.
# ---------------------------------------------------------------------------
class Hyper(ct.Structure):
    _fields_ = [("lr", ct.c_double), ("beta1", ct.c_double), ("beta2", ct.c_double),
                ("eps", ct.c_double), ("weight_decay", ct.c_double), ("adamw", ct.c_int32),
                ("step", ct.c_uint64), ("clip_coef", ct.c_double)]


def hyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, adamw=True, step=1,
          clip_coef=1.0) -> Hyper:
    if step < 1:
        raise ValueError("Adam steps count from 1")
    return Hyper(lr, beta1, beta2, eps, weight_decay, 1 if adamw else 0, step, clip_coef)


GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
             "-shared", "-Wall"]


def build(src: str = None, out: str = None) -> str:
    """Compile zero_oracle.c with gcc into liboracle.so (no fast-math, no FMA contraction)."""
    src = src or os.path.join(_HERE, "zero_oracle.c")
    out = out or LIB_PATH
    tmp = out + ".tmp"
    cmd = ["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building the oracle failed:\n" + res.stderr)
    os.replace(tmp, out)
    return out


_lib = None


def load(path: str):
    """Open a build of zero_oracle.c and declare its signatures."""
    L = ct.CDLL(path)
    P, U64, F, D, I = ct.c_void_p, ct.c_uint64, ct.c_float, ct.c_double, ct.c_int
    L.oracle_f32_to_f16.restype = ct.c_uint16
    L.oracle_f32_to_f16.argtypes = [F]
    L.oracle_f32_to_bf16.restype = ct.c_uint16
    L.oracle_f32_to_bf16.argtypes = [F]
    L.oracle_f16_value.restype = D
    L.oracle_f16_value.argtypes = [ct.c_uint16]
    L.oracle_bf16_value.restype = D
    L.oracle_bf16_value.argtypes = [ct.c_uint16]
    L.oracle_encode16.argtypes = [P, U64, I, P]
    L.oracle_reduce.argtypes = [ct.c_uint32, I, P, U64, F, I, P]
    L.oracle_reduce_add.argtypes = [ct.c_uint32, I, P, U64, F, P]
    L.oracle_accumulate.argtypes = [I, P, U64, I, P]
    L.oracle_grad_check.argtypes = [P, U64, P, P]
    L.oracle_clip_coef.restype = D
    L.oracle_clip_coef.argtypes = [D, D, D]
    L.oracle_adam_f64.argtypes = [U64, P, P, P, P, ct.POINTER(Hyper)]
    L.oracle_adam_f32.argtypes = [U64, P, P, P, P, ct.POINTER(Hyper)]
    L.oracle_owner_step.argtypes = [ct.c_uint32, I, P, U64, P, F, U64, P, P, P, P, P, U64, P,
                                    I, U64, ct.POINTER(Hyper)]
    L.oracle_num_threads.restype = I
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = load(LIB_PATH)
    return _lib


def _ptr(a: np.ndarray):
    return ct.c_void_p(a.ctypes.data)


def _storage(a: np.ndarray, dtype: int) -> np.ndarray:
    want = np.float32 if dtype == F32 else np.uint16
    if a.dtype != want or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"expected contiguous {want.__name__} storage for dtype {dtype}")
    return a


def _ptr_array(bufs: Sequence[np.ndarray]):
    arr = (ct.c_void_p * max(1, len(bufs)))()
    for r, b in enumerate(bufs):
        arr[r] = b.ctypes.data
    return arr


def encode16(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round fp32 values to fp16/bf16 bit patterns (nearest, ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_encode16(_ptr(x), x.size, dtype, _ptr(out))
    return out


def decode16(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Exact fp64 values of fp16/bf16 bit patterns."""
    f = lib().oracle_f16_value if dtype == F16 else lib().oracle_bf16_value
    return np.array([f(int(b)) for b in np.asarray(bits).ravel()], dtype=np.float64).reshape(
        np.shape(bits))


def reduce(grads: Sequence[np.ndarray], dtype: int, divisor: float, out: np.ndarray = None,
           accumulate: bool = False) -> np.ndarray:
    """fp32 rank reduce: ``(start + g_0 + ... + g_{R-1}) / divisor`` in rank order."""
    n = grads[0].size
    for g in grads:
        _storage(g, dtype)
        if g.size != n:
            raise ValueError("rank buffers differ in length")
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing output")
        out = np.empty(n, dtype=np.float32)
    lib().oracle_reduce(len(grads), dtype, _ptr_array(grads), n, divisor, int(accumulate),
                        _ptr(out))
    return out


def reduce_add(grads: Sequence[np.ndarray], dtype: int, divisor: float, out: np.ndarray) -> np.ndarray:
    """Per-backward reduce-and-accumulate: ``out += (g_0 + ... + g_{R-1}) / divisor``,
    the reduced value rounded to fp32 before the fp32 add."""
    n = grads[0].size
    for g in grads:
        _storage(g, dtype)
        if g.size != n:
            raise ValueError("rank buffers differ in length")
    _storage(out, F32)
    if out.size != n:
        raise ValueError("accumulator and rank buffers differ in length")
    lib().oracle_reduce_add(len(grads), dtype, _ptr_array(grads), n, divisor, _ptr(out))
    return out


def accumulate(g: np.ndarray, dtype: int, acc: np.ndarray, first: bool) -> np.ndarray:
    _storage(g, dtype)
    lib().oracle_accumulate(dtype, _ptr(g), g.size, int(first), _ptr(acc))
    return acc


def grad_check(g: np.ndarray) -> Tuple[int, float]:
    """(overflow flag, squared norm in fp64) of an fp32 gradient."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    flag = np.zeros(1, dtype=np.int32)
    s = np.zeros(1, dtype=np.float64)
    lib().oracle_grad_check(_ptr(g), g.size, _ptr(flag), _ptr(s))
    return int(flag[0]), float(s[0])


def adam_f64(g, w, m, v, h: Hyper):
    """fp64 state update in place (the pages' arithmetic, vectorised over elements)."""
    for a in (g, w, m, v):
        if a.dtype != np.float64 or not a.flags["C_CONTIGUOUS"]:
            raise TypeError("adam_f64 needs contiguous float64 arrays")
    lib().oracle_adam_f64(g.size, _ptr(g), _ptr(w), _ptr(m), _ptr(v), ct.byref(h))


def adam_f32(g, w, m, v, h: Hyper):
    """fp32 stored state, fp64 arithmetic, rounded once on store; in place."""
    for a in (g, w, m, v):
        if a.dtype != np.float32 or not a.flags["C_CONTIGUOUS"]:
            raise TypeError("adam_f32 needs contiguous float32 arrays")
    lib().oracle_adam_f32(g.size, _ptr(g), _ptr(w), _ptr(m), _ptr(v), ct.byref(h))


def owner_step(ranges: Sequence[Tuple[int, int]], h: Hyper, w: np.ndarray, m: np.ndarray,
               v: np.ndarray, local_base: int, *, grads: Sequence[np.ndarray] = (),
               gdtype: int = F32, grad_base: int = 0, divisor: float = 1.0,
               reduced_g: np.ndarray = None, p16: np.ndarray = None, pdtype: int = 0,
               param_base: int = 0) -> None:
    """The owner step over its real elements, in place.

    Flat index f reads ``grads[r][f - grad_base]`` (or ``reduced_g[f - local_base]``),
    updates ``w/m/v[f - local_base]`` and writes ``p16[f - param_base]``.
    """
    for a in (w, m, v):
        _storage(a, F32)
    for g in grads:
        _storage(g, gdtype)
    rb = np.array([b for b, _ in ranges], dtype=np.uint64)
    re_ = np.array([e for _, e in ranges], dtype=np.uint64)
    for b, e in ranges:
        if b < local_base or e - local_base > w.size:
            raise IndexError("range outside the owner-local arrays")
        if reduced_g is None and (b < grad_base or any(e - grad_base > g.size for g in grads)):
            raise IndexError("range outside the rank buffers")
        if p16 is not None and pdtype and (b < param_base or e - param_base > p16.size):
            raise IndexError("range outside the 16-bit buffer")
    if reduced_g is not None:
        _storage(reduced_g, F32)
    lib().oracle_owner_step(
        len(grads), gdtype, _ptr_array(grads), grad_base,
        _ptr(reduced_g) if reduced_g is not None else None, divisor, len(ranges),
        _ptr(rb) if len(ranges) else None, _ptr(re_) if len(ranges) else None,
        _ptr(w), _ptr(m), _ptr(v), local_base,
        _ptr(p16) if p16 is not None else None, pdtype if p16 is not None else 0, param_base,
        ct.byref(h))


def num_threads() -> int:
    return lib().oracle_num_threads()
