"""ZeRO owner-shard optimizer step on one MI355X: Python binding of libzero_shard.so.

Argument marshalling only.  Every step of the path runs in the HIP library
(``csrc/step.hip``, ``csrc/copy.hip``, ``csrc/launch.hip``, ``csrc/host.cpp``; C ABI in
``include/zero_shard.h``);
this module turns torch tensors into pointers, checks devices, dtypes,
contiguity and extents against what the kernels will touch, passes torch's
current stream, and raises on error codes.  There is no fallback: if the
library is missing, every call raises.

The functions carry the names of the C entry points.  ``OwnerShard`` bundles
one owner's layout, device chunk table and fp32 state for convenience; its
methods are sequences of the same calls.
"""
from __future__ import annotations

import ctypes as ct
import os
from fractions import Fraction
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .build import LIB_PATH, build

ZERO_OK, ZERO_EINVAL, ZERO_ERANGE, ZERO_EHIP = 0, -1, -2, -3
ZERO_NONE, ZERO_F16, ZERO_BF16, ZERO_F32 = 0, 1, 2, 3
ZERO_MAX_RANKS = 256

EXPORTED = ("zero_last_error", "zero_shard_layout", "zero_chunk_table", "zero_dense_offsets", "zero_state_bytes",
            "zero_reduce_owned", "zero_grad_check", "zero_clip_coef", "zero_step_decision", "zero_adam_step",
            "zero_owner_to_dense", "zero_dense_to_owner", "zero3_storage", "zero3_gather_spans",
            "zero3_partition_spans", "zero_copy_spans", "zero_stream_probe",
            "zero_check_workspace_bytes", "zero_chunk_groups", "zero_span_groups", "zero_reduce_owned_noalloc")

CHUNK_DTYPE = np.dtype([("flat", "<u8"), ("len", "<u4"), ("tensor", "<u4")])
SPAN_DTYPE = np.dtype([("src", "<u8"), ("dst", "<u8"), ("len", "<u4"), ("buf", "<u4")])
ZERO_MAX_COPY_SOURCES = 128
ZERO_MAX_PROBE_STREAMS = 64


class ZeroShardError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class AdamArgs(ct.Structure):
    _fields_ = [
        ("chunks", ct.c_void_p), ("n_chunks", ct.c_uint64), ("groups", ct.c_void_p),
        ("n_groups", ct.c_uint64), ("begin", ct.c_uint64),
        ("end", ct.c_uint64),
        ("rank_grads", ct.c_void_p), ("R", ct.c_uint32), ("grad_dtype", ct.c_int32),
        ("grad_base", ct.c_uint64), ("divisor", ct.c_float), ("reduced_g", ct.c_void_p),
        ("master", ct.c_void_p), ("exp_avg", ct.c_void_p), ("exp_avg_sq", ct.c_void_p),
        ("local_base", ct.c_uint64),
        ("param16", ct.c_void_p), ("param_dtype", ct.c_int32), ("param_base", ct.c_uint64),
        ("lr", ct.c_double), ("beta1", ct.c_double), ("beta2", ct.c_double), ("eps", ct.c_double),
        ("weight_decay", ct.c_double), ("adamw", ct.c_int32), ("step", ct.c_uint64),
        ("clip_coef", ct.c_double), ("grid_blocks", ct.c_uint32),
    ]


class Ratio(ct.Structure):
    _fields_ = [("num", ct.c_uint64), ("den", ct.c_uint64)]


_lib = None


def load(path: str):
    """Open a build of libzero_shard and declare its signatures."""
    L = ct.CDLL(path)
    P, U32, U64, I, F, D = ct.c_void_p, ct.c_uint32, ct.c_uint64, ct.c_int, ct.c_float, ct.c_double
    L.zero_last_error.restype = ct.c_char_p
    L.zero_last_error.argtypes = []
    for name in EXPORTED[1:]:
        getattr(L, name).restype = I
    L.zero_shard_layout.argtypes = [P, U32, U32, U32, P, P, P, P]
    L.zero_chunk_table.argtypes = [P, P, U32, U64, U64, U32, P, U64, P]
    L.zero_dense_offsets.argtypes = [P, U32, P, P]
    L.zero_state_bytes.argtypes = [U64, U64, U32, U32, U32, P]
    L.zero_reduce_owned.argtypes = [P, U32, I, U64, U64, U64, F, I, P, U64, P, P, P, ct.c_size_t, P]
    L.zero_reduce_owned_noalloc.argtypes = [P, U32, I, U64, U64, U64, F, I, P, U64, P, P, P]
    L.zero_grad_check.argtypes = [P, U64, P, P, P, ct.c_size_t, P]
    L.zero_clip_coef.argtypes = [D, D, D, ct.POINTER(F)]
    L.zero_step_decision.argtypes = [P, P, U32, D, D, ct.POINTER(ct.c_int32), ct.POINTER(F)]
    L.zero_adam_step.argtypes = [ct.POINTER(AdamArgs), P]
    L.zero_owner_to_dense.argtypes = [P, U64, P, U64, U64, U64, P, P, U32, P, U64, P, U64, P]
    L.zero_dense_to_owner.argtypes = [P, U64, P, U64, U64, U64, P, P, U32, P, U64, P, U64, P]
    L.zero3_storage.argtypes = [P, U32, U32, P, U32, P, P, P]
    L.zero3_gather_spans.argtypes = [P, U32, U32, P, U32, U32, P, U64, P]
    L.zero3_partition_spans.argtypes = [P, U32, U32, U32, U32, P, U64, P]
    L.zero_copy_spans.argtypes = [P, U64, P, P, U32, P, U64, U32, P, U64, P]
    L.zero_span_groups.argtypes = [P, U64, U32, U32, P, U64, P]
    L.zero_stream_probe.argtypes = [P, P, U32, P, P, U32, U64, I, P]
    L.zero_check_workspace_bytes.argtypes = [U64, P]
    L.zero_chunk_groups.argtypes = [P, U64, U32, P, U64, P]
    return L


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "(there is no fallback path)")
        _lib = load(LIB_PATH)
    return _lib


def _check(rc: int) -> None:
    if rc != ZERO_OK:
        raise ZeroShardError(rc, lib().zero_last_error().decode())


def _u64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint64))


def _p(a: np.ndarray):
    return ct.c_void_p(a.ctypes.data) if a is not None and a.size else None


# ---------------------------------------------------------------- host calls
def zero_shard_layout(numels: Sequence[int], ranks: int, align: int):
    """(tensor offsets, padded total, owner begins, owner ends) of the flat buffer."""
    n = _u64(numels)
    off = np.zeros(max(1, n.size), dtype=np.uint64)
    total = np.zeros(1, dtype=np.uint64)
    b = np.zeros(max(1, ranks), dtype=np.uint64)
    e = np.zeros(max(1, ranks), dtype=np.uint64)
    _check(lib().zero_shard_layout(_p(n), n.size, ranks, align, _p(off), _p(total), _p(b), _p(e)))
    return off[: n.size], int(total[0]), b[:ranks], e[:ranks]


def zero_chunk_table(numels: Sequence[int], offsets: Sequence[int], begin: int, end: int,
                     max_chunk: int) -> np.ndarray:
    """The owner's chunks as a structured array (flat, len, tensor)."""
    n, off = _u64(numels), _u64(offsets)
    if n.size != off.size:
        raise ValueError("numels and offsets differ in length")
    count = np.zeros(1, dtype=np.uint64)
    _check(lib().zero_chunk_table(_p(n), _p(off), n.size, begin, end, max_chunk, None, 0, _p(count)))
    out = np.zeros(int(count[0]), dtype=CHUNK_DTYPE)
    _check(lib().zero_chunk_table(_p(n), _p(off), n.size, begin, end, max_chunk,
                                  _p(out) if out.size else None, out.size, _p(count)))
    return out


def zero_dense_offsets(numels: Sequence[int]):
    """(start of each tensor in the dense unpadded layout, dense total)."""
    n = _u64(numels)
    off = np.zeros(max(1, n.size), dtype=np.uint64)
    total = np.zeros(1, dtype=np.uint64)
    _check(lib().zero_dense_offsets(_p(n), n.size, _p(off), _p(total)))
    return off[: n.size], int(total[0])


def groups_pay(n_groups: int, n_items: int) -> bool:
    """Whether a group table is worth its indirection: a group kernel block
    first reads its group bounds, then its chunks or spans, and that extra
    dependent load cost 17% on a span copy of long spans.  Packing pays when
    it at least halves the block count (512-element spans: +84%)."""
    return 2 * n_groups <= n_items


def zero_chunk_groups(chunks: np.ndarray, max_group: int) -> np.ndarray:
    """Group table (first chunk of each group, then len(chunks)) packing runs of
    short chunks for zero_adam_step; uint64, n_groups + 1 entries."""
    ch = np.ascontiguousarray(chunks, dtype=CHUNK_DTYPE)
    count = np.zeros(1, dtype=np.uint64)
    _check(lib().zero_chunk_groups(_p(ch), ch.size, max_group, None, 0, _p(count)))
    out = np.zeros(int(count[0]) + 1, dtype=np.uint64)
    _check(lib().zero_chunk_groups(_p(ch), ch.size, max_group, _p(out), out.size, _p(count)))
    return out


def zero_state_bytes(params: int, ranks: int, param: int = 2, grad: int = 2,
                     optimizer: int = 12) -> dict:
    out = (Ratio * 4)()
    _check(lib().zero_state_bytes(params, ranks, param, grad, optimizer, out))
    names = ("DP", "ZeRO-1", "ZeRO-2", "ZeRO-3")
    return {k: Fraction(out[i].num, out[i].den) for i, k in enumerate(names)}


def zero_clip_coef(sumsq: float, max_norm: float = 1.0, eps: float = 1e-6) -> float:
    c = ct.c_float()
    _check(lib().zero_clip_coef(sumsq, max_norm, eps, ct.byref(c)))
    return c.value


def zero_step_decision(overflow: Sequence[int], sumsq: Sequence[float], max_norm: float = 1.0,
                       eps: float = 1e-6):
    """(update, clip factor) from every owner's (flag, squared-norm partial), in
    owner order; the factor is None when the step is skipped."""
    fl = np.ascontiguousarray(np.asarray(overflow, dtype=np.int32))
    ss = np.ascontiguousarray(np.asarray(sumsq, dtype=np.float64))
    if fl.size != ss.size:
        raise ValueError("one flag and one partial per owner")
    up, c = ct.c_int32(), ct.c_float()
    _check(lib().zero_step_decision(_p(fl), _p(ss), fl.size, max_norm, eps, ct.byref(up), ct.byref(c)))
    return (True, c.value) if up.value else (False, None)


# ---------------------------------------------------------------- device calls
def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    return {torch.float16: ZERO_F16, torch.bfloat16: ZERO_BF16, torch.float32: ZERO_F32}[t.dtype]


def _dev(t, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.device.index != _torch().cuda.current_device():
        # the kernels run on the current device's stream
        raise ValueError(f"{name} lives on {t.device}, not on the current device "
                         f"cuda:{_torch().cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _stream():
    return ct.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _need(t, name: str, elems: int) -> None:
    if t.numel() < elems:
        raise ValueError(f"{name} holds {t.numel()} elements, {elems} needed")


def _rank_ptrs(rank_grads, base: int, last: int, name="rank_grads"):
    if not rank_grads:
        raise ValueError("no rank buffers")
    dt = rank_grads[0].dtype
    dev = rank_grads[0].device
    arr = (ct.c_void_p * len(rank_grads))()
    for r, g in enumerate(rank_grads):
        _dev(g, f"{name}[{r}]", dt)
        if g.device != dev:
            raise ValueError("rank buffers on different devices")
        _need(g, f"{name}[{r}]", last - base)
        arr[r] = g.data_ptr()
    return arr, _dtype_code(rank_grads[0])


def zero_reduce_owned(rank_grads, begin: int, n: int, divisor: float, out, *, grad_base: int = 0,
                      out_base: int = 0, accumulate: int = 0, check=None) -> None:
    """Rank reduce over flat indices [begin, begin+n) into ``out[f - out_base]``.

    ``accumulate``: 0 ``out = sum/D``; 1 (or True) ``out = (out + sum)/D``;
    2 ``out = out + sum/D`` (per-backward reduce-and-accumulate).

    ``check`` = (overflow int32[1], sumsq float64[1], workspace uint8[>= check_workspace_bytes(n)])
    device tensors to also compute the overflow flag and squared norm in the same pass.
    """
    torch = _torch()
    arr, code = _rank_ptrs(rank_grads, grad_base, begin + n)
    _dev(out, "out", torch.float32)
    _need(out, "out", begin + n - out_base)
    ov = ss = ws = None
    ws_bytes = 0
    if check is not None:
        ov, ss, ws = check
        _dev(ov, "overflow", torch.int32)
        _dev(ss, "sumsq", torch.float64)
        _dev(ws, "workspace")
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().zero_reduce_owned(
        arr, len(rank_grads), code, grad_base, begin, n, divisor, int(accumulate),
        ct.c_void_p(out.data_ptr()), out_base,
        ct.c_void_p(ov.data_ptr()) if ov is not None else None,
        ct.c_void_p(ss.data_ptr()) if ss is not None else None,
        ct.c_void_p(ws.data_ptr()) if ws is not None else None, ws_bytes, _stream()))


def zero_reduce_owned_noalloc(rank_grads, begin: int, n: int, divisor: float, out, *, grad_base: int = 0,
                              out_base: int = 0, accumulate: int = 0, check=None) -> None:
    """``zero_reduce_owned`` whose check needs no workspace: ``check`` = (overflow
    int32[1], sumsq float64[1]); the partials go to the library's own device
    array (calls on one GPU must not overlap)."""
    torch = _torch()
    arr, code = _rank_ptrs(rank_grads, grad_base, begin + n)
    _dev(out, "out", torch.float32)
    _need(out, "out", begin + n - out_base)
    ov = ss = None
    if check is not None:
        ov, ss = check
        _dev(ov, "overflow", torch.int32)
        _dev(ss, "sumsq", torch.float64)
    _check(lib().zero_reduce_owned_noalloc(
        arr, len(rank_grads), code, grad_base, begin, n, divisor, int(accumulate),
        ct.c_void_p(out.data_ptr()), out_base,
        ct.c_void_p(ov.data_ptr()) if ov is not None else None,
        ct.c_void_p(ss.data_ptr()) if ss is not None else None, _stream()))


def zero_grad_check(g, overflow, sumsq, workspace) -> None:
    torch = _torch()
    _dev(g, "g", torch.float32)
    _dev(overflow, "overflow", torch.int32)
    _dev(sumsq, "sumsq", torch.float64)
    _dev(workspace, "workspace")
    _check(lib().zero_grad_check(
        ct.c_void_p(g.data_ptr()), g.numel(), ct.c_void_p(overflow.data_ptr()),
        ct.c_void_p(sumsq.data_ptr()), ct.c_void_p(workspace.data_ptr()),
        workspace.numel() * workspace.element_size(), _stream()))


def check_workspace_bytes(n: int) -> int:
    """Bytes of device workspace a check over n elements needs."""
    out = np.zeros(1, dtype=np.uint64)
    _check(lib().zero_check_workspace_bytes(n, _p(out)))
    return int(out[0])


def check_workspace(n: int, device=None):
    """A device buffer for the overflow / norm reduction over n elements."""
    torch = _torch()
    return torch.empty(check_workspace_bytes(n), dtype=torch.uint8, device=device or "cuda")


def chunks_to_device(chunks: np.ndarray, device=None):
    torch = _torch()
    flat = np.ascontiguousarray(chunks).view(np.uint8)
    t = torch.from_numpy(flat.copy()).to(device or "cuda")
    return t


def zero_adam_step(*, chunks_dev, n_chunks: int, begin: int, end: int, master, exp_avg, exp_avg_sq,
                   local_base: int, step: int, lr: float, beta1: float, beta2: float, eps: float,
                   weight_decay: float = 0.0, adamw: bool = True, rank_grads=None, grad_base: int = 0,
                   divisor: float = 1.0, reduced_g=None, param16=None, param_base: int = 0,
                   clip_coef: float = 1.0, grid_blocks: int = 0, groups_dev=None, n_groups: int = 0) -> None:
    """Fused reduce + Adam/AdamW + 16-bit write-back over a device chunk table
    (optionally packed by a device group table from ``zero_chunk_groups``).

    The kernel touches only flat indices in [begin, end) (chunk pieces outside are
    ignored), so every buffer is checked to hold those.
    """
    torch = _torch()
    last = end
    if chunks_dev is not None:
        _dev(chunks_dev, "chunks")
        if chunks_dev.numel() * chunks_dev.element_size() < n_chunks * CHUNK_DTYPE.itemsize:
            raise ValueError("chunk table smaller than n_chunks")
    for name, t in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        _dev(t, name, torch.float32)
        _need(t, name, last - local_base)
    a = AdamArgs()
    a.chunks = chunks_dev.data_ptr() if chunks_dev is not None else None
    a.n_chunks, a.begin, a.end = n_chunks, begin, end
    if groups_dev is not None:
        _dev(groups_dev, "groups", torch.int64)
        if groups_dev.numel() < n_groups + 1:
            raise ValueError("group table smaller than n_groups + 1")
        a.groups, a.n_groups = groups_dev.data_ptr(), n_groups
    elif n_groups:
        raise ValueError("n_groups given without a group table")
    keep = None
    if reduced_g is not None:
        _dev(reduced_g, "reduced_g", torch.float32)
        _need(reduced_g, "reduced_g", last - local_base)
        a.reduced_g = reduced_g.data_ptr()
    else:
        keep, code = _rank_ptrs(rank_grads, grad_base, last)
        a.rank_grads = ct.cast(keep, ct.c_void_p)
        a.R, a.grad_dtype, a.grad_base = len(rank_grads), code, grad_base
    a.divisor = divisor
    a.master, a.exp_avg, a.exp_avg_sq = master.data_ptr(), exp_avg.data_ptr(), exp_avg_sq.data_ptr()
    a.local_base = local_base
    if param16 is not None:
        _dev(param16, "param16")
        if param16.dtype not in (torch.float16, torch.bfloat16):
            raise TypeError("param16 must be float16 or bfloat16")
        _need(param16, "param16", last - param_base)
        a.param16, a.param_dtype, a.param_base = param16.data_ptr(), _dtype_code(param16), param_base
    a.lr, a.beta1, a.beta2, a.eps, a.weight_decay = lr, beta1, beta2, eps, weight_decay
    a.adamw, a.step, a.clip_coef, a.grid_blocks = int(adamw), step, clip_coef, grid_blocks
    _check(lib().zero_adam_step(ct.byref(a), _stream()))
    del keep


def _group_ptr(groups_dev, n_groups):
    if groups_dev is None:
        if n_groups:
            raise ValueError("n_groups given without a group table")
        return None, 0
    _dev(groups_dev, "groups", _torch().int64)
    if groups_dev.numel() < n_groups + 1:
        raise ValueError("group table smaller than n_groups + 1")
    return ct.c_void_p(groups_dev.data_ptr()), n_groups


def _dense_call(name, chunks_dev, n_chunks, begin, end, tensor_offset_dev, dense_offset_dev, owner,
                owner_base, dense, groups_dev=None, n_groups=0):
    torch = _torch()
    _dev(owner, "owner", torch.float32)
    _dev(dense, "dense", torch.float32)
    _dev(tensor_offset_dev, "tensor_offset", torch.int64)
    _dev(dense_offset_dev, "dense_offset", torch.int64)
    if tensor_offset_dev.numel() != dense_offset_dev.numel():
        raise ValueError("tensor and dense offset tables differ in length")
    _need(owner, "owner", end - owner_base)
    if chunks_dev is not None and chunks_dev.numel() * chunks_dev.element_size() < n_chunks * CHUNK_DTYPE.itemsize:
        raise ValueError("chunk table smaller than n_chunks")
    L = lib()
    gptr, ng = _group_ptr(groups_dev, n_groups)
    common = (ct.c_void_p(chunks_dev.data_ptr()) if chunks_dev is not None else None, n_chunks, gptr, ng,
              begin, end, ct.c_void_p(tensor_offset_dev.data_ptr()), ct.c_void_p(dense_offset_dev.data_ptr()),
              tensor_offset_dev.numel())
    if name == "zero_owner_to_dense":
        _check(L.zero_owner_to_dense(*common, ct.c_void_p(owner.data_ptr()), owner_base,
                                     ct.c_void_p(dense.data_ptr()), dense.numel(), _stream()))
    else:
        _check(L.zero_dense_to_owner(*common, ct.c_void_p(dense.data_ptr()), dense.numel(),
                                     ct.c_void_p(owner.data_ptr()), owner_base, _stream()))


def zero_owner_to_dense(chunks_dev, n_chunks, begin, end, tensor_offset_dev, dense_offset_dev, owner,
                        owner_base, dense, groups_dev=None, n_groups: int = 0) -> None:
    """dense[dense_offset[k] + f - tensor_offset[k]] = owner[f - owner_base] for the owner's real f."""
    _dense_call("zero_owner_to_dense", chunks_dev, n_chunks, begin, end, tensor_offset_dev,
                dense_offset_dev, owner, owner_base, dense, groups_dev, n_groups)


def zero_dense_to_owner(chunks_dev, n_chunks, begin, end, tensor_offset_dev, dense_offset_dev, dense,
                        owner, owner_base, groups_dev=None, n_groups: int = 0) -> None:
    """owner[f - owner_base] = dense[dense_offset[k] + f - tensor_offset[k]] for the owner's real f."""
    _dense_call("zero_dense_to_owner", chunks_dev, n_chunks, begin, end, tensor_offset_dev,
                dense_offset_dev, owner, owner_base, dense, groups_dev, n_groups)


# ---------------------------------------------------------------- ZeRO-3 partition / gather
def _live(live):
    return np.ascontiguousarray(np.asarray(list(live), dtype=np.uint32))


def zero3_storage(numels: Sequence[int], ranks: int, live: Sequence[int] = ()):
    """(shard sizes, resident, gathered) element counts of per-tensor ZeRO-3 partitioning."""
    n, lv = _u64(numels), _live(live)
    shard = np.zeros(max(1, n.size), dtype=np.uint64)
    res, gat = np.zeros(1, dtype=np.uint64), np.zeros(1, dtype=np.uint64)
    _check(lib().zero3_storage(_p(n), n.size, ranks, _p(lv), lv.size, _p(shard), _p(res), _p(gat)))
    return shard[: n.size], int(res[0]), int(gat[0])


# Span length of the copy tables: one block copies one span, and 4096 elements
# (8 KiB of bf16 each way) measured fastest for the stage-3 gather (2048: -8%,
# 8192: -5%).
DEFAULT_SPAN = 4096


def _spans(fn, *args, max_span):
    count = np.zeros(1, dtype=np.uint64)
    _check(fn(*args, max_span, None, 0, _p(count)))
    out = np.zeros(int(count[0]), dtype=SPAN_DTYPE)
    _check(fn(*args, max_span, _p(out) if out.size else None, out.size, _p(count)))
    return out


def zero3_gather_spans(numels, ranks: int, live, max_span: int = DEFAULT_SPAN) -> np.ndarray:
    n, lv = _u64(numels), _live(live)
    return _spans(lib().zero3_gather_spans, _p(n), n.size, ranks, _p(lv), lv.size, max_span=max_span)


def zero3_partition_spans(numels, ranks: int, rank: int, max_span: int = DEFAULT_SPAN) -> np.ndarray:
    n = _u64(numels)
    return _spans(lib().zero3_partition_spans, _p(n), n.size, ranks, rank, max_span=max_span)


def spans_to_device(spans: np.ndarray, device=None):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(spans).view(np.uint8).copy()).to(device or "cuda")


def zero_span_groups(spans: np.ndarray, elem_bytes: int, max_group: int = DEFAULT_SPAN) -> np.ndarray:
    """Group table (first span of each group, then len(spans)) packing runs of
    short spans for zero_copy_spans; uint64, n_groups + 1 entries."""
    sp = np.ascontiguousarray(spans, dtype=SPAN_DTYPE)
    count = np.zeros(1, dtype=np.uint64)
    _check(lib().zero_span_groups(_p(sp), sp.size, elem_bytes, max_group, None, 0, _p(count)))
    out = np.zeros(int(count[0]) + 1, dtype=np.uint64)
    _check(lib().zero_span_groups(_p(sp), sp.size, elem_bytes, max_group, _p(out), out.size, _p(count)))
    return out


def zero_copy_spans(spans_dev, n_spans: int, srcs, dst, groups_dev=None, n_groups: int = 0) -> None:
    """dst[span.dst + i] = srcs[span.buf][span.src + i] over a device span table
    (optionally packed by a device group table from ``zero_span_groups``)."""
    torch = _torch()
    if not srcs or len(srcs) > ZERO_MAX_COPY_SOURCES:
        raise ValueError(f"between 1 and {ZERO_MAX_COPY_SOURCES} source buffers")
    _dev(dst, "dst")
    if dst.element_size() not in (2, 4):
        raise TypeError("elements must be 2 or 4 bytes")
    arr = (ct.c_void_p * len(srcs))()
    sizes = np.zeros(len(srcs), dtype=np.uint64)
    for i, t in enumerate(srcs):
        _dev(t, f"srcs[{i}]", dst.dtype)
        arr[i] = t.data_ptr()
        sizes[i] = t.numel()
    if spans_dev is not None:
        _dev(spans_dev, "spans")
        if spans_dev.numel() * spans_dev.element_size() < n_spans * SPAN_DTYPE.itemsize:
            raise ValueError("span table smaller than n_spans")
    gptr, ng = _group_ptr(groups_dev, n_groups)
    _check(lib().zero_copy_spans(ct.c_void_p(spans_dev.data_ptr()) if spans_dev is not None else None,
                                 n_spans, arr, _p(sizes), len(srcs), ct.c_void_p(dst.data_ptr()),
                                 dst.numel(), dst.element_size(), gptr, ng, _stream()))


def zero_stream_probe(srcs, dsts, order: int = 0, src_widths=None, dst_widths=None) -> None:
    """Bandwidth probe: every destination gets the bytewise XOR of all sources.

    A stream of width w (1 or 2; default 1) is touched w 16-byte vectors per
    thread, as the kernels stream 16-bit (w = 1) and fp32 (w = 2) data; every
    stream's byte size is its width times one common unit (a multiple of 16).
    No destinations: reads only; no sources: writes zeros.  ``order`` 0 deals
    the pieces to the XCDs in turn, 1 gives each XCD one contiguous run.
    """
    if len(srcs) > ZERO_MAX_PROBE_STREAMS or len(dsts) > ZERO_MAX_PROBE_STREAMS or not (srcs or dsts):
        raise ValueError(f"at most {ZERO_MAX_PROBE_STREAMS} sources and destinations, not none of both")
    sw = np.ascontiguousarray(np.asarray(src_widths if src_widths is not None else [1] * len(srcs), dtype=np.uint8))
    dw = np.ascontiguousarray(np.asarray(dst_widths if dst_widths is not None else [1] * len(dsts), dtype=np.uint8))
    if sw.size != len(srcs) or dw.size != len(dsts) or not np.all((sw == 1) | (sw == 2)) or \
            not np.all((dw == 1) | (dw == 2)):
        raise ValueError("one width of 1 or 2 per stream")
    streams = list(zip(srcs, sw.tolist())) + list(zip(dsts, dw.tolist()))
    first, w0 = streams[0]
    unit = first.numel() * first.element_size() // w0
    sa, da = (ct.c_void_p * max(1, len(srcs)))(), (ct.c_void_p * max(1, len(dsts)))()
    for arr, ts, ws, name in ((sa, srcs, sw, "srcs"), (da, dsts, dw, "dsts")):
        for i, t in enumerate(ts):
            _dev(t, f"{name}[{i}]")
            if t.numel() * t.element_size() != unit * int(ws[i]):
                raise ValueError("every probe stream must hold its width times one common unit of bytes")
            arr[i] = t.data_ptr()
    _check(lib().zero_stream_probe(sa, _p(sw), len(srcs), da, _p(dw), len(dsts), unit, int(order), _stream()))


# ---------------------------------------------------------------- convenience
class OwnerShard:
    """One owner's layout, device chunk table and fp32 master/moment state.

    Owner-local arrays start at ``local_base = begin & ~7`` and hold
    ``end - local_base`` elements, so their 128-bit vectors line up with the
    flat buffer's.
    """

    def __init__(self, numels: Sequence[int], ranks: int, owner: int, align: int = 64,
                 max_chunk: int = 2048, device=None):
        torch = _torch()
        self.numels = [int(x) for x in numels]
        self.offsets, self.padded_total, begins, ends = zero_shard_layout(self.numels, ranks, align)
        self.ranks, self.owner = ranks, owner
        self.begin, self.end = int(begins[owner]), int(ends[owner])
        self.local_base = self.begin & ~7
        self.local_size = self.end - self.local_base
        self.chunks = zero_chunk_table(self.numels, self.offsets, self.begin, self.end, max_chunk)
        self.device = torch.device(device or "cuda")
        self.chunks_dev = chunks_to_device(self.chunks, self.device)
        # short chunks packed several to a block, when that saves enough blocks
        self.groups = zero_chunk_groups(self.chunks, max_chunk)
        self.n_groups = self.groups.size - 1
        self.groups_dev = None
        if groups_pay(self.n_groups, self.chunks.size):
            self.groups_dev = torch.from_numpy(self.groups.astype(np.int64)).to(self.device)
        self.n_real = int(self.chunks["len"].sum()) if self.chunks.size else 0
        self.align = align
        self.dense_offsets, self.dense_total = zero_dense_offsets(self.numels)
        self.tensor_offset_dev = torch.from_numpy(self.offsets.astype(np.int64)).to(self.device)
        self.dense_offset_dev = torch.from_numpy(self.dense_offsets.astype(np.int64)).to(self.device)

    def _group_args(self) -> dict:
        if self.groups_dev is None:
            return {}
        return {"groups_dev": self.groups_dev, "n_groups": self.n_groups}

    def alloc_state(self):
        torch = _torch()
        mk = lambda: torch.zeros(max(8, self.local_size), dtype=torch.float32, device=self.device)
        self.master, self.exp_avg, self.exp_avg_sq = mk(), mk(), mk()
        return self.master, self.exp_avg, self.exp_avg_sq

    def adam_step(self, *, step: int, hyper: dict, rank_grads=None, grad_base: int = 0,
                  divisor: float = 1.0, reduced_g=None, param16=None, param_base: int = 0,
                  clip_coef: float = 1.0, grid_blocks: int = 0) -> None:
        zero_adam_step(chunks_dev=self.chunks_dev, n_chunks=self.chunks.size, begin=self.begin,
                       end=self.end, master=self.master, exp_avg=self.exp_avg,
                       exp_avg_sq=self.exp_avg_sq, local_base=self.local_base, step=step,
                       rank_grads=rank_grads, grad_base=grad_base, divisor=divisor,
                       reduced_g=reduced_g, param16=param16, param_base=param_base,
                       **self._group_args(),
                       clip_coef=clip_coef, grid_blocks=grid_blocks, **hyper)

    def check_buffers(self):
        """(owner-local fp32 gradient, overflow flag int32[1], squared norm
        float64[1], check workspace) used by ``checked_step``, allocated on first
        use and kept.  The flag and the norm share one 16-byte buffer, so one
        copy brings both to the host."""
        torch = _torch()
        if getattr(self, "_check_bufs", None) is None:
            g = torch.zeros(max(8, self.local_size), dtype=torch.float32, device=self.device)
            flag_norm = torch.zeros(16, dtype=torch.uint8, device=self.device)
            ws = check_workspace(max(1, self.end - self.begin), self.device)
            self._flag_norm = flag_norm
            self._check_bufs = (g, flag_norm[0:4].view(torch.int32), flag_norm[8:16].view(torch.float64), ws)
        return self._check_bufs

    def reduce_and_check(self, *, rank_grads, grad_base: int = 0, divisor: float = 1.0, events=None):
        """First half of the checked step: the rank reduce with the fused check into
        the owner-local fp32 gradient, then one 16-byte copy of (overflow flag,
        squared-norm partial) to the host.  Returns that pair for this owner;
        an empty owner returns (0, 0.0) without a launch.  The reduce runs over
        the owner's whole flat range, so the rank buffers hold zeros in the
        padding between tensors (no parameter lives there).  ``divisor`` folds
        in a static loss scale.  ``events``: optional (start, end) CUDA events
        recorded around the reduce launch."""
        if self.end == self.begin:
            return 0, 0.0
        g, ov, ss, ws = self.check_buffers()
        if events is not None:
            events[0].record()
        zero_reduce_owned(rank_grads, self.begin, self.end - self.begin, divisor, g,
                          grad_base=grad_base, out_base=self.local_base, check=(ov, ss, ws))
        if events is not None:
            events[1].record()
        host = self._flag_norm.cpu().numpy()  # waits for the reduce
        return int(host[0:4].view(np.int32)[0]), float(host[8:16].view(np.float64)[0])

    def apply_update(self, *, step: int, hyper: dict, coef: float, param16=None, param_base: int = 0,
                     grid_blocks: int = 0) -> None:
        """Second half: AdamW from the stored reduced gradient scaled by ``coef``
        (nothing to do for an empty owner)."""
        if self.end == self.begin:
            return
        g = self.check_buffers()[0]
        self.adam_step(step=step, hyper=hyper, reduced_g=g, param16=param16, param_base=param_base,
                       clip_coef=coef, grid_blocks=grid_blocks)

    def checked_step(self, *, step: int, hyper: dict, rank_grads, grad_base: int = 0, divisor: float = 1.0,
                     max_norm: float = 1.0, param16=None, param_base: int = 0, grid_blocks: int = 0,
                     events=None, exchange=None, apply_events=None):
        """The two-pass step with an overflow skip and a global-norm clip.

        ``reduce_and_check`` gives this owner's (flag, partial).  The decision
        needs every owner's: ``exchange(flag, partial)`` returns the lists of
        all owners' flags and partials in owner order (across GPUs, an
        all-gather of 12 bytes per owner); without it this owner's pair stands
        for the whole gradient.  ``zero_step_decision`` then skips when any
        flag is set, else gives ``min(1, max_norm / (sqrt(sum of partials) +
        1e-6))``, and ``apply_update`` runs AdamW from the stored gradient.

        Returns ``(updated, clip_coef)``; every owner returns the same pair, and
        the caller advances its step count only when ``updated`` is True.
        ``events`` / ``apply_events``: optional (start, end) CUDA events
        recorded around the reduce and around the AdamW launch.
        """
        flag, sumsq = self.reduce_and_check(rank_grads=rank_grads, grad_base=grad_base, divisor=divisor,
                                            events=events)
        flags, sums = ([flag], [sumsq]) if exchange is None else exchange(flag, sumsq)
        updated, coef = zero_step_decision(flags, sums, max_norm)
        if updated:
            if apply_events is not None:
                apply_events[0].record()
            self.apply_update(step=step, hyper=hyper, coef=coef, param16=param16, param_base=param_base,
                              grid_blocks=grid_blocks)
            if apply_events is not None:
                apply_events[1].record()
        return updated, coef

    # -- export / import of fp32 shard data in the dense per-tensor layout
    def to_dense(self, owner_array, dense) -> None:
        """Write this owner's real elements of an owner-local fp32 array into dense weights."""
        zero_owner_to_dense(self.chunks_dev, self.chunks.size, self.begin, self.end, self.tensor_offset_dev,
                            self.dense_offset_dev, owner_array, self.local_base, dense, **self._group_args())

    def from_dense(self, dense, owner_array) -> None:
        """Fill this owner's real elements of an owner-local fp32 array from dense weights."""
        zero_dense_to_owner(self.chunks_dev, self.chunks.size, self.begin, self.end, self.tensor_offset_dev,
                            self.dense_offset_dev, dense, owner_array, self.local_base, **self._group_args())

    # -- checkpoint of the owner's optimizer state
    def save(self, path: str, step: int) -> None:
        """Owner checkpoint: fp32 master, both moments, the step count and the layout."""
        np.savez(path, master=self.master.cpu().numpy(), exp_avg=self.exp_avg.cpu().numpy(),
                 exp_avg_sq=self.exp_avg_sq.cpu().numpy(), step=np.int64(step),
                 numels=np.array(self.numels, dtype=np.int64), ranks=np.int64(self.ranks),
                 owner=np.int64(self.owner), align=np.int64(self.align))

    def load(self, path: str) -> int:
        """Restore a checkpoint written by save() for the same layout; returns its step."""
        torch = _torch()
        with np.load(path, allow_pickle=False) as z:
            same = (list(z["numels"]) == self.numels and int(z["ranks"]) == self.ranks
                    and int(z["owner"]) == self.owner and int(z["align"]) == self.align)
            if not same:
                raise ValueError("checkpoint was written for a different layout or owner")
            self.master = torch.from_numpy(z["master"]).to(self.device)
            self.exp_avg = torch.from_numpy(z["exp_avg"]).to(self.device)
            self.exp_avg_sq = torch.from_numpy(z["exp_avg_sq"]).to(self.device)
            return int(z["step"])
