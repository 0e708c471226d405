"""Benchmark of the ZeRO owner-shard optimizer step on one MI355X.

One step = one pass of the owner's whole hot path over one batch of synthetic
input (inputs resident in HBM before the timed region):
  --config 4 (default): 7e10-parameter flat buffer, R=64, owner 1 (1.09375e9
      parameters), the largest configuration that fits one GPU: fp16 grads
      scaled by 2^16; reduce + overflow/norm check, host skip/clip decision,
      AdamW from the stored fp32 gradient; inf/NaN injected in one step of
      every four (those steps are skipped and count no updated parameters).
  --config 2: 1.5e9-parameter flat buffer, R=4, owner 1 (3.75e8 parameters):
      fused fp16 rank reduce + AdamW + fp16 write-back, one launch.
  --config 3: Llama-style 289-tensor list (6,607,339,520 parameters), 64-element
      alignment, R=8, owner 1: fused bf16 reduce + AdamW + bf16 write-back.
  --config 5: 10,000 log-uniform tensors (~2e9), R=16: eight bf16 microstep
      accumulations into the local fp32 buffer, then the owner's fused
      fp32-rank reduce + AdamW + bf16 write-back.

Prints one JSON line: owned parameters updated per second, achieved HBM GB/s of
the dominant kernel against the 8 TB/s peak, and the CPU oracle timed on a
bounded sample of the same workload (with its GB/s and the GPU's speed-up
over it).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "owned-shard params updated/sec + achieved HBM GB/s (fraction of MI355X peak)"
PEAK_GBPS = 8000.0
HP = dict(lr=1e-3, beta1=0.8, beta2=0.999, eps=1e-8, weight_decay=3e-7, adamw=True)
FIRST_STEP = 11  # the state stands for an optimizer after ten warm-up updates
DEFAULT_CHUNK = 2048  # chunk-table granularity (elements) of the timed launches


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4, choices=(2, 3, 4, 5))
    ap.add_argument("--schedule", default="accumulate", choices=("accumulate", "per-backward"),
                    help="config 5 only: accumulate microsteps locally then reduce (default), or reduce "
                         "every microstep and add the owned mean to an fp32 accumulator")
    ap.add_argument("--grid", type=int, default=0, help="fused-step grid blocks (0: library default, one block per chunk)")
    ap.add_argument("--chunk", type=int, default=DEFAULT_CHUNK, help="max chunk elements")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--op", default="step", choices=("step", "export", "gather3", "small"),
                    help="step: the owner's optimizer step; export: copy the owner's fp32 master "
                         "into the dense per-tensor layout (checkpoint consolidation); gather3: the "
                         "ZeRO-3 gather of four Llama-style layers from 8 ranks' bf16 shard buffers; "
                         "small: the fused step over 2,000,000 padded 100-element tensors (packed chunk groups)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-probe ceilings measured before the workload")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB fp32 device copy (counter calibration)")
    return ap.parse_args()


def kernel_source_hash(copy: bool = False) -> str:
    """Hash of the sources of the step kernels, or of the copy kernels (export,
    stage-3 gather); counter records are tied to it."""
    from zero_sharded_optimizer_owned_amd.build import COPY_SOURCES, CSRC, STEP_SOURCES

    h = hashlib.sha256()
    for name in COPY_SOURCES if copy else STEP_SOURCES:
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


# Workload names used in profiles/ file names.
WORKLOAD_TAG = {2: "flat-1.5e9-R4", 3: "llama-6.6e9-R8", 4: "flat-7e10-R64", 5: "10k-tensors-2e9-R16"}


def traffic_record(name: str, copy: bool = False):
    """Counter-derived HBM bytes per launch, if taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(copy):
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------- workloads
# read:write streams of equal size whose byte mix matches each dominant kernel's
# algorithmic traffic per parameter (e.g. config 2: 20 B read, 14 B written);
# for the 64-rank reduce also its structure: 64 sources of 2 bytes per
# parameter, and its 4-byte destination as two streams of 2 bytes
PROBE_MIX = {"adam_step_f16_f16": (10, 7), "adam_step_bf16_bf16": (2, 1), "reduce_check_f16_r64": (64, 2),
             "accumulate_bf16": (3, 2), "reduce_add_mean_bf16_r16": (9, 1), "owner_to_dense": (1, 1),
             "span_kernel<uint16_t>": (1, 1)}


# each dominant kernel's exact stream structure: the widths of its source and
# destination streams (1: 16-bit data, 16 bytes per 8 elements; 2: fp32 data,
# 32 bytes per 8 elements), as zero_stream_probe takes them
PROBE_STRUCTURE = {
    "adam_step_f16_f16": ([1] * 4 + [2] * 3, [2] * 3 + [1]),      # 4 ranks, w m v in; w m v p16 out
    "adam_step_bf16_bf16": ([1] * 8 + [2] * 3, [2] * 3 + [1]),    # 8 ranks, w m v in; w m v p16 out
    "reduce_check_f16_r64": ([1] * 64, [2]),                      # 64 ranks in; fp32 g out
    "accumulate_bf16": ([1, 2], [2]),                             # bf16 g and fp32 acc in; acc out
    "reduce_add_mean_bf16_r16": ([1] * 16 + [2], [2]),            # 16 ranks and acc in; acc out
    "owner_to_dense": ([2], [2]),
    "span_kernel<uint16_t>": ([1], [1]),
    # second kernels of a step
    "adam_step_reduced_f16": ([2] * 4, [2] * 3 + [1]),            # g, w, m, v in; w m v p16 out
    "adam_step_reduced_bf16": ([2] * 4, [2] * 3 + [1]),
    "adam_step_f32_bf16_r16": ([2] * 19, [2] * 3 + [1]),          # 16 fp32 ranks, w m v in
}

# The second kernel of a step (after the dominant one), timed beside it.
SECOND_KERNEL = {(4, "accumulate"): "adam_step_reduced_f16", (5, "accumulate"): "adam_step_f32_bf16_r16",
                 (5, "per-backward"): "adam_step_reduced_bf16"}


def structure_name(kname: str) -> str:
    src, dst = PROBE_STRUCTURE[kname]
    part = lambda ws: "+".join(f"{ws.count(w)}x{w}" for w in (1, 2) if ws.count(w))
    return f"{part(src)}:{part(dst)}"


def probe_structure_gbps(kname: str, elements: int, launches: int = 3, reps: int = 3) -> float:
    """HBM GB/s of the streaming probe with the kernel's exact stream structure
    (PROBE_STRUCTURE) at the kernel's own size: `elements` 8-element units per
    stream, i.e. the kernel's algorithmic bytes per launch; best of both piece
    orders."""
    import torch

    import zero_sharded_optimizer_owned_amd as zs

    src_w, dst_w = PROBE_STRUCTURE[kname]
    unit = elements // 8 * 16  # bytes per width unit: 2 bytes per element
    srcs = [torch.zeros(unit * w, dtype=torch.uint8, device="cuda") for w in src_w]
    dsts = [torch.empty(unit * w, dtype=torch.uint8, device="cuda") for w in dst_w]
    best = float("inf")
    for order in (0, 1):
        for _ in range(3):
            zs.zero_stream_probe(srcs, dsts, order, src_widths=src_w, dst_widths=dst_w)
        for _ in range(reps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            s.record()
            for _ in range(launches):
                zs.zero_stream_probe(srcs, dsts, order, src_widths=src_w, dst_widths=dst_w)
            e.record()
            torch.cuda.synchronize()
            best = min(best, s.elapsed_time(e) / launches)
    del srcs, dsts
    torch.cuda.empty_cache()
    return unit * (sum(src_w) + sum(dst_w)) / (best / 1e3) / 1e9


def probe_gbps(n_src: int, n_dst: int, total_bytes: float = 8e9, launches: int = 5, reps: int = 3) -> float:
    """HBM GB/s of the library's streaming probe for an n_src:n_dst mix of
    equal streams, about `total_bytes` moved per launch (far above the caches):
    the best of `reps` timings of `launches` launches after five warm-up ones,
    in either piece order (round-robin over the XCDs or XCD-contiguous runs;
    few streams go faster in contiguous runs, many in round-robin)."""
    import torch

    import zero_sharded_optimizer_owned_amd as zs

    per = int(total_bytes // (n_src + n_dst)) // (1 << 20) * (1 << 20)
    srcs = [torch.zeros(per, dtype=torch.uint8, device="cuda") for _ in range(n_src)]
    dsts = [torch.empty(per, dtype=torch.uint8, device="cuda") for _ in range(n_dst)]
    best = float("inf")
    for order in (0, 1):
        for _ in range(5):
            zs.zero_stream_probe(srcs, dsts, order)
        for _ in range(reps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            s.record()
            for _ in range(launches):
                zs.zero_stream_probe(srcs, dsts, order)
            e.record()
            torch.cuda.synchronize()
            best = min(best, s.elapsed_time(e) / launches)
    del srcs, dsts
    torch.cuda.empty_cache()
    return (n_src + n_dst) * per / (best / 1e3) / 1e9


def step_stats(ms: list) -> dict | None:
    if not ms:
        return None
    v = sorted(ms)
    mid = len(v) // 2
    med = v[mid] if len(v) % 2 else 0.5 * (v[mid - 1] + v[mid])
    return {"n": len(v), "median": round(med, 4), "min": round(v[0], 4), "max": round(v[-1], 4),
            "mean": round(sum(v) / len(v), 4)}


def ceilings(kname: str, elements: int, second=None) -> dict:
    """Measured ceilings for the dominant kernel: one stream read, one written,
    a plain copy, the probe with the kernel's own read:write byte mix over
    equal streams, and the probe with the kernel's exact stream structure and
    size (``elements`` per stream).  ``second``: (kernel, elements) of the
    step's second kernel, whose exact-structure probe is measured too."""
    n_src, n_dst = PROBE_MIX[kname]
    out = {"read_gbps": round(probe_gbps(1, 0), 1), "write_gbps": round(probe_gbps(0, 1), 1),
           "copy_gbps": round(probe_gbps(1, 1), 1), "mix": f"{n_src}:{n_dst}",
           "mix_gbps": round(probe_gbps(n_src, n_dst), 1), "structure": structure_name(kname),
           "structure_gbps": round(probe_structure_gbps(kname, elements), 1), "kernel": "zero_stream_probe"}
    if second is not None:
        out["second_structure"] = structure_name(second[0])
        out["second_structure_gbps"] = round(probe_structure_gbps(*second), 1)
    return out


def with_ceiling(roofline: dict, ceil: dict) -> dict:
    a = roofline["achieved"]
    return dict(ceil, frac_of_copy=round(a / ceil["copy_gbps"], 4), frac_of_mix=round(a / ceil["mix_gbps"], 4),
                frac_of_structure=round(a / ceil["structure_gbps"], 4))


def dominant_elements(args, owned: bool = False) -> int:
    """Elements the dominant kernel of a run processes per launch (``owned``: the
    owner's real elements, which the second kernel updates), from the layout
    alone (the ceilings are measured before the workload takes its memory)."""
    import zero_sharded_optimizer_owned_amd as zs

    if args.op == "gather3":
        _, _, gathered = zs.zero3_storage(llama_numels(), 8, list(range(1, 37)))
        return gathered
    if args.op == "small":
        numels, R = [100] * 2_000_000, 4
    else:
        numels, R = {2: ([1_500_000_000], 4), 3: (llama_numels(), 8), 4: ([70_000_000_000], 64),
                     5: (config5_numels(), 16)}[args.config]
    off, total, b, e = zs.zero_shard_layout(numels, R, 64)
    if args.config == 5 and args.schedule == "accumulate" and args.op == "step" and not owned:
        return total
    begin, end = int(b[1]), int(e[1])
    if (args.config == 4 or args.schedule == "per-backward") and args.op == "step" and not owned:
        return end - begin
    return sum(max(0, min(end, int(o) + n) - max(begin, int(o))) for o, n in zip(off, numels))


def llama_numels():
    d, ff, vocab = 4096, 11008, 32000
    layer = [d * d] * 4 + [d * ff, d * ff, ff * d, d, d]
    return [vocab * d] + layer * 32


def config5_numels(seed=5):
    import numpy as np

    import synth

    s = synth.log_uniform_sizes(seed, 10_000, 64, 1 << 24).astype(np.float64)
    s[0] = 1 << 24          # one tensor at the top of the range
    s[1:11] = 64            # at least ten at the bottom
    rest = s[11:]
    scale = (2e9 - (1 << 24) - 640) / rest.sum()
    s[11:] = np.maximum(64, np.floor(rest * scale))
    return [int(x) for x in s]


def fill(t, seed, stream, rank, index0, dist, scale, step=0):
    import synth

    synth.device_fill(t, synth.stream_key(seed, stream, rank, step), index0, dist, scale)


class Workload:
    """Device buffers and the step function of one configuration."""

    def __init__(self, cfg: int, chunk: int, grid: int, schedule: str = "accumulate"):
        import torch

        import synth
        import zero_sharded_optimizer_owned_amd as zs

        self.cfg, self.grid = cfg, grid
        self.schedule = schedule
        if schedule != "accumulate" and cfg != 5:
            raise ValueError("--schedule applies to config 5 only")
        dev = torch.device("cuda")
        self.dev = dev
        owner = 1
        if cfg == 2:
            numels, R, A, gdt, pdt = [1_500_000_000], 4, 64, torch.float16, torch.float16
            self.name = "flat 1.5e9 params, R=4, owner 1 of 4 (3.75e8), fp16 grads, fp16 write-back"
        elif cfg == 3:
            numels, R, A, gdt, pdt = llama_numels(), 8, 64, torch.bfloat16, torch.bfloat16
            self.name = ("Llama-style 289 tensors (6,607,339,520 params), 64-elem alignment, R=8, owner 1 "
                         "of 8, bf16 grads, bf16 write-back")
        elif cfg == 4:
            numels, R, A, gdt, pdt = [70_000_000_000], 64, 64, torch.float16, torch.float16
            self.name = ("flat 7e10 params, R=64, owner 1 of 64 (1.09375e9), fp16 grads x 2^16, overflow skip, "
                         "clip 1.0, fp16 write-back")
        else:
            numels, R, A, gdt, pdt = config5_numels(), 16, 64, torch.float32, torch.bfloat16
            self.name = ("10,000 log-uniform tensors (~2e9 params), R=16, owner 1 of 16, 8 bf16 microsteps "
                         "into fp32, bf16 write-back")
        self.numels, self.R = numels, R
        self.sh = zs.OwnerShard(numels, R, owner, align=A, max_chunk=chunk, device=dev)
        sh = self.sh
        lb, end = sh.local_base, sh.end
        seed = cfg
        # owner-local rank slices (what a reduce-scatter would deliver), flat-indexed from lb
        self.grads = []
        self.grad_scale = 65536.0 * 1e-3 if cfg == 4 else 1e-3
        if cfg != 5:
            for r in range(R):
                t = torch.empty(end - lb, dtype=gdt, device=dev)
                fill(t, seed, synth.STREAM_GRAD, r, lb, synth.DIST_NORMAL, self.grad_scale)
                self.grads.append(t)
        sh.alloc_state()
        fill(sh.master, seed, synth.STREAM_MASTER, 0, lb, synth.DIST_NORMAL, 0.02)
        fill(sh.exp_avg, seed, synth.STREAM_EXP_AVG, 0, lb, synth.DIST_NORMAL, 5e-4)
        fill(sh.exp_avg_sq, seed, synth.STREAM_EXP_AVG_SQ, 0, lb, synth.DIST_SQUARE, 1e-4)
        # 16-bit compute copy: the full flat buffer (ZeRO-1/2) except for the 70e9 case,
        # where only the owner's slice is held (ZeRO-3 style), param_base = lb
        if cfg == 4:
            self.p16, self.param_base = torch.zeros(end - lb, dtype=pdt, device=dev), lb
            # owner-local fp32 gradient, flag, norm and check workspace of the two-pass step
            self.g32, self.ov, self.ss, self.ws = sh.check_buffers()
            self.divisor = float(R) * 65536.0
        else:
            self.p16 = torch.zeros(sh.padded_total, dtype=pdt, device=dev)
            self.param_base = 0
            self.divisor = float(R)
        if cfg == 5 and schedule == "per-backward":
            self._setup_per_backward(seed)
            self.name += " (per-backward reduce + fp32 owned accumulator)"
        elif cfg == 5:
            self._setup_microsteps(seed)
        self.t = FIRST_STEP
        self.max_norm = 1.0  # config 4's clip threshold
        self.calls = 0
        self.skipped = 0
        self.kernel_bytes = self.algorithmic_bytes()
        torch.cuda.synchronize()

    def _setup_microsteps(self, seed):
        import torch

        import synth
        import zero_sharded_optimizer_owned_amd as zs

        sh = self.sh
        n = sh.padded_total
        # local rank's eight bf16 microstep gradients over the whole flat buffer
        self.micro = []
        for k in range(8):
            t = torch.empty(n, dtype=torch.bfloat16, device=self.dev)
            fill(t, seed, synth.STREAM_MICRO, self.sh.owner, 0, synth.DIST_NORMAL, 1e-3, step=k)
            self.micro.append(t)
        self.acc = torch.empty(n, dtype=torch.float32, device=self.dev)
        # the other ranks' accumulated gradients for this owner's slice: each is the
        # same eight-microstep accumulation of that rank's own microstep gradients
        lb, end = sh.local_base, sh.end
        tmp = torch.empty(end - lb, dtype=torch.bfloat16, device=self.dev)
        for r in range(self.R):
            if r == sh.owner:
                self.grads.append(None)
                continue
            acc_r = torch.empty(end - lb, dtype=torch.float32, device=self.dev)
            for k in range(8):
                fill(tmp, seed, synth.STREAM_MICRO, r, lb, synth.DIST_NORMAL, 1e-3, step=k)
                zs.zero_reduce_owned([tmp], lb, end - lb, 1.0, acc_r, grad_base=lb, out_base=lb,
                                     accumulate=k > 0)
            self.grads.append(acc_r)
        # the owner's own slice is a view of its accumulation buffer
        self.grads[sh.owner] = self.acc[lb:end]

    def _setup_per_backward(self, seed):
        """Owner slices of every rank's eight microstep gradients (what a reduce-scatter
        per backward call delivers) and the owner's fp32 accumulator."""
        import torch

        import synth

        sh = self.sh
        lb, end = sh.local_base, sh.end
        self.micro_slices = []
        for k in range(8):
            row = []
            for r in range(self.R):
                t = torch.empty(end - lb, dtype=torch.bfloat16, device=self.dev)
                fill(t, seed, synth.STREAM_MICRO, r, lb, synth.DIST_NORMAL, 1e-3, step=k)
                row.append(t)
            self.micro_slices.append(row)
        self.acc_owned = torch.empty(end - lb, dtype=torch.float32, device=self.dev)
        self.grads = [None]

    def kernel_elements(self) -> int:
        """Elements the dominant kernel processes per launch."""
        if self.cfg == 5 and self.schedule == "accumulate":
            return self.sh.padded_total
        if self.cfg == 4 or self.schedule == "per-backward":
            return self.sh.end - self.sh.begin
        return self.sh.n_real

    def algorithmic_bytes(self) -> int:
        """Bytes the dominant kernel (the one that takes most of the step) moves per launch."""
        n = self.sh.n_real
        if self.cfg == 4:
            # the 64-rank reduce with the fused check: 64 fp16 reads + one fp32 write
            return (self.sh.end - self.sh.begin) * (self.R * 2 + 4)
        if self.cfg == 5 and self.schedule == "accumulate":
            # one later microstep of the local accumulation: bf16 read, fp32 read and write
            return self.sh.padded_total * 10
        if self.schedule == "per-backward":
            # one microstep's reduce of 16 bf16 slices into the accumulator: 16*2 + 4 + 4
            return (self.sh.end - self.sh.begin) * (self.R * 2 + 8)
        gw = self.grads[0].element_size() if self.grads[0] is not None else 4
        return n * (self.R * gw + 24 + self.p16.element_size())

    def second_bytes(self) -> int:
        """Algorithmic bytes of the step's second kernel: AdamW from a stored fp32
        gradient (configs 4 and 5 per-backward: 4 + 12 read, 12 + 2 written) or
        config 5's fused owner step (16 fp32 ranks + 12 read, 14 written)."""
        n = self.sh.n_real
        if self.cfg == 5 and self.schedule == "accumulate":
            return n * (self.R * 4 + 26)
        return n * 30

    def step_bytes(self, overflow: bool) -> int:
        n = self.sh.n_real
        if self.cfg == 4:
            return n * (self.R * 2 + 4) + (0 if overflow else n * 30)
        if self.schedule == "per-backward":
            span = self.sh.end - self.sh.begin
            return span * (self.R * 2 + 4) + 7 * span * (self.R * 2 + 8) + n * 30
        if self.cfg == 5:
            P = self.sh.padded_total
            return P * (6 + 7 * 10) + n * (self.R * 4 + 26)
        return self.kernel_bytes

    # one full step of the owner's hot path; ``timing``: events around the dominant
    # kernel, ``timing2``: around the second kernel (configs 4 and 5)
    def step(self, timing=None, timing2=None):
        import torch

        import zero_sharded_optimizer_owned_amd as zs

        sh = self.sh
        if self.schedule == "per-backward":
            for k, row in enumerate(self.micro_slices):
                if timing is not None and k == 7:
                    timing[0].record()
                zs.zero_reduce_owned(row, sh.begin, sh.end - sh.begin, float(self.R), self.acc_owned,
                                     grad_base=sh.local_base, out_base=sh.local_base,
                                     accumulate=0 if k == 0 else 2)
                if timing is not None and k == 7:
                    timing[1].record()
            if timing2 is not None:
                timing2[0].record()
            sh.adam_step(step=self.t, hyper=HP, reduced_g=self.acc_owned, param16=self.p16,
                         param_base=self.param_base, grid_blocks=self.grid)
            if timing2 is not None:
                timing2[1].record()
            self.t += 1
            return False
        if self.cfg == 5:
            for k, g in enumerate(self.micro):
                if timing is not None and k == 7:
                    timing[0].record()
                zs.zero_reduce_owned([g], 0, sh.padded_total, 1.0, self.acc, accumulate=k > 0)
                if timing is not None and k == 7:
                    timing[1].record()
            if timing2 is not None:
                timing2[0].record()
            sh.adam_step(step=self.t, hyper=HP, rank_grads=self.grads, grad_base=sh.local_base,
                         divisor=self.divisor, param16=self.p16, param_base=self.param_base,
                         grid_blocks=self.grid)
            if timing2 is not None:
                timing2[1].record()
            self.t += 1
            return False
        self.calls += 1
        if self.cfg == 4:
            inject = self.calls % 4 == 0  # one step in four carries an inf and a NaN
            if inject:  # +inf in one rank, NaN in another (input preparation, two stores)
                saved = (self.grads[5][12345].clone(), self.grads[17][777_777].clone())
                self.grads[5][12345] = float("inf")
                self.grads[17][777_777] = float("nan")
            # reduce + check, 16 bytes to the host, then AdamW from g unless overflowed
            updated, _ = sh.checked_step(step=self.t, hyper=HP, rank_grads=self.grads, grad_base=sh.local_base,
                                         divisor=self.divisor, max_norm=self.max_norm, param16=self.p16,
                                         param_base=self.param_base, grid_blocks=self.grid, events=timing,
                                         apply_events=timing2)
            if inject:
                self.grads[5][12345] = saved[0]
                self.grads[17][777_777] = saved[1]
            if not updated:
                self.skipped += 1
                return True
            self.t += 1
            return False
        if timing is not None:
            timing[0].record()
        sh.adam_step(step=self.t, hyper=HP, rank_grads=self.grads, grad_base=sh.local_base,
                     divisor=self.divisor, param16=self.p16, param_base=self.param_base,
                     grid_blocks=self.grid)
        if timing is not None:
            timing[1].record()
        self.t += 1
        return False


# ---------------------------------------------------------------- CPU oracle leg
def cpu_baseline(w: Workload, seconds: float):
    """The oracle on a bounded prefix of the same owner's work, on the host cores."""
    import numpy as np

    import oracle
    import synth

    sh = w.sh
    cfg = w.cfg
    # real elements in the sample: sized so that generating its inputs stays a few seconds
    budget = {2: 1 << 24, 3: 1 << 23, 4: 1 << 21, 5: 1 << 20}[cfg]
    ranges, left = [], budget
    for c in sh.chunks:
        if left <= 0:
            break
        take = min(int(c["len"]), left)
        ranges.append((int(c["flat"]), int(c["flat"]) + take))
        left -= take
    lo, hi = ranges[0][0], ranges[-1][1]
    lb = lo & ~7
    seed = cfg

    def gen(key, start, stop, dist, scale, code):  # inputs on all host cores (untimed)
        return synth.host_values(key, start, stop - start, dist, scale, code)

    gcode = {2: synth.F16, 3: synth.BF16, 4: synth.F16, 5: synth.F32}[cfg]
    scale = w.grad_scale if cfg != 5 else 1e-3
    micro = None  # the per-step microstep work timed with the owner step (config 5)
    if w.schedule == "per-backward":
        # each of the eight microsteps reduces the 16 ranks' owned values into the owner's
        # accumulator (timed below; the eight microsteps reuse one microstep's values)
        rows = [gen(synth.stream_key(seed, synth.STREAM_MICRO, r, 0), lo, hi, synth.DIST_NORMAL, 1e-3, synth.BF16)
                for r in range(w.R)]
        acc = np.zeros(hi - lo, dtype=np.float32)

        def micro():
            acc[:] = oracle.reduce(rows, synth.BF16, float(w.R))
            for _ in range(7):
                oracle.reduce_add(rows, synth.BF16, float(w.R), acc)
        grads = None
    elif cfg == 5:
        # the owner's 16 rank slices: each the eight-microstep accumulation of its rank
        grads = []
        for r in range(w.R):
            acc_r = np.zeros(hi - lb, dtype=np.float32)
            for k in range(8):
                g = gen(synth.stream_key(seed, synth.STREAM_MICRO, r, k), lb, hi, synth.DIST_NORMAL, 1e-3,
                        synth.BF16)
                oracle.accumulate(g, synth.BF16, acc_r, first=(k == 0))
            grads.append(acc_r)
        # the local rank's eight microsteps over its whole flat buffer, which is
        # padded_total / owned elements per owned element (timed below; the eight
        # microsteps reuse one microstep's values)
        flat_per_owned = sh.padded_total / sh.n_real
        m = int(round((hi - lb) * flat_per_owned))
        gm = gen(synth.stream_key(seed, synth.STREAM_MICRO, sh.owner, 0), 0, m, synth.DIST_NORMAL, 1e-3, synth.BF16)
        acc_local = np.zeros(m, dtype=np.float32)

        def micro():
            for k in range(8):
                oracle.accumulate(gm, synth.BF16, acc_local, first=(k == 0))
    else:
        grads = [gen(synth.stream_key(seed, synth.STREAM_GRAD, r), lb, hi, synth.DIST_NORMAL, scale, gcode)
                 for r in range(w.R)]
    mk = lambda st, dist, s: gen(synth.stream_key(seed, st, 0), lb, hi, dist, s, synth.F32)
    w0 = mk(synth.STREAM_MASTER, synth.DIST_NORMAL, 0.02)
    m0 = mk(synth.STREAM_EXP_AVG, synth.DIST_NORMAL, 5e-4)
    v0 = mk(synth.STREAM_EXP_AVG_SQ, synth.DIST_SQUARE, 1e-4)
    pcode = synth.F16 if cfg in (2, 4) else synth.BF16
    p16 = np.zeros(hi - lb, dtype=np.uint16)
    n_real = sum(e - b for b, e in ranges)
    done, el, reps = 0, 0.0, 0
    while True:
        wc, mc, vc = w0.copy(), m0.copy(), v0.copy()
        t_start = time.perf_counter()
        if micro is not None:
            micro()
        if w.schedule == "per-backward":
            gfull = np.zeros(hi - lb, dtype=np.float32)
            gfull[lo - lb:] = acc
            oracle.owner_step(ranges, oracle.hyper(step=FIRST_STEP, **HP), wc, mc, vc, lb, reduced_g=gfull,
                              p16=p16, pdtype=pcode, param_base=lb)
        elif cfg == 4:
            g = oracle.reduce([x[lo - lb:hi - lb] for x in grads], gcode, w.divisor)
            flag, sumsq = oracle.grad_check(g)
            gfull = np.zeros(hi - lb, dtype=np.float32)
            gfull[lo - lb:] = g
            oracle.owner_step(ranges, oracle.hyper(step=FIRST_STEP, clip_coef=oracle.clip_coef(sumsq), **HP),
                              wc, mc, vc, lb, reduced_g=gfull, p16=p16, pdtype=pcode, param_base=lb)
        else:
            oracle.owner_step(ranges, oracle.hyper(step=FIRST_STEP, **HP), wc, mc, vc, lb, grads=grads,
                              gdtype=gcode, grad_base=lb, divisor=w.divisor, p16=p16, pdtype=pcode,
                              param_base=lb)
        el += time.perf_counter() - t_start
        done += n_real
        reps += 1
        if el >= seconds or reps >= 1000:
            break
    if w.schedule == "per-backward":
        what = "eight reduce-and-adds of the 16 ranks' owned values, then AdamW + cast"
    elif cfg == 4:
        what = "reduce + check + clip + AdamW + cast"
    elif cfg == 5:
        what = (f"eight microstep accumulations over {m} local flat elements "
                f"({flat_per_owned:.1f} per owned element), then reduce + AdamW + cast")
    else:
        what = "reduce + AdamW + cast"
    rate = done / el
    # the same algorithmic bytes per updated parameter as the GPU's updating step
    per_param = w.step_bytes(False) / sh.n_real
    return {"value": rate, "unit": "params/s", "cores": oracle.num_threads(), "kind": "oracle",
            "gbps": round(rate * per_param / 1e9, 3), "bytes_per_param": round(per_param, 3),
            "sample": f"first {n_real} real elements of the owner's shard, {reps} oracle step(s) "
                      f"({what}; inputs pre-generated)"}



class Stage3Gather:
    """ZeRO-3 working set: the first four layers (36 tensors) of the Llama-style list,
    gathered from 8 ranks' bf16 shard buffers (each holds its ceil(n/8) shard of all
    289 tensors) into full padded buffers."""

    SEED = 6

    def __init__(self, n_layers: int = 4, R: int = 8):
        import numpy as np
        import torch

        import synth
        import zero_sharded_optimizer_owned_amd as zs

        self.numels, self.R = llama_numels(), R
        self.live = list(range(1, 1 + 9 * n_layers))
        self.shard_numel, self.resident, self.gathered = zs.zero3_storage(self.numels, R, self.live)
        self.shards = []
        for r in range(R):
            t = torch.empty(self.resident, dtype=torch.bfloat16, device="cuda")
            fill(t, self.SEED, synth.STREAM_MASTER, r, 0, synth.DIST_NORMAL, 0.02)
            self.shards.append(t)
        self.out = torch.empty(self.gathered, dtype=torch.bfloat16, device="cuda")
        self.spans = zs.zero3_gather_spans(self.numels, R, self.live)
        self.spans_dev = zs.spans_to_device(self.spans)
        # short spans packed several to a block when that pays (here it does not:
        # only the norms' 512-element shards are short)
        groups = zs.zero_span_groups(self.spans, 2)
        self.n_groups = groups.size - 1
        self.groups_dev = (torch.from_numpy(groups.astype(np.int64)).to("cuda")
                           if zs.groups_pay(self.n_groups, self.spans.size) else None)
        self.so = np.concatenate([[0], np.cumsum(self.shard_numel)[:-1]]).astype(np.int64)
        torch.cuda.synchronize()

    def run(self):
        import zero_sharded_optimizer_owned_amd as zs

        zs.zero_copy_spans(self.spans_dev, self.spans.size, self.shards, self.out, groups_dev=self.groups_dev,
                           n_groups=self.n_groups if self.groups_dev is not None else 0)

    def expected(self, pos):
        """Generator values at gather-buffer positions (rank r's shard element so_k + j)."""
        import numpy as np

        import synth

        want = np.empty(pos.size, dtype=np.uint16)
        base = 0
        for k in self.live:
            s = int(self.shard_numel[k])
            sel = (pos >= base) & (pos < base + self.R * s)
            rel = pos[sel] - base
            r, j = rel // s, rel % s
            for rr in np.unique(r):
                m = r == rr
                idx = (self.so[k] + j[m]).astype(np.uint64)
                vals = synth.values(synth.stream_key(self.SEED, synth.STREAM_MASTER, int(rr)), idx,
                                    synth.DIST_NORMAL, 0.02, synth.BF16)
                tmp = want[sel]
                tmp[m] = vals
                want[sel] = tmp
            base += self.R * s
        return want


def gather3_bench(args, ceil):
    import torch

    g = Stage3Gather()
    for _ in range(args.warmup):
        g.run()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(args.steps):
        g.run()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    nbytes = 4 * g.gathered  # each bf16 element read once and written once
    line = {
        "metric": "ZeRO-3 gathered params/sec + achieved HBM GB/s (fraction of MI355X peak)",
        "value": round(g.gathered / (ms / 1e3), 1), "unit": "params/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Llama-style list (289 tensors), R=8 per-tensor shards, gather of layers 0-3 "
                               "(36 tensors) into full padded buffers", "op": "gather3",
                   "gathered_params": g.gathered, "resident_per_rank": g.resident, "spans": int(g.spans.size)},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (ms / 1e3) / 1e9, 1), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(nbytes / (ms / 1e3) / 1e9 / PEAK_GBPS, 4),
                     "traffic": traffic_record("span_copy_bf16__llama-layers0-3-R8", copy=True),
                     "kernel": "span_kernel<uint16_t>", "kernel_ms": round(ms, 4), "bytes_per_launch": nbytes},
    }
    if ceil:
        line["ceiling"] = with_ceiling(line["roofline"], ceil)
    if not args.no_cpu_baseline:
        import numpy as np

        import oracle
        import synth

        # the oracle's plain loops on a small model of the same shape (R=8, 9 tensors of one layer / 64)
        sizes = [n // 64 for n in llama_numels()[1:10]]
        dense = synth.values_f32(synth.stream_key(6, synth.STREAM_MASTER, 0), synth.arange(0, sum(sizes)),
                                 synth.DIST_NORMAL, 0.02)
        t0 = time.perf_counter()
        shards = oracle.stage3_shards(sizes, 8, dense)
        t1 = time.perf_counter()
        outg = oracle.stage3_gather(sizes, 8, shards, list(range(len(sizes))))
        t2 = time.perf_counter()
        line["cpu_baseline"] = {"value": outg.size / (t2 - t1), "unit": "params/s", "cores": 1, "kind": "oracle",
                                "sample": f"gather of one layer scaled by 1/64 ({outg.size} elements; "
                                          f"partition loop {t1 - t0:.1f} s untimed)"}
    print(json.dumps(line), flush=True)


def whole_line_bytes(ranges, streams, line: int = 128, sector: int = 32) -> int:
    """Bytes that the owner's real ranges take in whole memory units: a read
    stream fetches every 128-byte line that holds one of its elements, a write
    stream writes every 32-byte sector that holds one.  ``streams``: (element
    bytes, index of the stream's first element (its base is 256-byte aligned),
    True for a read)."""
    total = 0
    for b, e in ranges:
        for size, base, read in streams:
            unit = line if read else sector
            lo, hi = (b - base) * size, (e - base) * size
            total += (-(-hi // unit) - lo // unit) * unit
    return total


def small_bench(args, ceil):
    """The fused fp16 step (R=4, AdamW, fp16 write-back) of owner 1 over
    2,000,000 tensors of 100 elements each, padded to 128 (1.7 GB per step, far
    above the caches): short chunks, packed several to a block by the chunk
    group table (one block per chunk is timed beside it)."""
    import torch

    import synth
    import zero_sharded_optimizer_owned_amd as zs

    numels, R = [100] * 2_000_000, 4
    sh = zs.OwnerShard(numels, R, 1, align=64, max_chunk=DEFAULT_CHUNK, device="cuda")
    sh.alloc_state()
    lb = sh.local_base
    fill(sh.master, 7, synth.STREAM_MASTER, 0, lb, synth.DIST_NORMAL, 0.02)
    fill(sh.exp_avg, 7, synth.STREAM_EXP_AVG, 0, lb, synth.DIST_NORMAL, 5e-4)
    fill(sh.exp_avg_sq, 7, synth.STREAM_EXP_AVG_SQ, 0, lb, synth.DIST_SQUARE, 1e-4)
    grads = []
    for r in range(R):
        t = torch.empty(sh.end - lb, dtype=torch.float16, device="cuda")
        fill(t, 7, synth.STREAM_GRAD, r, lb, synth.DIST_NORMAL, 1e-3)
        grads.append(t)
    p16 = torch.zeros(sh.padded_total, dtype=torch.float16, device="cuda")

    def step(t, grouped=True):
        saved = sh.groups_dev
        if not grouped:
            sh.groups_dev = None
        sh.adam_step(step=t, hyper=HP, rank_grads=grads, grad_base=lb, divisor=float(R), param16=p16)
        sh.groups_dev = saved

    def timed(grouped):
        for i in range(args.warmup):
            step(FIRST_STEP + i, grouped)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(args.steps):
            step(FIRST_STEP + args.warmup + i, grouped)
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / args.steps

    ms_chunk = timed(False)
    ms = timed(True)
    n = sh.n_real
    nbytes = n * (R * 2 + 26)
    # what whole lines (reads) and sectors (writes) of the padded slots come to:
    # 4 fp16 rank slices and master/m/v read, master/m/v and the fp16 copy written
    ranges = [(int(c["flat"]), int(c["flat"]) + int(c["len"])) for c in sh.chunks]
    streams = [(2, lb, True)] * R + [(4, lb, True)] * 3 + [(4, lb, False)] * 3 + [(2, 0, False)]
    line_bytes = whole_line_bytes(ranges, streams)
    achieved = nbytes / (ms / 1e3) / 1e9
    line = {
        "metric": "owned-shard params updated/sec + achieved HBM GB/s (fraction of MI355X peak)",
        "value": round(n / (ms / 1e3), 1), "unit": "params/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "2,000,000 tensors of 100 elements (padded to 128), R=4, owner 1 of 4, fp16 grads, "
                               "fp16 write-back; chunk groups", "op": "small", "owned_params": n,
                   "chunks": int(sh.chunks.size), "groups": int(sh.n_groups)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": traffic_record("adam_group_step_f16_f16__2M-tensors-100-R4"),
                     "kernel": "adam_group_step_f16_f16",
                     "kernel_ms": round(ms, 4), "bytes_per_launch": nbytes, "elements_per_launch": n,
                     "bytes_per_element": float(R * 2 + 26)},
        "one_block_per_chunk": {"ms": round(ms_chunk, 4),
                                "achieved_gbps": round(nbytes / (ms_chunk / 1e3) / 1e9, 1)},
        "whole_line_bytes_per_launch": line_bytes,
        "whole_line_gbps": round(line_bytes / (ms / 1e3) / 1e9, 1),
    }
    if ceil:
        line["ceiling"] = with_ceiling(line["roofline"], ceil)
    print(json.dumps(line), flush=True)


def export_bench(w: Workload, args, ceil):
    """Time the consolidation copy of the owner's fp32 master into dense per-tensor weights."""
    import numpy as np
    import torch

    import oracle

    sh = w.sh
    dense = torch.zeros(sh.dense_total, dtype=torch.float32, device="cuda")
    for _ in range(args.warmup):
        sh.to_dense(sh.master, dense)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(args.steps):
        sh.to_dense(sh.master, dense)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    n = sh.n_real
    nbytes = 8 * n
    line = {
        "metric": "owned-shard fp32 export params/sec + achieved HBM GB/s (fraction of MI355X peak)",
        "value": round(n / (ms / 1e3), 1), "unit": "params/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name + "; export of the owner's master to dense per-tensor fp32",
                   "config": args.config, "op": "export", "owned_params": n},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (ms / 1e3) / 1e9, 1), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(nbytes / (ms / 1e3) / 1e9 / PEAK_GBPS, 4),
                     "traffic": traffic_record(f"owner_to_dense__{WORKLOAD_TAG[args.config]}", copy=True),
                     "kernel": "owner_to_dense", "kernel_ms": round(ms, 4), "bytes_per_launch": nbytes},
    }
    if ceil:
        line["ceiling"] = with_ceiling(line["roofline"], ceil)
    if not args.no_cpu_baseline:
        # the oracle's plain loop over the owner's first 2^16 real elements
        import synth

        m = 1 << 16
        first = [(int(c["flat"]), int(c["flat"]) + int(c["len"])) for c in sh.chunks[:max(1, m // 512)]]
        lo, hi = first[0][0], first[-1][1]
        arr = synth.values_f32(synth.stream_key(w.cfg, synth.STREAM_MASTER, 0), synth.arange(lo & ~7, hi),
                               synth.DIST_NORMAL, 0.02)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            numels = [b - a for a, b in first]
            oracle.consolidate(numels, [a for a, _ in first], [(lo, hi)], [arr], [lo & ~7])
            reps += 1
        el = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": reps * (hi - lo) / el, "unit": "params/s", "cores": 1, "kind": "oracle",
                                "sample": f"{hi - lo} real elements of the owner's shard (pure-Python loop)"}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU exchange "
              "around the owner step is not implemented here.", file=sys.stderr)
        sys.exit(2)
    import torch

    import zero_sharded_optimizer_owned_amd as zs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    zs.lib()
    if args.op == "gather3":
        kname = "span_kernel<uint16_t>"
    elif args.op == "small":
        kname = "adam_step_f16_f16"
    elif args.op == "export":
        kname = "owner_to_dense"
    elif args.schedule == "per-backward":
        kname = "reduce_add_mean_bf16_r16"
    else:
        kname = {2: "adam_step_f16_f16", 3: "adam_step_bf16_bf16", 4: "reduce_check_f16_r64",
                 5: "accumulate_bf16"}[args.config]
    # before the workload takes its memory
    kname2 = SECOND_KERNEL.get((args.config, args.schedule)) if args.op == "step" else None
    second = (kname2, dominant_elements(args, owned=True)) if kname2 else None
    ceil = None if args.no_ceiling else ceilings(kname, dominant_elements(args), second)
    if args.calibrate_copy:
        # a plain copy of known size: 2^28 fp32 read + 2^28 fp32 written per launch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.op == "gather3":
        return gather3_bench(args, ceil)
    if args.op == "small":
        return small_bench(args, ceil)
    w = Workload(args.config, args.chunk, args.grid, args.schedule)
    if args.op == "export":
        return export_bench(w, args, ceil)
    for _ in range(args.warmup):
        w.step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    starts2 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends2 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    overflow_steps = 0
    w.skipped = 0
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]  # step boundaries
    wall0 = time.perf_counter()
    marks[0].record()
    launched = []
    for i in range(args.steps):
        skipped = w.step(timing=(starts[i], ends[i]), timing2=(starts2[i], ends2[i]))
        marks[i + 1].record()
        launched.append(not skipped)
        overflow_steps += int(skipped)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = marks[0].elapsed_time(marks[-1])
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    ms_step = total_ms / args.steps
    kms = [s.elapsed_time(e) for s, e in zip(starts, ends)]  # the dominant kernel runs every step
    kernel_ms = sum(kms) / len(kms)
    n = w.sh.n_real
    updated = n * (args.steps - overflow_steps)
    value = updated / (total_ms / 1e3)
    step_bytes = sum(w.step_bytes(not ok) for ok in launched)
    gbps_step = step_bytes / (total_ms / 1e3) / 1e9
    achieved = w.kernel_bytes / (kernel_ms / 1e3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBPS, 4),
                "traffic": traffic_record(f"{kname}__{WORKLOAD_TAG[args.config]}"),
                "kernel": kname, "kernel_ms": round(kernel_ms, 4),
                "bytes_per_launch": w.kernel_bytes, "elements_per_launch": w.kernel_elements(),
                "bytes_per_element": round(w.kernel_bytes / w.kernel_elements(), 3)}
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "params/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "config": args.config, "schedule": w.schedule, "owned_params": n,
                   "ranks": w.R, "padded_total": w.sh.padded_total, "chunks": int(w.sh.chunks.size),
                   "parallelism": "1 GPU (owner shard; no collectives)"},
        "gbps": round(gbps_step, 1), "frac_of_peak": round(gbps_step / PEAK_GBPS, 4),
        "overflow_steps": overflow_steps, "wall_s": round(wall, 3),
        "step_ms": step_stats(step_ms),
        "roofline": roofline,
    }
    if ceil:
        line["ceiling"] = with_ceiling(roofline, ceil)
    k2 = [s2.elapsed_time(e2) for s2, e2, ok in zip(starts2, ends2, launched) if ok] if kname2 else []
    if k2:  # the step's second kernel, on the steps that run it (config 4: updating steps)
        ms2 = sum(k2) / len(k2)
        bytes2 = w.second_bytes()
        sk = {"kernel": kname2, "kernel_ms": round(ms2, 4), "bytes_per_launch": bytes2,
              "achieved": round(bytes2 / (ms2 / 1e3) / 1e9, 1),
              "frac": round(bytes2 / (ms2 / 1e3) / 1e9 / PEAK_GBPS, 4)}
        if ceil:
            sk["structure"] = ceil["second_structure"]
            sk["structure_gbps"] = ceil["second_structure_gbps"]
            sk["frac_of_structure"] = round(sk["achieved"] / ceil["second_structure_gbps"], 4)
        line["second_kernel"] = sk
    if args.config == 4:  # updating and skipped (overflow) steps separately, and the 4-step cycle
        line["step_ms_update"] = step_stats([t for t, ok in zip(step_ms, launched) if ok])
        line["step_ms_overflow"] = step_stats([t for t, ok in zip(step_ms, launched) if not ok])
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)
        cpu["gpu_speedup"] = round(value / cpu["value"], 1)  # the GPU's params/s over the oracle's
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
