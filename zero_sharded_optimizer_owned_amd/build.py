"""Build libzero_shard.so for gfx950 (hipcc, in place next to this file)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libzero_shard.so")
SOURCES = ("host.cpp", "launch.hip", "step.hip", "copy.hip", "probe.hip")
# The sources whose kernels make up the optimizer step (hashed to tie counter
# records to the code they were taken on).
STEP_SOURCES = ("step.hip", "launch.hip", "launch.h", "internal.h", "scan.h")
# The same for the copy kernels (checkpoint export/import, stage-3 gather).
COPY_SOURCES = ("copy.hip", "launch.hip", "launch.h", "internal.h", "scan.h")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # every fused multiply-add is written explicitly in the kernels
    "-ffp-contract=off",
    # IEEE fp32 division and square root, denormals kept (bit-exact reduce)
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no mixed-precision FMAs: the compiler would otherwise fold the fp16
    # conversion of an fma result into one v_fma_mix (one rounding of the
    # exact a*b+c to fp16) instead of rounding the fp32 master weight that is
    # stored, so the 16-bit copy would not always be that weight's rounding
    "-Xclang", "-target-feature", "-Xclang", "-fma-mix-insts",
    "-Wall",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, f) for f in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = ["hipcc", *HIPCC_FLAGS, "-I", INCLUDE, *srcs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building libzero_shard.so failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(" ".join(cmd))
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
