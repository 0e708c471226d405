"""Host checks of bench.py: its refusals, and the committed counter records it reads."""
import glob
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    res = _run("--gpus", "2")
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_without_a_gpu_it_fails_loudly():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    res = _run("--steps", "1", "--warmup", "0")
    assert res.returncode == 1 and "needs a GPU" in res.stderr and res.stdout == ""


RECORDS = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json")))


def test_there_are_traffic_records_for_every_workload():
    names = {os.path.basename(p)[:-len("_traffic.json")] for p in RECORDS}
    for cfg, tag in bench.WORKLOAD_TAG.items():
        assert any(n.endswith("__" + tag) for n in names), f"no counter record for config {cfg}"
    assert "owner_to_dense__llama-6.6e9-R8" in names and "span_copy_bf16__llama-layers0-3-R8" in names


@pytest.mark.parametrize("path", RECORDS, ids=[os.path.basename(p) for p in RECORDS])
def test_traffic_record_is_consistent(path):
    rec = json.load(open(path))
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    # the counters were scaled by a plain copy's reading: fetch x2, write x1 on this chip
    assert abs(rec["fetch_scale"] - 2.0) < 0.01 and abs(rec["write_scale"] - 1.0) < 0.01
    # a kernel moves at least its algorithmic bytes, and these move at most 25% more
    assert 0.999 * rec["algorithmic_bytes"] <= rec["bytes_per_launch"] <= 1.25 * rec["algorithmic_bytes"]
    assert len(rec["kernel_source_sha256_16"]) == 16
    # its summary sits beside it
    assert os.path.exists(path.replace("_traffic.json", "_counters.md"))


def test_every_timed_kernel_has_a_probe_mix():
    for kname in ("adam_step_f16_f16", "adam_step_bf16_bf16", "reduce_check_f16_r64", "accumulate_bf16",
                  "reduce_add_mean_bf16_r16", "owner_to_dense", "span_kernel<uint16_t>"):
        reads, writes = bench.PROBE_MIX[kname]
        assert reads > 0 and writes > 0


def test_every_timed_kernel_has_an_exact_structure():
    """The exact-structure probe of each timed kernel: its stream widths add up to
    its algorithmic bytes per element (2 bytes per width unit)."""
    per_element = {"adam_step_f16_f16": 34, "adam_step_bf16_bf16": 42, "reduce_check_f16_r64": 132,
                   "accumulate_bf16": 10, "reduce_add_mean_bf16_r16": 40, "owner_to_dense": 8,
                   "span_kernel<uint16_t>": 4, "adam_step_reduced_f16": 30, "adam_step_reduced_bf16": 30,
                   "adam_step_f32_bf16_r16": 90}
    for kname, b in per_element.items():
        src, dst = bench.PROBE_STRUCTURE[kname]
        assert 2 * (sum(src) + sum(dst)) == b, kname
    for kname in bench.SECOND_KERNEL.values():
        assert kname in bench.PROBE_STRUCTURE
