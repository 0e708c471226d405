"""The benchmark's output contract, checked on a short run of the default workload.

bench.py runs in a child process (as the benchmark is run), for two timed steps
of the default configuration (config 4: the 1.09375e9-parameter owner of a
7e10-parameter model over 64 ranks) with a one-second CPU-oracle sample, and
its one JSON line must carry every field the contract names, consistent with
itself: value = updated parameters / time, roofline.frac = achieved / peak,
the dominant kernel's algorithmic bytes = its elements x bytes per element
(64 fp16 reads + one fp32 write), and a CPU baseline of the oracle with its
GB/s and the GPU's speed-up.
"""
import json
import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def test_default_bench_line_keeps_the_contract():
    print("bench.py --steps 2 --warmup 1 --no-ceiling --cpu-seconds 1", flush=True)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                          "--no-ceiling", "--cpu-seconds", "1"], capture_output=True, text=True, timeout=240,
                         cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, "bench.py prints exactly one line"
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["scaling"] == "weak" and d["vs_baseline"] is None
    assert d["unit"] == "params/s" and d["dtype"] == "f32" and d["data"] == "synthetic"
    cfg = d["config"]
    assert "workload" in cfg and cfg["config"] == 4 and cfg["owned_params"] == 1_093_750_000
    assert cfg["ranks"] == 64 and cfg["padded_total"] == 70_000_000_000
    # value: parameters updated per second over the timed steps (skipped steps update none)
    updated = cfg["owned_params"] * (d["steps"] - d["overflow_steps"])
    assert d["value"] == pytest.approx(updated / (d["steps"] * d["ms_per_step"] * 1e-3), rel=1e-3)
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["kernel"] == "reduce_check_f16_r64"
    assert r["bytes_per_launch"] == r["elements_per_launch"] * r["bytes_per_element"] == 1_093_750_000 * 132
    assert r["achieved"] == pytest.approx(r["bytes_per_launch"] / (r["kernel_ms"] * 1e-3) / 1e9, rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    assert 0.3 < r["frac"] < 1.0
    # counter-measured bytes, or null once the kernel source has changed since the counters
    assert r["traffic"] is None or r["traffic"] >= r["bytes_per_launch"]
    if d["steps"] > d["overflow_steps"]:  # AdamW from the stored gradient, on the updating steps
        k2 = d["second_kernel"]
        assert k2["kernel"] == "adam_step_reduced_f16" and k2["bytes_per_launch"] == 1_093_750_000 * 30
        assert k2["achieved"] == pytest.approx(k2["bytes_per_launch"] / (k2["kernel_ms"] * 1e-3) / 1e9, rel=1e-3)
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "params/s" and c["value"] > 0 and c["cores"] >= 1
    assert c["sample"] and c["bytes_per_param"] == 162.0
    assert c["gbps"] == pytest.approx(c["value"] * 162 / 1e9, rel=1e-3)
    assert c["gpu_speedup"] == pytest.approx(d["value"] / c["value"], rel=0.01)
