"""The oracle and the library's host code built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc/g++, CPU only) and driven over random inputs
by the test programs in tests/sanitize/: any out-of-bounds access, use after
free or undefined operation aborts the program."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-static-libasan"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")


def _build_and_run(cmd, exe):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        if "sanitize" in res.stderr and ("cannot find" in res.stderr or "unrecognized" in res.stderr):
            pytest.skip("sanitizer runtime not available: " + res.stderr[-300:])
        raise AssertionError("build failed:\n" + res.stderr[-3000:])
    run = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "clean" in run.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _build_and_run(["gcc", "-std=c11", "-ffp-contract=off", *SAN, os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "zero_oracle.c"), "-lm", "-o", exe], exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers not found")
def test_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_driver")
    _build_and_run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    "-D__HIP_PLATFORM_AMD__", os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
                    os.path.join(ROOT, "zero_sharded_optimizer_owned_amd", "csrc", "host.cpp"), "-o", exe], exe)
