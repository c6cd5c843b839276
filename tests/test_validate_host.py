"""The HIP-free validator and shape chooser, compiled on their own with g++
under AddressSanitizer and UndefinedBehaviorSanitizer (host code only) and
driven through every status it can return."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "reduce_residual_add_amd", "csrc")
FIT = os.path.join(ROOT, "_build", "twnorm_fit_table.inc")


def test_validator_under_sanitizers(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    if not os.path.exists(FIT):
        pytest.skip("build products not present (run the build first)")
    exe = tmp_path / "validate_host"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", os.path.dirname(FIT), os.path.join(CSRC, "twnorm_validate.cpp"),
           os.path.join(ROOT, "tests", "validate_host_driver.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "OK (0 failures)" in r.stdout
