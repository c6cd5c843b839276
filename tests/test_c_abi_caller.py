"""The C ABI from a plain C99 program (tests/c_abi_driver.c): no Python,
C++ or torch in the calling process.  Inputs come from the seeded generators
and are handed over in a file; the program's outputs are checked against the
oracle.  The CPU test only builds the program; the GPU test runs it as a
child process."""
import os
import shutil
import struct
import subprocess
import sys

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "reduce_residual_add_amd")
LIB = os.path.join(PKG, "libtwnorm.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_driver(out_dir):
    """Compile the C caller with gcc against include/twnorm.h, libtwnorm.so
    and the HIP runtime; returns the executable's path."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("HIP headers not available")
    if not os.path.exists(LIB):
        pytest.skip("libtwnorm.so not built")
    exe = os.path.join(str(out_dir), "c_abi_driver")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_driver.c"), "-L", PKG, "-ltwnorm",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{PKG}:{os.path.join(ROCM, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_caller_builds(tmp_path):
    exe = build_driver(tmp_path)
    assert os.access(exe, os.X_OK)


CASES = [
    # (n, rows, hidden, dtype)
    (3, 37, 5120, "bf16"),
    (8, 5, 8192, "bf16"),
    (2, 9, 1000, "f32"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("n,rows,hidden,dtype", CASES, ids=[f"n{a}-r{b}-h{c}-{d}" for a, b, c, d in CASES])
def test_c_caller_matches_oracle(twn, tmp_path, n, rows, hidden, dtype):
    from gpu_helpers import assert_parity, reference
    exe = build_driver(tmp_path)
    inp = workloads.make_random(n, rows, hidden, dtype, seed=rows * n + 3)
    code = 0 if dtype == "bf16" else 1
    src = tmp_path / "in.bin"
    with open(src, "wb") as f:
        f.write(struct.pack("<iiqqf", n, code, rows, hidden, inp["eps"]))
        for p in inp["partials"]:
            f.write(np.ascontiguousarray(p).tobytes())
        f.write(np.ascontiguousarray(inp["residual"]).tobytes())
        f.write(np.ascontiguousarray(inp["weight"]).tobytes())
    dst = tmp_path / "out.bin"
    print(f"[C caller] n={n} rows={rows} H={hidden} {dtype}", flush=True)
    sys.stdout.flush()
    r = subprocess.run([exe, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "refused as expected: TW_ERR_INVALID_ARG" in r.stderr
    storage = np.uint16 if dtype == "bf16" else np.float32
    got = np.fromfile(dst, dtype=storage).reshape(2, rows, hidden)
    ref_out, ref_res, b_out, b_res = reference(inp)
    assert_parity(got[1], ref_res, dtype, "residual_out from C", b_res)
    assert_parity(got[0], ref_out, dtype, "out from C", b_out)
