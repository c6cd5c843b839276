"""Property tests of the validator's alias rules.  The HIP-free validator is
built with g++ into a test-only shared library (tests/validate_shim.cpp), so
no call here can reach the HIP runtime.  Hypothesis places every tensor at a
16-byte offset inside a small window (8 KiB for the fused and AllGather
calls, where about half of the layouts then overlap; 1 KiB for the reduce),
so that overlaps of every kind are common, and the validator's status must
match the rules of include/twnorm.h written out below."""
import ctypes
import os
import shutil
import subprocess

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "reduce_residual_add_amd", "csrc")
FIT = os.path.join(ROOT, "_build", "twnorm_fit_table.inc")
OK, ALIAS = 0, -3
BF16 = 0
BASE = 0x7F0000000000
HIDDEN = 64                    # 128 bytes per bf16 row
ROW = HIDDEN * 2


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    if not os.path.exists(FIT):
        pytest.skip("build products not present (run the build first)")
    so = tmp_path_factory.mktemp("shim") / "libtwvalidate_shim.so"
    cmd = ["g++", "-std=c++17", "-O1", "-shared", "-fPIC", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-I", os.path.dirname(FIT), os.path.join(CSRC, "twnorm_validate.cpp"),
           os.path.join(ROOT, "tests", "validate_shim.cpp"), "-o", str(so)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lib = ctypes.CDLL(str(so))
    vp, i64 = ctypes.c_void_p, ctypes.c_longlong
    lib.shim_check_fused.argtypes = [ctypes.POINTER(vp), ctypes.c_int, i64, i64, ctypes.c_int, vp,
                                     vp, ctypes.c_float, vp, vp, ctypes.c_int]
    lib.shim_check_fused_allgather.argtypes = [ctypes.POINTER(vp), ctypes.c_int, i64, i64,
                                               ctypes.c_int, vp, vp, ctypes.c_float,
                                               ctypes.POINTER(vp), ctypes.c_int, i64, i64, vp,
                                               ctypes.c_int]
    lib.shim_check_reduce.argtypes = [ctypes.POINTER(vp), ctypes.c_int, i64, i64, ctypes.c_int, vp,
                                      ctypes.c_int]
    return lib


def _span(addr, nbytes):
    return (addr, addr + nbytes)


def _overlap(a, b):
    return a[0] < b[1] and b[0] < a[1]


def _addr(slot):
    return BASE + 16 * slot


_slot = st.integers(min_value=0, max_value=511)          # 8 KiB window
_slot_small = st.integers(min_value=0, max_value=63)     # 1 KiB window
_SETTINGS = settings(max_examples=400, deadline=None, derandomize=True,
                     suppress_health_check=[HealthCheck.function_scoped_fixture])


def _inputs_alias(parts, res, w, rout, tb):
    """Rules on residual_out: it may not overlap a partial or the weight, and
    may overlap the residual only by being exactly it (the in-place update)."""
    RO = _span(rout, tb)
    return (any(_overlap(RO, _span(p, tb)) for p in parts) or _overlap(RO, _span(w, ROW))
            or (rout != res and _overlap(RO, _span(res, tb))))


def _output_alias(o, nbytes, parts, res, w, rout, tb):
    """An output may overlap no input and not residual_out."""
    O = _span(o, nbytes)
    return (any(_overlap(O, _span(p, tb)) for p in parts) or _overlap(O, _span(res, tb))
            or _overlap(O, _span(w, ROW)) or _overlap(O, _span(rout, tb)))


@_SETTINGS
@given(n=st.integers(1, 4), rows=st.integers(1, 3), part_slots=st.lists(_slot, min_size=4, max_size=4),
       res=_slot, w=_slot, out=_slot, rout=_slot, in_place=st.booleans())
def test_fused_alias_rules_hold(shim, n, rows, part_slots, res, w, out, rout, in_place):
    tb = rows * ROW
    parts = [_addr(s) for s in part_slots[:n]]
    res_a, w_a, out_a = _addr(res), _addr(w), _addr(out)
    rout_a = res_a if in_place else _addr(rout)
    expect = ALIAS if (_inputs_alias(parts, res_a, w_a, rout_a, tb)
                       or _output_alias(out_a, tb, parts, res_a, w_a, rout_a, tb)) else OK
    arr = (ctypes.c_void_p * n)(*parts)
    got = shim.shim_check_fused(arr, n, rows, HIDDEN, BF16, res_a, w_a, 1e-5, out_a, rout_a, 0)
    assert got == expect, (parts, res_a, w_a, out_a, rout_a, tb, got)


@_SETTINGS
@given(n=st.integers(1, 3), rows=st.integers(1, 2), extra=st.integers(0, 2),
       part_slots=st.lists(_slot, min_size=3, max_size=3), res=_slot, w=_slot, rout=_slot,
       ag_slots=st.lists(_slot, min_size=1, max_size=3), in_place=st.booleans(),
       offset_frac=st.floats(0, 1))
def test_allgather_alias_rules_hold(shim, n, rows, extra, part_slots, res, w, rout, ag_slots,
                                    in_place, offset_frac):
    tb = rows * ROW
    total = rows + extra
    offset = int(round(offset_frac * extra))
    parts = [_addr(s) for s in part_slots[:n]]
    res_a, w_a = _addr(res), _addr(w)
    rout_a = res_a if in_place else _addr(rout)
    ags = [_addr(s) for s in ag_slots]
    gb = total * ROW
    alias = _inputs_alias(parts, res_a, w_a, rout_a, tb)
    for j, g in enumerate(ags):
        alias = alias or _output_alias(g, gb, parts, res_a, w_a, rout_a, tb)
        alias = alias or any(_overlap(_span(g, gb), _span(h, gb)) for h in ags[:j])
    expect = ALIAS if alias else OK
    arr = (ctypes.c_void_p * n)(*parts)
    ag_arr = (ctypes.c_void_p * len(ags))(*ags)
    got = shim.shim_check_fused_allgather(arr, n, rows, HIDDEN, BF16, res_a, w_a, 1e-5, ag_arr,
                                          len(ags), offset, total, rout_a, 0)
    assert got == expect, (parts, res_a, w_a, rout_a, ags, total, offset, got)


@_SETTINGS
@given(n=st.integers(1, 4), rows=st.integers(1, 3),
       part_slots=st.lists(_slot_small, min_size=4, max_size=4), red=_slot_small,
       onto=st.integers(-1, 3))
def test_reduce_alias_rules_hold(shim, n, rows, part_slots, red, onto):
    """reduced may be exactly one of the partials (written in place) but may
    not partly overlap any of them."""
    tb = rows * ROW
    parts = [_addr(s) for s in part_slots[:n]]
    red_a = parts[onto] if 0 <= onto < n else _addr(red)
    alias = any(p != red_a and _overlap(_span(red_a, tb), _span(p, tb)) for p in parts)
    expect = ALIAS if alias else OK
    arr = (ctypes.c_void_p * n)(*parts)
    got = shim.shim_check_reduce(arr, n, rows, HIDDEN, BF16, red_a, 0)
    assert got == expect, (parts, red_a, tb, got)
