"""The C ABI without a GPU: the library loads, exports every function that
include/twnorm.h and include/twnorm_bench.h declare, and every error path returns its status before
any HIP call.  Pointers here are fake, 16-byte aligned addresses that the
validator compares but never dereferences."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("twnorm.h", "twnorm_bench.h")]

import reduce_residual_add_amd as twn  # noqa: E402

OK, INV, UNS, ALIAS = twn.TW_OK, twn.TW_ERR_INVALID_ARG, twn.TW_ERR_UNSUPPORTED, twn.TW_ERR_ALIAS
BF16, F32 = twn.TW_BF16, twn.TW_F32

MB = 1 << 20


def _declared_functions():
    names = set()
    for path in HEADERS:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(tw_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(twn.LIB_PATH):
        # a fresh checkout: build it (hipcc cross-compiles gfx950 without a GPU)
        from reduce_residual_add_amd import build
        build.build()
    return twn.load()


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert "tw_fused_reduce_rmsnorm" in declared and "tw_reduce" in declared
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"
    assert sorted(twn.EXPORTED) == declared


def test_version_and_status_strings(lib):
    assert lib.tw_abi_version() == twn.TW_ABI_VERSION
    for code, name in [(OK, b"TW_OK"), (INV, b"TW_ERR_INVALID_ARG"), (UNS, b"TW_ERR_UNSUPPORTED"),
                       (ALIAS, b"TW_ERR_ALIAS"), (twn.TW_ERR_HIP, b"TW_ERR_HIP")]:
        assert lib.tw_status_string(code) == name


class Bufs:
    """Fake, disjoint, 16-byte aligned device addresses."""

    def __init__(self, n=2, rows=4, hidden=64, dtype=BF16):
        self.n, self.rows, self.hidden, self.dtype = n, rows, hidden, dtype
        base = 0x7F0000000000
        self.parts = [base + i * 64 * MB for i in range(n)]
        self.residual = base + 1024 * MB
        self.weight = base + 1100 * MB
        self.out = base + 1200 * MB
        self.res_out = base + 1300 * MB

    def fused(self, lib, **kw):
        a = dict(parts=self.parts, n=self.n, rows=self.rows, hidden=self.hidden, dtype=self.dtype,
                 residual=self.residual, weight=self.weight, eps=1e-5, out=self.out,
                 res_out=self.res_out, cu=0)
        a.update(kw)
        parts = a["parts"]
        arr = None if parts is None else (ctypes.c_void_p * max(1, len(parts)))(*parts)
        return lib.tw_fused_reduce_rmsnorm(arr, a["n"], a["rows"], a["hidden"], a["dtype"],
                                           a["residual"], a["weight"], a["eps"], a["out"],
                                           a["res_out"], a["cu"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(parts=None), INV),
    (dict(n=0), INV),
    (dict(n=17), INV),
    (dict(rows=-1), INV),
    (dict(hidden=0), INV),
    (dict(hidden=-64), INV),
    (dict(eps=-1e-5), INV),
    (dict(eps=float("nan")), INV),
    (dict(eps=float("inf")), INV),
    (dict(cu=-1), INV),
    (dict(dtype=7), INV),
    (dict(residual=None), INV),
    (dict(weight=None), INV),
    (dict(out=None), INV),
    (dict(res_out=None), INV),
    (dict(hidden=12), UNS),                 # 24 bytes per row: not a multiple of 16
    (dict(hidden=16 * 64 * 8 * 8 + 8), UNS),  # row beyond the widest shape
    (dict(hidden=1 << 60), INV),            # byte count overflow
], ids=lambda v: str(v))
def test_fused_invalid_args(lib, kw, expect):
    st = Bufs().fused(lib, **kw)
    assert st == expect, (kw, st, twn.last_error())
    assert twn.last_error() != ""


def test_fused_null_partial_and_misaligned(lib):
    b = Bufs()
    assert b.fused(lib, parts=[b.parts[0], None]) == INV
    assert b.fused(lib, parts=[b.parts[0] + 8, b.parts[1]]) == UNS
    assert b.fused(lib, residual=b.residual + 2) == UNS
    assert b.fused(lib, weight=b.weight + 4) == UNS
    assert b.fused(lib, out=b.out + 8) == UNS
    assert b.fused(lib, res_out=b.res_out + 8) == UNS
    assert b.fused(lib, dtype=F32, hidden=6) == UNS     # 24 bytes


def test_fused_alias_rules(lib):
    b = Bufs()
    tensor = b.rows * b.hidden * 2
    assert b.fused(lib, out=b.parts[1]) == ALIAS
    assert b.fused(lib, out=b.residual) == ALIAS
    assert b.fused(lib, out=b.weight) == ALIAS
    assert b.fused(lib, out=b.res_out) == ALIAS
    assert b.fused(lib, out=b.residual + tensor - 16) == ALIAS       # partial overlap
    assert b.fused(lib, res_out=b.parts[0]) == ALIAS
    assert b.fused(lib, res_out=b.weight) == ALIAS
    assert b.fused(lib, res_out=b.residual + 16) == ALIAS            # shifted in-place
    # exact in-place residual update is allowed; rows == 0 is a no-op, so
    # these return OK without a HIP call
    assert b.fused(lib, res_out=b.residual, rows=0) == OK
    assert b.fused(lib, rows=0) == OK
    # partials may repeat (reading a buffer twice is harmless)
    assert b.fused(lib, parts=[b.parts[0], b.parts[0]], rows=0) == OK
    # adjacent (touching, not overlapping) buffers are fine
    assert b.fused(lib, out=b.residual + tensor, rows=0) == OK


def test_reduce_rmsnorm_copy_validation(lib):
    b = Bufs()
    arr = (ctypes.c_void_p * 2)(*b.parts)
    assert lib.tw_reduce(arr, 0, 4, 64, BF16, b.out, 0, None) == INV
    assert lib.tw_reduce(arr, 2, 4, 64, BF16, None, 0, None) == INV
    assert lib.tw_reduce(arr, 2, 4, 64, BF16, b.parts[1] + 16, 0, None) == ALIAS
    assert lib.tw_reduce(arr, 2, 0, 64, BF16, b.parts[1], 0, None) == OK  # in place, no-op
    assert lib.tw_reduce(arr, 2, 4, 60, BF16, b.out, 0, None) == UNS
    assert lib.tw_rmsnorm(None, 4, 64, BF16, b.residual, b.weight, 1e-5, b.out, b.res_out, 0,
                          None) == INV
    assert lib.tw_rmsnorm(b.parts[0], 4, 64, BF16, b.residual, b.weight, 1e-5, b.parts[0],
                          b.res_out, 0, None) == ALIAS
    assert lib.tw_rmsnorm(b.parts[0], 0, 64, BF16, b.residual, b.weight, 1e-5, b.out,
                          b.residual, 0, None) == OK
    assert lib.tw_stream_copy(b.parts[0], b.parts[1], 100, 0, None) == UNS
    assert lib.tw_stream_copy(b.parts[0], b.parts[0] + 16, 1024, 0, None) == ALIAS
    assert lib.tw_stream_copy(None, b.parts[1], 1024, 0, None) == INV
    assert lib.tw_stream_copy(b.parts[0], b.parts[1], 0, 0, None) == OK


def test_stream_mix_validation(lib):
    """Every check of tw_stream_mix fails before any HIP call.  The addresses
    are fake: a call expected to succeed passes bytes == 0 (a no-op), so no
    kernel is ever launched on them."""
    b = Bufs()
    base = 0x7F0000000000 + 4096 * MB
    srcs = [base + i * 64 * MB for i in range(17)]
    dsts = [base + (32 + j) * 64 * MB for j in range(16)]

    def call(s=srcs[:9], d=dsts[:2], n_src=None, n_dst=None, nbytes=0, cu=0):
        sa = None if s is None else (ctypes.c_void_p * max(1, len(s)))(*s)
        da = None if d is None else (ctypes.c_void_p * max(1, len(d)))(*d)
        n_src = len(s) if n_src is None else n_src
        n_dst = len(d) if n_dst is None else n_dst
        return lib.tw_stream_mix(sa, n_src, da, n_dst, nbytes, cu, None)
    assert call() == OK
    assert call(s=srcs, d=dsts) == OK                    # 17 sources, 16 destinations
    assert call(s=None, n_src=1) == INV
    assert call(d=None, n_dst=1) == INV
    assert call(n_src=0) == INV
    assert call(s=srcs + [srcs[0]]) == INV              # 18 sources
    assert call(n_dst=0) == INV
    assert call(d=dsts + [dsts[0]]) == INV              # 17 destinations
    assert call(nbytes=-16) == INV
    assert call(cu=-1) == INV
    assert call(s=[srcs[0], None]) == INV
    assert call(d=[dsts[0], None]) == INV
    assert call(nbytes=1000) == UNS
    assert call(s=[srcs[0] + 4]) == UNS
    assert call(d=[dsts[0] + 8]) == UNS
    assert call(s=[srcs[0], srcs[0]]) == OK                     # sources may coincide
    assert call(d=[srcs[1] + 1024], nbytes=4096) == ALIAS       # dst inside a src
    assert call(d=[dsts[0], dsts[0] + 2048], nbytes=4096) == ALIAS
    del b


def test_allgather_validation(lib):
    b = Bufs()
    tensor = b.rows * b.hidden * 2
    base = 0x7F0000000000 + 2048 * MB
    ag = [base + j * 64 * MB for j in range(4)]

    def call(ag_list=ag, n_ag=None, off=0, total=16, rows=b.rows, res_out=b.res_out, **kw):
        parts = (ctypes.c_void_p * 2)(*b.parts)
        arr = None if ag_list is None else (ctypes.c_void_p * max(1, len(ag_list)))(*ag_list)
        if n_ag is None:
            n_ag = 1 if ag_list is None else len(ag_list)
        return lib.tw_fused_reduce_rmsnorm_allgather(parts, 2, rows, b.hidden, BF16, b.residual,
                                                     b.weight, 1e-5, arr, n_ag, off, total,
                                                     res_out, 0, None)
    assert call(ag_list=None) == INV
    assert call(n_ag=0) == INV
    assert call(n_ag=17, ag_list=ag * 5) == INV
    assert call(ag_list=[ag[0], None]) == INV
    assert call(off=-1) == INV
    assert call(off=13, total=16) == INV              # 13 + 4 rows > 16
    assert call(off=0, total=3) == INV
    assert call(ag_list=[ag[0] + 8]) == UNS
    assert call(ag_list=[ag[0], ag[0] + 1024]) == ALIAS   # second starts inside the first (2 KiB)
    assert call(ag_list=[b.parts[1]]) == ALIAS
    assert call(ag_list=[b.residual - 16 * 64 * 2 + tensor]) == ALIAS
    assert call(ag_list=[b.weight]) == ALIAS
    assert call(ag_list=[b.res_out]) == ALIAS
    assert call(rows=0) == OK                       # validated no-op
    assert call(rows=0, off=12, total=12) == OK


def test_masked_stream_argument_checks(lib):
    h = ctypes.c_void_p()
    assert lib.tw_cu_masked_stream(8, None) == INV
    assert lib.tw_cu_masked_stream(0, ctypes.byref(h)) == INV
    assert lib.tw_cu_masked_stream(-3, ctypes.byref(h)) == INV
    assert lib.tw_cu_complement_stream(8, None) == INV
    assert lib.tw_cu_complement_stream(0, ctypes.byref(h)) == INV


def test_error_is_cleared_by_next_call(lib):
    b = Bufs()
    assert b.fused(lib, n=0) == INV
    assert twn.last_error() != ""
    assert b.fused(lib, rows=0) == OK
    assert twn.last_error() == ""


def test_shape_choice(lib):
    # (dtype, hidden, n) -> (waves, chunks per lane, team lanes)
    assert twn.query_fused_shape(F32, 64, 2) == (0, 0, 16)      # 16 chunks: narrow-row team
    assert twn.query_fused_shape(BF16, 8, 1) == (0, 0, 1)
    assert twn.query_fused_shape(BF16, 256, 3) == (0, 0, 32)
    assert twn.query_fused_shape(BF16, 8192, 8) == (4, 4, 0)     # measured shapes
    assert twn.query_fused_shape(BF16, 8192, 2) == (8, 2, 0)
    assert twn.query_fused_shape(BF16, 8192, 4) == (4, 4, 0)
    assert twn.query_fused_shape(BF16, 7168, 2) == (7, 2, 0)
    assert twn.query_fused_shape(BF16, 16384, 4) == (4, 8, 0)
    assert twn.query_fused_shape(BF16, 16384, 1) == (16, 2, 0)
    assert twn.query_fused_shape(BF16, 16384, 2) == (8, 4, 0)
    assert twn.query_fused_shape(BF16, 16384, 8) == (4, 8, 0)
    assert twn.query_fused_shape(BF16, 4096, 2) == (1, 8, 0)     # one wave per row
    assert twn.query_fused_shape(BF16, 4096, 4) == (8, 1, 0)
    assert twn.query_fused_shape(BF16, 4096, 8) == (1, 8, 0)
    assert twn.query_fused_shape(BF16, 12288, 8) == (4, 6, 0)
    assert twn.query_fused_shape(BF16, 5120, 4) == (4, 3, 0)     # default rule: 4 waves
    assert twn.query_fused_shape(BF16, 5120, 2) == (5, 2, 0)
    assert twn.query_fused_shape(BF16, 2048, 2) == (1, 4, 0)     # <= 256 chunks: one wave per row
    assert twn.query_fused_shape(BF16, 512, 8) == (1, 1, 0)
    assert twn.query_fused_shape(F32, 256, 2) == (1, 1, 0)
    assert twn.query_fused_shape(BF16, 768, 2) == (1, 2, 0)
    assert twn.query_fused_shape(BF16, 1536, 16) == (1, 3, 0)
    assert twn.query_fused_shape(F32, 1024, 8) == (1, 4, 0)
    assert twn.query_fused_shape(BF16, 3072, 8) == (1, 6, 0)     # measured mid widths
    assert twn.query_fused_shape(BF16, 3072, 6) == (4, 2, 0)     # 384 chunks: 4 waves, fewest slots
    assert twn.query_fused_shape(BF16, 3072, 4) == (6, 1, 0)
    assert twn.query_fused_shape(BF16, 2560, 8) == (5, 1, 0)
    assert twn.query_fused_shape(BF16, 2560, 12) == (4, 2, 0)
    assert twn.query_fused_shape(BF16, 3584, 16) == (1, 8, 0)
    assert twn.query_fused_shape(BF16, 3584, 5) == (4, 2, 0)
    w, k, t = twn.query_fused_shape(BF16, 5120, 4)
    assert t == 0 and w * 64 * k >= 640
    w, k, t = twn.query_fused_shape(BF16, 16 * 64 * 8 * 8, 2)   # the widest row
    assert (w, k) == (16, 8)
    # fewer rows than CUs: as many wavefronts as the row fills, fewest slots
    assert twn.query_fused_shape(BF16, 8192, 8, rows=1, cus=256) == (16, 1, 0)
    assert twn.query_fused_shape(BF16, 8192, 8, rows=255, cus=256) == (16, 1, 0)
    assert twn.query_fused_shape(BF16, 8192, 8, rows=256, cus=256) == (4, 4, 0)
    # on at most half of the CUs: the shapes measured for that regime
    assert twn.query_fused_shape(BF16, 8192, 8, rows=2048, cus=8) == (8, 2, 0)
    assert twn.query_fused_shape(BF16, 8192, 8, rows=2048, cus=128) == (8, 2, 0)
    assert twn.query_fused_shape(BF16, 8192, 8, rows=2048, cus=129) == (4, 4, 0)
    assert twn.query_fused_shape(BF16, 5120, 4, rows=4096, cus=32) == (10, 1, 0)
    assert twn.query_fused_shape(BF16, 5120, 16, rows=2048, cus=8) == (10, 1, 0)
    assert twn.query_fused_shape(BF16, 7168, 8, rows=2048, cus=32) == (7, 2, 0)
    assert twn.query_fused_shape(BF16, 7168, 16, rows=2048, cus=32) == (4, 4, 0)
    assert twn.query_fused_shape(BF16, 7168, 8, rows=2048, cus=256) == (4, 4, 0)
    assert twn.query_fused_shape(BF16, 12288, 3, rows=2048, cus=8) == (8, 3, 0)
    assert twn.query_fused_shape(BF16, 12288, 8, rows=2048, cus=8) == (4, 6, 0)
    assert twn.query_fused_shape(BF16, 4096, 4, rows=2048, cus=32) == (2, 4, 0)
    assert twn.query_fused_shape(BF16, 4096, 5, rows=2048, cus=32) == (8, 1, 0)
    assert twn.query_fused_shape(BF16, 4096, 2, rows=4096, cus=32) == (2, 4, 0)
    assert twn.query_fused_shape(BF16, 2048, 2, rows=4096, cus=32) == (1, 4, 0)   # none measured
    assert twn.query_fused_shape(BF16, 8192, 8, rows=64, cus=8, device_cus=8) == (4, 4, 0)
    assert twn.query_fused_shape(BF16, 5120, 4, rows=8, cus=256) == (10, 1, 0)
    assert twn.query_fused_shape(BF16, 4096, 2, rows=8, cus=256) == (8, 1, 0)
    assert twn.query_fused_shape(BF16, 16384, 2, rows=8, cus=256) == (16, 2, 0)
    assert twn.query_fused_shape(F32, 64, 2, rows=1, cus=256) == (0, 0, 16)   # still a team
    # CU-limited calls launch workgroups of at most 10 wavefronts
    assert twn.query_fused_shape(BF16, 8192, 8, rows=4, cus=8) == (10, 2, 0)
    assert twn.query_fused_shape(BF16, 5120, 4, rows=5, cus=16) == (10, 1, 0)
    assert twn.query_fused_shape(BF16, 16384, 5, rows=4096, cus=8) == (4, 8, 0)
    assert twn.query_fused_shape(BF16, 16384, 5, rows=4096, cus=256) == (4, 8, 0)
    assert twn.query_fused_shape(BF16, 40960, 2, rows=4, cus=8) == (10, 8, 0)
    with pytest.raises(twn.TwError, match="10 wavefronts"):
        twn.query_fused_shape(BF16, 40968, 2, rows=4, cus=8)
    with pytest.raises(twn.TwError):
        twn.query_fused_shape(F32, 20484, 2, rows=4, cus=8)
    assert twn.query_fused_shape(F32, 20480, 2, rows=4, cus=8) == (10, 8, 0)
    with pytest.raises(twn.TwError):
        twn.query_fused_shape(BF16, 8192, 8, rows=-1)
    with pytest.raises(twn.TwError):
        twn.query_fused_shape(BF16, 8192, 8, rows=4, cus=0)
    with pytest.raises(twn.TwError):
        twn.query_fused_shape(BF16, 8192, 8, rows=4, cus=300, device_cus=256)
    with pytest.raises(twn.TwError):
        twn.query_fused_shape(BF16, 12, 2)
    with pytest.raises(twn.TwError):
        twn.query_fused_shape(BF16, 1024, 17)
    # forced shapes
    twn.set_fused_shape(8, 2)
    try:
        assert twn.query_fused_shape(BF16, 8192, 8) == (8, 2, 0)
        with pytest.raises(twn.TwError):
            twn.query_fused_shape(BF16, 16384, 8)   # 8 x 64 x 2 < 2048 chunks
    finally:
        twn.set_fused_shape(0, 0)
    twn.set_fused_shape(16, 1)
    try:
        assert twn.query_fused_shape(BF16, 8192, 8, rows=4096, cus=256) == (16, 1, 0)
        with pytest.raises(twn.TwError, match="CU-limited"):
            twn.query_fused_shape(BF16, 8192, 8, rows=4096, cus=8)   # more than 10 wavefronts
        with pytest.raises(twn.TwError, match="CU-limited"):
            twn.query_fused_shape(BF16, 256, 8, rows=4, cus=8)     # narrow rows too
    finally:
        twn.set_fused_shape(0, 0)
    for bad in [(17, 1), (4, 5), (0, 2), (2, 0), (-1, 1), (4, 4, -1)]:
        with pytest.raises(twn.TwError):
            twn.set_fused_shape(*bad)


K_VALUES = [1, 2, 3, 4, 6, 8]


def _fit_table():
    """kFitMask[dtype][n][bucket] from the include the build generated out
    of the compiler's kernel-resource-usage remarks."""
    import numpy as np
    path = os.path.join(ROOT, "_build", "twnorm_fit_table.inc")
    if not os.path.exists(path):
        pytest.skip("build products not present")
    text = open(path).read()
    m = re.search(r"kFitMask\[2\]\[17\]\[3\] = \{(.*?)\n\};", text, re.S)
    return np.array([int(x) for x in re.findall(r"\d+", m.group(1))]).reshape(2, 17, 3)


def _bucket(w):
    return 0 if w <= 4 else (1 if w <= 8 else 2)


def test_auto_shapes_never_spill(lib):
    """Whenever some (waves, K) covering the row runs without scratch, the
    automatic choice is one of those."""
    mask = _fit_table()
    for dt, b in ((BF16, 2), (F32, 4)):
        for n in range(1, 17):
            for chunks in list(range(33, 200, 7)) + [256, 512, 640, 1000, 1024, 1025, 2048, 3072,
                                                      4096, 6000, 8192]:
                hidden = chunks * 16 // b
                w, k, t = twn.query_fused_shape(dt, hidden, n)
                assert t == 0 and w * 64 * k >= chunks and w <= 16
                free = [(-(-chunks // (64 * kk)), kk) for kk in K_VALUES
                        if -(-chunks // (64 * kk)) <= 16 and
                        (mask[dt][n][_bucket(-(-chunks // (64 * kk)))] >> K_VALUES.index(kk)) & 1]
                if free:
                    assert (mask[dt][n][_bucket(w)] >> K_VALUES.index(k)) & 1, (dt, n, hidden, w, k)


def test_last_error_is_per_thread(lib):
    """Each thread sees the detail of its own last failure (ctypes releases
    the GIL during the calls, so the threads run the library concurrently)."""
    import threading
    b = Bufs()
    results = {}

    def worker(tid):
        msgs = set()
        for i in range(400):
            if tid % 2 == 0:
                st = b.fused(lib, n=0)                     # n out of range
                want = "n must be in [1, 16]"
            else:
                st = b.fused(lib, hidden=12)               # 24-byte rows
                want = "multiple of 16"
            msg = twn.last_error()
            msgs.add((st, want in msg))
        results[tid] = msgs

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for tid, msgs in results.items():
        want_status = INV if tid % 2 == 0 else UNS
        assert msgs == {(want_status, True)}, (tid, msgs)


def test_shape_override_is_per_thread(lib):
    """tw_set_fused_shape applies to the calling thread only: another
    thread's shape choice (and so its calls) is unchanged."""
    import threading
    auto = twn.query_fused_shape(BF16, 8192, 8, rows=1024)
    seen = {}
    twn.set_fused_shape(2, 8)
    try:
        assert twn.query_fused_shape(BF16, 8192, 8, rows=1024) == (2, 8, 0)
        t = threading.Thread(target=lambda: seen.update(other=twn.query_fused_shape(BF16, 8192, 8,
                                                                                     rows=1024)))
        t.start()
        t.join()
    finally:
        twn.set_fused_shape(0, 0)
    assert seen["other"] == auto
    assert twn.query_fused_shape(BF16, 8192, 8, rows=1024) == auto


def test_shutdown_is_idempotent_and_final():
    """In a fresh process: tw_shutdown twice returns TW_OK, and afterwards
    the CU-masked stream queries refuse instead of creating queues again
    (checked before any HIP call, so no GPU is needed)."""
    import subprocess
    import sys
    code = ("import ctypes, reduce_residual_add_amd as t; L = t.load(); "
            "a = L.tw_shutdown(); b = L.tw_shutdown(); h = ctypes.c_void_p(); "
            "c = L.tw_cu_masked_stream(8, ctypes.byref(h)); "
            "d = L.tw_cu_complement_stream(8, ctypes.byref(h)); "
            "print(a, b, c, d, t.last_error())")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    a, b, c, d, *msg = r.stdout.strip().splitlines()[-1].split(" ")
    assert (int(a), int(b), int(c), int(d)) == (OK, OK, UNS, UNS)
    assert "tw_shutdown" in " ".join(msg)
