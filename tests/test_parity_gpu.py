"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle on
the same seeded inputs.  Needs an MI355X; every case prints what it runs
before touching the GPU."""
import os
import sys

import numpy as np
import pytest

import workloads
from oracle import twnorm_oracle as O
from gpu_helpers import (assert_parity, from_dev, inputs_to_dev, reference,
                         to_dev, tolerance_report)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _assert_rows(inp, out, res_out, what, rows=None):
    """Oracle parity of the given rows (all if None) of stored results."""
    ref_out, ref_res, b_out, b_res = reference(inp, rows)
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    assert_parity(sel(res_out), ref_res, inp["dtype"], f"{what} residual_out", b_res)
    assert_parity(sel(out), ref_out, inp["dtype"], f"{what} out", b_out)


def _assert_all_rows(inp, out, res_out, what, chunk=256):
    """Every row against the oracle, `chunk` rows at a time."""
    rows = inp["rows"]
    for a in range(0, rows, chunk):
        _assert_rows(inp, out, res_out, f"{what} rows {a}:{min(rows, a + chunk)}",
                     slice(a, min(rows, a + chunk)))


def _run_fused(twn, inp, n_cu_limit=0, in_place=False):
    import torch
    parts, res, w = inputs_to_dev(inp)
    out = torch.full_like(res, 7.0)
    res_out = res if in_place else torch.full_like(res, 7.0)
    twn.fused_reduce_rmsnorm(parts, res, w, inp["eps"], out=out, residual_out=res_out,
                             n_cu_limit=n_cu_limit)
    torch.cuda.synchronize()
    return from_dev(out, inp["dtype"]), from_dev(res_out, inp["dtype"])


# ---------------------------------------------------------------------------
# Every workload at its full size, every row against the oracle, in the
# launch configurations the benchmark times.  The outputs start as a 7.0
# sentinel, so a row the kernel skipped fails too.
# ---------------------------------------------------------------------------
CASES = [(w.name, cu) for w in workloads.WORKLOADS for cu in w.cu_limits]


@pytest.mark.parametrize("name,cu", CASES, ids=[f"{n}-cu{c}" for n, c in CASES])
def test_fused_full_size(twn, name, cu):
    w = workloads.get(name)
    _say(f"[fused full] {name} n={w.n} rows={w.rows} H={w.hidden} {w.dtype} n_cu_limit={cu}")
    inp = workloads.make(w, seed=0)
    out, res_out = _run_fused(twn, inp, n_cu_limit=cu)
    _assert_all_rows(inp, out, res_out, f"{name} cu{cu}")


# ---------------------------------------------------------------------------
# Smaller shapes the oracle checks in full: several tiles, ragged tails,
# every kernel shape (narrow-row teams, 1..16 waves, 1..8 chunks per lane).
# ---------------------------------------------------------------------------
SHAPES = [
    # (n, rows, hidden, dtype)
    (1, 5, 8, "bf16"),        # one chunk per row: team of 1 lane
    (2, 37, 64, "f32"),       # 16 chunks: team of 16
    (3, 33, 200, "bf16"),     # 25 chunks: team of 32, 7 idle lanes
    (2, 9, 256, "bf16"),      # 32 chunks
    (5, 17, 520, "bf16"),     # 65 chunks: first wide-row shape, ragged
    (4, 64, 1000, "f32"),     # 250 chunks
    (2, 129, 4096, "bf16"),
    (4, 50, 5120, "bf16"),    # 640 chunks
    (8, 40, 8192, "bf16"),
    (7, 23, 8200, "bf16"),    # 1025 chunks: one slot past a round shape
    (16, 11, 3072, "bf16"),   # the most partials
    (3, 13, 12288, "f32"),    # 3072 chunks, fp32
    (2, 3, 65536, "bf16"),    # the widest supported row
    (9, 1, 1024, "bf16"),     # a single row
    (2, 9, 7168, "bf16"),     # the measured shapes of other common widths
    (2, 5, 12288, "bf16"),
    (8, 3, 12288, "bf16"),
    (4, 3, 16384, "bf16"),
    (16, 2, 65536, "bf16"),   # the most partials on the widest row (every shape spills)
    (4, 3, 32768, "f32"),     # the widest fp32 row
]


@pytest.mark.parametrize("n,rows,hidden,dtype", SHAPES, ids=[f"n{a}-r{b}-h{c}-{d}" for a, b, c, d in SHAPES])
def test_fused_shapes(twn, n, rows, hidden, dtype):
    _say(f"[fused shape] n={n} rows={rows} H={hidden} {dtype} shape={twn.query_fused_shape(0 if dtype == 'bf16' else 1, hidden, n)}")
    inp = workloads.make_random(n, rows, hidden, dtype, seed=hidden + n)
    out, res_out = _run_fused(twn, inp)
    _assert_rows(inp, out, res_out, f"n={n} rows={rows} H={hidden} {dtype}")


@pytest.mark.parametrize("waves,k", [(16, 1), (8, 2), (4, 4), (6, 3), (3, 6), (2, 8), (1, 8), (5, 4)])
def test_fused_forced_shapes(twn, waves, k):
    """Every wide-row instantiation (both launch bounds) gives oracle parity."""
    import torch
    _say(f"[forced shape] waves={waves} k={k}")
    inp = workloads.make_random(8, 19, 4096, "bf16", seed=waves * 10 + k)
    twn.set_fused_shape(waves, k)
    try:
        out, res_out = _run_fused(twn, inp)
    finally:
        twn.set_fused_shape(0, 0)
    _assert_rows(inp, out, res_out, f"forced {waves}x{k}")
    del torch


# ---------------------------------------------------------------------------
# Unfused comparison path
# ---------------------------------------------------------------------------
def _row_slice(inp, sl):
    """The rows `sl` of a storage dict (the weight and eps unchanged)."""
    parts = [p[sl] for p in inp["partials"]]
    return dict(inp, partials=parts, residual=inp["residual"][sl], rows=parts[0].shape[0])


@pytest.mark.parametrize("name", ["tiny", "page1", "zero_padded", "shard70b"])
def test_unfused_pair(twn, name):
    """tw_reduce then tw_rmsnorm at the workload's full size (the pair the
    benchmark times), every row against the oracle."""
    import torch
    w = workloads.get(name)
    _say(f"[unfused] {name} rows={w.rows}")
    inp = workloads.make(w, seed=2)
    parts, res, wt = inputs_to_dev(inp)
    red = twn.reduce(parts)
    out, res_out = twn.rmsnorm(red, res, wt, inp["eps"])
    torch.cuda.synchronize()
    red_h, out_h, res_h = (from_dev(t, w.dtype) for t in (red, out, res_out))
    for a in range(0, w.rows, 512):
        sl = slice(a, min(w.rows, a + 512))
        part = _row_slice(inp, sl)
        # reduce alone: the stored sum of the partials (n - 1 float32 roundings)
        ref_red = O.reduce_from_storage(part)
        mag = sum(np.abs(O.decode(p, w.dtype)) for p in part["partials"])
        assert_parity(red_h[sl], ref_red, w.dtype, f"reduce rows {sl}", (w.n + 1) * 2.0 ** -24 * mag)
        # The pair's definition rounds the intermediate to the storage type
        # before the add + norm (it makes a round trip through HBM).  That
        # double rounding can exceed the tolerance against the fused
        # definition (e.g. 1/2 ulp of the sum plus 1/2 ulp of x near |x| = 4),
        # so the reference is the oracle's own reduce, stored, then its
        # add + norm.
        ref_out, ref_res = O.rmsnorm_from_storage(O.encode(ref_red, w.dtype), part)
        rep = tolerance_report(out_h[sl], ref_out, w.dtype)
        assert rep["fails"] == 0, (sl, rep)
        rep = tolerance_report(res_h[sl], ref_res, w.dtype)
        assert rep["fails"] == 0, (sl, rep)


def test_rmsnorm_alone(twn):
    """tw_rmsnorm on a seeded `reduced` tensor (not one the GPU produced)."""
    import torch
    _say("[rmsnorm alone]")
    inp = workloads.make_random(1, 77, 5120, "bf16", seed=99)
    red, res, wt = inputs_to_dev(inp)
    out, res_out = twn.rmsnorm(red[0], res, wt, inp["eps"])
    torch.cuda.synchronize()
    # the reduced tensor is the single "partial" of inp: the oracle's
    # rmsnorm_from_storage on it is the fused definition with n = 1
    ref_out, ref_res = O.rmsnorm_from_storage(inp["partials"][0], inp)
    _, _, b_out, b_res = reference(inp)
    assert_parity(from_dev(res_out, "bf16"), ref_res, "bf16", "residual_out", b_res)
    assert_parity(from_dev(out, "bf16"), ref_out, "bf16", "out", b_out)


# ---------------------------------------------------------------------------
# Zero-padded column partials: exact arithmetic makes these bit-exact
# ---------------------------------------------------------------------------
def test_zero_padded_bit_exact(twn):
    import torch
    w = workloads.get("zero_padded")
    _say("[zero-padded bit-exact] full size")
    inp = workloads.make(w, seed=0)
    parts, res, wt = inputs_to_dev(inp)
    red = twn.reduce(parts)
    out, res_out = twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"])
    torch.cuda.synchronize()
    block = w.hidden // w.n
    concat = np.concatenate([inp["partials"][i][:, i * block:(i + 1) * block] for i in range(w.n)], axis=1)
    # each column has one nonzero partial, so the sum is that partial exactly
    assert np.array_equal(from_dev(red, "bf16"), concat)
    # residual_out = RNE(p_k + r): float32 holds p_k + r exactly when the
    # exponents are within 15 of each other; check those elements bit-exactly
    pk = O.decode(concat, "bf16")
    r = O.decode(inp["residual"], "bf16")
    exact_sum = pk + r
    f32_exact = exact_sum.astype(np.float32).astype(np.float64) == exact_sum
    got = from_dev(res_out, "bf16")
    expect = O.bf16_encode_rne(exact_sum)
    assert f32_exact.mean() > 0.99
    assert np.array_equal(got[f32_exact], expect[f32_exact])


# ---------------------------------------------------------------------------
# Determinism: the same row gives the same bits under any sharding, CU limit,
# repetition or in-place choice.
# ---------------------------------------------------------------------------
def test_determinism(twn):
    import torch
    w = workloads.get("shard70b")
    _say("[determinism] shard70b")
    inp = workloads.make(w, seed=5, rows=512)
    parts, res, wt = inputs_to_dev(inp)
    base_out, base_res = twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"])
    torch.cuda.synchronize()
    b_out, b_res = from_dev(base_out, "bf16"), from_dev(base_res, "bf16")
    # repeated calls
    for _ in range(3):
        o, r = twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"])
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(o, "bf16"), b_out) and np.array_equal(from_dev(r, "bf16"), b_res)
    # CU limits (the same three the full-size tests use: a process may hold
    # at most three distinct limits)
    for cu in (8, 16, 32, 0, 256, 1000):
        _say(f"[determinism] n_cu_limit={cu}")
        o, r = twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"], n_cu_limit=cu)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(o, "bf16"), b_out), cu
        assert np.array_equal(from_dev(r, "bf16"), b_res), cu
    # calls queued directly on the library's CU-masked stream (no join)
    ms = twn.cu_masked_stream(16)
    with torch.cuda.stream(ms):
        o, r = twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"], n_cu_limit=16)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(o, "bf16"), b_out) and np.array_equal(from_dev(r, "bf16"), b_res)
    # token shards: row ranges through pointer offsets (views), stitched back
    cuts = [0, 1, 130, 131, 400, 512]
    out = torch.empty_like(res)
    res_out = torch.empty_like(res)
    for a, b in zip(cuts[:-1], cuts[1:]):
        twn.fused_reduce_rmsnorm([p[a:b] for p in parts], res[a:b], wt, inp["eps"],
                                 out=out[a:b], residual_out=res_out[a:b])
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(out, "bf16"), b_out)
    assert np.array_equal(from_dev(res_out, "bf16"), b_res)
    # in place residual update
    res2 = res.clone()
    o, r = twn.fused_reduce_rmsnorm(parts, res2, wt, inp["eps"], residual_out=res2)
    torch.cuda.synchronize()
    assert r.data_ptr() == res2.data_ptr()
    assert np.array_equal(from_dev(o, "bf16"), b_out)
    assert np.array_equal(from_dev(res2, "bf16"), b_res)


def test_rmsnorm_equals_fused_with_one_partial(twn):
    import torch
    _say("[rmsnorm == fused n=1]")
    inp = workloads.make_random(1, 64, 8192, "bf16", seed=3)
    parts, res, wt = inputs_to_dev(inp)
    o1, r1 = twn.rmsnorm(parts[0], res, wt, 1e-5)
    o2, r2 = twn.fused_reduce_rmsnorm(parts, res, wt, 1e-5)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(r1, r2)


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------
def test_zero_rows_is_noop(twn):
    import torch
    _say("[edge] rows=0")
    p = torch.zeros((0, 4096), dtype=torch.bfloat16, device="cuda")
    res = torch.zeros_like(p)
    w = torch.ones(4096, dtype=torch.bfloat16, device="cuda")
    out, res_out = twn.fused_reduce_rmsnorm([p, p], res, w, 1e-5)
    torch.cuda.synchronize()
    assert out.shape == (0, 4096)


def test_special_values(twn):
    """eps = 0 on an all-zero row gives NaN (0 * inf), as in the oracle; a NaN
    or inf in one row stays in that row; the paired worked-example rows come
    out as the hand-derived values."""
    import torch
    _say("[edge] special values")
    h = 64
    rows = 4
    p0 = np.zeros((rows, h), np.float32)
    p1 = np.zeros((rows, h), np.float32)
    r = np.zeros((rows, h), np.float32)
    # row 0: all zero -> NaN with eps = 0
    # row 1: hand-derived case, mean square 4 -> [1, -1, 1, 1] * w over 4 columns x 16
    r[1] = np.tile([1, 1, -1, 1], 16)
    p0[1] = np.tile([1, -3, 0, 0], 16)
    p1[1] = np.tile([0, 0, 3, 1], 16)
    # row 2: contains inf
    p0[2] = 1.0
    p0[2, 5] = np.inf
    # row 3: ordinary values
    p0[3] = np.linspace(-2, 2, h)
    for dt in ("f32", "bf16"):
        store = (lambda a: a) if dt == "f32" else (lambda a: O.bf16_encode_rne(a.astype(np.float64)))
        w = np.ones(h, np.float32)
        parts = [to_dev(store(p0), dt), to_dev(store(p1), dt)]
        out, res_out = twn.fused_reduce_rmsnorm(parts, to_dev(store(r), dt), to_dev(store(w), dt), 0.0)
        torch.cuda.synchronize()
        o = O.decode(from_dev(out, dt), dt)
        assert np.all(np.isnan(o[0]))
        assert np.array_equal(o[1], np.tile([1.0, -1.0, 1.0, 1.0], 16))
        assert np.all(np.isnan(o[2]) | (o[2] == 0))   # inf / inf -> NaN, finite / inf -> 0
        ref = O.rmsnorm(O.decode(store(p0[3:4]), dt), np.ones(h), 0.0)
        assert tolerance_report(from_dev(out, dt)[3:4], ref, dt)["fails"] == 0


def test_subnormal_inputs(twn):
    """bf16 subnormal residuals and partials are neither flushed nor
    rounded: float32 holds every bf16 subnormal and the sum of two of them
    exactly, so residual_out equals the oracle's value bit for bit; out is
    checked to the usual bar.  Whole chip and 8 CUs."""
    _say("[edge] subnormal inputs")
    rows, h = 6, 8192
    rng = np.random.default_rng(11)

    def subnormal_bits(hi):
        bits = rng.integers(1, hi, size=(rows, h)).astype(np.uint16)
        return bits | (rng.integers(0, 2, size=(rows, h)).astype(np.uint16) << 15)

    r = subnormal_bits(128)
    r[:, :8] = 0x3F80                       # a few ones, so no row's mean square is tiny
    p0 = subnormal_bits(64)
    p1 = np.zeros((rows, h), np.uint16)      # adding a zero partial is exact too
    p0[1] = 0                                # row 1: the residual alone
    inp = dict(partials=[p0, p1], residual=r, weight=np.full(h, 0x3F80, np.uint16), eps=1e-5,
               dtype="bf16", n=2, rows=rows, hidden=h)
    ref_out, ref_res = O.fused_from_storage(inp)
    for cu in (0, 8):
        out, res_out = _run_fused(twn, inp, n_cu_limit=cu)
        assert np.array_equal(res_out, O.bf16_encode_rne(ref_res)), f"residual_out at cu {cu}"
        assert np.array_equal(res_out[1], r[1])
        _assert_rows(inp, out, res_out, f"subnormal inputs cu{cu}")


def test_fourth_cu_limit_is_refused(twn):
    """A fourth distinct CU limit in one process is refused with a clear
    error before anything is enqueued (each limit holds a hardware queue)."""
    import torch
    _say("[cu limits] fourth distinct limit")
    inp = workloads.make_random(2, 8, 1024, "bf16", seed=1)
    parts, res, wt = inputs_to_dev(inp)
    for cu in (8, 16, 32):
        twn.fused_reduce_rmsnorm(parts, res, wt, 1e-5, n_cu_limit=cu)
    out = torch.zeros_like(res)
    with pytest.raises(twn.TwError, match="distinct CU masks"):
        twn.fused_reduce_rmsnorm(parts, res, wt, 1e-5, out=out, n_cu_limit=64)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out)) == 0
    # the three cached limits keep working
    twn.fused_reduce_rmsnorm(parts, res, wt, 1e-5, out=out, n_cu_limit=16)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out)) > 0


# ---------------------------------------------------------------------------
# AllGather store: every rank's shard lands in every rank's gather buffer
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,ranks", [("page1", 2), ("shard70b", 8), ("tiny", 2)])
def test_allgather_store_simulated_ranks(twn, name, ranks):
    """Token-boundary ReduceScatter -> add + norm -> AllGather on `ranks`
    simulated ranks: rank r owns rows [r*R, (r+1)*R) of the T-token sequence,
    reads only its rows of the partials and residual, and writes its
    normalised rows into all `ranks` gather buffers.  Afterwards every gather
    buffer holds the full normalised sequence, identical to normalising all T
    rows at once ("TokenWeave 策略详解", §3.2-§3.4)."""
    import torch
    w = workloads.get(name)
    rows_per_rank = w.rows   # each rank's full shard, as the benchmark times it
    T = rows_per_rank * ranks
    _say(f"[allgather] {name} ranks={ranks} T={T}")
    inp = workloads.make(w, seed=9, rows=T)
    parts, res, wt = inputs_to_dev(inp)
    sentinel = 3.0
    gathers = [torch.full((T, w.hidden), sentinel, dtype=res.dtype, device="cuda") for _ in range(ranks)]
    res_out = torch.empty_like(res)
    for r in range(ranks):
        sl = slice(r * rows_per_rank, (r + 1) * rows_per_rank)
        twn.fused_reduce_rmsnorm_allgather([p[sl] for p in parts], res[sl], wt, inp["eps"], gathers,
                                           r * rows_per_rank, residual_out=res_out[sl])
    torch.cuda.synchronize()
    g0 = from_dev(gathers[0], w.dtype)
    for g in gathers[1:]:
        assert torch.equal(g, gathers[0])
    _assert_all_rows(inp, g0, from_dev(res_out, w.dtype), "gathered", chunk=1024)
    # the same rows through the plain fused call give the same bits
    out_plain, _ = twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"])
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(out_plain, w.dtype), g0)


def test_allgather_store_leaves_other_rows(twn):
    import torch
    _say("[allgather] partial range")
    inp = workloads.make_random(3, 5, 8192, "bf16", seed=4)
    parts, res, wt = inputs_to_dev(inp)
    T = 16
    gathers = [torch.full((T, 8192), -2.0, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    twn.fused_reduce_rmsnorm_allgather(parts, res, wt, 1e-5, gathers, 7)
    torch.cuda.synchronize()
    ref_out, _, b_out, _ = reference(inp)
    for g in gathers:
        gh = from_dev(g, "bf16")
        assert_parity(gh[7:12], ref_out, "bf16", "written rows", b_out)
        untouched = np.concatenate([gh[:7], gh[12:]])
        assert np.all(untouched == O.bf16_encode_rne(np.array([-2.0]))[0])


AG_CASES = [
    # (n partials, rows, hidden, dtype, gather buffers, row offset, total rows, n_cu_limit)
    (2, 9, 4096, "bf16", 1, 0, 9, 0),          # one buffer: the plain fused call's store
    (5, 11, 8200, "bf16", 16, 13, 40, 0),      # the most gather buffers, ragged row
    (3, 37, 200, "bf16", 16, 3, 64, 0),        # narrow rows: the team kernel stores 16 times
    (4, 6, 3000, "f32", 5, 2, 8, 0),           # fp32
    (8, 300, 8192, "bf16", 8, 100, 2400, 8),   # on 8 CUs (persistent grid)
]


@pytest.mark.parametrize("case", AG_CASES, ids=lambda c: f"n{c[0]}-r{c[1]}-h{c[2]}-{c[3]}-ag{c[4]}-cu{c[7]}")
def test_allgather_store_shapes(twn, case):
    """The AllGather store across its shapes: 1-16 gather buffers, the wide-
    and narrow-row kernels, fp32, a CU limit.  Every gather buffer holds the
    normalised rows at the offset, against the oracle, and nothing else."""
    import torch
    n, rows, hidden, dtype, n_ag, off, total, cu = case
    _say(f"[allgather shapes] n={n} rows={rows} H={hidden} {dtype} buffers={n_ag} offset={off} cu={cu}")
    inp = workloads.make_random(n, rows, hidden, dtype, seed=700 + n_ag + hidden)
    parts, res, wt = inputs_to_dev(inp)
    tdt = res.dtype
    gathers = [torch.full((total, hidden), -2.0, dtype=tdt, device="cuda") for _ in range(n_ag)]
    res_out = twn.fused_reduce_rmsnorm_allgather(parts, res, wt, inp["eps"], gathers, off,
                                                 n_cu_limit=cu)
    torch.cuda.synchronize()
    ref_out, ref_res, b_out, b_res = reference(inp)
    assert_parity(from_dev(res_out, dtype), ref_res, dtype, "residual_out", b_res)
    minus2 = O.encode(np.array([-2.0]), dtype)[0]
    for j, g in enumerate(gathers):
        gh = from_dev(g, dtype)
        assert_parity(gh[off:off + rows], ref_out, dtype, f"gather buffer {j}", b_out)
        rest = np.concatenate([gh[:off], gh[off + rows:]])
        assert np.all(rest == minus2), f"gather buffer {j}: rows outside the shard were written"


def test_many_rows_per_workgroup(twn):
    """Rows far beyond the resident grid.  On the whole chip every row gets a
    workgroup of its own; on 8 CUs, and under a cap of one workgroup per CU,
    the grid is persistent and every workgroup walks tens to thousands of rows
    through the software-pipelined loop (the narrow-row kernel loops too).
    Every row of every run is checked against the oracle."""
    for n, rows, hidden, dtype in [(3, 20011, 1024, "bf16"), (2, 40000, 64, "f32")]:
        inp = workloads.make_random(n, rows, hidden, dtype, seed=rows)
        for cu, cap in ((0, 0), (8, 0), (0, 1)):
            _say(f"[many rows] n={n} rows={rows} H={hidden} {dtype} n_cu_limit={cu} cap={cap}")
            twn.set_fused_shape(0, 0, cap)
            try:
                out, res_out = _run_fused(twn, inp, n_cu_limit=cu)
            finally:
                twn.set_fused_shape(0, 0, 0)
            _assert_all_rows(inp, out, res_out, f"many rows n={n} cu{cu} cap{cap}", chunk=4096)


def test_decode_rows_on_cu_limits(twn):
    """Decode-sized calls (fewer rows than the CU limit) on 8 and 16 CUs: one
    workgroup of at most 10 wavefronts per row.  Every row against the oracle,
    and bit-identical to the whole-chip call, which uses 16 wavefronts."""
    cases = [(8, 1, 8192, 8), (8, 7, 8192, 8), (4, 5, 5120, 16), (2, 3, 4096, 8),
             (2, 15, 16384, 16), (3, 2, 40960, 8)]
    for i, (n, rows, hidden, cu) in enumerate(cases):
        _say(f"[decode on CUs] n={n} rows={rows} H={hidden} n_cu_limit={cu}")
        inp = workloads.make_random(n, rows, hidden, "bf16", seed=500 + i)
        out_cu, res_cu = _run_fused(twn, inp, n_cu_limit=cu)
        _assert_rows(inp, out_cu, res_cu, f"decode rows={rows} H={hidden} cu{cu}")
        out0, res0 = _run_fused(twn, inp)
        assert np.array_equal(out_cu, out0) and np.array_equal(res_cu, res0)


def test_cu_limited_call_refuses_rows_past_its_workgroups(twn):
    """A CU-limited call on rows wider than 10 wavefronts can cover returns
    TW_ERR_UNSUPPORTED and writes nothing; the whole-chip call takes them."""
    import torch
    _say("[cu limit] 65536-wide rows refused on 8 CUs")
    inp = workloads.make_random(2, 3, 65536, "bf16", seed=17)
    parts, res, wt = inputs_to_dev(inp)
    out = torch.full_like(res, 7.0)
    res_out = torch.full_like(res, 7.0)
    with pytest.raises(twn.TwError, match="10 wavefronts"):
        twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"], out=out, residual_out=res_out,
                                 n_cu_limit=8)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((res_out == 7.0).all())


def test_same_partial_twice(twn):
    """Passing one buffer twice sums it twice (reads may repeat)."""
    import torch
    _say("[same partial twice]")
    inp = workloads.make_random(1, 33, 4096, "bf16", seed=8)
    parts, res, wt = inputs_to_dev(inp)
    out, res_out = twn.fused_reduce_rmsnorm([parts[0], parts[0]], res, wt, 1e-5)
    torch.cuda.synchronize()
    twice = dict(inp, partials=[inp["partials"][0], inp["partials"][0]], n=2)
    _assert_rows(twice, from_dev(out, "bf16"), from_dev(res_out, "bf16"), "same partial twice")


def test_results_unchanged_beside_a_gemm(twn):
    """Fused calls on a CU-masked stream while a hipBLASLt GEMM runs on
    another stream (the two-split overlap): the fused results match the
    oracle and are bit-identical to a solo run, and the GEMM's results are
    bit-identical to its solo run.  Uses the 32-CU mask the other tests
    already hold (a process may hold three); the 128-CU split the benchmark
    reports runs in a fresh process (test_two_split_overlap_at_128_cus)."""
    import torch
    _say("[overlap] fused on 32 CUs beside a GEMM")
    w = workloads.get("shard70b")
    inp = workloads.make(w, seed=12, rows=512)
    parts, res, wt = inputs_to_dev(inp)
    a = torch.randn(1024, 3584, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(3584, 8192, device="cuda", dtype=torch.bfloat16)
    solo_c = torch.matmul(a, b)
    solo_out, solo_res = twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"])
    torch.cuda.synchronize()
    _assert_rows(inp, from_dev(solo_out, "bf16"), from_dev(solo_res, "bf16"), "solo")
    ms = twn.cu_masked_stream(32)
    side = torch.cuda.Stream()
    outs = []
    with torch.cuda.stream(side):
        cs = [torch.matmul(a, b) for _ in range(4)]
    with torch.cuda.stream(ms):
        for _ in range(4):
            outs.append(twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"], n_cu_limit=32))
    torch.cuda.synchronize()
    for o, r in outs:
        assert torch.equal(o, solo_out) and torch.equal(r, solo_res)
    for c in cs:
        assert torch.equal(c, solo_c)


def test_two_split_overlap_at_128_cus(twn):
    """The split the benchmark reports: fused calls for one token split on
    the first 128 CUs, the other split's GEMM either unmasked beside them or
    on the 128 complementary CUs.  Runs in a fresh process, which holds only
    those two CU masks; every overlapped fused result is checked against the
    oracle there, and every GEMM against its solo run."""
    import subprocess
    import os
    child = os.path.join(os.path.dirname(os.path.abspath(__file__)), "overlap_split_child.py")
    _say("[overlap] 128-CU split in a child process")
    r = subprocess.run([sys.executable, "-u", child, "128"], capture_output=True, text=True,
                       timeout=600)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "OVERLAP_OK k=128" in r.stdout


def test_graph_capture_replays(twn):
    """The entry points allocate nothing and never synchronise, so a caller
    can capture them in a HIP graph.  Three fused calls (and one unfused
    pair) are captured, then replayed several times with eager work between
    replays; every replay must reproduce the eager results bit for bit."""
    import torch
    _say("[graph] capture + replays")
    w = workloads.get("shard70b")
    inp = workloads.make(w, seed=21, rows=96)
    parts, res, wt = inputs_to_dev(inp)
    eager_out, eager_res = twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"])
    eager_red = twn.reduce(parts)
    eager_out2, _ = twn.rmsnorm(eager_red, res, wt, inp["eps"])
    torch.cuda.synchronize()
    outs = [torch.empty_like(res) for _ in range(3)]
    ress = [torch.empty_like(res) for _ in range(3)]
    red = torch.empty_like(res)
    out2 = torch.empty_like(res)
    res2 = torch.empty_like(res)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the graph
        twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"], out=outs[0], residual_out=ress[0])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(3):
            twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"], out=outs[i], residual_out=ress[i])
        twn.reduce(parts, out=red)
        twn.rmsnorm(red, res, wt, inp["eps"], out=out2, residual_out=res2)
    for rep in range(4):
        for t in outs + ress + [red, out2, res2]:
            t.fill_(-1.0)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(outs[i], eager_out), (rep, i)
            assert torch.equal(ress[i], eager_res), (rep, i)
        assert torch.equal(red, eager_red) and torch.equal(out2, eager_out2), rep


def test_graph_capture_of_cu_limited_call(twn):
    """A CU-limited call (event join to the 8-CU stream) captured in a HIP
    graph replays with the whole-chip result's bits, on the capturing stream
    (not confined to the 8 CUs: graph nodes carry no CU mask) and on the
    masked stream itself (confined to them)."""
    import torch
    _say("[graph] CU-limited call captured and replayed")
    inp = workloads.make_random(8, 300, 8192, "bf16", seed=23)
    parts, res, wt = inputs_to_dev(inp)
    ref_out, ref_res = twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"])
    out = torch.empty_like(res)
    rout = torch.empty_like(res)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the graph (creates the masked stream)
        twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"], out=out, residual_out=rout,
                                 n_cu_limit=8)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"], out=out, residual_out=rout,
                                 n_cu_limit=8)
    for rep in range(3):
        out.fill_(-1.0)
        rout.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(rout, ref_res), rep
    # replayed on the masked stream itself, where the CU limit holds
    masked = twn.cu_masked_stream(8)
    for rep in range(2):
        out.fill_(-1.0)
        rout.fill_(-1.0)
        torch.cuda.synchronize()
        with torch.cuda.stream(masked):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(rout, ref_res), ("masked", rep)
    _assert_rows(inp, from_dev(out, "bf16"), from_dev(rout, "bf16"), "graph replay on 8 CUs")


@pytest.mark.parametrize("n", list(range(1, 17)))
def test_every_partial_count(twn, n):
    """Each partial count is its own kernel instantiation: run every one of
    them on the wide-row bf16 and fp32 kernels and on the narrow-row kernel."""
    _say(f"[every n] n={n}")
    for rows, hidden, dtype in [(7, 8192, "bf16"), (5, 1536, "f32"), (9, 128, "bf16"), (3, 40, "f32")]:
        inp = workloads.make_random(n, rows, hidden, dtype, seed=100 * n + hidden)
        out, res_out = _run_fused(twn, inp)
        _assert_rows(inp, out, res_out, f"n={n} H={hidden} {dtype}")


@pytest.mark.parametrize("n", list(range(1, 17)))
def test_reduce_every_partial_count(twn, n):
    """tw_reduce, the unfused path's first kernel, is instantiated per partial
    count and format: every one against the oracle's stored sum, on totals
    that end inside a block (5 x 1000 bf16, 3 x 1540 fp32), with the output
    written over the first partial in the last case (an exact alias the ABI
    allows)."""
    import torch
    _say(f"[reduce every n] n={n}")
    for rows, hidden, dtype, in_place in [(5, 1000, "bf16", False), (3, 1540, "f32", False),
                                          (4, 2056, "bf16", True)]:
        inp = workloads.make_random(n, rows, hidden, dtype, seed=300 * n + hidden)
        parts, _, _ = inputs_to_dev(inp)
        red = twn.reduce(parts, out=parts[0] if in_place else None)
        torch.cuda.synchronize()
        if in_place:
            assert red.data_ptr() == parts[0].data_ptr()
        ref = O.reduce_from_storage(inp)
        mag = sum(np.abs(O.decode(p, dtype)) for p in inp["partials"])
        bound = (n + 1) * 2.0 ** -24 * mag if dtype == "bf16" else None
        assert_parity(from_dev(red, dtype), ref, dtype, f"reduce n={n} H={hidden} {dtype}", bound)


# ---------------------------------------------------------------------------
# Traffic-pattern measurement aid (not part of the method): every destination
# word is the wrap-around uint32 sum of the source words; bytes past the end
# stay untouched.  Checked against numpy integer arithmetic.
# ---------------------------------------------------------------------------
MIX_CASES = [
    # (n_src, n_dst, bytes, n_cu_limit)
    (1, 1, 4096, 0),                   # less than one block
    (3, 2, 3 * 16384 + 48, 0),         # ragged last block, 4-slot layout
    (9, 2, (16 << 20) + 16, 0),        # the shard70b pattern, one chunk past
    (10, 3, 5 * 8192 + 4080, 0),       # 2-slot layout, ragged
    (17, 2, 1 << 20, 0),               # the most sources
    (9, 2, (2 << 20) + 512, 8),        # CU-limited persistent grid
]


@pytest.mark.parametrize("n_src,n_dst,nbytes,cu", MIX_CASES,
                         ids=[f"s{a}-d{b}-{c}B-cu{d}" for a, b, c, d in MIX_CASES])
def test_stream_mix_sums_words(twn, n_src, n_dst, nbytes, cu):
    import torch
    _say(f"[stream mix] n_src={n_src} n_dst={n_dst} bytes={nbytes} n_cu_limit={cu}")
    words = nbytes // 4
    rng = np.random.default_rng(1000 * n_src + n_dst)
    host = [rng.integers(0, 2 ** 32, size=words, dtype=np.uint32) for _ in range(n_src)]
    want = np.zeros(words, dtype=np.uint32)
    for h in host:
        want += h                       # wraps modulo 2**32
    srcs = [torch.from_numpy(h.view(np.int32)).cuda() for h in host]
    guard = 64
    full = [torch.full((words + guard,), 7, dtype=torch.int32, device="cuda") for _ in range(n_dst)]
    dsts = [f[:words] for f in full]
    twn.stream_mix(srcs, dsts, n_cu_limit=cu)
    torch.cuda.synchronize()
    for j, f in enumerate(full):
        got = f.cpu().numpy().view(np.uint32)
        assert np.array_equal(got[:words], want), f"dsts[{j}] differs"
        assert (got[words:] == 7).all(), f"dsts[{j}] written past its end"


# ---------------------------------------------------------------------------
# The order of the sum of squares depends on the row width alone: every
# launch shape (wavefronts x chunk slots, and the narrow-row kernel) gives
# bit-identical results.  This is what lets the shape follow the row count
# without breaking batch invariance.
# ---------------------------------------------------------------------------
INVARIANCE_CASES = [
    # (n, rows, hidden, dtype)
    (8, 6, 8192, "bf16"),     # 1024 chunks, 16 groups
    (5, 4, 8200, "bf16"),     # 1025 chunks: a one-chunk last group
    (4, 5, 5120, "bf16"),     # 640 chunks
    (2, 7, 4096, "f32"),      # 1024 chunks of fp32
    (3, 9, 200, "bf16"),      # 25 chunks: the narrow-row kernel by default
    (2, 3, 1000, "f32"),      # 250 chunks, ragged last group
    (2, 6, 296, "bf16"),      # 37 chunks: one wave per row, one ragged group
    (8, 3, 3072, "bf16"),     # 384 chunks: a measured one-wave shape (1 x 6)
]


@pytest.mark.parametrize("n,rows,hidden,dtype", INVARIANCE_CASES,
                         ids=[f"n{a}-r{b}-h{c}-{d}" for a, b, c, d in INVARIANCE_CASES])
def test_results_independent_of_launch_shape(twn, n, rows, hidden, dtype):
    import torch
    inp = workloads.make_random(n, rows, hidden, dtype, seed=7 * hidden + n)
    chunks = hidden * (2 if dtype == "bf16" else 4) // 16
    auto = twn.query_fused_shape(0 if dtype == "bf16" else 1, hidden, n)
    _say(f"[shape invariance] n={n} rows={rows} H={hidden} {dtype} auto={auto}")
    ref_out, ref_res = _run_fused(twn, inp)
    tried = 0
    for waves in (1, 2, 3, 4, 5, 8, 16):
        for k in (1, 2, 3, 4, 6, 8):
            if waves * 64 * k < chunks or waves * 64 * k > 4 * max(chunks, 64) + 64 * 8:
                continue
            _say(f"  forced waves={waves} k={k}")
            twn.set_fused_shape(waves, k)
            try:
                out, res_out = _run_fused(twn, inp)
            finally:
                twn.set_fused_shape(0, 0)
            assert np.array_equal(res_out, ref_res), f"residual_out differs at {waves}x{k}"
            assert np.array_equal(out.view(np.uint8), ref_out.view(np.uint8)), \
                f"out differs at {waves}x{k} (auto {auto})"
            tried += 1
    assert tried >= 3
    torch.cuda.synchronize()
    _assert_rows(inp, ref_out, ref_res, "automatic shape")


# ---------------------------------------------------------------------------
# Tensors past 4 GiB: row offsets beyond 32 bits.  A seeded 1024-row tile is
# repeated on the device (data movement only), so every tile of the outputs
# must be bit-identical to the first (rows depend on nothing but their own
# data); the first tile is checked in full against the oracle, so every row,
# on both sides of the 4 GiB boundary, is covered.
# ---------------------------------------------------------------------------
def test_fused_tensors_beyond_4gib(twn):
    import torch
    n, hidden, block = 2, 8192, 1024
    rows = 266240                      # 260 tiles x 16 KiB rows = 4.06 GiB per tensor
    need = (n + 3) * rows * hidden * 2
    free, _ = torch.cuda.mem_get_info()
    if free < need + (4 << 30):
        pytest.skip(f"needs {need / 2**30:.1f} GiB of free device memory")
    _say(f"[beyond 4 GiB] n={n} rows={rows} H={hidden} bf16 ({need / 2**30:.1f} GiB)")
    inp = workloads.make_random(n, block, hidden, "bf16", seed=44)
    reps = rows // block
    assert reps * block == rows and (rows - block) * hidden * 2 > (1 << 32)
    parts = [to_dev(p, "bf16").repeat(reps, 1) for p in inp["partials"]]
    res = to_dev(inp["residual"], "bf16").repeat(reps, 1)
    wt = to_dev(inp["weight"], "bf16")
    out = torch.full_like(res, 7.0)
    res_out = torch.full_like(res, 7.0)
    twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"], out=out, residual_out=res_out)
    torch.cuda.synchronize()
    o_tiles = out.view(reps, block, hidden)
    r_tiles = res_out.view(reps, block, hidden)
    for t in range(1, reps):
        assert torch.equal(o_tiles[t], o_tiles[0]), f"out tile {t} differs from tile 0"
        assert torch.equal(r_tiles[t], r_tiles[0]), f"residual_out tile {t} differs from tile 0"
    _assert_rows(inp, from_dev(o_tiles[0], "bf16"), from_dev(r_tiles[0], "bf16"), "tile 0")
    del parts, res, out, res_out, o_tiles, r_tiles
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Host threads: several threads issue fused calls concurrently, each on its
# own stream; every result is bit-identical to the single-threaded one.
# ---------------------------------------------------------------------------
def test_concurrent_host_threads(twn):
    import threading
    import torch
    _say("[threads] 4 host threads x 20 calls, own streams")
    cases = [workloads.make_random(n, rows, h, "bf16", seed=90 + n)
             for n, rows, h in ((2, 64, 4096), (4, 33, 5120), (8, 300, 8192), (3, 7, 200))]
    dev = [inputs_to_dev(c) for c in cases]
    ref = []
    for c, (parts, res, wt) in zip(cases, dev):
        o, r = twn.fused_reduce_rmsnorm(parts, res, wt, c["eps"])
        torch.cuda.synchronize()
        ref.append((from_dev(o, "bf16"), from_dev(r, "bf16")))
    errors = []

    def worker(i):
        try:
            c, (parts, res, wt) = cases[i], dev[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [twn.fused_reduce_rmsnorm(parts, res, wt, c["eps"]) for _ in range(20)]
            s.synchronize()
            for o, r in outs:
                if not (np.array_equal(from_dev(o, "bf16"), ref[i][0])
                        and np.array_equal(from_dev(r, "bf16"), ref[i][1])):
                    errors.append(f"thread {i}: result differs")
                    return
        except Exception as e:  # reported below
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors


# ---------------------------------------------------------------------------
# A seeded sweep of random configurations: partial count, dtype, width (any
# multiple of 16 bytes up to the widest row), row count and in-place use,
# each checked element by element against the oracle.
# ---------------------------------------------------------------------------
def _random_configs(count, seed, rows_lo, rows_hi, wide_top=2048, cu_choices=(0,)):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        dtype = "bf16" if rng.random() < 0.75 else "f32"
        per_chunk = 8 if dtype == "bf16" else 4
        max_chunks = (64 * 1024 if dtype == "bf16" else 32 * 1024) // per_chunk
        # widths spread over every scale: mostly up to wide_top chunks, some wider
        top = max_chunks if rng.random() < 0.15 else wide_top
        chunks = max(1, int(np.exp(rng.uniform(0, np.log(top)))))
        cu = int(rng.choice(cu_choices))
        if chunks > 10 * 64 * 8:   # wider than a CU-limited call's workgroups take
            cu = 0
        out.append((int(rng.integers(1, 17)), int(rng.integers(rows_lo, rows_hi + 1)),
                    chunks * per_chunk, dtype, bool(rng.random() < 0.3), cu))
    return out


# TW_RANDOM_SCALE=k multiplies both sweeps' case counts (one-off extended runs)
_SCALE = max(1, int(os.environ.get("TW_RANDOM_SCALE", "1")))
# decode-sized calls (fewer rows than CUs) on the whole chip
RANDOM_CASES = _random_configs(120 * _SCALE, 2024, 1, 48)
# calls of several hundred rows, on the whole chip or on 8 or 32 CUs
RANDOM_WIDE_CASES = _random_configs(24 * _SCALE, 4048, 256, 700, wide_top=1536,
                                    cu_choices=(0, 0, 8, 32))


def _run_random_cases(twn, cases, seed0, label):
    _say(f"[{label}] {len(cases)} cases")
    for i, (n, rows, hidden, dtype, in_place, cu) in enumerate(cases):
        _say(f"  case {i}: n={n} rows={rows} H={hidden} {dtype} in_place={in_place} cu={cu}")
        inp = workloads.make_random(n, rows, hidden, dtype, seed=seed0 + i)
        out, res_out = _run_fused(twn, inp, n_cu_limit=cu, in_place=in_place)
        _assert_rows(inp, out, res_out, f"{label} case {i}")


def test_fused_random_configs(twn):
    _run_random_cases(twn, RANDOM_CASES, 10_000, "random configs")


def test_fused_random_configs_many_rows(twn):
    _run_random_cases(twn, RANDOM_WIDE_CASES, 20_000, "random configs, many rows")


# ---------------------------------------------------------------------------
# The binding refuses mismatched GPU tensors before anything is enqueued.
# ---------------------------------------------------------------------------
def test_binding_rejects_mismatched_tensors(twn):
    import torch
    _say("[binding] mismatched tensors")
    inp = workloads.make_random(3, 8, 1024, "bf16", seed=5)
    parts, res, wt = inputs_to_dev(inp)
    out = torch.zeros_like(res)
    bad = [
        dict(partials=[parts[0], parts[1].float(), parts[2]]),                  # dtype
        dict(partials=[parts[0], parts[1][:4], parts[2]]),                       # shape
        dict(partials=[parts[0], parts[1].t().contiguous().t(), parts[2]]),      # layout
        dict(weight=wt[:512]),                                                   # weight shape
        dict(weight=wt.float()),                                                 # weight dtype
        dict(residual_out=torch.zeros(8, 1024, dtype=torch.bfloat16)),           # host tensor
        dict(partials=[]),                                                       # no partials
    ]
    for i, kw in enumerate(bad):
        args = dict(partials=parts, residual=res, weight=wt, out=out, residual_out=None)
        args.update(kw)
        with pytest.raises((ValueError, TypeError)):
            twn.fused_reduce_rmsnorm(args["partials"], args["residual"], args["weight"], 1e-5,
                                     out=args["out"], residual_out=args["residual_out"])
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out)) == 0


def test_concurrent_threads_with_cu_limits(twn):
    """Three host threads issue CU-limited calls (8, 16 and 32 CUs: masked
    streams created and joined concurrently) on their own streams; every
    result is bit-identical to the whole-chip result."""
    import threading
    import torch
    _say("[threads] CU-limited calls from 3 threads")
    inp = workloads.make_random(8, 96, 8192, "bf16", seed=77)
    parts, res, wt = inputs_to_dev(inp)
    o_ref, r_ref = twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"])
    torch.cuda.synchronize()
    ref = (from_dev(o_ref, "bf16"), from_dev(r_ref, "bf16"))
    errors = []

    def worker(cu):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"], n_cu_limit=cu)
                        for _ in range(10)]
            s.synchronize()
            for o, r in outs:
                if not (np.array_equal(from_dev(o, "bf16"), ref[0]) and np.array_equal(from_dev(r, "bf16"), ref[1])):
                    errors.append(f"cu {cu}: result differs")
                    return
        except Exception as e:  # reported below
            errors.append(f"cu {cu}: {e!r}")

    threads = [threading.Thread(target=worker, args=(cu,)) for cu in (8, 16, 32)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors


@pytest.mark.parametrize("nbytes,cu", [(16, 0), (4096 + 16, 0), ((1 << 20) + 48, 0), ((3 << 20) + 4080, 8)],
                         ids=["16B", "4KiB+16", "1MiB+48", "3MiB+4080-cu8"])
def test_stream_copy_copies_bytes(twn, nbytes, cu):
    """The plain-copy measurement aid (used to scale the hardware counters)
    copies every byte and nothing past the end."""
    import torch
    _say(f"[stream copy] bytes={nbytes} n_cu_limit={cu}")
    rng = np.random.default_rng(nbytes)
    src_h = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    src = torch.from_numpy(src_h).cuda()
    full = torch.full((nbytes + 256,), 7, dtype=torch.uint8, device="cuda")
    twn.stream_copy(src, full[:nbytes], n_cu_limit=cu)
    torch.cuda.synchronize()
    got = full.cpu().numpy()
    assert np.array_equal(got[:nbytes], src_h)
    assert (got[nbytes:] == 7).all()


def test_grid_cap_changes_no_bit(twn):
    """A persistent whole-chip grid capped at 1 or 2 workgroups per CU (each
    workgroup walks several rows through the pipelined loop) gives the same
    bits as the default grid of one workgroup per row."""
    import torch
    _say("[grid cap] 1 and 2 workgroups per CU")
    inp = workloads.make_random(8, 700, 8192, "bf16", seed=31)
    ref_out, ref_res = _run_fused(twn, inp)
    for cap in (1, 2):
        twn.set_fused_shape(0, 0, cap)
        try:
            out, res_out = _run_fused(twn, inp)
        finally:
            twn.set_fused_shape(0, 0, 0)
        assert np.array_equal(out, ref_out) and np.array_equal(res_out, ref_res), f"cap {cap}"
    torch.cuda.synchronize()
