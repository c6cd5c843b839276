"""Shared helpers of the GPU parity tests: moving seeded storage arrays to
the device and back, the oracle's reference with per-element error bounds,
and the tolerance of the comparison.

Tolerance (the reading of "max abs error <= 2e-2 and max rel error <= 1e-2
for bf16, <= 1e-5 relative for fp32"):
  bf16: element passes iff |got - ref| <= max(2e-2, 1e-2 * |ref|)
  fp32: element passes iff |got - ref| <= 1e-5 * max(1, |ref|)
The literal conjunction cannot hold for any correct kernel: a relative bound
is meaningless at |ref| ~ 0, and one bf16 half-ulp above 8 is 0.031 > 2e-2.

Two stronger bf16 checks come on top:
  * one ulp: every bf16 result whose float32 error bound (below) is at most
    a quarter of a bf16 ulp of the exact value must lie within one bf16 ulp
    of the oracle's correctly rounded value.  The bound is computed per
    element from the inputs, so only results next to a cancellation -- where
    the specified float32 order legitimately moves a tiny result by several
    ulps -- are left to the tolerance alone, and they are counted;
  * exactness: in every comparison of at least 4096 outputs at least 99.9%
    must be exactly the correctly rounded value.

Float32 error bounds (u = 2^-24, the float32 unit roundoff), per element of
a row with N partials:
  residual_out: the kernel rounds N times (p_0 + ... + p_{N-1}, then + r),
    so |x_f32 - x| <= e_x = (N + 1) u (|r| + sum_i |p_i|).
  out = x * inv * w: the row's sum of squares is a sum of positive terms
    whose rounding depth is at most the chunk's elements + 6 butterfly levels
    + the row's 64-chunk groups; with the error of x it gives a relative
    error rel_ss <= (depth + 2) u + sum_j (2 |x_j| e_x + e_x^2) / sum_j x_j^2;
    the mean, eps, square root and reciprocal add at most 4 u, so
    rel_inv <= rel_ss / 2 + 4 u, and
    |out_f32 - out| <= |out| (rel_inv + 3 u) + inv |w| e_x (1 + rel_inv).
These bounds are checked on the CPU against a float32 model of the kernel's
order of operations (tests/test_helpers.py).
"""
import os

import numpy as np

from oracle import twnorm_oracle as O


def to_dev(arr, dtype, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def from_dev(t, dtype):
    import torch
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().astype(np.float32)


def inputs_to_dev(inp, device="cuda"):
    dt = inp["dtype"]
    parts = [to_dev(p, dt, device) for p in inp["partials"]]
    return parts, to_dev(inp["residual"], dt, device), to_dev(inp["weight"], dt, device)


U32 = 2.0 ** -24   # float32 unit roundoff


def bf16_ulp(v):
    """Spacing of the bf16 grid at |v| (2^-133 below the normal range)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, ex = np.frexp(np.where(np.isfinite(a), a, 1.0))
    e = np.maximum(ex.astype(np.int64) - 1, -126)
    return np.where(np.isfinite(a), np.ldexp(1.0, e - 7), np.inf)


def fp32_bounds(inp, ref_out, ref_res, rows=None):
    """Per-element bounds (float64 [rows, H]) on how far the kernel's float32
    results can lie from the exact out and residual_out (module docstring)."""
    dt = inp["dtype"]
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    mag = np.abs(O.decode(sel(inp["residual"]), dt))
    for p in inp["partials"]:
        mag = mag + np.abs(O.decode(sel(p), dt))
    n = len(inp["partials"])
    e_x = (n + 1) * U32 * mag
    x = np.asarray(ref_res, dtype=np.float64)
    h = x.shape[-1]
    elems = 8 if dt == "bf16" else 4
    chunks = h // elems
    depth = elems + 6 + (chunks + 63) // 64
    ss = np.sum(x * x, axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel_ss = (depth + 2) * U32 + np.sum(2 * np.abs(x) * e_x + e_x * e_x, axis=-1) / ss
        rel_ss = np.where(ss > 0, rel_ss, np.inf)
        rel_inv = rel_ss / 2 + 4 * U32
        inv = 1.0 / np.sqrt(ss / h + O.eps_as_passed(inp["eps"]))
    w = np.abs(O.decode(inp["weight"], dt))
    with np.errstate(invalid="ignore"):
        b_out = (np.abs(ref_out) * (rel_inv + 3 * U32)[..., None]
                 + (inv * (1 + rel_inv))[..., None] * w * e_x)
    b_out = np.where(np.isnan(b_out), np.inf, b_out)
    return b_out, e_x


def reference(inp, rows=None):
    """The oracle's float64 (out, residual_out) for `rows` (an index array
    or slice; all rows if None) of a storage dict, with their float32 error
    bounds: returns (out, res, bound_out, bound_res)."""
    dt = inp["dtype"]
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    out, res = O.fused([O.decode(sel(p), dt) for p in inp["partials"]],
                       O.decode(sel(inp["residual"]), dt), O.decode(inp["weight"], dt),
                       O.eps_as_passed(inp["eps"]))
    b_out, b_res = fp32_bounds(inp, out, res, rows)
    return out, res, b_out, b_res


def tolerance_report(got_storage, ref, dtype, bound=None):
    """Returns dict(fails, max_abs, max_rel, max_ulp, ...) for stored results
    vs float64 oracle values.  `bound` (bf16) is the per-element float32
    error bound that decides where the one-ulp check applies."""
    got = O.decode(got_storage, dtype)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    if dtype == "bf16":
        tol = np.maximum(2e-2, 1e-2 * np.abs(ref))
    else:
        tol = 1e-5 * np.maximum(1.0, np.abs(ref))
    big = np.abs(ref) >= 1.0
    rep = dict(fails=int(np.count_nonzero(~(d <= tol))),
               max_abs=float(d.max()) if d.size else 0.0,
               max_rel=float((d[big] / np.abs(ref[big])).max()) if np.any(big) else 0.0)
    if dtype == "bf16":
        rne = O.bf16_encode_rne(ref)
        dist = bf16_ulp_distance(got_storage, rne)
        # One ulp wherever float32 rounding provably stays below a quarter of
        # a bf16 ulp; elements next to a cancellation are left to the
        # tolerance above, and counted.
        if bound is None:
            well = np.ones(ref.shape, dtype=bool)
        else:
            well = np.asarray(bound) <= bf16_ulp(ref) / 4
        rep["max_ulp"] = int(dist[well].max()) if np.any(well) else 0
        rep["ulp_exempt"] = int(np.count_nonzero(~well))
        rep["max_ulp_all"] = int(dist.max()) if d.size else 0
        # share of outputs that are exactly the correctly rounded value
        rep["exact_frac"] = float(np.count_nonzero(dist == 0) / dist.size) if d.size else 1.0
        rep["n"] = int(d.size)
    return rep


def bf16_ulp_distance(a_bits, b_bits):
    """Distance in representable bf16 steps between two bit arrays."""
    def ordered(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), 0x8000 + u)
    return np.abs(ordered(np.asarray(a_bits)) - ordered(np.asarray(b_bits)))


def assert_parity(got_storage, ref, dtype, what="", bound=None):
    """Tolerance, one-ulp and exactness checks (module docstring).  bf16
    comparisons pass the float32 error bound of every element."""
    if dtype == "bf16" and bound is None:
        raise ValueError("bf16 parity needs the per-element float32 error bound")
    rep = tolerance_report(got_storage, ref, dtype, bound)
    if os.environ.get("TW_PRINT_EXACT"):
        print(f"EXACT {what} {rep.get('exact_frac')} n={rep.get('n')} "
              f"exempt={rep.get('ulp_exempt')} max_ulp_all={rep.get('max_ulp_all')}", flush=True)
    assert rep["fails"] == 0, f"{what}: {rep}"
    if dtype == "bf16":
        assert rep["max_ulp"] <= 1, f"{what}: more than one bf16 ulp from the oracle: {rep}"
        if rep["n"] >= 4096:
            assert rep["exact_frac"] >= 0.999, \
                f"{what}: fewer than 99.9% of outputs are the correctly rounded value: {rep}"
    return rep
