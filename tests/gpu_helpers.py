"""Shared helpers of the GPU parity tests: moving seeded storage arrays to
the device and back, and the tolerance of the comparison.

Tolerance (the reading of "max abs error <= 2e-2 and max rel error <= 1e-2
for bf16, <= 1e-5 relative for fp32"):
  bf16: element passes iff |got - ref| <= max(2e-2, 1e-2 * |ref|)
  fp32: element passes iff |got - ref| <= 1e-5 * max(1, |ref|)
The literal conjunction cannot hold for any correct kernel: a relative bound
is meaningless at |ref| ~ 0, and one bf16 half-ulp above 8 is 0.031 > 2e-2.
Every bf16 result of at least 1/256 of the array's largest magnitude is also
checked to lie within one bf16 ulp of the oracle's correctly rounded value
(float32 accumulation error is far below half an ulp there, so only
rounding-boundary cases may differ by one; tinier results can sit next to a
cancellation, where float32 order legitimately moves them by several ulps at
~1e-8 absolute), and in every
comparison of at least 4096 outputs at least 99.9% of them must be exactly
that correctly rounded value (the chance that float32 error crosses a bf16
rounding boundary is of order 1e-4 per output).
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


def tolerance_report(got_storage, ref, dtype):
    """Returns dict(fails, max_abs, max_rel, max_ulp) for stored results vs
    float64 oracle values."""
    got = O.decode(got_storage, dtype)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    if dtype == "bf16":
        bound = np.maximum(2e-2, 1e-2 * np.abs(ref))
    else:
        bound = 1e-5 * np.maximum(1.0, np.abs(ref))
    big = np.abs(ref) >= 1.0
    rep = dict(fails=int(np.count_nonzero(~(d <= bound))),
               max_abs=float(d.max()) if d.size else 0.0,
               max_rel=float((d[big] / np.abs(ref[big])).max()) if np.any(big) else 0.0)
    if dtype == "bf16":
        rne = O.bf16_encode_rne(ref)
        dist = bf16_ulp_distance(got_storage, rne)
        # The one-ulp bound holds where float32 rounding is far below half a
        # bf16 ulp.  Near a cancellation (|ref| much smaller than the terms
        # summed) the specified float32 order can move a tiny result by
        # several ulps at ~1e-8 absolute, so those elements are left to the
        # tolerance above.
        mag = np.abs(ref)
        well = mag >= (mag.max() / 256.0 if mag.size else 0.0)
        rep["max_ulp"] = int(dist[well].max()) if np.any(well) else 0
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


def assert_parity(got_storage, ref, dtype, what=""):
    rep = tolerance_report(got_storage, ref, dtype)
    if os.environ.get("TW_PRINT_EXACT"):
        print(f"EXACT {what} {rep.get('exact_frac')} n={rep.get('n')}", flush=True)
    assert rep["fails"] == 0, f"{what}: {rep}"
    if dtype == "bf16":
        assert rep["max_ulp"] <= 1, f"{what}: more than one bf16 ulp from the oracle: {rep}"
        if rep["n"] >= 4096:
            assert rep["exact_frac"] >= 0.999, \
                f"{what}: fewer than 99.9% of outputs are the correctly rounded value: {rep}"
    return rep


def sample_rows(rows, k=384, seed=0):
    """First, last and a seeded sample of rows (all rows if few)."""
    if rows <= k:
        return np.arange(rows)
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(rows, size=k - 4, replace=False).tolist()) | {0, 1, rows - 2, rows - 1}
    return np.array(sorted(pick))
