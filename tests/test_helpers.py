"""CPU checks of the GPU tests' comparison helpers."""
import numpy as np
import pytest

import workloads
from gpu_helpers import bf16_ulp, bf16_ulp_distance, reference, tolerance_report


def test_ulp_helper_pins():
    """The ulp distance used above counts representable steps across zero."""
    a = np.array([0x3F80, 0x3F80, 0x0000, 0x8000, 0x8001], np.uint16)
    b = np.array([0x3F80, 0x3F81, 0x8000, 0x0001, 0x0001], np.uint16)
    assert bf16_ulp_distance(a, b).tolist() == [0, 1, 0, 1, 2]


def test_tolerance_reading():
    """bf16 passes iff |d| <= max(2e-2, 1e-2 |ref|); fp32 iff |d| <= 1e-5 max(1, |ref|)."""
    from oracle import twnorm_oracle as O
    ref = np.array([0.0, 0.5, 8.5, -100.0])
    ok = O.bf16_encode_rne(ref + np.array([0.019, -0.019, 0.08, 0.9]))
    assert tolerance_report(ok, ref, "bf16")["fails"] == 0
    bad = O.bf16_encode_rne(ref + np.array([0.03, 0.0, 0.0, 0.0]))
    assert tolerance_report(bad, ref, "bf16")["fails"] == 1
    f = np.array([1e-6, 2.0], np.float32)
    assert tolerance_report(f, np.array([0.0, 2.0 + 1.9e-5]), "f32")["fails"] == 0
    assert tolerance_report(f, np.array([2e-5, 2.0]), "f32")["fails"] == 1


def test_cancellation_moves_tiny_results_by_several_ulps():
    """Why the one-ulp check needs a per-element error bound: summing in
    float32 in index order (the kernel's specified arithmetic) next to a
    cancellation legitimately lands several bf16 ulps from the correctly
    rounded exact sum, at ~1e-8 absolute."""
    import numpy as np
    from oracle import twnorm_oracle as O
    terms = [-1.1875, 0.8828125, -1.555308699607849e-07, 0.3046875]   # bf16-exact values
    for t in terms:
        assert O.bf16_decode(O.bf16_encode_rne(np.array([t])))[0] == t
    s32 = np.float32(0.0)
    for t in terms:
        s32 = np.float32(s32 + np.float32(t))
    exact = sum(terms)
    ulps = bf16_ulp_distance(O.bf16_encode_rne(np.array([float(s32)])),
                             O.bf16_encode_rne(np.array([exact])))[0]
    assert ulps == 7
    assert abs(float(s32) - exact) < 1e-8


# ---------------------------------------------------------------------------
# The per-element float32 error bounds of gpu_helpers, pinned against a
# float32 model of the kernel's order of operations: partials added in index
# order, then the residual; squares summed per 16-byte chunk by fused
# multiply-adds, per group of 64 chunks by a pairwise tree in lane order, the
# groups in row order; then 1 / sqrt(ss / H + eps) and (x * inv) * w.  The
# model exists only to test the bound; no GPU result is compared with it.
# ---------------------------------------------------------------------------
def _fma32(a, b, c):
    """float32 fused multiply-add: the float64 product of two float32 values
    is exact; adding c and rounding once more can differ from a true fma by
    far less than the bound's slack."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def _kernel_order_f32(inp):
    dt = inp["dtype"]
    dec = lambda a: np.asarray(O.decode(a, dt), dtype=np.float32)   # exact
    acc = dec(inp["partials"][0])
    for p in inp["partials"][1:]:
        acc = acc + dec(p)                                     # float32 adds
    x = dec(inp["residual"]) + acc
    rows, h = x.shape
    e = 8 if dt == "bf16" else 4
    chunks = h // e
    groups = (chunks + 63) // 64
    xc = np.zeros((rows, groups * 64, e), dtype=np.float32)
    xc[:, :chunks, :] = x.reshape(rows, chunks, e)
    q = np.zeros((rows, groups * 64), dtype=np.float32)
    for k in range(e):
        q = _fma32(xc[:, :, k], xc[:, :, k], q)
    v = q.reshape(rows, groups, 64)
    while v.shape[-1] > 1:                                    # pairwise, lane order
        v = v[..., 0::2] + v[..., 1::2]
    ss = np.zeros(rows, dtype=np.float32)
    for g in range(groups):
        ss = ss + v[:, g, 0]
    eps = np.float32(inp["eps"])
    inv = np.float32(1.0) / np.sqrt(ss / np.float32(h) + eps)
    out = (x * inv[:, None]) * dec(inp["weight"])
    return out.astype(np.float64), x.astype(np.float64)


from oracle import twnorm_oracle as O  # noqa: E402


def _bound_holds(inp):
    ref_out, ref_res, b_out, b_res = reference(inp)
    got_out, got_res = _kernel_order_f32(inp)
    assert np.all(np.abs(got_res - ref_res) <= b_res)
    assert np.all(np.abs(got_out - ref_out) <= b_out)
    return ref_out, ref_res, b_out, b_res


@pytest.mark.parametrize("name", ["tiny", "page1", "zero_padded", "shard70b"])
def test_error_bound_holds_on_the_workloads(name):
    inp = workloads.make(workloads.get(name), seed=3, rows=6)
    ref_out, ref_res, b_out, b_res = _bound_holds(inp)
    if inp["dtype"] == "bf16":
        # the bound exempts almost nothing on these inputs
        assert np.mean(b_res <= bf16_ulp(ref_res) / 4) > 0.99
        assert np.mean(b_out <= bf16_ulp(ref_out) / 4) > 0.99


@pytest.mark.parametrize("n,hidden,dtype,std", [(16, 8192, "bf16", 4.0), (3, 65536, "bf16", 1.0),
                                                (7, 1000, "f32", 1.0), (2, 8, "bf16", 1e-3)])
def test_error_bound_holds_on_wide_and_deep_rows(n, hidden, dtype, std):
    _bound_holds(workloads.make_random(n, 3, hidden, dtype, seed=n + hidden, partial_std=std))


def test_error_bound_exempts_the_cancellation_case():
    """The cancellation example above: the element lands 7 ulps away, which
    the bound allows, and the one-ulp check exempts it."""
    terms = [-1.1875, 0.8828125, -1.555308699607849e-07, 0.3046875]
    h = 64
    cols = lambda t: np.full((1, h), t)
    inp = dict(partials=[O.bf16_encode_rne(cols(t)) for t in terms[:3]],
               residual=O.bf16_encode_rne(cols(terms[3])),
               weight=O.bf16_encode_rne(np.ones(h)), eps=1e-5, dtype="bf16", n=3, rows=1,
               hidden=h)
    ref_out, ref_res, b_out, b_res = _bound_holds(inp)
    got_out, got_res = _kernel_order_f32(inp)
    dist = bf16_ulp_distance(O.bf16_encode_rne(got_res), O.bf16_encode_rne(ref_res))
    assert dist.max() == 7
    assert np.all(b_res > bf16_ulp(ref_res) / 4)       # exempt from the one-ulp check
    rep = tolerance_report(O.bf16_encode_rne(got_res), ref_res, "bf16", b_res)
    assert rep["fails"] == 0 and rep["max_ulp"] == 0 and rep["ulp_exempt"] == h


def test_one_ulp_check_catches_a_wrong_element():
    """A result two ulps off in a well-conditioned element fails the
    one-ulp check even though it is inside the tolerance."""
    inp = workloads.make(workloads.get("shard70b"), seed=1, rows=2)
    ref_out, ref_res, b_out, b_res = reference(inp)
    got = O.bf16_encode_rne(ref_out)
    # an element near 0.75, where two ulps (2^-7) are well inside 2e-2
    i = np.unravel_index(np.argmin(np.abs(np.abs(ref_out) - 0.75)), ref_out.shape)
    got[i] = got[i] + 2                     # two steps away from zero (sign bit untouched)
    rep = tolerance_report(got, ref_out, "bf16", b_out)
    assert rep["fails"] == 0 and rep["max_ulp"] == 2
