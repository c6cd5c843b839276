"""Pins for the CPU oracle: values the pages print (worked example), closed
forms, a library special case, exact brute force and invariants.

Sources: "TokenWeave 策略详解：以大模型推理为例" (§1 output formula, §3 token
split, appendix hidden=4 example) and "张量并行Tensor Parallelism" (MLP
section, Y = sum of the ranks' partials).
"""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from oracle import twnorm_oracle as O
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Pin checks, written as functions returning an error message (or None) so
# that the planted-mistake test below can run them against broken oracles.
# ---------------------------------------------------------------------------


def check_golden(oracle) -> str | None:
    for case in _golden()["cases"]:
        parts = [np.array(p, dtype=np.float64) for p in case["partials"]]
        out, res = oracle.fused(parts, np.array(case["residual"], dtype=np.float64),
                                np.array(case["weight"], dtype=np.float64), case["eps"])
        if not np.array_equal(res, np.array(case["residual_out"], dtype=np.float64)):
            return f"{case['name']}: residual_out {res} != {case['residual_out']}"
        exp = np.array(case["out"], dtype=np.float64)
        if not np.allclose(out, exp, rtol=1e-15, atol=1e-15):
            return f"{case['name']}: out {out} != {exp}"
    return None


def check_library_special_case(oracle) -> str | None:
    """N = 1 and residual = 0 is plain RMSNorm: compare with torch's
    rms_norm in float64 on the CPU."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(7)
    for h in (8, 64, 5120):
        x = rng.standard_normal((5, h)) * 1.7
        w = rng.uniform(0.5, 1.5, h)
        eps = 1e-5
        out, _ = oracle.fused([x], np.zeros_like(x), w, eps)
        ref = F.rms_norm(torch.from_numpy(x), (h,), torch.from_numpy(w), eps).numpy()
        if not np.allclose(out, ref, rtol=1e-13, atol=1e-13):
            return f"rms_norm mismatch at H={h}: {np.max(np.abs(out - ref))}"
        # with a nonzero residual the norm is applied to partial + residual
        r = rng.standard_normal((5, h))
        out, _ = oracle.fused([x], r, w, eps)
        ref = F.rms_norm(torch.from_numpy(x + r), (h,), torch.from_numpy(w), eps).numpy()
        if not np.allclose(out, ref, rtol=1e-13, atol=1e-13):
            return f"rms_norm(p+r) mismatch at H={h}"
    return None


def _exact_case(oracle, parts, resid, w, eps) -> str | None:
    """Exact rational reference for one tiny case; sqrt at 50 digits."""
    getcontext().prec = 50
    rows, h = len(resid), len(resid[0])
    out, res = oracle.fused([np.array(p, dtype=np.float64) for p in parts],
                            np.array(resid, dtype=np.float64), np.array(w, dtype=np.float64), eps)
    for t in range(rows):
        x = []
        for j in range(h):
            s = Fraction(0)
            for p in parts:
                s += Fraction(p[t][j])
            x.append(Fraction(resid[t][j]) + s)
        ms = sum(v * v for v in x) / h + Fraction(eps)
        root = Decimal(ms.numerator) / Decimal(ms.denominator)
        root = root.sqrt()
        for j in range(h):
            if Fraction(res[t][j]) != x[j]:
                return f"residual_out[{t},{j}] {res[t][j]} != {x[j]}"
            exact = Decimal(x[j].numerator) / Decimal(x[j].denominator) / root * Decimal(w[j])
            got = Decimal(float(out[t][j]))
            if abs(got - exact) > Decimal("1e-15") * max(Decimal(1), abs(exact)):
                return f"out[{t},{j}] {got} != {exact}"
    return None


def check_brute_force(oracle) -> str | None:
    vals = [-2.0, -1.0, -0.5, 0.0, 0.5, 1.0, 2.0, 1.5, -0.25]
    rng = np.random.default_rng(123)
    for trial in range(60):
        n = int(rng.integers(1, 4))
        h = int(rng.integers(1, 9))
        rows = int(rng.integers(1, 3))
        parts = [[[float(rng.choice(vals)) for _ in range(h)] for _ in range(rows)] for _ in range(n)]
        resid = [[float(rng.choice(vals)) for _ in range(h)] for _ in range(rows)]
        w = [float(rng.choice([0.5, 0.75, 1.0, 1.25, 1.5])) for _ in range(h)]
        eps = float(rng.choice([1e-6, 1e-5, 0.25]))
        msg = _exact_case(oracle, parts, resid, w, eps)
        if msg:
            return f"trial {trial}: {msg}"
    return None


def check_token_split(oracle) -> str | None:
    """Reduce-scatter along token rows, add + norm per shard, all-gather;
    equals all-reduce then add + norm on all rows ([TW] §2-§3, §3.4)."""
    rng = np.random.default_rng(5)
    n, t, h = 2, 64, 96
    parts = [rng.standard_normal((t, h)) for _ in range(n)]
    resid = rng.standard_normal((t, h))
    w = rng.uniform(0.5, 1.5, h)
    full_out, full_res = oracle.fused(parts, resid, w, 1e-5)
    shard = t // n
    outs, ress = [], []
    for r in range(n):
        sl = slice(r * shard, (r + 1) * shard)
        o, x = oracle.fused([p[sl] for p in parts], resid[sl], w, 1e-5)
        outs.append(o)
        ress.append(x)
    if not np.allclose(oracle.allgather_rows(outs), full_out, rtol=1e-15, atol=1e-15):
        return "token split changes out"
    if not np.allclose(oracle.allgather_rows(ress), full_res, rtol=0, atol=0):
        return "token split changes residual_out"
    return None


def check_zero_padded_columns(oracle) -> str | None:
    """Appendix (零填充 + AllReduce 求和): partial i is zero outside its own
    column block, so the reduce equals the concatenation of the blocks."""
    w = workloads.get("zero_padded")
    inp = workloads.make(w, seed=3, rows=8)
    s = oracle.reduce_from_storage(inp)
    block = w.hidden // w.n
    concat = np.concatenate([oracle.decode(inp["partials"][i], "bf16")[:, i * block:(i + 1) * block]
                             for i in range(w.n)], axis=1)
    if not np.array_equal(s, concat):
        return "column-block reduce is not the concatenation"
    return None


def check_closed_forms(oracle) -> str | None:
    # constant row c*1 with eps 0 -> sign(c) * w
    w = np.linspace(0.5, 1.5, 12)
    for c in (1.5, -0.75, 3.0):
        out, _ = oracle.fused([np.full((1, 12), c)], np.zeros((1, 12)), w, 0.0)
        if not np.allclose(out[0], np.sign(c) * w, rtol=1e-15, atol=0):
            return f"constant row {c}"
    # one-hot v * e_k with eps 0 -> sign(v) * sqrt(H) * w_k, for several H
    for h in (16, 64, 4096, 5120):
        x = np.zeros((1, h))
        x[0, 3] = -2.5
        wv = np.full(h, 0.75)
        out, _ = oracle.fused([x], np.zeros((1, h)), wv, 0.0)
        if not math.isclose(out[0, 3], -math.sqrt(h) * 0.75, rel_tol=1e-14):
            return f"one-hot H={h}: {out[0, 3]} vs {-math.sqrt(h) * 0.75}"
        if np.count_nonzero(out) != 1:
            return "one-hot leaks"
    # residual only (all partials zero) is plain RMSNorm of the residual
    r = np.array([[3.0, -4.0, 0.0, 0.0]])
    out, res = oracle.fused([np.zeros((1, 4)), np.zeros((1, 4))], r, np.ones(4), 0.0)
    # mean square 25/4, root 2.5 -> [1.2, -1.6, 0, 0]
    if not np.allclose(out, [[1.2, -1.6, 0, 0]], rtol=1e-15, atol=0) or not np.array_equal(res, r):
        return "residual-only row"
    return None


def check_invariants(oracle) -> str | None:
    inp = workloads.make(workloads.get("shard70b"), seed=11, rows=4)
    parts = [oracle.decode(p, "bf16") for p in inp["partials"]]
    r = oracle.decode(inp["residual"], "bf16")
    w = oracle.decode(inp["weight"], "bf16")
    base_out, base_res = oracle.fused(parts, r, w, 1e-5)
    # permutation of the partials (sums of a few bf16 values are exact in fp64)
    perm = [parts[i] for i in (3, 0, 7, 5, 1, 6, 2, 4)]
    o2, r2 = oracle.fused(perm, r, w, 1e-5)
    if not (np.array_equal(o2, base_out) and np.array_equal(r2, base_res)):
        return "permutation changes the result"
    # an all-zero extra partial changes nothing
    o3, r3 = oracle.fused(parts + [np.zeros_like(r)], r, w, 1e-5)
    if not (np.array_equal(o3, base_out) and np.array_equal(r3, base_res)):
        return "zero partial changes the result"
    # scaling everything by 2^k leaves out unchanged when eps = 0
    o4, _ = oracle.fused(parts, r, w, 0.0)
    o5, _ = oracle.fused([p * 2.0 ** 7 for p in parts], r * 2.0 ** 7, w, 0.0)
    if not np.array_equal(o4, o5):
        return "scale invariance"
    # RMS(out / w) = sqrt(ms / (ms + eps)) per row
    ms = np.mean(base_res ** 2, axis=1)
    rms = np.sqrt(np.mean((base_out / w) ** 2, axis=1))
    if not np.allclose(rms, np.sqrt(ms / (ms + 1e-5)), rtol=1e-14, atol=0):
        return "RMS of the normalised row"
    return None


def _bf16_bits_by_hand(values) -> np.ndarray:
    """bf16 storage of values that bf16 holds exactly: the high half of the
    float32 bit pattern (asserting the low half is zero, i.e. no rounding)."""
    bits32 = np.asarray(values, dtype=np.float32).view(np.uint32)
    assert np.all((bits32 & 0xFFFF) == 0), "value is not bf16-exact"
    return (bits32 >> 16).astype(np.uint16)


def _storage_case(case, dtype) -> dict:
    """A golden case as a ``workloads.make``-style storage dict."""
    store = _bf16_bits_by_hand if dtype == "bf16" else (lambda v: np.asarray(v, dtype=np.float32))
    res = np.array(case["residual"], dtype=np.float64)
    return dict(partials=[store(p) for p in case["partials"]], residual=store(res),
                weight=store(case["weight"]), eps=case["eps"], dtype=dtype,
                n=len(case["partials"]), rows=res.shape[0], hidden=res.shape[1])


def check_storage_wrappers(oracle) -> str | None:
    """The wrappers on stored bits (what every GPU comparison calls) give the
    hand-derived golden values in both storage formats: fused_from_storage
    on the stored inputs, and rmsnorm_from_storage on the stored sum of the
    partials (every golden sum is exact in both formats)."""
    for case in _golden()["cases"]:
        want_res = np.array(case["residual_out"], dtype=np.float64)
        want_out = np.array(case["out"], dtype=np.float64)
        for dt in ("bf16", "f32"):
            inp = _storage_case(case, dt)
            out, res = oracle.fused_from_storage(inp)
            if not np.array_equal(res, want_res):
                return f"fused_from_storage {case['name']} {dt}: residual_out {res}"
            if not np.allclose(out, want_out, rtol=1e-15, atol=1e-15):
                return f"fused_from_storage {case['name']} {dt}: out {out}"
            summed = want_res - np.array(case["residual"], dtype=np.float64)
            reduced = _bf16_bits_by_hand(summed) if dt == "bf16" else summed.astype(np.float32)
            out, res = oracle.rmsnorm_from_storage(reduced, inp)
            if not np.array_equal(res, want_res):
                return f"rmsnorm_from_storage {case['name']} {dt}: residual_out {res}"
            if not np.allclose(out, want_out, rtol=1e-15, atol=1e-15):
                return f"rmsnorm_from_storage {case['name']} {dt}: out {out}"
    return None


def check_eps_as_passed(oracle) -> str | None:
    """The kernel receives eps as a C float.  float32(0.1) is 13421773 / 2^27
    and float32(1e-5) is 10995116 / 2^40 (the nearest multiples of 2^-27 and
    2^-40 with 24 significant bits); 2^-20 is exact.  A constant row
    2^-10 (mean square 2^-20) with eps = 0.1 then has the exact result
    2^-10 / sqrt(2^-20 + 13421773 / 2^27) * w, which differs from the result
    with the float64 eps 0.1 by 7.45e-9 relative: the cast is visible."""
    for eps, want in ((0.1, Fraction(13421773, 2 ** 27)), (1e-5, Fraction(10995116, 2 ** 40)),
                      (2.0 ** -20, Fraction(1, 2 ** 20)), (0.0, Fraction(0))):
        if Fraction(oracle.eps_as_passed(eps)) != want:
            return f"eps_as_passed({eps}) = {oracle.eps_as_passed(eps)!r}"
    getcontext().prec = 50
    ms_plus_eps = Fraction(1, 2 ** 20) + Fraction(13421773, 2 ** 27)
    root = (Decimal(ms_plus_eps.numerator) / Decimal(ms_plus_eps.denominator)).sqrt()
    w = [1.0, 0.5, 2.0, 1.5]
    for dt in ("bf16", "f32"):
        case = dict(partials=[[[2.0 ** -11] * 4], [[2.0 ** -11] * 4]], residual=[[0.0] * 4],
                    weight=w, eps=0.1)
        out, res = oracle.fused_from_storage(_storage_case(case, dt))
        if not np.array_equal(res, np.full((1, 4), 2.0 ** -10)):
            return f"eps case {dt}: residual_out {res}"
        for j in range(4):
            exact = Decimal(1) / Decimal(1024) / root * Decimal(w[j])
            if abs(Decimal(float(out[0, j])) - exact) > Decimal("1e-15") * abs(exact):
                return f"eps case {dt}: out[{j}] {out[0, j]!r} != {exact}"
    return None


ALL_PINS = [check_golden, check_library_special_case, check_brute_force, check_token_split,
            check_zero_padded_columns, check_closed_forms, check_invariants,
            check_storage_wrappers, check_eps_as_passed]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    msg = pin(O)
    assert msg is None, msg


# ---------------------------------------------------------------------------
# Planted mistakes: each broken copy of the oracle must fail at least one pin
# ---------------------------------------------------------------------------


class _Mutant:
    """A copy of the oracle's public functions with one step replaced."""

    def __init__(self, **over):
        for name in ("fused", "reduce_from_storage", "decode", "allgather_rows",
                     "fused_from_storage", "rmsnorm_from_storage", "eps_as_passed"):
            setattr(self, name, getattr(O, name))
        for k, v in over.items():
            setattr(self, k, v)


def _fused_with(reduce=O.reduce_partials, add=O.residual_add, norm=O.rmsnorm):
    def f(partials, residual, weight, eps):
        x = add(residual, reduce(partials))
        return norm(x, weight, eps), x
    return f


def _norm_divisor(div):
    def norm(x, w, eps):
        x = np.asarray(x, dtype=np.float64)
        ms = np.sum(x * x, axis=-1) / div(x.shape[-1])
        return x / np.sqrt(ms + eps)[..., None] * w
    return norm


MUTANTS = {
    "drop_residual": _fused_with(add=lambda r, s: s),
    "drop_last_partial": _fused_with(reduce=lambda ps: O.reduce_partials(ps[:-1]) if len(ps) > 1 else O.reduce_partials(ps)),
    "subtract_partial": _fused_with(reduce=lambda ps: O.reduce_partials(ps[:1]) - (O.reduce_partials(ps[1:]) if len(ps) > 1 else 0)),
    "divisor_half_hidden": _fused_with(norm=_norm_divisor(lambda h: max(1, h // 2))),
    "divisor_h_minus_1": _fused_with(norm=_norm_divisor(lambda h: max(1, h - 1))),
    "eps_on_sum": _fused_with(norm=lambda x, w, eps: x / np.sqrt((np.sum(x * x, -1) + eps) / x.shape[-1])[..., None] * w),
    "eps_outside_sqrt": _fused_with(norm=lambda x, w, eps: x / (np.sqrt(np.mean(x * x, -1)) + eps)[..., None] * w),
    "no_weight": _fused_with(norm=lambda x, w, eps: O.rmsnorm(x, np.ones_like(w), eps)),
    "weight_reversed": _fused_with(norm=lambda x, w, eps: O.rmsnorm(x, np.asarray(w)[::-1], eps)),
    "mean_over_tokens": _fused_with(norm=lambda x, w, eps: x / np.sqrt(np.mean(x * x, axis=0, keepdims=True) + eps) * w),
    "sqrt_not_inverse": _fused_with(norm=lambda x, w, eps: x * np.sqrt(np.mean(x * x, -1) + eps)[..., None] * w),
    "sum_not_mean": _fused_with(norm=_norm_divisor(lambda h: 1)),
    "eps_squared": _fused_with(norm=lambda x, w, eps: O.rmsnorm(x, w, eps * eps)),
    "weight_shifted": _fused_with(norm=lambda x, w, eps: O.rmsnorm(x, np.roll(np.asarray(w), 1), eps)),
    "residual_out_is_norm": None,   # handled below
}


def _mutant_residual_out_is_norm(partials, residual, weight, eps):
    out, _ = O.fused(partials, residual, weight, eps)
    return out, out


MUTANTS["residual_out_is_norm"] = _mutant_residual_out_is_norm


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    m = _Mutant(fused=MUTANTS[name])
    failures = []
    for pin in ALL_PINS:
        try:
            msg = pin(m)
        except Exception as e:  # a crash also counts as caught
            msg = f"raised {e!r}"
        if msg:
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name} passes every pin"


# Planted mistakes in the wrappers on stored bits: each must fail a pin.
def _ffs_swapped_residual_weight(inp):
    dt = inp["dtype"]
    return O.fused([O.decode(p, dt) for p in inp["partials"]], O.decode(inp["weight"], dt),
                   O.decode(inp["residual"], dt), O.eps_as_passed(inp["eps"]))


def _ffs_eps_uncast(inp):
    dt = inp["dtype"]
    return O.fused([O.decode(p, dt) for p in inp["partials"]], O.decode(inp["residual"], dt),
                   O.decode(inp["weight"], dt), float(inp["eps"]))


def _ffs_wrong_decode(inp):
    """bf16 bits read as IEEE half precision."""
    def dec(a, dt):
        return np.asarray(a).view(np.float16).astype(np.float64) if dt == "bf16" else O.decode(a, dt)
    dt = inp["dtype"]
    return O.fused([dec(p, dt) for p in inp["partials"]], dec(inp["residual"], dt),
                   dec(inp["weight"], dt), O.eps_as_passed(inp["eps"]))


def _ffs_first_partial_only(inp):
    return O.fused_from_storage(dict(inp, partials=inp["partials"][:1]))


def _rfs_drops_residual(reduced, inp):
    dt = inp["dtype"]
    x = O.decode(reduced, dt)
    return O.fused([x], np.zeros_like(x), O.decode(inp["weight"], dt), O.eps_as_passed(inp["eps"]))


def _rfs_unit_weight(reduced, inp):
    dt = inp["dtype"]
    return O.fused([O.decode(reduced, dt)], O.decode(inp["residual"], dt),
                   np.ones(inp["hidden"]), O.eps_as_passed(inp["eps"]))


WRAPPER_MUTANTS = {
    "fused_from_storage_swaps_residual_and_weight": dict(fused_from_storage=_ffs_swapped_residual_weight),
    "fused_from_storage_eps_not_cast": dict(fused_from_storage=_ffs_eps_uncast),
    "fused_from_storage_wrong_bf16_decode": dict(fused_from_storage=_ffs_wrong_decode),
    "fused_from_storage_first_partial_only": dict(fused_from_storage=_ffs_first_partial_only),
    "rmsnorm_from_storage_drops_residual": dict(rmsnorm_from_storage=_rfs_drops_residual),
    "rmsnorm_from_storage_unit_weight": dict(rmsnorm_from_storage=_rfs_unit_weight),
    "eps_as_passed_keeps_float64": dict(eps_as_passed=lambda eps: float(eps)),
}


@pytest.mark.parametrize("name", sorted(WRAPPER_MUTANTS))
def test_pins_catch_planted_wrapper_mistake(name):
    m = _Mutant(**WRAPPER_MUTANTS[name])
    failures = []
    for pin in ALL_PINS:
        try:
            msg = pin(m)
        except Exception as e:  # a crash also counts as caught
            msg = f"raised {e!r}"
        if msg:
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name} passes every pin"


def test_pins_catch_broken_bf16_decode():
    """A decode that drops the low mantissa bits (or shifts the wrong way)
    must break the column-block pin or the codec pin."""
    def bad_decode(arr, dtype):
        v = O.decode(arr, dtype)
        return np.trunc(v * 4) / 4
    m = _Mutant(decode=bad_decode)
    assert check_zero_padded_columns(m) is not None


# ---------------------------------------------------------------------------
# bf16 codec
# ---------------------------------------------------------------------------


def test_bf16_golden_rounding():
    for case in _golden()["bf16_rounding"]["cases"]:
        got = int(O.bf16_encode_rne(np.array([case["value"]]))[0])
        assert got == int(case["bits"], 16), (case, hex(got))


def test_bf16_encode_matches_torch_cast_on_float32():
    """For float32 inputs, direct RNE from float64 equals torch's CPU
    float32 -> bfloat16 cast (RNE), on 2^20 random patterns + specials."""
    import torch
    rng = np.random.default_rng(2024)
    bits = rng.integers(0, 2 ** 32, size=2 ** 20, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    specials = np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 3.4e38, -3.4e38, 1e-40, -1e-40,
                         1.00390625, 1.01171875, np.inf, -np.inf], dtype=np.float32)
    f = np.concatenate([f, specials])
    finite = np.isfinite(f) | np.isinf(f)
    f = f[finite]
    ours = O.bf16_encode_rne(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref), np.flatnonzero(ours != ref)[:10]


def test_bf16_nan_and_decode_roundtrip():
    out = O.bf16_encode_rne(np.array([np.nan, -np.nan]))
    assert (out[0] & 0x7FFF) > 0x7F80 and (out[1] & 0x7FFF) > 0x7F80
    allbits = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    dec = O.bf16_decode(allbits)
    ok = ~np.isnan(dec)
    assert np.array_equal(O.bf16_encode_rne(dec[ok]), allbits[ok])
    import torch
    ref = torch.from_numpy(allbits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(dec[ok], ref[ok].astype(np.float64))


def test_eps_zero_on_zero_row_is_nan():
    with np.errstate(divide="ignore", invalid="ignore"):
        out, res = O.fused([np.zeros((1, 8))], np.zeros((1, 8)), np.ones(8), 0.0)
    assert np.all(np.isnan(out)) and np.all(res == 0)
