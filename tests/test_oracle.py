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


ALL_PINS = [check_golden, check_library_special_case, check_brute_force, check_token_split,
            check_zero_padded_columns, check_closed_forms, check_invariants]


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
        for name in ("fused", "reduce_from_storage", "decode", "allgather_rows"):
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
