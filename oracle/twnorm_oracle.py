"""CPU oracle for the fused reduce + residual-add + RMSNorm step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, headers, helpers or constants); the only module both sides
use is ``workloads`` (seeded draws, no arithmetic of the method).

What it computes is the plain definition, in float64, row by row.  The pages
state that the reordered, fused pipeline reaches exactly the result of the
plain one ("TokenWeave 策略详解：以大模型推理为例", appendix "融合内核中的体现"
and its closing summary: mathematically equivalent to gathering first and
processing locally), so no step of the fused kernel's design appears here.

Sources (cited by page title and section):
  [TW]  "TokenWeave 策略详解：以大模型推理为例" (nanhubrain.csdn.net)
  [TP]  "张量并行Tensor Parallelism" (scmmm.top)

Readings taken where the pages are silent (each is also listed in the design
notes of the repository):
  * RMSNorm is y = x / sqrt(mean_j x_j^2 + eps) * w; eps is added to the mean
    inside the square root (the pages name RMSNorm but do not define it).
  * The mean runs over the full hidden size H of the token ([TW] §1: the
    statistic uses all of a token's features), never H/N.
  * The updated residual residual + sum(partials) is an output too
    ([TP] Self-Attention: X = X + Y; [TW] §5: the residual is fused in
    registers).  The norm uses the unrounded sum, not its stored copy.
  * eps reaches the GPU as a C ``float``; the oracle uses float64(float32(eps)).
  * Stored bf16 values are round-to-nearest-even of the float64 result, taken
    directly (no float32 step, so no double rounding).

Every function here is pinned by ``tests/test_oracle.py`` against values the
pages fix (worked example, closed forms), a library routine for the special
case N=1 and residual=0 (torch.nn.functional.rms_norm), exact rational brute
force on tiny inputs, and invariants (token-split, permutation, zero partial).
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# bf16 codec (hand-written; bf16 is the top 16 bits of an IEEE float32)
# ---------------------------------------------------------------------------


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64, exactly (shift into the high half
    of a float32, then widen; both steps are exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    as_f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return as_f32.astype(np.float64)


def bf16_encode_rne(x: np.ndarray) -> np.ndarray:
    """float64 -> uint16 bf16 bits, round to nearest, ties to even, taken
    directly from the float64 value.  Overflow rounds to +/-inf; NaN maps to
    the quiet NaN 0x7FC0 (sign kept)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    sign = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(x)
    # bf16 has 8 significand bits (7 stored).  For a finite a > 0 pick the
    # exponent e with 2^e <= a < 2^(e+1); the bf16 grid spacing there is
    # 2^(e-7), and below the normal range (e < -126) it stays 2^-133.
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        _, e2 = np.frexp(a)              # a = m * 2^e2 with 0.5 <= m < 1
        e = e2.astype(np.int64) - 1
        e = np.maximum(e, -126)
        quantum = np.ldexp(1.0, (e - 7).astype(np.int64))
        q = a / quantum                  # exact: a power-of-two scaling
        q_floor = np.floor(q)
        frac = q - q_floor
        up = (frac > 0.5) | ((frac == 0.5) & (np.fmod(q_floor, 2.0) == 1.0))
        mag = (q_floor + up) * quantum   # exact multiple of the grid
    mag = np.where(np.isfinite(a), mag, a)
    # Re-encode the (now bf16-representable) magnitude through float32 bits;
    # magnitudes beyond the largest bf16 become inf.
    big = mag >= 2.0 ** 128
    with np.errstate(over="ignore"):
        f32 = mag.astype(np.float32)
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(big, np.uint16(0x7F80), bits)
    bits = np.where(sign, bits | np.uint16(0x8000), bits)
    bits = np.where(nan, np.where(sign, np.uint16(0xFFC0), np.uint16(0x7FC0)), bits)
    out[...] = bits
    return out


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64 values (exact for both formats)."""
    if dtype == "bf16":
        return bf16_decode(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> storage (bf16 bits by direct RNE, or float32)."""
    if dtype == "bf16":
        return bf16_encode_rne(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def eps_as_passed(eps: float) -> float:
    """The eps the kernel sees: a C float, widened exactly."""
    return float(np.float32(eps))


# ---------------------------------------------------------------------------
# The method, step by step, in float64
# ---------------------------------------------------------------------------


def reduce_partials(partials: Sequence[np.ndarray]) -> np.ndarray:
    """s = sum_i p_i, elementwise over [rows, H].

    [TW] §3.2 (each shard sums the other ranks' contributions for its own
    token rows) and the appendix's hidden=4 example ([a,b,0,0] + [0,0,c,d]);
    [TP] MLP section (Y = sum_i Y_i for row-parallel partials).
    """
    if len(partials) == 0:
        raise ValueError("need at least one partial")
    s = np.zeros_like(np.asarray(partials[0], dtype=np.float64))
    for p in partials:
        s = s + np.asarray(p, dtype=np.float64)
    return s


def residual_add(residual: np.ndarray, s: np.ndarray) -> np.ndarray:
    """x = residual + s  ([TW] §1 output formula; [TP] Self-Attention,
    X = X + Y)."""
    return np.asarray(residual, dtype=np.float64) + s


def mean_square(x: np.ndarray) -> np.ndarray:
    """ms[t] = (1/H) * sum_j x[t, j]^2 over the full hidden size H of each
    token ([TW] §1: the per-token statistic uses all of its features)."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1]
    return np.sum(x * x, axis=-1) / h


def rmsnorm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """out[t, j] = x[t, j] / sqrt(ms[t] + eps) * w[j]  ([TW] §1 output
    formula "RMSNorm(...) * weight" and §3.3; eps on the mean is the textbook
    RMSNorm reading)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    inv = 1.0 / np.sqrt(mean_square(x) + eps)
    return x * inv[..., None] * w


def fused(partials: Sequence[np.ndarray], residual: np.ndarray, weight: np.ndarray,
          eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """The whole step on float64 values: returns (out, residual_out).

    residual_out = residual + sum_i p_i                     (the new residual)
    out          = RMSNorm(residual_out) * weight            ([TW] §1, §3.3, §5)
    """
    s = reduce_partials(partials)
    x = residual_add(residual, s)
    return rmsnorm(x, weight, eps), x


# ---------------------------------------------------------------------------
# Convenience wrappers on storage arrays (as produced by ``workloads``)
# ---------------------------------------------------------------------------


def fused_from_storage(inp: dict) -> Tuple[np.ndarray, np.ndarray]:
    """Decode a ``workloads.make`` dict exactly and run :func:`fused`.
    Returns float64 (out, residual_out)."""
    dt = inp["dtype"]
    parts = [decode(p, dt) for p in inp["partials"]]
    return fused(parts, decode(inp["residual"], dt), decode(inp["weight"], dt),
                 eps_as_passed(inp["eps"]))


def reduce_from_storage(inp: dict) -> np.ndarray:
    dt = inp["dtype"]
    return reduce_partials([decode(p, dt) for p in inp["partials"]])


def rmsnorm_from_storage(reduced: np.ndarray, inp: dict) -> Tuple[np.ndarray, np.ndarray]:
    """The norm half of the unfused comparison path on a stored ``reduced``
    tensor: x = residual + reduced; returns (out, residual_out) in float64."""
    dt = inp["dtype"]
    return fused([decode(reduced, dt)], decode(inp["residual"], dt),
                 decode(inp["weight"], dt), eps_as_passed(inp["eps"]))


def allgather_rows(shards: Sequence[np.ndarray]) -> np.ndarray:
    """AllGather of token-row shards: concatenate the per-rank [rows_r, H]
    results along tokens ([TW] §3.4)."""
    return np.concatenate([np.asarray(s) for s in shards], axis=0)
