"""Seeded synthetic inputs for the fused reduce + residual-add + RMSNorm path.

This module only draws random values and stores them in the activation
format; it holds none of the method's arithmetic.  It is the one piece of
code shared by the CPU oracle (``oracle/``) and the HIP path
(``reduce_residual_add_amd``); neither of those imports the other.

Workloads (all token-sharded slices of one GPU's rows, "rows" = T/N):

* ``tiny``         N=2 partials of [16, 64] fp32, eps 1e-6.
* ``page1``        N=2, 1024 rows (one shard of seq 2048), H=4096 bf16 -- the
                   N=2 / seq_len 2048 / hidden 4096 example of
                   "TokenWeave 策略详解：以大模型推理为例", §1 and §3.
* ``zero_padded``  N=4, 4096 rows, H=5120 bf16; partial i is nonzero only in
                   its own column block [i*H/4, (i+1)*H/4) -- the zero-padded
                   column partials of the same page's appendix
                   ("实现方法：零填充 + AllReduce 求和").
* ``shard70b``     N=8 dense partials of [1024, 8192] bf16 -- the row-parallel
                   partial sums Y_i of "张量并行Tensor Parallelism", MLP section,
                   at a 70B-class hidden size.
* ``cu_restricted`` N=8, 2048 rows, H=8192 bf16, the shard70b distributions.

Recipe: every tensor is drawn in float32 from ``numpy.random.Generator(PCG64)``
seeded by ``SeedSequence([seed, config_index]).spawn(N + 2)`` (one child per
partial, then residual, then weight).  bf16 tensors are the round-to-nearest-
even cast of those float32 draws, done by torch on the CPU.  N(0, s) means
standard deviation s; U(a, b) is uniform on [a, b).  The weight has the
activation dtype.

Storage convention returned by :func:`make`: bf16 tensors are ``numpy.uint16``
arrays of raw bit patterns, fp32 tensors are ``numpy.float32`` arrays.  Both
are C-contiguous [rows, hidden] (weight: [hidden]).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import List, Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    index: int            # position in WORKLOADS; also the seed-sequence key
    n: int                # number of partial buffers
    rows: int             # token rows of this shard
    hidden: int           # H
    dtype: str            # "bf16" or "f32"
    partial_std: float
    residual_std: float
    weight_lo: float
    weight_hi: float
    eps: float
    layout: str = "dense"            # "dense" or "column_blocks"
    cu_limits: Tuple[int, ...] = (0,)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def fused_bytes(self) -> int:
        """Algorithmic HBM bytes of one fused call: N partial reads, one
        residual read, residual_out and out writes, plus the weight once."""
        b = self.elem_bytes
        return (self.n + 3) * self.rows * self.hidden * b + self.hidden * b

    def unfused_bytes(self) -> int:
        """Reduce kernel (N reads + 1 write) then norm kernel (2 reads + 2
        writes + weight)."""
        b = self.elem_bytes
        return (self.n + 5) * self.rows * self.hidden * b + self.hidden * b

    def with_rows(self, rows: int) -> "Workload":
        return replace(self, rows=rows)


WORKLOADS: List[Workload] = [
    Workload("tiny", 0, 2, 16, 64, "f32", 1.0, 1.0, 0.5, 1.5, 1e-6),
    Workload("page1", 1, 2, 1024, 4096, "bf16", 1.0, 1.0, 0.5, 1.5, 1e-5),
    Workload("zero_padded", 2, 4, 4096, 5120, "bf16", 1.0, 1.0, 0.5, 1.5, 1e-5,
             layout="column_blocks"),
    Workload("shard70b", 3, 8, 1024, 8192, "bf16", 0.5, 1.0, 0.8, 1.2, 1e-5),
    Workload("cu_restricted", 4, 8, 2048, 8192, "bf16", 0.5, 1.0, 0.8, 1.2, 1e-5,
             cu_limits=(8, 16, 32, 0)),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def get(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    return BY_NAME[name_or_index]


def f32_to_storage(values: np.ndarray, dtype: str) -> np.ndarray:
    """Store float32 draws in the activation format (bf16 bits via torch's
    CPU round-to-nearest-even cast, or float32 unchanged)."""
    values = np.ascontiguousarray(values, dtype=np.float32)
    if dtype == "f32":
        return values
    import torch
    t = torch.from_numpy(values).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _rngs(w: Workload, seed: int):
    children = np.random.SeedSequence([seed, w.index]).spawn(w.n + 2)
    return [np.random.Generator(np.random.PCG64(c)) for c in children]


def make(w: Workload, seed: int = 0, rows: Optional[int] = None) -> dict:
    """Draw one set of inputs for workload ``w``.

    ``rows`` overrides the row count (smaller parity cases of the same
    distributions); the first ``r`` rows of a draw with more rows are NOT the
    same values, each size is its own draw.
    Returns a dict with keys partials (list), residual, weight, eps, dtype,
    n, rows, hidden.
    """
    if rows is None:
        rows = w.rows
    h = w.hidden
    rng = _rngs(w, seed)
    partials = []
    for i in range(w.n):
        if w.layout == "column_blocks":
            block = h // w.n
            v = np.zeros((rows, h), dtype=np.float32)
            v[:, i * block:(i + 1) * block] = (
                rng[i].standard_normal((rows, block), dtype=np.float32) * np.float32(w.partial_std))
        else:
            v = rng[i].standard_normal((rows, h), dtype=np.float32) * np.float32(w.partial_std)
        partials.append(f32_to_storage(v, w.dtype))
    r = rng[w.n].standard_normal((rows, h), dtype=np.float32) * np.float32(w.residual_std)
    wt = rng[w.n + 1].uniform(w.weight_lo, w.weight_hi, size=h).astype(np.float32)
    return dict(partials=partials, residual=f32_to_storage(r, w.dtype),
                weight=f32_to_storage(wt, w.dtype), eps=w.eps, dtype=w.dtype,
                n=w.n, rows=rows, hidden=h)


def make_random(n: int, rows: int, hidden: int, dtype: str, seed: int,
                partial_std: float = 1.0, residual_std: float = 1.0,
                weight_lo: float = 0.5, weight_hi: float = 1.5) -> dict:
    """Dense draws of an arbitrary shape (edge-case and ragged-tail tests)."""
    children = np.random.SeedSequence([seed, 1000 + n, rows, hidden]).spawn(n + 2)
    rng = [np.random.Generator(np.random.PCG64(c)) for c in children]
    partials = [f32_to_storage(rng[i].standard_normal((rows, hidden), dtype=np.float32)
                               * np.float32(partial_std), dtype) for i in range(n)]
    r = rng[n].standard_normal((rows, hidden), dtype=np.float32) * np.float32(residual_std)
    wt = rng[n + 1].uniform(weight_lo, weight_hi, size=hidden).astype(np.float32)
    return dict(partials=partials, residual=f32_to_storage(r, dtype),
                weight=f32_to_storage(wt, dtype), eps=1e-5, dtype=dtype,
                n=n, rows=rows, hidden=hidden)
