"""The seeded input generators: deterministic, right shapes, right
distributions, and the zero-padded column structure."""
import numpy as np
import pytest

import workloads
from oracle import twnorm_oracle as O


@pytest.mark.parametrize("w", workloads.WORKLOADS, ids=lambda w: w.name)
def test_shapes_and_determinism(w):
    rows = min(w.rows, 64)
    a = workloads.make(w, seed=0, rows=rows)
    b = workloads.make(w, seed=0, rows=rows)
    c = workloads.make(w, seed=1, rows=rows)
    assert len(a["partials"]) == w.n
    sdt = np.uint16 if w.dtype == "bf16" else np.float32
    for i in range(w.n):
        assert a["partials"][i].shape == (rows, w.hidden) and a["partials"][i].dtype == sdt
        assert a["partials"][i].flags["C_CONTIGUOUS"]
        assert np.array_equal(a["partials"][i], b["partials"][i])
        assert not np.array_equal(a["partials"][i], c["partials"][i])
    assert a["residual"].shape == (rows, w.hidden)
    assert a["weight"].shape == (w.hidden,)
    assert np.array_equal(a["weight"], b["weight"])


@pytest.mark.parametrize("name", ["page1", "shard70b", "zero_padded"])
def test_distributions(name):
    w = workloads.get(name)
    inp = workloads.make(w, seed=0, rows=256)
    dec = lambda a: O.decode(a, w.dtype)
    p = dec(inp["partials"][0])
    if w.layout == "column_blocks":
        p = p[:, : w.hidden // w.n]
    assert abs(p.mean()) < 0.02
    assert abs(p.std() - w.partial_std) < 0.02 * w.partial_std + 0.01
    r = dec(inp["residual"])
    assert abs(r.std() - w.residual_std) < 0.02
    wt = dec(inp["weight"])
    assert wt.min() >= w.weight_lo - 1e-2 and wt.max() <= w.weight_hi + 1e-2
    assert abs(wt.mean() - 0.5 * (w.weight_lo + w.weight_hi)) < 0.03


def test_zero_padded_structure():
    w = workloads.get("zero_padded")
    inp = workloads.make(w, seed=0, rows=32)
    block = w.hidden // w.n
    for i, p in enumerate(inp["partials"]):
        mask = np.zeros(w.hidden, dtype=bool)
        mask[i * block:(i + 1) * block] = True
        assert np.all(p[:, ~mask] == 0)
        assert np.count_nonzero(p[:, mask]) > 0.99 * p[:, mask].size


def test_algorithmic_bytes_table():
    # (N+3) * rows * H * b + H * b, the fused path's touch-once traffic
    assert workloads.get("shard70b").fused_bytes() == 184_565_760
    assert workloads.get("page1").fused_bytes() == 41_951_232
    assert workloads.get("zero_padded").fused_bytes() == 293_611_520
    assert workloads.get("cu_restricted").fused_bytes() == 369_115_136
    assert workloads.get("tiny").fused_bytes() == 20_736
    assert workloads.get("shard70b").unfused_bytes() == 218_120_192
