#!/usr/bin/env python3
"""Benchmark: fused reduce of N partials + residual add + RMSNorm on one
MI355X, reported as algorithmic HBM GB/s, fraction of the 8 TB/s peak and
token-rows/s.

Default workload: N=8 partials of [1024, 8192] bf16 (one 8-way shard of
8192 tokens at a 70B-class hidden size).  A step is one fused call over one
rotating set of resident buffers; S sets totalling at least twice the 256 MB
Infinity Cache are cycled so the timed bytes come from HBM, not the cache.

Prints ONE JSON line.  Besides the headline it carries the per-call
distribution (median, p10, p90 over ~1 ms batches timed right after the
headline's steps) and a per_config block: every other
workload at its full size (the CU-restricted one on 8, 16, 32 CUs and the
whole chip), each with its oracle check of a row slice, and the unfused
pair on the headline's buffers.  --report PATH also writes a detailed JSON: the
unfused pair, the AllGather store, decode-size rows, the two-split overlap
beside a GEMM, row-count scaling, the plain-copy
ceiling, the ceiling of the fused call's own traffic pattern, the same step
as plain eager PyTorch ops, the isolated single call's time, the oracle
on every host core, and a cache-resident figure.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--report PATH]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused reduce+RMSNorm HBM GB/s (% of peak) and token-rows/s at H=8192, N=8"
PEAK_GBS = 8000.0              # MI355X HBM3E, published
MALL_BYTES = 256 * 1024 * 1024  # Infinity Cache
PROFILE_DIR = os.path.join(ROOT, "profiles")
COPY_CAL_BYTES = 512 * 1024 * 1024   # plain copy of known size for counter scaling
KERNEL_SOURCES = ["reduce_residual_add_amd/csrc/twnorm_kernels.hpp",
                  "reduce_residual_add_amd/csrc/twnorm_launch_impl.hpp",
                  "reduce_residual_add_amd/csrc/twnorm_validate.cpp"]


def _strip_comments(src: str) -> str:
    """C++ source without comments and whitespace (so that editing comments
    does not mark the kernel as changed)."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "".join(src.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def counter_traffic(workload: str, cu: int = 0):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload (at n_cu_limit `cu`, 0 = whole chip), or None if absent or
    taken on a different kernel source."""
    tag = f"_cu{cu}" if cu > 0 else ""
    path = os.path.join(PROFILE_DIR, f"fused_{workload}{tag}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_hash and m_bytes) or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="shard70b")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cu", type=int, default=0, help="n_cu_limit of the timed calls (0 = whole chip)")
    p.add_argument("--rotate", type=int, default=0, help="rotating buffer sets (0 = auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--report", default="", help="write a detailed JSON report here")
    p.add_argument("--overlap-cus", type=int, default=128,
                   help="CUs given to the fused call in the --report two-split overlap")
    p.add_argument("--unfused-steps", type=int, default=0,
                   help="after the timed steps, run this many unfused reduce + norm pairs "
                        "(for hardware-counter runs)")
    p.add_argument("--allgather-steps", type=int, default=0,
                   help="after the timed steps, run this many fused calls with the AllGather "
                        "store into N gather buffers (for hardware-counter runs)")
    p.add_argument("--no-per-config", action="store_true",
                   help="skip the per_config block (every other workload and CU limit, and "
                        "the unfused pair, timed in the same run)")
    p.add_argument("--calibration-copies", type=int, default=0,
                   help="after the timed steps, run this many plain copies of "
                        f"{COPY_CAL_BYTES >> 20} MiB (hardware-counter calibration)")
    return p.parse_args(argv)


# ---------------------------------------------------------------------------
# device buffers
# ---------------------------------------------------------------------------


def _to_dev(arr, dtype):
    import numpy as np
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def make_sets(inp, n_sets):
    """n_sets resident copies of the inputs (+ outputs); set 0 holds the
    host draw, the others are device clones at other addresses."""
    import torch
    dt = inp["dtype"]
    base = dict(parts=[_to_dev(p, dt) for p in inp["partials"]], res=_to_dev(inp["residual"], dt),
                w=_to_dev(inp["weight"], dt))
    sets = []
    for s in range(n_sets):
        if s == 0:
            d = dict(base)
        else:
            d = dict(parts=[p.clone() for p in base["parts"]], res=base["res"].clone(), w=base["w"].clone())
        d["out"] = torch.empty_like(d["res"])
        d["res_out"] = torch.empty_like(d["res"])
        d["red"] = torch.empty_like(d["res"])
        sets.append(d)
    torch.cuda.synchronize()
    return sets


def n_rotating_sets(set_bytes, requested):
    if requested > 0:
        return requested
    s = 3
    while s * set_bytes < 2 * MALL_BYTES:
        s += 1
    return s


def time_batches(step_fns, est_us_per_call, stream=None, batches=30, batch_ms=1.0):
    """Per-call time distribution over `batches` batches of back-to-back
    calls, each batch about `batch_ms` of GPU time and a whole number of
    passes over the rotating sets (or, with more sets than four batches
    hold, consecutive calls of the rotation), with one event between
    consecutive batches.
    An event recorded between two kernels on MI355X costs about 1 us of GPU
    time (measured: 30.3 -> 31.4 us per call with an event every 3 calls), so
    the headline mean is timed without them and this pass runs after it, with
    batches long enough that the events cost about 0.1%."""
    import torch
    n = len(step_fns)
    want = max(1, int(round(batch_ms * 1e3 / max(est_us_per_call, 1e-3))))
    # whole passes over the sets, unless one pass alone is far longer than a
    # batch (thousands of sets of a latency-bound workload): then each batch
    # continues the rotation where the previous one stopped
    calls = max(1, int(round(want / n))) * n if n <= 4 * want else want
    for f in step_fns:
        f()
    torch.cuda.synchronize()
    s = stream if stream is not None else torch.cuda.current_stream()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(batches + 1)]
    gate(s)
    marks[0].record(s)
    k = 0
    for b in range(batches):
        for _ in range(calls):
            step_fns[k % n]()
            k += 1
        marks[b + 1].record(s)
    torch.cuda.synchronize()
    per_call = [marks[b].elapsed_time(marks[b + 1]) * 1e3 / calls for b in range(batches)]
    return batch_distribution(per_call, calls)


def batch_distribution(per_call_us, calls_per_batch):
    """Median, p10 and p90 (nearest rank) of per-call times in microseconds,
    one value per batch."""
    v = sorted(per_call_us)
    if not v:
        return None

    def pct(q):
        return round(v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))], 3)
    return {"batches": len(v), "calls_per_batch": calls_per_batch, "median_us": pct(0.5),
            "p10_us": pct(0.1), "p90_us": pct(0.9)}


# GPU-side delay queued ahead of a start event (about 45 us on MI355X): while
# it runs, the host enqueues the first timed calls, so the timed region holds
# the calls back to back instead of also holding the host's latency to issue
# the first one after an idle stream (about 1% of a 20-call region).
GATE_CYCLES = 100_000


def gate(stream):
    import torch
    with torch.cuda.stream(stream):
        torch.cuda._sleep(GATE_CYCLES)


def time_steps(step_fns, steps, warmup, stream=None):
    """Warm up, then time exactly `steps` calls between two events recorded
    on the stream the kernels run on (default: the current stream), with a
    device synchronisation on both sides and the start event behind the
    gate delay; returns (ms per step, wall s)."""
    import torch
    n = len(step_fns)
    for i in range(warmup):
        step_fns[i % n]()
    torch.cuda.synchronize()
    s = stream if stream is not None else torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    gate(s)
    start.record(s)
    for i in range(steps):
        step_fns[i % n]()
    end.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def time_single_calls(step_fns, calls=60, stream=None):
    """One call at a time between two events, behind the gate delay, with a
    device synchronisation after each: the isolated call's time (no
    neighbour to overlap its start or end), over `calls` calls of the
    rotating sets.  Returns the median, p10 and p90 in microseconds."""
    import torch
    n = len(step_fns)
    s = stream if stream is not None else torch.cuda.current_stream()
    for f in step_fns:
        f()
    torch.cuda.synchronize()
    per_call = []
    for i in range(calls):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        gate(s)
        a.record(s)
        step_fns[i % n]()
        b.record(s)
        torch.cuda.synchronize()
        per_call.append(a.elapsed_time(b) * 1e3)
    d = batch_distribution(per_call, 1)
    return {"calls": calls, "median_us": d["median_us"], "p10_us": d["p10_us"],
            "p90_us": d["p90_us"]}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded row sample (the only use of oracle/)
# ---------------------------------------------------------------------------


def cpu_baseline(inp, w, gpu_out, gpu_res_out, target_seconds, all_core_threads=0):
    """The oracle on one host thread over a bounded sample of the inputs
    (GB/s, rows/s, and its check of the GPU's first rows); with
    all_core_threads > 0 also the same oracle on that many threads, each
    working through its own 64-row slices (numpy releases the GIL inside its
    array loops), as `all_cores`."""
    import numpy as np
    from oracle import twnorm_oracle as O
    rows_total = inp["rows"]
    chunk = min(rows_total, 64)
    done_rows = 0
    spent = 0.0
    first = None
    start = 0
    while (done_rows == 0 or spent < target_seconds) and spent < 30.0:
        sl = slice(start, start + chunk)
        sub = dict(inp, partials=[p[sl] for p in inp["partials"]], residual=inp["residual"][sl])
        t0 = time.perf_counter()
        ref_out, ref_res = O.fused_from_storage(sub)
        spent += time.perf_counter() - t0
        if first is None:
            first = (sl, ref_out, ref_res)
        done_rows += chunk
        start = (start + chunk) % rows_total
        if start + chunk > rows_total:
            start = 0
    rows_per_s = done_rows / spent
    bytes_per_row = (w.n + 3) * w.hidden * w.elem_bytes
    # parity of the GPU's first rows against the oracle rows just computed
    sl, ref_out, ref_res = first
    got_out = O.decode(gpu_out[sl], w.dtype)
    got_res = O.decode(gpu_res_out[sl], w.dtype)

    def fails(got, ref):
        d = np.abs(got - ref)
        bound = (np.maximum(2e-2, 1e-2 * np.abs(ref)) if w.dtype == "bf16"
                 else 1e-5 * np.maximum(1.0, np.abs(ref)))
        return int(np.count_nonzero(~(d <= bound))), float(d.max())

    f_out, m_out = fails(got_out, ref_out)
    f_res, m_res = fails(got_res, ref_res)
    all_cores = None
    if all_core_threads > 0:
        from concurrent.futures import ThreadPoolExecutor
        starts = list(range(0, rows_total - chunk + 1, chunk)) or [0]

        def worker(t):
            done, i = 0, t
            t_end = time.perf_counter() + min(target_seconds, 5.0)
            while time.perf_counter() < t_end:
                st = starts[i % len(starts)]
                s2 = slice(st, st + chunk)
                O.fused_from_storage(dict(inp, partials=[p[s2] for p in inp["partials"]],
                                          residual=inp["residual"][s2]))
                done += chunk
                i += all_core_threads
            return done

        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=all_core_threads) as ex:
            rows_mt = sum(ex.map(worker, range(all_core_threads)))
        wall = time.perf_counter() - t0
        all_cores = {"threads": all_core_threads, "rows": rows_mt, "wall_s": round(wall, 2),
                     "rows_per_s": round(rows_mt / wall, 1),
                     "value": round(rows_mt / wall * bytes_per_row / 1e9, 4), "unit": "GB/s"}
    result = {
        "value": round(rows_per_s * bytes_per_row / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"float64 numpy oracle on {done_rows} token rows ({chunk}-row slices of the "
                  f"same {w.name} inputs, {spent:.1f} s, single thread); "
                  f"{rows_per_s:.1f} rows/s",
        "rows_per_s": round(rows_per_s, 2),
        "host_cpu": _cpu_model(),
        "affinity_cores": len(os.sched_getaffinity(0)),
        "parity_rows": f"{sl.start}:{sl.stop}",
        "parity_fails": f_out + f_res,
        "parity_max_abs": max(m_out, m_res),
    }
    if all_cores is not None:
        result["all_cores"] = all_cores
    return result


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _from_dev(t, dtype):
    import numpy as np
    import torch
    t = t.detach().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# ---------------------------------------------------------------------------
# main measurement
# ---------------------------------------------------------------------------


def measure_fused(twn, w, sets, cu, steps, warmup, stream=None, with_distribution=False):
    """Per-step time of the fused call.  With cu > 0 and `stream` the
    library's CU-masked stream, the kernels are queued and timed there
    directly (no per-call join to another stream).  With_distribution adds
    the per-call distribution over ~1 ms batches from a second pass."""
    fns = [twn.PreparedFused(d["parts"], d["res"], d["w"], w.eps, d["out"], d["res_out"],
                             n_cu_limit=cu, stream=stream) for d in sets]
    ms, wall = time_steps(fns, steps, warmup, stream=stream)
    if with_distribution:
        return ms, wall, time_batches(fns, ms * 1e3, stream=stream)
    return ms, wall


def measure_unfused(twn, w, sets, steps, warmup):
    def pair(d):
        def f():
            twn.reduce(d["parts"], out=d["red"])
            twn.rmsnorm(d["red"], d["res"], d["w"], w.eps, out=d["out"], residual_out=d["res_out"])
        return f
    return time_steps([pair(d) for d in sets], steps, warmup)


def measure_fused_graph(twn, w, sets, calls=64, replays=20):
    """Per-call time of `calls` fused calls captured in one HIP graph and
    replayed: the GPU-side cost without host launch overhead (which matters
    for small, launch-bound calls)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for d in sets:
            twn.fused_reduce_rmsnorm(d["parts"], d["res"], d["w"], w.eps, out=d["out"],
                                     residual_out=d["res_out"])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            d = sets[i % len(sets)]
            twn.fused_reduce_rmsnorm(d["parts"], d["res"], d["w"], w.eps, out=d["out"],
                                     residual_out=d["res_out"])
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / (replays * calls)


def measure_rows_scaling(twn, w, base_set, row_counts=(512, 1024, 2048, 4096, 8192)):
    """Per-call time of the fused call at several row counts of the same
    (dtype, H, N), each over rotating sets totalling at least twice the
    Infinity Cache.  The larger inputs repeat the workload's rows on the
    device: the values do not change the timing.  Returns {rows: {us, gbs}}."""
    import torch
    out = {}
    per_row = (w.n + 3) * w.hidden * w.elem_bytes
    for rows in row_counts:
        reps = -(-rows // w.rows)
        grow = lambda t: t.repeat(reps, 1)[:rows].contiguous()
        n_sets = n_rotating_sets(rows * per_row, 0)
        sets = []
        for _ in range(n_sets):
            res = grow(base_set["res"])
            sets.append(dict(parts=[grow(p) for p in base_set["parts"]], res=res, w=base_set["w"],
                             out=torch.empty_like(res), res_out=torch.empty_like(res)))
        torch.cuda.synchronize()
        steps = max(60, (300 * 1024) // rows)
        ms = sorted(measure_fused(twn, w, sets, 0, steps, 20)[0] for _ in range(3))[1]
        byt = rows * per_row + w.hidden * w.elem_bytes
        out[str(rows)] = {"us_per_call": round(ms * 1e3, 2), "gbs": round(byt / (ms * 1e-3) / 1e9, 1),
                          "rotating_sets": n_sets}
        del sets
        torch.cuda.empty_cache()
    return out


def measure_allgather(twn, w, sets, steps, warmup):
    """The fused step with the AllGather store: each call writes its rows
    into N gather buffers of N * rows rows (one per simulated rank), at the
    offset of the shard it plays (cycling over the N shards)."""
    import torch
    ranks = w.n
    total = ranks * w.rows
    gathers = [torch.empty((total, w.hidden), dtype=sets[0]["res"].dtype, device="cuda")
               for _ in range(ranks)]
    fns = []
    for i in range(len(sets) * ranks):
        d = sets[i % len(sets)]
        off = (i % ranks) * w.rows
        fns.append(lambda d=d, off=off: twn.fused_reduce_rmsnorm_allgather(
            d["parts"], d["res"], d["w"], w.eps, gathers, off, residual_out=d["res_out"]))
    ms, _ = time_steps(fns, steps, warmup)
    # the same traffic without the arithmetic: N partials and the residual
    # read; residual_out and the N gather slices written
    mix_fns = []
    for i in range(len(sets) * ranks if ranks + 1 <= 16 else 0):
        d = sets[i % len(sets)]
        off = (i % ranks) * w.rows
        dsts = [d["res_out"]] + [g[off:off + w.rows] for g in gathers]
        mix_fns.append(lambda d=d, dsts=dsts: twn.stream_mix(list(d["parts"]) + [d["res"]], dsts))
    mix_ms = time_steps(mix_fns, steps, warmup)[0] if mix_fns else float("nan")
    b = w.elem_bytes
    nbytes = (w.n + 2 + ranks) * w.rows * w.hidden * b + w.hidden * b
    del gathers
    return ms, nbytes, mix_ms


def measure_overlap(twn, w, sets, k, iters=40):
    """Two-split overlap: fused calls for one token split on the first k CUs
    while the row-parallel GEMM of the other split (the MLP down-projection
    of an 8-way tensor-parallel 70B-class layer: [rows, 3584] x [3584, H],
    bf16, hipBLASLt via torch) runs on the other CUs.  Each side queues
    `iters` calls and joins once, so no per-call cross-queue dependency is
    timed.  Returns a dict of per-iteration times in microseconds."""
    import torch
    a = torch.randn(w.rows, 3584, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(3584, w.hidden, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(w.rows, w.hidden, device="cuda", dtype=torch.bfloat16)
    masked = twn.cu_masked_stream(k)
    comp = twn.cu_complement_stream(k)
    fused = [twn.PreparedFused(d["parts"], d["res"], d["w"], w.eps, d["out"], d["res_out"],
                               n_cu_limit=k, stream=masked) for d in sets]

    def gemm():
        torch.matmul(a, b, out=c)

    def timed(work):   # work() enqueues; returns microseconds per iteration
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        work()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / iters

    def fused_on_masked():
        for i in range(iters):
            fused[i % len(fused)]()

    def gemm_on(stream):
        with torch.cuda.stream(stream):
            for _ in range(iters):
                gemm()

    def both():
        fused_on_masked()
        gemm_on(comp)

    side = torch.cuda.Stream()   # default priority, no CU mask
    side2 = torch.cuda.Stream()
    fused_full = [twn.PreparedFused(d["parts"], d["res"], d["w"], w.eps, d["out"], d["res_out"],
                                    n_cu_limit=0, stream=side2) for d in sets]

    def both_unmasked_gemm():
        fused_on_masked()
        gemm_on(side)

    def both_unmasked():   # no CU mask on either side: the hardware shares every CU
        for i in range(iters):
            fused_full[i % len(fused_full)]()
        gemm_on(side)

    for f in (fused_on_masked, lambda: gemm_on(comp), lambda: gemm_on(torch.cuda.current_stream())):
        f()   # warm-up (hipBLASLt heuristics, code objects)
    res = {
        "k_cus": k,
        "gemm_all_cus_us": timed(lambda: gemm_on(torch.cuda.current_stream())),
        "gemm_on_complement_us": timed(lambda: gemm_on(comp)),
        "fused_on_k_cus_us": timed(fused_on_masked),
        "overlapped_us": timed(both),
        "overlapped_gemm_unmasked_us": timed(both_unmasked_gemm),
        "overlapped_both_unmasked_us": timed(both_unmasked),
    }
    gflop = 2.0 * w.rows * 3584 * w.hidden / 1e9
    res["gemm_tflops_all_cus"] = gflop / res["gemm_all_cus_us"] * 1e3   # GFLOP/us = PFLOP/s
    return res


def measure_mix(twn, w, sets, steps, warmup):
    """The fused call's traffic pattern without its arithmetic
    (tw_stream_mix): the N partials and the residual read, residual_out and
    out written, on the same rotating buffers.  Returns (ms per call, bytes
    moved per call)."""
    fns = []
    for d in sets:
        srcs = list(d["parts"]) + [d["res"]]
        dsts = [d["res_out"], d["out"]]
        fns.append(lambda srcs=srcs, dsts=dsts: twn.stream_mix(srcs, dsts))
    ms, _ = time_steps(fns, steps, warmup)
    return ms, (w.n + 3) * w.rows * w.hidden * w.elem_bytes


def measure_torch_eager(w, sets, steps, warmup):
    """The same step written as plain eager PyTorch ops (float32 arithmetic,
    stores in the storage dtype), on the same rotating buffers: context for
    what the fusion saves, not part of the library."""
    import torch

    def step(d):
        x = d["parts"][0].float()
        for p in d["parts"][1:]:
            x += p.float()
        x += d["res"].float()
        d["res_out"].copy_(x)
        inv = torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + w.eps)
        d["out"].copy_(x * inv * d["w"].float())

    fns = [lambda d=d: step(d) for d in sets]
    ms, _ = time_steps(fns, steps, warmup)
    return ms


def measure_copy(twn, total_bytes, steps, warmup):
    import torch
    n = total_bytes // 2
    bufs = [(torch.empty(n, dtype=torch.uint8, device="cuda"), torch.empty(n, dtype=torch.uint8, device="cuda"))
            for _ in range(2)]
    fns = [lambda a=a, b=b: twn.stream_copy(a, b) for a, b in bufs]
    ms, _ = time_steps(fns, steps, warmup)
    return ms, n


# CU limits of the CU-restricted workload's sweep (0 = the whole chip).
SWEEP_CU_LIMITS = (0, 8, 16, 32)


def _steps_for(us_per_call, target_ms=20.0, lo=30, hi=2000):
    """Timed steps that keep one measurement near `target_ms` of GPU time."""
    return int(min(hi, max(lo, target_ms * 1e3 / max(us_per_call, 1e-3))))


def measure_config(twn, w, seed, cu_limits, dev_cus, cpu_seconds):
    """One workload at its full size, at each CU limit: per-call time over
    rotating sets, GB/s, fraction of peak, the per-batch distribution, and
    the oracle's check of a row slice of the outputs the timed calls left."""
    import torch
    import workloads
    inp = workloads.make(w, seed=seed)
    n_sets = n_rotating_sets(w.fused_bytes(), 0)
    launch_bound = w.fused_bytes() < (1 << 20)
    if launch_bound:
        # A call this small is bound by launch latency, not HBM: its data
        # stays cache-resident and more sets would change nothing.
        n_sets = min(n_sets, 64)
    sets = make_sets(inp, n_sets)
    code = twn.TW_BF16 if w.dtype == "bf16" else twn.TW_F32
    entries = {}
    for cu in cu_limits:
        stream = twn.cu_masked_stream(cu) if cu > 0 else None
        probe, _ = measure_fused(twn, w, sets, cu, 3 * n_sets, n_sets, stream=stream)
        steps = _steps_for(probe * 1e3)
        steps -= steps % n_sets
        ms, _, dist = measure_fused(twn, w, sets, cu, steps, max(n_sets, 10), stream=stream,
                                    with_distribution=True)
        gbs = w.fused_bytes() / (ms * 1e-3) / 1e9
        call_cus = cu if 0 < cu < dev_cus else dev_cus
        e = {"n_cu_limit": cu, "us_per_call": round(ms * 1e3, 3), "gbs": round(gbs, 1),
             "frac_of_peak": round(gbs / PEAK_GBS, 4),
             "token_rows_per_s": round(w.rows / (ms * 1e-3), 1), "steps": steps,
             "rotating_sets": n_sets, "per_call_distribution": dist,
             "launch_shape": list(twn.query_fused_shape(code, w.hidden, w.n, w.rows, call_cus,
                                                        dev_cus)),
             "traffic_per_call": counter_traffic(w.name, cu if call_cus < dev_cus else 0)}
        torch.cuda.synchronize()
        d0 = sets[0]
        # the timed calls ended on the last set; set 0 holds the outputs of
        # one of them at this CU limit
        cb = cpu_baseline(inp, w, _from_dev(d0["out"], w.dtype), _from_dev(d0["res_out"], w.dtype),
                          cpu_seconds)
        e["oracle_parity_rows"] = cb["parity_rows"]
        e["oracle_parity_fails"] = cb["parity_fails"]
        e["oracle_parity_max_abs"] = cb["parity_max_abs"]
        e["cpu_oracle_gbs"] = cb["value"]
        if launch_bound and cu == 0:
            e["latency_bound"] = True
            e["us_per_call_graph_replay"] = round(measure_fused_graph(twn, w, sets) * 1e3, 3)
        entries[f"cu{cu}"] = e
    del sets
    torch.cuda.empty_cache()
    return {"workload": w.name, "n_partials": w.n, "rows": w.rows, "hidden": w.hidden,
            "dtype": w.dtype, "algorithmic_bytes_per_call": w.fused_bytes(),
            "traffic_per_call": counter_traffic(w.name), "by_cu_limit": entries}


def measure_per_config(twn, args, w_main, main_sets, main_ms, dev_cus):
    """Every other workload (and the CU-restricted sweep) timed in the same
    run as the headline, plus the unfused pair on the headline's buffers."""
    import workloads
    out = {}
    # The sweep needs three CU masks of its own; a process may hold three.
    cu_ok = args.cu == 0 and not args.report
    for w in workloads.WORKLOADS:
        if w.name == w_main.name and args.cu == 0:
            continue
        limits = w.cu_limits if cu_ok else (0,)
        out[w.name] = measure_config(twn, w, args.seed, limits, dev_cus, cpu_seconds=0.3)
        if not cu_ok and w.cu_limits != (0,):
            out[w.name]["note"] = "CU-limited runs skipped: this run holds other CU masks"
    ums, _ = measure_unfused(twn, w_main, main_sets, _steps_for(main_ms * 1e3 * 1.3), 10)
    out["unfused_pair"] = {"workload": w_main.name, "us_per_step": round(ums * 1e3, 3),
                           "algorithmic_bytes": w_main.unfused_bytes(),
                           "gbs_on_unfused_bytes": round(w_main.unfused_bytes() / (ums * 1e-3) / 1e9, 1),
                           "fused_speedup": round(ums / main_ms, 4)}
    return out


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the library's path "
                                   "covers one GPU's token shard and has no multi-GPU transport",
                          "n_gpus": args.gpus}))
        return 2
    import torch
    import reduce_residual_add_amd as twn
    import workloads

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    twn.load()
    w = workloads.get(args.workload)
    inp = workloads.make(w, seed=args.seed)
    set_bytes = w.fused_bytes() + w.rows * w.hidden * w.elem_bytes   # + the unfused intermediate
    n_sets = n_rotating_sets(set_bytes, args.rotate)
    sets = make_sets(inp, n_sets)

    dev_cus = torch.cuda.get_device_properties(0).multi_processor_count
    call_cus = args.cu if 0 < args.cu < dev_cus else dev_cus
    masked = twn.cu_masked_stream(args.cu) if args.cu > 0 else None
    ms, wall, dist = measure_fused(twn, w, sets, args.cu, args.steps, args.warmup, stream=masked,
                                   with_distribution=True)
    bytes_call = w.fused_bytes()
    gbs = bytes_call / (ms * 1e-3) / 1e9
    rows_per_s = w.rows / (ms * 1e-3)

    metric = METRIC if w.name == "shard70b" else (
        f"fused reduce+RMSNorm HBM GB/s (% of peak) and token-rows/s, {w.name} workload "
        f"(H={w.hidden}, N={w.n}, {w.rows} rows)")
    result = {
        "metric": metric,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "n_partials": w.n, "rows": w.rows, "hidden": w.hidden,
                   "dtype": w.dtype, "eps": w.eps, "n_cu_limit": args.cu,
                   "rotating_sets": n_sets, "parallelism": "single GPU"},
        "launch_shape": dict(zip(("waves_per_row", "chunks_per_lane", "team_lanes"),
                                 twn.query_fused_shape(twn.TW_BF16 if w.dtype == "bf16" else twn.TW_F32,
                                                       w.hidden, w.n, w.rows, call_cus, dev_cus))),
        "pct_of_peak": round(100.0 * gbs / PEAK_GBS, 2),
        "token_rows_per_s": round(rows_per_s, 1),
        "per_call_distribution": dist,
        "algorithmic_bytes_per_step": bytes_call,
        "wall_s_timed": round(wall, 4),
        "timed_region": ("exactly `steps` calls between two HIP events on the kernels' stream, "
                         "device-synchronised on both sides; a GPU-side delay queued before the "
                         "start event keeps the host's first-launch latency out"),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_GBS, 4),
                     "traffic": counter_traffic(w.name, args.cu if call_cus < dev_cus else 0)},
    }
    if args.cu > 0:
        # the same calls issued from the default stream: each one pays the
        # event join to the masked stream and back
        jms, _ = measure_fused(twn, w, sets, args.cu, max(20, args.steps // 5), 5)
        result["ms_per_step_joined_from_default_stream"] = round(jms, 6)

    if args.unfused_steps > 0:
        for i in range(args.unfused_steps):
            d = sets[i % len(sets)]
            twn.reduce(d["parts"], out=d["red"])
            twn.rmsnorm(d["red"], d["res"], d["w"], w.eps, out=d["out"], residual_out=d["res_out"])
        torch.cuda.synchronize()

    if args.allgather_steps > 0:
        gathers = [torch.empty((w.n * w.rows, w.hidden), dtype=sets[0]["res"].dtype, device="cuda")
                   for _ in range(w.n)]
        for i in range(args.allgather_steps):
            d = sets[i % len(sets)]
            twn.fused_reduce_rmsnorm_allgather(d["parts"], d["res"], d["w"], w.eps, gathers,
                                               (i % w.n) * w.rows, residual_out=d["res_out"])
        torch.cuda.synchronize()
        del gathers

    if args.calibration_copies > 0:
        src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(args.calibration_copies):
            twn.stream_copy(src, dst)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = COPY_CAL_BYTES
        del src, dst

    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        d0 = sets[0]
        # recompute set 0 once so its outputs are the ones checked
        twn.fused_reduce_rmsnorm(d0["parts"], d0["res"], d0["w"], w.eps, out=d0["out"],
                                 residual_out=d0["res_out"])
        torch.cuda.synchronize()
        result["cpu_baseline"] = cpu_baseline(inp, w, _from_dev(d0["out"], w.dtype),
                                              _from_dev(d0["res_out"], w.dtype), args.cpu_seconds,
                                              len(os.sched_getaffinity(0)) if args.report else 0)

    if not args.no_per_config:
        result["per_config"] = measure_per_config(twn, args, w, sets, ms, dev_cus)

    if args.report:
        rep = {"main": result, "kernel_source_sha256": kernel_source_hash()}
        ums, _ = measure_unfused(twn, w, sets, max(50, args.steps // 4), 10)
        rep["unfused_pair"] = {"ms_per_step": ums, "algorithmic_bytes": w.unfused_bytes(),
                               "gbs_on_unfused_bytes": w.unfused_bytes() / (ums * 1e-3) / 1e9,
                               "speedup_fused_vs_unfused": ums / ms}
        ams, abytes, amix = measure_allgather(twn, w, sets, max(50, args.steps // 4), 10)
        rep["allgather_store"] = {"ms_per_step": ams, "algorithmic_bytes": abytes,
                                  "gather_buffers": w.n, "gbs": abytes / (ams * 1e-3) / 1e9,
                                  "traffic_pattern_ms": amix,
                                  "fused_time_over_pattern_time": ams / amix}
        # decode-size rows: latency per call at a few row counts of the same
        # (dtype, H, N); below the CU count the kernel runs its latency shape
        dec = {}
        for rows in (1, 8, 64):
            wd = w.with_rows(rows)
            dsets = make_sets(workloads.make(wd, seed=args.seed), 8)
            dms, _ = measure_fused(twn, wd, dsets, 0, 400, 40)
            gms = measure_fused_graph(twn, wd, dsets)
            dec[str(rows)] = {"launch_shape": list(twn.query_fused_shape(
                                  twn.TW_BF16 if w.dtype == "bf16" else twn.TW_F32, w.hidden, w.n,
                                  rows, call_cus, dev_cus)),
                              "us_per_call": round(dms * 1e3, 3),
                              "us_per_call_graph_replay": round(gms * 1e3, 3),
                              "gbs": round(wd.fused_bytes() / (dms * 1e-3) / 1e9, 1)}
            del dsets
        rep["decode_rows"] = dec
        ov = measure_overlap(twn, w, sets, args.overlap_cus)
        full_fused_us = ms * 1e3
        ov["fused_all_cus_us"] = full_fused_us
        ov["sequential_all_cus_us"] = ov["gemm_all_cus_us"] + full_fused_us
        ov["overlap_speedup_vs_sequential"] = ov["sequential_all_cus_us"] / ov["overlapped_us"]
        ov["overlap_gemm_unmasked_speedup_vs_sequential"] = (ov["sequential_all_cus_us"] /
                                                             ov["overlapped_gemm_unmasked_us"])
        ov["overlap_both_unmasked_speedup_vs_sequential"] = (ov["sequential_all_cus_us"] /
                                                             ov["overlapped_both_unmasked_us"])
        rep["two_split_overlap"] = ov
        if w.dtype == "bf16" and w.rows >= 64:
            rep["rows_scaling"] = measure_rows_scaling(twn, w, sets[0])
        cms, cbytes = measure_copy(twn, 2 * MALL_BYTES, 200, 20)
        copy_gbs = 2 * cbytes / (cms * 1e-3) / 1e9
        rep["copy_ceiling"] = {"ms": cms, "bytes_moved": 2 * cbytes, "gbs": copy_gbs,
                               "fused_frac_of_copy_ceiling": gbs / copy_gbs}
        mms, mbytes = measure_mix(twn, w, sets, max(50, args.steps // 4), 10)
        rep["mix_ceiling"] = {"ms": mms, "bytes_moved": mbytes,
                              "gbs": mbytes / (mms * 1e-3) / 1e9,
                              "fused_time_over_mix_time": ms / mms}
        tms = measure_torch_eager(w, sets, max(20, args.steps // 10), 5)
        rep["torch_eager_same_step"] = {"ms": tms, "gbs_on_fused_bytes": bytes_call / (tms * 1e-3) / 1e9,
                                        "fused_speedup": tms / ms}
        fns = [twn.PreparedFused(d["parts"], d["res"], d["w"], w.eps, d["out"], d["res_out"],
                                 n_cu_limit=args.cu, stream=masked) for d in sets]
        rep["single_call"] = time_single_calls(fns, stream=masked)
        del fns
        # cache-resident figure (one buffer set, repeated): NOT an HBM number
        wms, _ = measure_fused(twn, w, sets[:1], args.cu, 200, 20)
        rep["warm_same_buffers_not_hbm"] = {"ms": wms, "gbs": bytes_call / (wms * 1e-3) / 1e9}
        with open(args.report, "w") as f:
            json.dump(rep, f, indent=1)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
