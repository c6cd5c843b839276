"""Child process of test_two_split_overlap_at_128_cus (not collected by
pytest): the two-split overlap at k CUs, checked against the oracle.

One token split's fused calls run on the library's stream limited to the
first k CUs while the other split's row-parallel GEMM (the MLP down-
projection of an 8-way tensor-parallel 70B-class layer, [1024, 3584] x
[3584, 8192] bf16, torch / hipBLASLt) runs beside them, first unmasked on an
ordinary stream, then on the k-complement stream; last, whole-chip fused
calls on an ordinary stream beside the unmasked GEMM ("TokenWeave: Efficient
Compute-Communication Overlap for Distributed LLM Inference", the split into
two token blocks, one computing while the other communicates).  Each fused
call writes its own outputs; all of them must match the oracle, and every
GEMM its solo result.  Prints OVERLAP_OK on success.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path[:0] = [ROOT, os.path.dirname(os.path.abspath(__file__))]

import torch  # noqa: E402

import reduce_residual_add_amd as twn  # noqa: E402
import workloads  # noqa: E402
from gpu_helpers import assert_parity, from_dev, inputs_to_dev, reference  # noqa: E402


def main(k: int) -> int:
    twn.load()
    w = workloads.get("shard70b")
    print(f"[overlap child] shard70b n={w.n} rows={w.rows} H={w.hidden}, fused on {k} CUs",
          flush=True)
    inp = workloads.make(w, seed=12)
    parts, res, wt = inputs_to_dev(inp)
    ref_out, ref_res, b_out, b_res = reference(inp)
    g = torch.Generator(device="cuda").manual_seed(5)
    a = torch.randn(w.rows, 3584, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(3584, w.hidden, device="cuda", dtype=torch.bfloat16, generator=g)
    solo_c = torch.matmul(a, b)
    torch.cuda.synchronize()
    masked = twn.cu_masked_stream(k)
    comp = twn.cu_complement_stream(k)
    side = torch.cuda.Stream()
    side2 = torch.cuda.Stream()
    calls = 4
    for gemm_stream, fused_stream, cu, label in (
            (side, masked, k, "GEMM unmasked"), (comp, masked, k, "GEMM on the complement"),
            (side, side2, 0, "GEMM unmasked beside whole-chip fused calls")):
        print(f"[overlap child] {label}", flush=True)
        outs = [(torch.full_like(res, 7.0), torch.full_like(res, 7.0)) for _ in range(calls)]
        cs = [torch.empty_like(solo_c) for _ in range(calls)]
        torch.cuda.synchronize()
        with torch.cuda.stream(gemm_stream):
            for c in cs:
                torch.matmul(a, b, out=c)
        with torch.cuda.stream(fused_stream):
            for o, r in outs:
                twn.fused_reduce_rmsnorm(parts, res, wt, inp["eps"], out=o, residual_out=r,
                                         n_cu_limit=cu)
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(outs):
            assert_parity(from_dev(r, "bf16"), ref_res, "bf16", f"{label} call {i} residual_out",
                          b_res)
            assert_parity(from_dev(o, "bf16"), ref_out, "bf16", f"{label} call {i} out", b_out)
        for i, c in enumerate(cs):
            assert torch.equal(c, solo_c), f"{label}: GEMM {i} differs from its solo run"
    print(f"OVERLAP_OK k={k}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(int(sys.argv[1]) if len(sys.argv) > 1 else 128))
