"""Benchmark of the block-scaled FP4 routed-expert MLP on one MI355X.

A step is one call of mx_grouped_expert_mlp over the whole batch: activation
quantisation, routing permute/scan, L1 gate/up GEMM with the fused SiLU*up and
MXFP4 re-quant, L2 down GEMM with the gate weight, and the weighted combine.
Workload: 48 local experts, 4096 tokens, top-8, hidden 7168, intermediate 3072,
MXFP4 weights (uniform random codes, E8M0 exponents 120..130) and bf16 N(0,1)
activations, all synthetic and resident in HBM before timing starts.

Prints one JSON line. `value` is TFLOP/s over 6 * tokens * k * hidden * inter
algorithmic FLOPs per step. `roofline` is for the dominant kernel (the L1
GEMM), timed with HIP events recorded on the stream it runs on, during the
timed steps. `cpu_baseline` times the CPU oracle on a bounded sample (all
pairs routed to the first few experts).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "expert-MLP TFLOP/s & frac of FP4 peak, 48 experts x 4096 tok top-8 (1 GPU)"
PEAK_FP4_TFLOPS = 10100.0     # MI355X dense MXFP4 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-experts", type=int, default=4,
                    help="experts in the oracle's bounded CPU sample")
    return ap.parse_args()


def dev_tensors(torch, d, names):
    return {n: torch.from_numpy(np.ascontiguousarray(d[n])).cuda() for n in names}


def bf16_dev(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def time_steps(torch, fn, steps, warmup, profile=None):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if profile:
        profile[0]()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stats = profile[1]() if profile else None
    return (t1 - t0) * 1e3 / steps, stats


def secondary(torch, mx, workloads):
    """Shared expert at decode/prefill sizes and dequant bandwidth (context lines)."""
    out = {}
    H, I = workloads.HIDDEN, workloads.INTER
    d = workloads.expert_weights(0)
    w = dev_tensors(torch, d, ("w1", "w1s", "w3", "w3s", "w2", "w2s"))
    wbytes = sum(v.numel() for v in w.values())
    for M in (1, 8, 128, 4096):
        x = bf16_dev(torch, workloads.activations(1, M))
        ws = torch.empty(mx.expert_mlp_workspace_size(M, H, I), dtype=torch.uint8, device="cuda")
        y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
        fn = lambda: mx.expert_mlp(x, w["w1"], w["w1s"], w["w3"], w["w3s"], w["w2"], w["w2s"], out=y, workspace=ws)
        ms, _ = time_steps(torch, fn, 20, 3)
        flops = 6.0 * M * H * I
        out[f"shared_expert_M{M}"] = {"ms": round(ms, 4), "TFLOP/s": round(flops / ms / 1e9, 2),
                                      "weight_GB/s": round(wbytes / ms / 1e6, 1)}
    # dequant (8 rotating buffer sets so the working set exceeds the 256 MB cache)
    dq = workloads.dequant_inputs(0)
    c = torch.from_numpy(dq["w1"]).cuda()
    s = torch.from_numpy(dq["w1s"]).cuda()
    sets = [(c.clone(), s.clone(), torch.empty((3072, 7168), dtype=torch.bfloat16, device="cuda")) for _ in range(8)]
    it = [0]

    def deq():
        cc, ss, oo = sets[it[0] % 8]
        it[0] += 1
        mx.dequant("mxfp4", cc, ss, 3072, 7168, out=oo)
    ms, _ = time_steps(torch, deq, 40, 8)
    nbytes = c.numel() + s.numel() + 3072 * 7168 * 2
    out["dequant_mxfp4_w1"] = {"ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1),
                               "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 3)}
    q = torch.from_numpy(dq["fp8"]).cuda()
    qs = torch.from_numpy(dq["fp8s"]).cuda()
    qsets = [(q.clone(), qs.clone(), torch.empty((7168, 1536), dtype=torch.bfloat16, device="cuda")) for _ in range(8)]

    def deq8():
        cc, ss, oo = qsets[it[0] % 8]
        it[0] += 1
        mx.dequant("fp8_b128", cc, ss, 7168, 1536, out=oo)
    ms, _ = time_steps(torch, deq8, 40, 8)
    nbytes = q.numel() + qs.numel() + 7168 * 1536 * 2
    out["dequant_fp8_block"] = {"ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1),
                                "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 3)}
    return out


def cpu_baseline(d, n_exp):
    """The oracle, untuned, on all pairs routed to experts 0..n_exp-1."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    ids = d["ids"].copy()
    pairs = int((ids < n_exp).sum())
    t0 = time.perf_counter()
    oracle.grouped_expert_mlp(d["x"], ids, d["w"], d["w1"][:n_exp], d["w1s"][:n_exp], d["w3"][:n_exp],
                              d["w3s"][:n_exp], d["w2"][:n_exp], d["w2s"][:n_exp])
    sec = time.perf_counter() - t0
    flops = 6.0 * pairs * d["x"].shape[1] * d["w1"].shape[1]
    return {"value": round(flops / sec / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(sec, 2),
            "sample": f"all {pairs} token-expert pairs routed to experts 0..{n_exp - 1} of the same "
                      f"batch (fp64 NumPy oracle, {len(os.sched_getaffinity(0))} host cores visible)"}


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (expert parallelism "
              "across GPUs is a design note only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import mxfp4_block_scaled_e2m1_amd as mx
    import workloads

    T, E, K = 4096, workloads.N_LOCAL_EXPERTS, workloads.TOP_K
    H, I = workloads.HIDDEN, workloads.INTER
    d = workloads.grouped(tokens=T, n_experts=E, k=K, seed=0)
    w = dev_tensors(torch, d, ("w1", "w1s", "w3", "w3s", "w2", "w2s", "ids", "w"))
    x = bf16_dev(torch, d["x"])
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.grouped_expert_mlp_workspace_size(T, H, I, K, E), dtype=torch.uint8, device="cuda")

    def step():
        mx.grouped_expert_mlp(x, w["ids"], w["w"], w["w1"], w["w1s"], w["w3"], w["w3s"], w["w2"], w["w2s"],
                              out=y, workspace=ws)

    ms, phases = time_steps(torch, step, a.steps, a.warmup, profile=(mx.profile_start, mx.profile_stop))
    flops = 6.0 * T * K * H * I
    value = flops / ms / 1e9   # TFLOP/s
    l1_ms, l1_n = phases["l1_gemm"]
    l1_avg = l1_ms / l1_n
    l1_flops = 2.0 * T * K * (2 * I) * H
    achieved = l1_flops / l1_avg / 1e9
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4 (E2M1 x E8M0 operands, fp32 accumulation)", "data": "synthetic",
        "config": {"workload": "routed expert MLP: 48 local experts x 4096 tokens, top-8, hidden 7168, "
                               "inter 3072, MXFP4 weights and activations",
                   "experts": E, "tokens": T, "top_k": K, "hidden": H, "inter": I,
                   "parallelism": "single GPU"},
        "frac_of_fp4_peak": round(value / PEAK_FP4_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": "l1_gemm (gate/up GEMM + SiLU*up + MXFP4 re-quant)",
                     "achieved": round(achieved, 2), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP4_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops_per_launch": l1_flops, "avg_launch_ms": round(l1_avg, 4)},
        "phases_ms_per_step": {k: round(v[0] / v[1], 4) for k, v in phases.items()},
    }
    if not a.no_secondary:
        rec["secondary"] = secondary(torch, mx, workloads)
    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(d, a.cpu_experts)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
