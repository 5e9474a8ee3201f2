"""Benchmark of the block-scaled FP4 routed-expert MLP on one MI355X.

A step is one call of mx_grouped_expert_mlp over the whole batch: activation
quantisation, routing permute/scan, L1 gate/up GEMM with the fused SiLU*up and
MXFP4 re-quant, L2 down GEMM with the gate weight, and the weighted combine.
Workload: 48 local experts, 4096 tokens, top-8, hidden 7168, intermediate 3072,
MXFP4 weights (uniform random codes, E8M0 exponents 120..130) and bf16 N(0,1)
activations, all synthetic and resident in HBM before timing starts.

Prints one JSON line. `value` is TFLOP/s over 6 * tokens * k * hidden * inter
algorithmic FLOPs per step, timed with nothing else recorded. `roofline` is for
the dominant kernel (the L1 GEMM), timed with HIP events recorded on the stream
it runs on, in a second pass of the same steps; its `traffic` is the HBM byte count per launch from rocprofv3
FETCH_SIZE / WRITE_SIZE runs scaled by a copy of known size (see
`L1_TRAFFIC`), reported only while the GEMM sources are the ones it was
measured on. `cpu_baseline` times the CPU oracle on a bounded sample (all
pairs routed to the first few experts). `secondary` holds the other
configurations: the shared expert (few-token sizes replayed from a hipGraph
over 16 rotating weight copies, so the weights come from HBM), the skewed
16384-token batch with NVFP4 re-quantisation and its 8-token tail, and the
dequant kernels. `measured_peaks` holds the ceilings the library's probes reach
on this GPU (FP4 MFMA loop, HBM reads into registers and into LDS, a device
copy) beside the published peaks that `roofline` is quoted against.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "expert-MLP TFLOP/s & frac of FP4 peak, 48 experts x 4096 tok top-8 (1 GPU)"
PEAK_FP4_TFLOPS = 10100.0     # MI355X dense MXFP4 MFMA
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
CALIB_COPY_BYTES = 1 << 28    # --calibration-copy: one device copy of 256 MiB (read 256 MiB, write 256 MiB)

# HBM traffic of one L1 GEMM launch (48 x 4096 x top-8), from two rocprofv3 --pmc
# runs of `bench.py --steps 2 --warmup 1 --no-secondary --no-cpu-baseline
# --calibration-copy` (FETCH_SIZE, then WRITE_SIZE), each scaled by what the same
# counter reads for the calibration copy. Valid for the GEMM sources whose
# digest is recorded; None otherwise.
L1_TRAFFIC = {
    "gemm_digest": "928d7cfc70a761d6",
    "bytes_per_launch": 1681777120,          # 794956 KiB fetched x 1.99947 + 52867 KiB written x 1.000
    "profile": "profiles/grouped_e48_t4096_hbm_bytes.md",
}
GEMM_SOURCES = ("gemm.hip", "gemm_common.h", "mx_device.h", "mx_internal.h")


def log(msg):
    """Progress on stderr (the JSON line stays alone on stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-experts", type=int, default=24,
                    help="experts in the oracle's bounded CPU sample")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="run one device copy of known size first (for PMC byte-counter scaling)")
    return ap.parse_args()


def gemm_digest():
    h = hashlib.sha256()
    for n in GEMM_SOURCES:
        with open(os.path.join(ROOT, "mxfp4_block_scaled_e2m1_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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


def graph_replay_us(torch, calls, reps=20):
    """Capture `calls` (one list entry per rotating input set) into a hipGraph and
    return the mean microseconds per call over `reps` replays."""
    for c in calls:
        c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls[0]()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        for c in calls:
            c()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * len(calls))


def secondary(torch, mx, workloads):
    """Shared expert, skewed NVFP4 batch and dequant bandwidth (context lines)."""
    out = {}
    H, I = workloads.HIDDEN, workloads.INTER
    d = workloads.expert_weights(0)
    w0 = dev_tensors(torch, d, ("w1", "w1s", "w3", "w3s", "w2", "w2s"))
    wbytes = sum(v.numel() for v in w0.values())
    # 16 weight copies (~561 MB) so that successive calls miss the 256 MB cache
    copies = [w0] + [{k: v.clone() for k, v in w0.items()} for _ in range(15)]
    for c in copies:   # load-time step: tile-major weight scales and codes
        c["pk"] = mx.pack_weight_scales(c["w1s"], c["w3s"], c["w2s"])
        c["pc"] = mx.pack_weight_codes(c["w1"], c["w3"], c["w2"])
    for M in (1, 8, 128):
        x = bf16_dev(torch, workloads.activations(1, M))
        ws = torch.empty(mx.expert_mlp_workspace_size(M, H, I), dtype=torch.uint8, device="cuda")
        y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
        calls = [lambda w=w: mx.expert_mlp(x, w["w1"], w["w1s"], w["w3"], w["w3s"], w["w2"], w["w2s"], out=y,
                                           workspace=ws, packed_scales=w["pk"], packed_codes=w["pc"])
                 for w in copies]
        us = graph_replay_us(torch, calls)
        out[f"shared_expert_M{M}"] = {"us_per_call": round(us, 2), "weight_GB/s": round(wbytes / us / 1e3, 1),
                                      "hbm_frac": round(wbytes / us / 1e3 / PEAK_HBM_GBS, 3),
                                      "timing": "hipGraph replay, 16 rotating weight copies"}
    del copies
    M = 4096
    x = bf16_dev(torch, workloads.activations(1, M))
    ws = torch.empty(mx.expert_mlp_workspace_size(M, H, I), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    fn = lambda: mx.expert_mlp(x, w0["w1"], w0["w1s"], w0["w3"], w0["w3s"], w0["w2"], w0["w2s"], out=y, workspace=ws,
                               packed_scales=w0["pk"], packed_codes=w0["pc"])
    ms, _ = time_steps(torch, fn, 20, 3)
    flops = 6.0 * M * H * I
    out["shared_expert_M4096"] = {"ms": round(ms, 4), "TFLOP/s": round(flops / ms / 1e9, 2),
                                  "frac_of_fp4_peak": round(flops / ms / 1e9 / PEAK_FP4_TFLOPS, 4)}
    out.update(skewed_nvfp4(torch, mx, workloads))
    out.update(fp8_linear(torch, mx, workloads))
    out.update(nvfp4_linear(torch, mx, workloads))
    # dequant (8 rotating buffer sets so the working set exceeds the 256 MB cache)
    dq = workloads.dequant_inputs(0)
    c = torch.from_numpy(dq["w1"]).cuda()
    s = torch.from_numpy(dq["w1s"]).cuda()
    sets = [(c.clone(), s.clone(), torch.empty((3072, 7168), dtype=torch.bfloat16, device="cuda")) for _ in range(8)]
    calls = [lambda cc=cc, ss=ss, oo=oo: mx.dequant("mxfp4", cc, ss, 3072, 7168, out=oo) for cc, ss, oo in sets]
    us = graph_replay_us(torch, calls)
    nbytes = c.numel() + s.numel() + 3072 * 7168 * 2
    out["dequant_mxfp4_w1"] = {"us_per_call": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1),
                               "hbm_frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 3),
                               "timing": "hipGraph replay, 8 rotating buffer sets"}
    del sets
    q = torch.from_numpy(dq["fp8"]).cuda()
    qs = torch.from_numpy(dq["fp8s"]).cuda()
    qsets = [(q.clone(), qs.clone(), torch.empty((7168, 1536), dtype=torch.bfloat16, device="cuda")) for _ in range(8)]
    calls = [lambda cc=cc, ss=ss, oo=oo: mx.dequant("fp8_b128", cc, ss, 7168, 1536, out=oo) for cc, ss, oo in qsets]
    us = graph_replay_us(torch, calls)
    nbytes = q.numel() + qs.numel() + 7168 * 1536 * 2
    out["dequant_fp8_block"] = {"us_per_call": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1),
                                "hbm_frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 3),
                                "timing": "hipGraph replay, 8 rotating buffer sets"}
    return out


def fp8_linear(torch, mx, workloads):
    """FP8 block-scaled linear (MXFP8 activations, E4M3 weights with 128 x 128
    E8M0 scales) over 4096 tokens: the pages' FP8 matrix [7168, 1536] and the
    shared expert's gate/up [6144, 7168] and down [7168, 3072] shapes. Per-phase
    times from HIP events on the launch stream (quantiser and GEMM)."""
    out = {}
    M = 4096
    for N, K in ((7168, 1536), (6144, 7168), (7168, 3072)):
        d = workloads.fp8_linear(M, N, K, seed=0)
        x = bf16_dev(torch, d["x"])
        w = torch.from_numpy(d["w"]).cuda()
        wsc = torch.from_numpy(d["ws"]).cuda()
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(mx.fp8_block_linear_workspace_size(M, K), dtype=torch.uint8, device="cuda")
        fn = lambda: mx.fp8_block_linear(x, w, wsc, out=y, workspace=ws)
        ms, phases = time_steps(torch, fn, 20, 3, profile=(mx.profile_start, mx.profile_stop))
        flops = 2.0 * M * N * K
        gemm_ms = phases["fp8_gemm"][0] / phases["fp8_gemm"][1]
        out[f"fp8_block_linear_M{M}_N{N}_K{K}"] = {
            "ms": round(ms, 4), "TFLOP/s": round(flops / ms / 1e9, 2),
            "gemm_ms": round(gemm_ms, 4), "gemm_TFLOP/s": round(flops / gemm_ms / 1e9, 2),
            "gemm_frac_of_fp8_peak": round(flops / gemm_ms / 1e9 / PEAK_FP8_TFLOPS, 4),
            "quant_ms": round(phases["quant_x8"][0] / phases["quant_x8"][1], 4)}
    # the FP8 shared expert (three FP8 linears around SiLU * up), 4096 tokens
    H, I = workloads.HIDDEN, workloads.INTER
    d = workloads.fp8_expert(M, H, I, seed=0)
    wd = {n: torch.from_numpy(d[n]).cuda() for n in ("w1", "w1s", "w3", "w3s", "w2", "w2s")}
    x = bf16_dev(torch, d["x"])
    y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.fp8_expert_mlp_workspace_size(M, H, I), dtype=torch.uint8, device="cuda")
    fn = lambda: mx.fp8_expert_mlp(x, wd["w1"], wd["w1s"], wd["w3"], wd["w3s"], wd["w2"], wd["w2s"], out=y,
                                   workspace=ws)
    ms, phases = time_steps(torch, fn, 20, 3, profile=(mx.profile_start, mx.profile_stop))
    flops = 6.0 * M * H * I
    out[f"fp8_shared_expert_M{M}"] = {
        "ms": round(ms, 4), "TFLOP/s": round(flops / ms / 1e9, 2),
        "frac_of_fp8_peak": round(flops / ms / 1e9 / PEAK_FP8_TFLOPS, 4),
        "phases_ms_per_step": {k: round(v[0] / 20, 4) for k, v in phases.items()}}
    return out


def nvfp4_linear(torch, mx, workloads):
    """NVFP4-weight linear (NVFP4 activations) over 4096 tokens at the down
    projection's shape [7168, 3072], on bf16 matrix cores (NVFP4's E4M3 block
    scale has no MFMA form on gfx950)."""
    M, N, K = 4096, workloads.HIDDEN, workloads.INTER
    d = workloads.nvfp4_linear(M, N, K, seed=0)
    x = bf16_dev(torch, d["x"])
    w = torch.from_numpy(d["w"]).cuda()
    wsc = torch.from_numpy(d["ws"]).cuda()
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.nvfp4_linear_workspace_size(M, K), dtype=torch.uint8, device="cuda")
    fn = lambda: mx.nvfp4_linear(x, w, wsc, float(d["wg"]), float(d["xg"]), out=y, workspace=ws)
    ms, phases = time_steps(torch, fn, 20, 3, profile=(mx.profile_start, mx.profile_stop))
    flops = 2.0 * M * N * K
    gemm_ms = phases["nv_gemm"][0] / phases["nv_gemm"][1]
    out = {f"nvfp4_linear_M{M}_N{N}_K{K}": {
        "ms": round(ms, 4), "TFLOP/s": round(flops / ms / 1e9, 2), "gemm_ms": round(gemm_ms, 4),
        "gemm_TFLOP/s": round(flops / gemm_ms / 1e9, 2),
        "gemm_frac_of_bf16_peak": round(flops / gemm_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
        "quant_ms": round(phases["quant_nvfp4"][0] / phases["quant_nvfp4"][1], 4)}}
    # one expert with NVFP4 weights (dual gate/up globals), 4096 tokens
    H, I = workloads.HIDDEN, workloads.INTER
    d = workloads.nvfp4_expert(M, H, I, seed=0)
    names = ("w1", "w1s", "w1g", "w3", "w3s", "w3g", "w2", "w2s", "w2g")
    args = [float(d[n]) if n.endswith("g") else torch.from_numpy(d[n]).cuda() for n in names]
    x = bf16_dev(torch, d["x"])
    y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.nvfp4_expert_mlp_workspace_size(M, H, I), dtype=torch.uint8, device="cuda")
    fn = lambda: mx.nvfp4_expert_mlp(x, *args, float(d["xg"]), float(d["hg"]), out=y, workspace=ws)
    ms, phases = time_steps(torch, fn, 20, 3, profile=(mx.profile_start, mx.profile_stop))
    flops = 6.0 * M * H * I
    out[f"nvfp4_weight_expert_M{M}"] = {
        "ms": round(ms, 4), "TFLOP/s": round(flops / ms / 1e9, 2),
        "frac_of_bf16_peak": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
        "phases_ms_per_step": {k: round(v[0] / 20, 4) for k, v in phases.items()}}
    del args, x, y, ws
    # the headline batch (48 experts x 4096 tokens, top-8) with NVFP4 weights
    T, E, K = 4096, workloads.N_LOCAL_EXPERTS, workloads.TOP_K
    d = workloads.grouped_nvfp4(tokens=T, seed=0)
    args = [torch.from_numpy(np.ascontiguousarray(d[n])).cuda() for n in names]
    x = bf16_dev(torch, d["x"])
    ids, gw = torch.from_numpy(d["ids"]).cuda(), torch.from_numpy(d["w"]).cuda()
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.grouped_nvfp4_expert_mlp_workspace_size(T, H, I, K, E), dtype=torch.uint8, device="cuda")
    fn = lambda: mx.grouped_nvfp4_expert_mlp(x, ids, gw, *args, float(d["xg"]), float(d["hg"]), out=y, workspace=ws)
    ms, phases = time_steps(torch, fn, 5, 2, profile=(mx.profile_start, mx.profile_stop))
    flops = 6.0 * T * K * H * I
    out["grouped_nvfp4_weights_e48_t4096"] = {
        "ms": round(ms, 4), "TFLOP/s": round(flops / ms / 1e9, 2),
        "frac_of_bf16_peak": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
        "phases_ms_per_step": {k: round(v[0] / 5, 4) for k, v in phases.items()}}
    return out


def skewed_nvfp4(torch, mx, workloads):
    """16384 tokens, Zipf(1.2) routing over 48 experts, NVFP4 re-quantisation of h.

    The global scale is an input of the call; its value does not change the work
    done, so a fixed power of two stands in for the warm-up value here."""
    T, E, K = 16384, workloads.N_LOCAL_EXPERTS, workloads.TOP_K
    H, I = workloads.HIDDEN, workloads.INTER
    # the global as the library reads it: one fp32 in device memory, written
    # once (a Python float would be copied to the device on every call, which
    # a captured graph cannot hold)
    g = torch.tensor([2.0 ** -6], dtype=torch.float32, device="cuda")
    d = workloads.skewed(tokens=T, seed=0)
    w = dev_tensors(torch, d, ("w1", "w1s", "w3", "w3s", "w2", "w2s", "ids", "w"))
    x = bf16_dev(torch, d["x"])
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.grouped_expert_mlp_workspace_size(T, H, I, K, E, "nvfp4"), dtype=torch.uint8, device="cuda")
    pk = mx.pack_weight_scales(w["w1s"], w["w3s"], w["w2s"])
    pc = mx.pack_weight_codes(w["w1"], w["w3"], w["w2"])

    def step():
        mx.grouped_expert_mlp(x, w["ids"], w["w"], w["w1"], w["w1s"], w["w3"], w["w3s"], w["w2"], w["w2s"],
                              requant="nvfp4", requant_global=g, out=y, workspace=ws, packed_scales=pk,
                              packed_codes=pc)
    ms, phases = time_steps(torch, step, 5, 2, profile=(mx.profile_start, mx.profile_stop))
    P = T * K
    flops = 6.0 * P * H * I
    ideal_ms = (4.0 * P * H * I / (PEAK_FP4_TFLOPS * 1e9)) + (2.0 * P * H * I / (PEAK_BF16_TFLOPS * 1e9))
    rec = {"skewed_e48_t16384_nvfp4": {
        "ms": round(ms, 4), "TFLOP/s": round(flops / ms / 1e9, 2),
        "frac_of_mixed_peak": round(ideal_ms / ms, 4),
        "mixed_peak_note": "L1 (2/3 of the FLOPs) at the FP4 peak, L2 (1/3) at the bf16 peak",
        "phases_ms_per_step": {k: round(v[0] / v[1], 4) for k, v in phases.items()}}}
    # decode tail: the first 8 tokens over the same weights
    xt = x[:8].contiguous()
    yt = torch.empty((8, H), dtype=torch.bfloat16, device="cuda")
    idt, wt = w["ids"][:8].contiguous(), w["w"][:8].contiguous()
    n_active = int(np.unique(d["ids"][:8]).size)
    tbytes = n_active * 35094528
    for rq in ("nvfp4", "mxfp4"):
        wst = torch.empty(mx.grouped_expert_mlp_workspace_size(8, H, I, K, E, rq), dtype=torch.uint8, device="cuda")
        tail = lambda: mx.grouped_expert_mlp(xt, idt, wt, w["w1"], w["w1s"], w["w3"], w["w3s"], w["w2"], w["w2s"],
                                             requant=rq, requant_global=g, out=yt, workspace=wst,
                                             packed_scales=pk, packed_codes=pc)
        us = graph_replay_us(torch, [tail])
        rec[f"skewed_decode_tail_t8_{rq}"] = {
            "us_per_call": round(us, 2), "active_experts": n_active, "weight_GB/s": round(tbytes / us / 1e3, 1),
            "hbm_frac": round(tbytes / us / 1e3 / PEAK_HBM_GBS, 3),
            "timing": "hipGraph replay (weights of the active experts)"}
    return rec


def gpu_clocks(torch):
    """Current shader and memory clock levels of the GPU the bench ran on
    (device 0 of this process), read from the amdgpu sysfs tables of its PCI
    device (the level marked '*'), right after the timed steps. File reads
    only: no child process. None where the files are missing."""
    p = torch.cuda.get_device_properties(0)
    bdf = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
    out = {"pci": bdf}
    for key, name in (("sclk", "pp_dpm_sclk"), ("mclk", "pp_dpm_mclk")):
        path = f"/sys/bus/pci/devices/{bdf}/{name}"
        try:
            cur = [ln.split(":", 1)[1].replace("*", "").strip() for ln in open(path).read().splitlines()
                   if ln.rstrip().endswith("*")]
        except OSError:
            continue
        if cur:
            out[key] = cur[0]
    return out if len(out) > 1 else None


def measured_peaks(torch, mx):
    """The ceilings this GPU reaches, measured with the library's probes beside
    the published peaks: the scaled FP4 MFMA in a register-only loop, a 1 GiB
    read into registers and into LDS (the GEMMs' copy instruction), and a
    512 MiB device copy. Each probe's result is checked before its rate is
    reported (MFMA sums against their closed form, read checksums against
    torch's, the copy byte for byte)."""
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps   # ms

    out = {}
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 20000
    rng = np.random.default_rng(0)
    operand_sets = {
        # codes 3 and 5 (1.5 and 3) in every nibble of A and B: each output of a
        # step is 32 * (1.5 * 1.5 + 3 * 3) = 360, a lane's sum 64 * 360 * iters
        "constant": (np.full((512, 16), 0x35353535, np.uint32), 64 * 360.0 * iters),
        # uniform random codes: the data the GEMMs see (more switching power);
        # every workgroup must produce the same sums as workgroup 0
        "random": (rng.integers(0, 2**32, (512, 16), dtype=np.uint64).astype(np.uint32), None),
    }
    for tag, (host, want) in operand_sets.items():
        ops = torch.from_numpy(host.view(np.int32)).cuda()
        best = None
        for wgs in (cus, 2 * cus, 4 * cus):
            res = mx.probe_mfma_fp4(ops, iters, wgs)
            ms = timed(lambda: mx.probe_mfma_fp4(ops, iters, wgs, out=res), 3)
            ok = torch.all(res == want).item() if want is not None else torch.all(res == res[0:1]).item()
            if not ok:
                raise RuntimeError(f"MFMA probe result check failed ({tag} operands)")
            tf = wgs * 8 * iters * 4 * 131072 / ms / 1e9
            if best is None or tf > best[0]:
                best = (tf, wgs)
        out[f"mfma_fp4_loop_{tag}_operands"] = {
            "TFLOP/s": round(best[0], 1), "spec_TFLOP/s": PEAK_FP4_TFLOPS,
            "frac_of_spec": round(best[0] / PEAK_FP4_TFLOPS, 4), "workgroups": best[1],
            "note": "512-thread workgroups, 4 independent accumulators per wave, operands in registers"}
    nbytes = 1 << 30
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
    want = None
    for mode, name in ((0, "read_to_registers"), (1, "read_to_lds_dma")):
        best = None
        for lpw, wgs in ((8, 8 * cus), (32, 2 * cus), (32, cus)):
            res = mx.probe_read(src, mode, lpw, wgs)
            ms = timed(lambda: mx.probe_read(src, mode, lpw, wgs, out=res), 5)
            got = int(np.bitwise_xor.reduce(res.cpu().numpy().view(np.uint32)))
            if want is None:
                want = int(np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32)))
            if got != want:
                raise RuntimeError(f"read probe checksum mismatch ({name})")
            gbs = nbytes / ms / 1e6
            if best is None or gbs > best[0]:
                best = (gbs, lpw, wgs)
        out[f"hbm_{name}"] = {"GB/s": round(best[0], 1), "spec_GB/s": PEAK_HBM_GBS,
                              "frac_of_spec": round(best[0] / PEAK_HBM_GBS, 4), "bytes": nbytes,
                              "loads_per_wave": best[1], "workgroups": best[2]}
    del src
    cb = 1 << 29
    a = torch.randint(0, 255, (cb,), dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    ms = timed(lambda: mx.probe_copy(a, b), 5)
    if not torch.equal(a, b):
        raise RuntimeError("copy probe output differs from its input")
    out["hbm_copy"] = {"GB/s": round(2 * cb / ms / 1e6, 1), "spec_GB/s": PEAK_HBM_GBS,
                       "frac_of_spec": round(2 * cb / ms / 1e6 / PEAK_HBM_GBS, 4),
                       "bytes_moved": 2 * cb, "note": "read + write of 512 MiB"}
    return out


def cpu_baseline(d, n_exp):
    """The oracle, untuned, on all pairs routed to experts 0..n_exp-1."""
    import oracle
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip() for i in info}))
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
            "kind": "oracle", "seconds": round(sec, 2), "blas": blas,
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
    # load-time step, outside the timed region: the weight scales re-laid
    # tile-major once (mx_pack_weight_scales), as a runner does after loading
    pk = mx.pack_weight_scales(w["w1s"], w["w3s"], w["w2s"])
    pc = mx.pack_weight_codes(w["w1"], w["w3"], w["w2"])

    def step():
        mx.grouped_expert_mlp(x, w["ids"], w["w"], w["w1"], w["w1s"], w["w3"], w["w3s"], w["w2"], w["w2s"],
                              out=y, workspace=ws, packed_scales=pk, packed_codes=pc)

    if a.calibration_copy:
        src = torch.empty(CALIB_COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log("inputs resident; timing the headline")
    # the headline: K steps with nothing else recorded
    ms, _ = time_steps(torch, step, a.steps, a.warmup)
    clocks = gpu_clocks(torch)
    # the phase split: the same K steps again, every kernel bracketed by HIP
    # events on the stream it runs on (the library's profiler)
    ms_prof, phases = time_steps(torch, step, a.steps, 1, profile=(mx.profile_start, mx.profile_stop))
    flops = 6.0 * T * K * H * I
    value = flops / ms / 1e9   # TFLOP/s
    l1_ms, l1_n = phases["l1_gemm"]
    l1_avg = l1_ms / l1_n
    l1_flops = 2.0 * T * K * (2 * I) * H
    achieved = l1_flops / l1_avg / 1e9
    traffic = None
    if L1_TRAFFIC is not None and L1_TRAFFIC["gemm_digest"] == gemm_digest():
        traffic = L1_TRAFFIC["bytes_per_launch"]
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4 (E2M1 x E8M0 operands, fp32 accumulation)", "data": "synthetic",
        "config": {"workload": "routed expert MLP: 48 local experts x 4096 tokens, top-8, hidden 7168, "
                               "inter 3072, MXFP4 weights and activations",
                   "experts": E, "tokens": T, "top_k": K, "hidden": H, "inter": I,
                   "parallelism": "single GPU",
                   "weight_prep": "E8M0 weight scales and FP4 weight codes re-laid tile-major once after load "
                                  "(mx_pack_weight_scales, mx_pack_weight_codes), not timed"},
        "frac_of_fp4_peak": round(value / PEAK_FP4_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": "l1_gemm (gate/up GEMM + SiLU*up + MXFP4 re-quant)",
                     "achieved": round(achieved, 2), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP4_TFLOPS, 4), "traffic": traffic,
                     "algorithmic_flops_per_launch": l1_flops, "avg_launch_ms": round(l1_avg, 4),
                     "timing": "HIP events around each launch, in a second pass of the same steps"},
        "phases_ms_per_step": {k: round(v[0] / v[1], 4) for k, v in phases.items()},
        "ms_per_step_with_phase_events": round(ms_prof, 4),
        "gpu_clocks_after_timed_steps": clocks,
    }
    log(f"headline {ms:.4f} ms per step")
    if not a.no_secondary:
        rec["measured_peaks"] = measured_peaks(torch, mx)
        log("measured peaks done")
        rec["secondary"] = secondary(torch, mx, workloads)
        log("secondary configurations done")
    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(d, a.cpu_experts)
        log("cpu baseline done")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
