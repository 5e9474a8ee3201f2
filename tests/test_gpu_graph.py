"""hipGraph capture and replay of the library calls (the pages' runner is
graph-safe: page "Current Bug: vLLM produces empty/garbage output", section
"Revised Plan", Phase 1). The calls allocate nothing and never synchronise, so
they can be captured; every replay must reproduce the eager result bit for bit,
with eager work and synchronisations between the replays."""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import bf16_t, bits, t

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    import mxfp4_block_scaled_e2m1_amd as m
    return m


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _check_replays(g, out, ref, scratch):
    for i in range(3):
        out.zero_()
        scratch.normal_()                 # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), ref), f"replay {i}"


@pytest.mark.parametrize("M", [1, 8, 40, 300])
def test_graph_shared_expert(mx, M):
    d = W.shared_expert(M, seed=3, hidden=1024, inter=512)
    w = {n: t(d[n]) for n in ("w1", "w1s", "w3", "w3s", "w2", "w2s")}
    x = bf16_t(d["x"])
    y = torch.empty((M, 1024), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.expert_mlp_workspace_size(M, 1024, 512), dtype=torch.uint8, device="cuda")
    fn = lambda: mx.expert_mlp(x, w["w1"], w["w1s"], w["w3"], w["w3s"], w["w2"], w["w2s"], out=y, workspace=ws)
    fn()
    torch.cuda.synchronize()
    ref = bits(y)
    g = _capture(fn)
    _check_replays(g, y, ref, torch.empty(1 << 20, device="cuda"))


@pytest.mark.parametrize("requant,T", [("mxfp4", 300), ("nvfp4", 300), ("mxfp4", 4), ("nvfp4", 20)])
def test_graph_grouped(mx, requant, T):
    """Tiled GEMMs (300 tokens) and the routed weight-streaming kernels (few rows per expert)."""
    d = W.grouped(tokens=T, n_experts=6, k=3, seed=9, hidden=512, inter=256)
    w = {n: t(d[n]) for n in ("w1", "w1s", "w3", "w3s", "w2", "w2s", "ids", "w")}
    x = bf16_t(d["x"])
    y = torch.empty((T, 512), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.grouped_expert_mlp_workspace_size(T, 512, 256, 3, 6, requant), dtype=torch.uint8,
                     device="cuda")
    g_scale = torch.tensor([2.0 ** -6], dtype=torch.float32, device="cuda")   # device global: no copy in capture
    fn = lambda: mx.grouped_expert_mlp(x, w["ids"], w["w"], w["w1"], w["w1s"], w["w3"], w["w3s"], w["w2"], w["w2s"],
                                       requant=requant, requant_global=g_scale, out=y, workspace=ws)
    fn()
    torch.cuda.synchronize()
    ref = bits(y)
    g = _capture(fn)
    _check_replays(g, y, ref, torch.empty(1 << 20, device="cuda"))


def test_graph_dequant_quant(mx):
    dq = W.dequant_inputs(0)
    c, s = t(dq["w2"]), t(dq["w2s"])
    out = torch.empty((7168, 3072), dtype=torch.bfloat16, device="cuda")
    fn = lambda: mx.dequant("mxfp4", c, s, 7168, 3072, out=out)
    fn()
    torch.cuda.synchronize()
    ref = bits(out)
    g = _capture(fn)
    _check_replays(g, out, ref, torch.empty(1 << 20, device="cuda"))


def test_graph_fp8_linear(mx):
    d = W.fp8_linear(300, 384, 512, seed=4)
    x, w, wsc = bf16_t(d["x"]), t(d["w"]), t(d["ws"])
    y = torch.empty((300, 384), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.fp8_block_linear_workspace_size(300, 512), dtype=torch.uint8, device="cuda")
    fn = lambda: mx.fp8_block_linear(x, w, wsc, out=y, workspace=ws)
    fn()
    torch.cuda.synchronize()
    ref = bits(y)
    g = _capture(fn)
    _check_replays(g, y, ref, torch.empty(1 << 20, device="cuda"))


@pytest.mark.parametrize("requant,T", [("mxfp4", 300), ("nvfp4", 20)])
def test_runner_replays_match_eager(mx, requant, T):
    """mx_moe_runner: buffers bound once, graph captured once; after refreshing
    x, ids and weights in place each replay equals an eager call on the new
    contents, bit for bit, also on another stream."""
    E, k, H, I = 6, 3, 512, 256
    d0 = W.grouped(tokens=T, n_experts=E, k=k, seed=9, hidden=H, inter=I)
    w = {n: t(d0[n]) for n in ("w1", "w1s", "w3", "w3s", "w2", "w2s")}
    x, ids, gw = bf16_t(d0["x"]), t(d0["ids"]), t(d0["w"])
    g_scale = torch.tensor([2.0 ** -6], dtype=torch.float32, device="cuda")
    # the runner reads tile-major weight scales and codes; the eager reference
    # reads the row-major weights (the results are the same bytes either way)
    pk = mx.pack_weight_scales(w["w1s"], w["w3s"], w["w2s"])
    pc = mx.pack_weight_codes(w["w1"], w["w3"], w["w2"])
    r = mx.MoeRunner(x, ids, gw, w["w1"], w["w1s"], w["w3"], w["w3s"], w["w2"], w["w2s"], requant=requant,
                     requant_global=g_scale, packed_scales=pk, packed_codes=pc)
    try:
        for seed in (9, 21, 33):
            d = W.grouped(tokens=T, n_experts=E, k=k, seed=seed, hidden=H, inter=I)
            x.copy_(bf16_t(d["x"]))
            ids.copy_(t(d["ids"]))
            gw.copy_(t(d["w"]))
            g_scale.fill_(2.0 ** -6 if seed != 21 else 2.0 ** -5 * 1.5)   # the global is read at each replay
            torch.cuda.synchronize()
            ref = bits(mx.grouped_expert_mlp(x, ids, gw, w["w1"], w["w1s"], w["w3"], w["w3s"], w["w2"], w["w2s"],
                                             requant=requant, requant_global=g_scale))
            r.out.zero_()
            s = torch.cuda.Stream() if seed == 33 else torch.cuda.current_stream()
            s.wait_stream(torch.cuda.current_stream())
            r.replay(stream=s)
            torch.cuda.synchronize()
            assert np.array_equal(bits(r.out), ref), seed
    finally:
        torch.cuda.synchronize()
        r.close()



@pytest.mark.parametrize("T", [300, 20])
def test_runner_after_device_writes_and_warmup_without_sync(mx, T):
    """Inputs written by device kernels on the caller's stream, the NVFP4 global from
    the on-device warm-up, then the runner created with no host synchronisation in
    between: its first output (the eager call of create) and its replays equal eager
    calls bit for bit. The global goes from the warm-up to the runner as a device
    pointer, never read back to the host."""
    E, k, H, I = 6, 3, 512, 256
    d0 = W.grouped(tokens=T, n_experts=E, k=k, seed=41, hidden=H, inter=I)
    w = {n: t(d0[n]) for n in ("w1", "w1s", "w3", "w3s", "w2", "w2s")}
    src_x, src_ids, src_gw = bf16_t(d0["x"]), t(d0["ids"]), t(d0["w"])
    torch.cuda.synchronize()
    x = torch.zeros_like(src_x)
    ids = torch.zeros_like(src_ids)
    gw = torch.zeros_like(src_gw)
    x.copy_(src_x)          # device-to-device copies, enqueued on the current stream
    ids.copy_(src_ids)
    gw.copy_(src_gw)
    g = mx.nvfp4_global_warmup(x, w["w1"], w["w1s"], w["w3"], w["w3s"], topk_ids=ids, topk_w=gw)
    r = mx.MoeRunner(x, ids, gw, w["w1"], w["w1s"], w["w3"], w["w3s"], w["w2"], w["w2s"], requant="nvfp4",
                     requant_global=g)
    try:
        first = bits(r.out)
        ref = bits(mx.grouped_expert_mlp(x, ids, gw, w["w1"], w["w1s"], w["w3"], w["w3s"], w["w2"], w["w2s"],
                                         requant="nvfp4", requant_global=g))
        assert np.array_equal(first, ref)
        # the same global as a host value gives the same output
        ref_host = bits(mx.grouped_expert_mlp(x, ids, gw, w["w1"], w["w1s"], w["w3"], w["w3s"], w["w2"],
                                              w["w2s"], requant="nvfp4", requant_global=float(g.item())))
        assert np.array_equal(ref_host, ref)
        # new inputs and a new warm-up global on the device, then a replay, still without a host sync
        d1 = W.grouped(tokens=T, n_experts=E, k=k, seed=42, hidden=H, inter=I)
        src_x.copy_(bf16_t(d1["x"]))
        torch.cuda.synchronize()
        x.copy_(src_x)
        mx.nvfp4_global_warmup(x, w["w1"], w["w1s"], w["w3"], w["w3s"], topk_ids=ids, topk_w=gw, out=g)
        r.replay()
        rep = bits(r.out)
        ref1 = bits(mx.grouped_expert_mlp(x, ids, gw, w["w1"], w["w1s"], w["w3"], w["w3s"], w["w2"], w["w2s"],
                                          requant="nvfp4", requant_global=g))
        assert np.array_equal(rep, ref1)
    finally:
        torch.cuda.synchronize()
        r.close()
