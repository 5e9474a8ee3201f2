"""Parity of the NVFP4 re-quantisation variant (E4M3 per 16 + fp32 global scale
between the two GEMMs; bf16 matrix cores for L2) with the oracle.

The global scale g comes from the oracle's warm-up reading (max |h| / (6 * 448)
over a warm-up pass): over every (token, expert) pair for the small cases and
over the first tokens for the 16384-token case, whose full warm-up would take
the fp64 oracle hours."""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import assert_mlp_close, assert_nvfp4_requant_close, bf16_t, bits, t

pytestmark = pytest.mark.gpu

WNAMES = ("w1", "w1s", "w3", "w3s", "w2", "w2s")


@pytest.fixture(scope="module")
def mx():
    import mxfp4_block_scaled_e2m1_amd as m
    return m


def _warmup_dense(d):
    _, inter = O.expert_mlp(d["x"], *(d[n] for n in WNAMES), intermediates=True)
    return float(O.nvfp4_warmup_global(inter["h"]))


def _warmup_grouped(d, tokens):
    """max |h| over the (token, expert) pairs of `tokens` -> g."""
    amax = 0.0
    ids = d["ids"][tokens]
    E = d["w1"].shape[0]
    for e in range(E):
        tt = np.nonzero((ids == e).any(axis=1))[0]
        if tt.size == 0:
            continue
        we = {n: d[n][e] for n in WNAMES}
        _, inter = O.expert_mlp(d["x"][tokens][tt], *(we[n] for n in WNAMES), intermediates=True)
        amax = max(amax, float(np.abs(O.bf16_to_f64(inter["h"])).max()))
    return float(np.float32(amax / (6.0 * 448.0)))


def _run_dense_nv(mx, d, M, H, I, g):
    nbytes = mx.expert_mlp_workspace_size(M, H, I, "nvfp4")
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = mx.expert_mlp(bf16_t(d["x"]), *(t(d[n]) for n in WNAMES), requant="nvfp4", requant_global=g,
                      workspace=ws)
    torch.cuda.synchronize()
    # GEMM-path workspace: xq, xs, hq, hs (E4M3 per 16), regions 256-byte aligned
    off, sl = 0, []
    for n in (M * H // 2, M * H // 32, M * I // 2, M * I // 16):
        sl.append(ws[off:off + n])
        off += (n + 255) // 256 * 256
    return bits(y), sl


@pytest.mark.parametrize("M,H,I", [(16, 256, 128), (1, 256, 128), (48, 512, 256)])
def test_nvfp4_dense_small(mx, M, H, I):
    d = W.tiny_mlp(0) if H == 256 else W.shared_expert(M, seed=4, hidden=H, inter=I)
    d["x"] = d["x"][:M]
    g = _warmup_dense(d)
    y, (xq, xs, hq, hs) = _run_dense_nv(mx, d, M, H, I, g)
    ref, inter = O.expert_mlp(d["x"], *(d[n] for n in WNAMES), requant="nvfp4", nv_global=g, intermediates=True)
    assert np.array_equal(xq.cpu().numpy().reshape(M, H // 2), inter["xq"])
    assert_nvfp4_requant_close(hq.cpu().numpy().reshape(M, I // 2), hs.cpu().numpy().reshape(M, I // 16),
                               inter["hq"], inter["hs"], g)
    assert_mlp_close(y, ref)


@pytest.mark.parametrize("M", [1, 8, 300])
def test_nvfp4_shared_expert_real_shape(mx, M):
    d = W.shared_expert(M, seed=0)
    g = _warmup_dense(d)
    y, (_, _, hq, hs) = _run_dense_nv(mx, d, M, 7168, 3072, g)
    ref, inter = O.expert_mlp(d["x"], *(d[n] for n in WNAMES), requant="nvfp4", nv_global=g, intermediates=True)
    assert_nvfp4_requant_close(hq.cpu().numpy().reshape(M, 1536), hs.cpu().numpy().reshape(M, 192),
                               inter["hq"], inter["hs"], g)
    assert_mlp_close(y, ref)


def test_nvfp4_global_scale_is_linear(mx):
    """Doubling g halves every E4M3 block scale exactly (while they stay normal:
    s >= 2^-5 before halving) and leaves every code and every output bit as is:
    the dequantised values code * s * g do not change."""
    d = W.shared_expert(40, seed=6, hidden=512, inter=256)
    g = _warmup_dense(d)
    y1, (_, _, hq1, hs1) = _run_dense_nv(mx, d, 40, 512, 256, g)
    y2, (_, _, hq2, hs2) = _run_dense_nv(mx, d, 40, 512, 256, 2 * g)
    s1 = O.e4m3_decode(hs1.cpu().numpy())
    s2 = O.e4m3_decode(hs2.cpu().numpy())
    nz = s1 != 0
    assert np.all(np.abs(s1[nz]) >= 2.0 ** -5)      # precondition of the exact halving
    assert np.array_equal(s2[nz], s1[nz] / 2)
    assert np.array_equal(hq1.cpu().numpy(), hq2.cpu().numpy())
    assert np.array_equal(y1, y2)


def _device_warmup(mx, d, routed):
    args = (bf16_t(d["x"]), t(d["w1"]), t(d["w1s"]), t(d["w3"]), t(d["w3s"]))
    if routed:
        g = mx.nvfp4_global_warmup(*args, topk_ids=t(d["ids"]), topk_w=t(d["w"]))
    else:
        g = mx.nvfp4_global_warmup(*args)
    torch.cuda.synchronize()
    return float(g.cpu().numpy()[0])


def _assert_same_global(g_dev, g_ref):
    """The device takes max |h| over its own bf16 h, which can differ from the
    oracle's by one bf16 step where a value sits at a rounding boundary; g then
    differs by that step. Otherwise it is the same fp32 number."""
    assert g_dev == g_ref or abs(g_dev - g_ref) <= g_ref * 2.0 ** -7, (g_dev, g_ref)


@pytest.mark.parametrize("M,H,I", [(37, 512, 256), (300, 384, 384), (64, 7168, 3072)])
def test_device_warmup_global_dense(mx, M, H, I):
    d = W.shared_expert(M, seed=6, hidden=H, inter=I)
    _assert_same_global(_device_warmup(mx, d, routed=False), _warmup_dense(d))


def test_device_warmup_global_routed_then_mlp(mx):
    """g from the device warm-up over a routed batch, then the NVFP4 MLP with it."""
    d = W.grouped(tokens=600, n_experts=8, k=4, seed=5, hidden=512, inter=256)
    g_ref = _warmup_grouped(d, np.arange(600))
    g = _device_warmup(mx, d, routed=True)
    _assert_same_global(g, g_ref)
    y = _run_grouped_nv(mx, d, g)
    ref = O.grouped_expert_mlp(d["x"], d["ids"], d["w"], *(d[n] for n in WNAMES), requant="nvfp4", nv_global=g)
    assert_mlp_close(y, ref)


def test_device_warmup_global_degenerate(mx):
    """All-zero h (zero activations) and an empty batch give g = 1, as the oracle's rule."""
    d = W.shared_expert(40, seed=1, hidden=256, inter=128)
    d["x"] = np.zeros_like(d["x"])
    assert _device_warmup(mx, d, routed=False) == 1.0
    assert float(O.nvfp4_warmup_global(np.zeros((4, 128), np.uint16))) == 1.0
    d["x"] = d["x"][:0]
    assert _device_warmup(mx, d, routed=False) == 1.0


def _run_grouped_nv(mx, d, g):
    y = mx.grouped_expert_mlp(bf16_t(d["x"]), t(d["ids"]), t(d["w"]), *(t(d[n]) for n in WNAMES),
                              requant="nvfp4", requant_global=g)
    torch.cuda.synchronize()
    return bits(y)


def test_nvfp4_grouped_multi_tile(mx):
    d = W.grouped(tokens=600, n_experts=8, k=4, seed=5, hidden=512, inter=256)
    g = _warmup_grouped(d, np.arange(600))
    y = _run_grouped_nv(mx, d, g)
    ref = O.grouped_expert_mlp(d["x"], d["ids"], d["w"], *(d[n] for n in WNAMES), requant="nvfp4", nv_global=g)
    assert_mlp_close(y, ref)


def test_nvfp4_grouped_single_expert_equals_shared(mx):
    d = W.shared_expert(200, seed=2, hidden=512, inter=256)
    g = _warmup_dense(d)
    gd = {n: d[n][None] for n in WNAMES}
    gd.update(x=d["x"], ids=np.zeros((200, 1), np.int32), w=np.ones((200, 1), np.float32))
    yg = _run_grouped_nv(mx, gd, g)
    yd, _ = _run_dense_nv(mx, d, 200, 512, 256, g)
    assert np.array_equal(yg, yd)


def test_nvfp4_skewed_sampled_tokens_and_decode_tail(mx):
    """The skewed 16384-token case with NVFP4 re-quantisation, plus its 8-token
    decode tail over the same weights."""
    d = W.skewed(tokens=16384, seed=0)
    g = _warmup_grouped(d, np.arange(16))
    y = _run_grouped_nv(mx, d, g)
    tok = np.array([3, 16383])
    ref = O.grouped_expert_mlp(d["x"], d["ids"], d["w"], *(d[n] for n in WNAMES), requant="nvfp4", nv_global=g,
                               tokens=tok)
    assert_mlp_close(y[tok], ref)
    assert np.all(np.isfinite(((y.astype(np.uint32) << 16).view(np.float32))))
    tail = dict(d, x=d["x"][:8], ids=d["ids"][:8], w=d["w"][:8])
    yt = _run_grouped_nv(mx, tail, g)
    reft = O.grouped_expert_mlp(tail["x"], tail["ids"], tail["w"], *(d[n] for n in WNAMES), requant="nvfp4",
                                nv_global=g)
    assert_mlp_close(yt, reft)


def test_nvfp4_grouped_stream(mx):
    """Few rows per expert with NVFP4 re-quantisation: the weight-streaming L2
    on the exactly dequantised h (bf16 matrix cores), against the oracle; one
    expert with more than 16 rows, one empty, foreign ids."""
    d = W.grouped(tokens=20, n_experts=6, k=3, seed=11, hidden=256, inter=128)
    d["ids"][:, 0] = 0
    d["ids"][d["ids"] == 5] = 4
    d["ids"][::3, 2] = -1
    g = _warmup_grouped(d, np.arange(20))
    y = _run_grouped_nv(mx, d, g)
    ref = O.grouped_expert_mlp(d["x"], d["ids"], d["w"], *(d[n] for n in WNAMES), requant="nvfp4", nv_global=g)
    assert_mlp_close(y, ref)


def test_nvfp4_grouped_stream_single_expert_close_to_shared(mx):
    """E = 1 over 12 tokens: the weight-streaming path against the dense
    NVFP4 path (tiled GEMMs): the same quantisation, sums in another order."""
    d = W.shared_expert(12, seed=7, hidden=512, inter=256)
    g = _warmup_dense(d)
    gd = {n: d[n][None] for n in WNAMES}
    gd.update(x=d["x"], ids=np.zeros((12, 1), np.int32), w=np.ones((12, 1), np.float32))
    yg = _run_grouped_nv(mx, gd, g)
    yd, _ = _run_dense_nv(mx, d, 12, 512, 256, g)
    assert_mlp_close(yg, yd, cos_min=0.99999)


# ---------------------------------------------------------------- NVFP4 weights
def _nv_linear_check(y_bits, d, rows=None):
    x = d["x"] if rows is None else d["x"][rows]
    _nv_bar(y_bits, x, d["w"], d["ws"], d["wg"], d["xg"])


def _nv_bar(y_bits, x, w, ws, wg, xg):
    """Identical NVFP4 operands on both sides, bf16 products exact, fp32 sums:
    outputs equal the oracle's correctly rounded value or lie one step from
    it, with |y - e| <= 2^-8 |e| + 2^-16 S (S: sum of the products' magnitudes)."""
    from gpu_util import bf16_f64
    ref = O.nvfp4_linear(x, w, ws, wg, xg)
    xq, xs = O.nvfp4_quantize(x, xg)
    a = O.nvfp4_dequant_f64(xq, xs, xg)
    b = O.nvfp4_dequant_f64(w, ws, wg)
    exact, mag = O.gemm_f64(a, b), O.gemm_f64(np.abs(a), np.abs(b))
    yv = bf16_f64(y_bits)
    assert np.all(np.isfinite(yv))
    assert np.mean(y_bits == ref) >= 0.99
    assert np.all(np.abs(yv - exact) <= np.abs(exact) * 2.0 ** -8 + mag * 2.0 ** -16)
    assert np.linalg.norm(yv - exact) / np.linalg.norm(exact) <= 4e-3


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (37, 384, 256), (300, 640, 1152), (64, 3072, 7168)])
def test_nvfp4_linear_matches_oracle(mx, M, N, K):
    d = W.nvfp4_linear(M, N, K, seed=M + N)
    y = mx.nvfp4_linear(bf16_t(d["x"]), t(d["w"]), t(d["ws"]), float(d["wg"]), float(d["xg"]))
    torch.cuda.synchronize()
    _nv_linear_check(bits(y), d)


@pytest.mark.parametrize("M,N,K", [(64, 256, 512), (300, 384, 1024)])
def test_nvfp4_linear_full_e4m3_range(mx, M, N, K):
    """Weight scales over every finite E4M3 byte and activation blocks over
    2^-20 .. 2^4 (their scales reach zero, the subnormals and 448): the fp16
    operands code x scale of the NVFP4-weight GEMM are exact and normal over
    that whole range (6 x 448 at most, 2^-10 at least), so the same bars hold."""
    d = W.nvfp4_linear_wide(M, N, K, seed=M + K)
    y = mx.nvfp4_linear(bf16_t(d["x"]), t(d["w"]), t(d["ws"]), float(d["wg"]), float(d["xg"]))
    torch.cuda.synchronize()
    _nv_linear_check(bits(y), d)


def test_nvfp4_linear_real_shape_sampled_rows(mx):
    """4096 tokens through the down projection's shape [7168, 3072]; rows from every m-tile."""
    d = W.nvfp4_linear(4096, seed=0)
    y = bits(mx.nvfp4_linear(bf16_t(d["x"]), t(d["w"]), t(d["ws"]), float(d["wg"]), float(d["xg"])))
    rows = np.array([0, 255, 256, 1000, 2047, 3333, 4095])
    _nv_linear_check(y[rows], d, rows)


NV_WN = ("w1", "w1s", "w1g", "w3", "w3s", "w3g", "w2", "w2s", "w2g")


def _nv_bar_q(y_bits, xq, xs, xg, w, ws, wg):
    """_nv_bar with the activation operand given as NVFP4 codes and scales (the
    GPU's own quantised h): same bars against the exact product."""
    from gpu_util import bf16_f64
    a = O.nvfp4_dequant_f64(xq, xs, xg)
    b = O.nvfp4_dequant_f64(w, ws, wg)
    exact, mag = O.gemm_f64(a, b), O.gemm_f64(np.abs(a), np.abs(b))
    ref = O.f64_to_bf16(exact)
    yv = bf16_f64(y_bits)
    assert np.all(np.isfinite(yv))
    assert np.mean(y_bits == ref) >= 0.99
    assert np.all(np.abs(yv - exact) <= np.abs(exact) * 2.0 ** -8 + mag * 2.0 ** -16)
    assert np.linalg.norm(yv - exact) / np.linalg.norm(exact) <= 4e-3


@pytest.mark.parametrize("M,H,I", [(5, 256, 128), (300, 512, 384), (64, 7168, 3072), (700, 640, 384)])
def test_nvfp4_expert_mlp_matches_oracle(mx, M, H, I):
    """The stages the GPU writes against the oracle: the fused gate/up GEMM's
    NVFP4 h (codes and E4M3 scales) against the oracle's, >= 99.9 % equal with
    every mismatch within one E2M1 step (its g and u are the NVFP4 linears'
    bf16 outputs, which may sit one bf16 step from the oracle's); y against the
    exact product of the GPU's own h and w2 at the linear's bar; end to end
    cosine >= 0.9999 and max error <= 5e-2 of max |y| (a one-step difference in
    g or u can move an element of h across an E2M1 rounding boundary)."""
    d = W.nvfp4_expert(M, H, I, seed=M + I)
    args = [t(d[n]) if not n.endswith("g") else float(d[n]) for n in NV_WN]
    ws = torch.empty(mx.nvfp4_expert_mlp_workspace_size(M, H, I), dtype=torch.uint8, device="cuda")
    y = bits(mx.nvfp4_expert_mlp(bf16_t(d["x"]), *args, float(d["xg"]), float(d["hg"]), workspace=ws))
    torch.cuda.synchronize()
    al = lambda n: (n + 255) // 256 * 256
    sizes = [M * H // 2, M * H // 16, M * I // 2, M * I // 16]
    off, sl = 0, []
    for n in sizes:
        sl.append(ws[off:off + n].cpu().numpy())
        off += al(n)
    hq, hs = sl[2].reshape(M, I // 2), sl[3].reshape(M, I // 16)
    g = O.nvfp4_linear(d["x"], d["w1"], d["w1s"], d["w1g"], d["xg"])
    u = O.nvfp4_linear(d["x"], d["w3"], d["w3s"], d["w3g"], d["xg"])
    rh = O.silu_mul_bf16(O.bf16_to_f64(g), O.bf16_to_f64(u))
    rq, rs = O.nvfp4_quantize(rh, d["hg"])
    assert_nvfp4_requant_close(hq, hs, rq, rs, float(d["hg"]))
    _nv_bar_q(y, hq, hs, d["hg"], d["w2"], d["w2s"], d["w2g"])
    ref = O.nvfp4_expert_mlp(d["x"], *(d[n] for n in NV_WN), d["xg"], d["hg"])
    assert_mlp_close(y, ref, rel_max=5e-2)


# ---------------------------------------------------------------- routed, NVFP4 weights
def _run_grouped_nvw(mx, d):
    args = [t(d[n]) for n in NV_WN]
    y = mx.grouped_nvfp4_expert_mlp(bf16_t(d["x"]), t(d["ids"]), t(d["w"]), *args, float(d["xg"]), float(d["hg"]))
    torch.cuda.synchronize()
    return bits(y)


def _oracle_grouped_nvw(d, tokens=None):
    return O.grouped_nvfp4_expert_mlp(d["x"], d["ids"], d["w"], *(d[n] for n in NV_WN), d["xg"], d["hg"],
                                      tokens=tokens)


def test_grouped_nvfp4_weights_matches_oracle(mx):
    """Per-expert weight globals, an expert with more rows than a tile, an
    empty expert, duplicated and foreign ids; end-to-end bar of R21."""
    d = W.grouped_nvfp4(tokens=300, n_experts=6, k=3, seed=4, hidden=256, inter=128)
    d["ids"][:, 0] = 0                # expert 0: every token (two 256-row tiles)
    d["ids"][d["ids"] == 5] = 4       # expert 5 empty
    d["ids"][::7, 2] = -1             # other ranks
    assert_mlp_close(_run_grouped_nvw(mx, d), _oracle_grouped_nvw(d), rel_max=5e-2)
    perm = np.random.default_rng(3).permutation(300)
    dp = dict(d, x=d["x"][perm], ids=d["ids"][perm], w=d["w"][perm])
    assert np.array_equal(_run_grouped_nvw(mx, dp), _run_grouped_nvw(mx, d)[perm])


def test_grouped_nvfp4_weights_single_expert_equals_dense(mx):
    """E = 1, k = 1, w = 1: the routed path (gathered rows, per-expert globals
    on the device) equals mx_nvfp4_expert_mlp bit for bit."""
    d = W.grouped_nvfp4(tokens=300, n_experts=1, k=1, seed=5, hidden=512, inter=256)
    d["w"] = np.ones_like(d["w"])
    yg = _run_grouped_nvw(mx, d)
    args = [t(d[n][0]) if not n.endswith("g") else float(d[n][0]) for n in NV_WN]
    yd = bits(mx.nvfp4_expert_mlp(bf16_t(d["x"]), *args, float(d["xg"]), float(d["hg"])))
    assert np.array_equal(yg, yd)


def test_grouped_nvfp4_weights_real_shape(mx):
    """48 experts at 7168 x 3072 with NVFP4 weights: two tokens of a top-8 batch."""
    d = W.grouped_nvfp4(tokens=2, seed=0)
    assert_mlp_close(_run_grouped_nvw(mx, d), _oracle_grouped_nvw(d), rel_max=5e-2)

