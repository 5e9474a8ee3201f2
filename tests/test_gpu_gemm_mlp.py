"""Parity of the scaled-MFMA GEMM, the shared expert and the routed experts with the oracle."""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import (as_np, assert_mlp_close, assert_requant_close, bf16_f64, bf16_t, bits, chunked_scale_bytes,
                      pack_weight_codes_ref,
                      pack_weight_scales_ref, packed_code_bytes, packed_scale_bytes, t, unpack_chunked,
                      unpack_tile_codes, unpack_tile_major)

_np = as_np
WN = ("w1", "w1s", "w3", "w3s", "w2", "w2s")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    import mxfp4_block_scaled_e2m1_amd as m
    return m


DECODE_MAX_TOKENS = 8    # mx_expert_mlp streams the weights once for up to 8 tokens


def _align(n):
    return (n + 255) // 256 * 256


def _ws_slices(mx, ws, M, H, I):
    """Dense workspace layout of mx_expert_mlp, each region 256-byte aligned:
    few tokens: h (bf16 SiLU output); weight-streaming path (9..512 tokens): xq,
    xs, hq, hs (chunked: whole 16-row chunks, scales per wave), h; GEMM path: xq,
    xs
    (row-major), hq, hs (both tile-major), xs_pk, and split-K partials when a
    GEMM is split.
    Returns (xq, xs, hq, hs), hq [M, I/2] and hs [M, I/32] row-major, or (h,)."""
    if M <= DECODE_MAX_TOKENS:
        return [ws[:M * I * 2]]
    mt, mq = (M + 255) // 256, (M + 15) // 16 * 16
    skinny = [mq * H // 2, chunked_scale_bytes(M), mq * I // 2, chunked_scale_bytes(M), M * I * 2]
    tile_major = sum(_align(n) for n in skinny) != mx.expert_mlp_workspace_size(M, H, I)
    gemm = [M * H // 2, M * H // 32, packed_code_bytes(mt, I), packed_scale_bytes(mt, I)]
    sizes = gemm if tile_major else skinny[:4]
    off, out = 0, []
    for n in sizes:
        out.append(ws[off:off + n])
        off += _align(n)
    if tile_major:
        out[2] = torch.from_numpy(unpack_tile_codes(out[2].cpu().numpy(), mt, I)[:M])
        out[3] = unpack_tile_major(out[3].cpu().numpy(), M, I)
    else:
        for i, k in ((0, H), (2, I)):
            q, s = unpack_chunked(out[i].cpu().numpy(), out[i + 1].cpu().numpy(), M, k)
            out[i], out[i + 1] = torch.from_numpy(np.ascontiguousarray(q)), torch.from_numpy(np.ascontiguousarray(s))
    return out


H_TINY = 1e-30   # fp32 exp(-g) overflows for g < -88.7: silu(g) * u below ~1e-36 flushes to +-0


def _check_h_and_requant(mx, h_slice, M, I, inter):
    """Few-token path: h (bf16) against the oracle's, and its re-quantisation.

    The GPU evaluates silu(g) * u in fp32 and rounds to bf16 once; the oracle
    rounds the fp64 value. They agree bit for bit except near bf16 rounding
    boundaries and for negligible values (|h| < 1e-30), which fp32 flushes."""
    h = h_slice.view(torch.int16).view(M, I)
    hb = h.cpu().numpy().view(np.uint16)
    ref = inter["h"]
    hv, rv = bf16_f64(hb), bf16_f64(ref)
    big = np.abs(rv) >= H_TINY
    same = np.mean(hb[big] == ref[big])
    assert same >= 0.999, same
    assert np.all(np.abs(hv - rv) <= np.abs(rv) * 2.0 ** -7 + H_TINY)
    codes, scales = mx.quantize_act("mxfp4", h.view(torch.bfloat16))
    assert_requant_close(codes.cpu().numpy(), scales.cpu().numpy(), inter["hq"], inter["hs"])


# ---------------------------------------------------------------- GEMM
@pytest.mark.parametrize("M,N,K", [(16, 256, 256), (130, 300, 384), (257, 512, 7168), (64, 7168, 3072),
                                   (200, 3072, 128), (1, 4, 256)])
def test_debug_gemm_f32(mx, M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    a, a_s = W.mxfp4_weight(rng, M, K)
    b, b_s = W.mxfp4_weight(rng, N, K)
    c = mx.debug_gemm_f32(t(a), t(a_s), t(b), t(b_s)).cpu().numpy().astype(np.float64)
    ref = O.gemm_f64(O.mxfp4_dequant_f64(a, a_s), O.mxfp4_dequant_f64(b, b_s))
    err = np.linalg.norm(c - ref) / np.linalg.norm(ref)
    assert err <= 1e-5, err


# ---------------------------------------------------------------- shared expert
def _run_dense(mx, d, M, H, I, packed=False):
    x = d["x"]
    nbytes = mx.expert_mlp_workspace_size(M, H, I)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    wd = [t(d[n]) for n in WN]
    pk = mx.pack_weight_scales(wd[1], wd[3], wd[5]) if packed else None
    pc = mx.pack_weight_codes(wd[0], wd[2], wd[4]) if packed == "all" else None
    y = mx.expert_mlp(bf16_t(x), *wd, workspace=ws, packed_scales=pk, packed_codes=pc)
    torch.cuda.synchronize()
    return bits(y), _ws_slices(mx, ws, M, H, I)


def _check_gemm_path(mx, d, M, H, I):
    """The output, and the quantised x and re-quantised h the workspace holds
    (only h in bf16 when the kernels quantise in registers)."""
    y, sl = _run_dense(mx, d, M, H, I)
    ref, inter = O.expert_mlp(d["x"], d["w1"], d["w1s"], d["w3"], d["w3s"], d["w2"], d["w2s"], intermediates=True)
    if len(sl) == 1:
        _check_h_and_requant(mx, sl[0], M, I, inter)
        assert_mlp_close(y, ref)
        return
    xq, xs, hq, hs = sl
    assert np.array_equal(xq.cpu().numpy().reshape(M, H // 2), inter["xq"])
    assert np.array_equal(xs.cpu().numpy().reshape(M, H // 32), inter["xs"])
    assert_requant_close(hq.cpu().numpy().reshape(M, I // 2), _np(hs).reshape(M, I // 32),
                         inter["hq"], inter["hs"])
    assert_mlp_close(y, ref)


def test_tiny_expert_mlp(mx):
    """The tiny configuration: 16 tokens, hidden 256, intermediate 128."""
    _check_gemm_path(mx, W.tiny_mlp(0), 16, 256, 128)


def test_tiny_expert_mlp_48_tokens(mx):
    d = W.tiny_mlp(0)
    d["x"] = W.bf16_normal(np.random.default_rng(7), (48, 256))
    _check_gemm_path(mx, d, 48, 256, 128)


@pytest.mark.parametrize("M", [1, 3, 8])
def test_tiny_expert_mlp_few_tokens(mx, M):
    """The tiny weights with the first M tokens: the weight-streaming path."""
    d = W.tiny_mlp(0)
    d["x"] = d["x"][:M]
    y, (h,) = _run_dense(mx, d, M, 256, 128)
    ref, inter = O.expert_mlp(d["x"], d["w1"], d["w1s"], d["w3"], d["w3s"], d["w2"], d["w2s"], intermediates=True)
    _check_h_and_requant(mx, h, M, 128, inter)
    assert_mlp_close(y, ref)


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 9, 17, 32, 33, 96, 97, 128, 300, 600])
def test_shared_expert_real_shape(mx, M):
    d = W.shared_expert(M, seed=0)
    y, sl = _run_dense(mx, d, M, 7168, 3072)
    ref, inter = O.expert_mlp(d["x"], d["w1"], d["w1s"], d["w3"], d["w3s"], d["w2"], d["w2s"], intermediates=True)
    if len(sl) == 1:
        _check_h_and_requant(mx, sl[0], M, 3072, inter)
    else:
        _, _, hq, hs = sl
        assert_requant_close(hq.cpu().numpy().reshape(M, 1536), _np(hs).reshape(M, 96), inter["hq"], inter["hs"])
    assert_mlp_close(y, ref)


@pytest.mark.parametrize("M,H,I", [(2, 2048, 1024), (8, 2048, 1024), (8, 1024, 512), (4, 512, 1024)])
def test_few_tokens_other_shapes(mx, M, H, I):
    """Few tokens at shapes besides the expert's: 2-step K runs per wave at
    hidden 2048, one step at hidden 1024 and 512 (intermediate 1024: more
    weight rows than the hidden size)."""
    d = W.shared_expert(M, seed=5, hidden=H, inter=I)
    y, (h,) = _run_dense(mx, d, M, H, I)
    ref, inter = O.expert_mlp(d["x"], d["w1"], d["w1s"], d["w3"], d["w3s"], d["w2"], d["w2s"], intermediates=True)
    _check_h_and_requant(mx, h, M, I, inter)
    assert_mlp_close(y, ref)


def test_few_tokens_calls_in_a_row(mx):
    """Calls in a row on one workspace, with different token counts, give the
    results of calls on fresh workspaces, bit for bit: nothing a call leaves in
    the workspace (h) leaks into the next."""
    H, I = 7168, 3072
    d = W.expert_weights(0)
    wd = [t(d[n]) for n in WN]
    xs = {M: bf16_t(W.activations(10 + M, M)) for M in (1, 3, 8)}
    fresh = {}
    for M, x in xs.items():
        ws = torch.empty(mx.expert_mlp_workspace_size(M, H, I), dtype=torch.uint8, device="cuda")
        fresh[M] = bits(mx.expert_mlp(x, *wd, workspace=ws))
    shared = torch.empty(mx.expert_mlp_workspace_size(8, H, I), dtype=torch.uint8, device="cuda")
    for M in (8, 1, 3, 8, 1):
        y = bits(mx.expert_mlp(xs[M], *wd, workspace=shared))
        assert np.array_equal(y, fresh[M]), M
    assert_mlp_close(fresh[3], O.expert_mlp(W.activations(13, 3), *[d[n] for n in WN]))


@pytest.mark.parametrize("M,H,I", [(130, 8320, 384), (200, 8448, 256), (256, 7168, 3072), (257, 7168, 3072)])
def test_shared_expert_split_k(mx, M, H, I):
    """Up to 256 tokens with hidden beyond the weight-streaming kernels' 8192,
    the dense L1 of one m-tile splits K over several workgroups (fp32 partials
    summed in split order, then the usual epilogue): 8 splits of 32.5 stages
    (H = 8320, ending in a half-width stage) and of 33 (H = 8448). At the real
    shape 256 and 257 tokens take the weight-streaming kernels in two and three
    groups of up to 128 (the third of one row)."""
    d = W.shared_expert(M, seed=4, hidden=H, inter=I)
    y, sl = _run_dense(mx, d, M, H, I)
    ref, inter = O.expert_mlp(d["x"], d["w1"], d["w1s"], d["w3"], d["w3s"], d["w2"], d["w2s"], intermediates=True)
    _, _, hq, hs = sl
    assert_requant_close(hq.cpu().numpy().reshape(M, I // 2), _np(hs).reshape(M, I // 32), inter["hq"], inter["hs"])
    assert_mlp_close(y, ref)


def test_shared_expert_prefill_sampled_rows(mx):
    M = 4096
    d = W.shared_expert(M, seed=0)
    y, _ = _run_dense(mx, d, M, 7168, 3072)
    rows = np.random.default_rng(3).choice(M, 24, replace=False)
    ref = O.expert_mlp(d["x"][rows], d["w1"], d["w1s"], d["w3"], d["w3s"], d["w2"], d["w2s"])
    assert_mlp_close(y[rows], ref)
    assert np.all(np.isfinite(((y.astype(np.uint32) << 16).view(np.float32))))


# ---------------------------------------------------------------- routed experts
def _run_grouped(mx, d, packed=False, requant="mxfp4", g=0.0):
    wd = [t(d[n]) for n in WN]
    pk = mx.pack_weight_scales(wd[1], wd[3], wd[5]) if packed else None
    pc = mx.pack_weight_codes(wd[0], wd[2], wd[4]) if packed == "all" else None
    y = mx.grouped_expert_mlp(bf16_t(d["x"]), t(d["ids"]), t(d["w"]), *wd, requant=requant, requant_global=g,
                              packed_scales=pk, packed_codes=pc)
    torch.cuda.synchronize()
    return bits(y)


def _oracle_grouped(d, tokens=None):
    return O.grouped_expert_mlp(d["x"], d["ids"], d["w"], d["w1"], d["w1s"], d["w3"], d["w3s"],
                                d["w2"], d["w2s"], tokens=tokens)


def test_grouped_multi_tile(mx):
    d = W.grouped(tokens=600, n_experts=8, k=4, seed=5, hidden=512, inter=256)
    y = _run_grouped(mx, d)
    assert_mlp_close(y, _oracle_grouped(d))


def test_grouped_single_expert_equals_shared(mx):
    d = W.shared_expert(200, seed=2, hidden=512, inter=256)
    g = {n: d[n][None] for n in ("w1", "w1s", "w3", "w3s", "w2", "w2s")}
    g["x"] = d["x"]
    g["ids"] = np.zeros((200, 1), np.int32)
    g["w"] = np.ones((200, 1), np.float32)
    yg = _run_grouped(mx, g)
    yd, _ = _run_dense(mx, d, 200, 512, 256)
    assert np.array_equal(yg, yd)


def test_grouped_permutation_empty_and_foreign_ids(mx):
    d = W.grouped(tokens=300, n_experts=6, k=3, seed=9, hidden=256, inter=128)
    d["ids"][d["ids"] == 5] = 4                 # expert 5 empty; duplicates within a token allowed
    y = _run_grouped(mx, d)
    perm = np.random.default_rng(1).permutation(300)
    dp = dict(d, x=d["x"][perm], ids=d["ids"][perm], w=d["w"][perm])
    yp = _run_grouped(mx, dp)
    assert np.array_equal(yp, y[perm])
    # ids outside [0, E) contribute nothing
    d2 = dict(d, ids=d["ids"].copy())
    d2["ids"][:, 2] = -1
    d2["ids"][::2, 1] = 6
    y2 = _run_grouped(mx, d2)
    assert_mlp_close(y2, _oracle_grouped(d2))


@pytest.mark.parametrize("E,k,T", [(1, 1, 1 << 20), (7, 4, 1 << 18), (512, 8, 1 << 17)])
def test_route_many_chunks(mx, E, k, T):
    """The route at 2^20 pairs (1024 chunks of 1024): one expert (the scan's
    1024 runs of one chunk), 7 (runs of 7 experts, which do not divide the
    scan block) and 512 (two runs of 512 chunks), with 2 % of the ids outside
    [0, E). Expert offsets, m-tile bases and every sorted row's token, slot and
    gate weight against a stable sort of the pairs by expert (the route of
    "Current Bug: vLLM produces empty/garbage output", "Revised Plan", Phase 1:
    pairs in expert order, pair order within an expert)."""
    from gpu_util import routed_ws_slices
    H = I = 128
    rng = np.random.default_rng(E)
    d = W.expert_weights(3, H, I, E)
    d["x"] = W.activations(4, T, H)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    foreign = rng.random((T, k)) < 0.02
    ids[foreign] = rng.choice(np.array([-1, E, E + 5], np.int32), int(foreign.sum()))
    w = rng.random((T, k)).astype(np.float32)
    wd = [t(d[n]) for n in WN]
    ws = torch.empty(mx.grouped_expert_mlp_workspace_size(T, H, I, k, E), dtype=torch.uint8, device="cuda")
    mx.grouped_expert_mlp(bf16_t(d["x"]), t(ids), t(w), *wd, workspace=ws)
    torch.cuda.synchronize()
    s = routed_ws_slices(ws, T, H, I, k, E)
    flat = ids.ravel()
    valid = (flat >= 0) & (flat < E)
    p = np.nonzero(valid)[0]
    order = p[np.argsort(flat[p], kind="stable")]
    counts = np.bincount(flat[valid], minlength=E)
    eo = np.concatenate([[0], np.cumsum(counts)])
    tb = np.concatenate([[0], np.cumsum((counts + 255) // 256)])
    assert np.array_equal(s["expert_off"], eo)
    assert np.array_equal(s["tile_base"], tb)
    n = int(eo[-1])
    assert np.array_equal(s["row_slot"][:n], order)
    assert np.array_equal(s["row_token"][:n], order // k)
    assert np.array_equal(s["row_weight"][:4 * n].view(np.float32), w.ravel()[order])


def test_grouped_headline_sampled_tokens(mx):
    d = W.grouped(tokens=4096, n_experts=48, k=8, seed=0)
    y = _run_grouped(mx, d, packed=True)
    tok = np.array([0, 1, 2, 4095])
    assert_mlp_close(y[tok], _oracle_grouped(d, tokens=tok))
    assert np.all(np.isfinite(((y.astype(np.uint32) << 16).view(np.float32))))


def test_grouped_skewed_sampled_tokens(mx):
    d = W.skewed(tokens=16384, seed=0)
    counts = np.bincount(d["ids"].ravel(), minlength=48)
    assert (counts == 0).sum() >= 1 and counts.max() > 4 * counts.mean()
    y = _run_grouped(mx, d)
    tok = np.array([7, 16383])
    assert_mlp_close(y[tok], _oracle_grouped(d, tokens=tok))
    # decode tail of 8 tokens over the same weights
    tail = dict(d, x=d["x"][:8], ids=d["ids"][:8], w=d["w"][:8])
    yt = _run_grouped(mx, tail)
    assert_mlp_close(yt, _oracle_grouped(tail))


# ---------------------------------------------------------------- tile-major weight scales
# ---------------------------------------------------------------- routed, few rows per expert
# The routed weight-streaming kernels run while T * k <= mean_rows * E:
STREAM_MEAN_ROWS = {"mxfp4": 6, "nvfp4": 24}


def _stream_ws_h(ws, T, H, I, k, E):
    """Routed weight-streaming workspace (regions 256-byte aligned): xq, xs,
    block counts, expert offsets, tile bases, row_token, row_slot, row_weight,
    h (bf16 [P, I], sorted rows), ... Returns (expert_off, row_token, h)."""
    P = T * k
    sizes = [T * H // 2, T * H // 32, -(-P // 1024) * E * 4, (E + 1) * 4, (E + 1) * 4, P * 4, P * 4, P * 4,
             P * I * 2]
    off, sl = 0, []
    for n in sizes:
        sl.append(ws[off:off + n])
        off += _align(n)
    eo = sl[3].cpu().numpy().view(np.int32)
    rt = sl[5].cpu().numpy().view(np.int32)
    h = sl[8].cpu().numpy().view(np.uint16).reshape(P, I)
    return eo, rt, h


def _stream_case(seed, T=16, E=16, k=2, H=256, I=128):
    d = W.grouped(tokens=T, n_experts=E, k=k, seed=seed, hidden=H, inter=I)
    d["ids"][:, 0] = 0              # expert 0: every token, and twice for the first three
    d["ids"][:3, 1] = 0             # (duplicates within a token allowed): two chunks of 16 rows
    d["ids"][d["ids"] == E - 1] = E - 2     # the last expert empty
    assert T * k <= STREAM_MEAN_ROWS["mxfp4"] * E
    return d


def test_grouped_stream_matches_oracle_and_h(mx):
    """Few rows per expert: the weight-streaming kernels. Output against the
    oracle, and h of every sorted row against the oracle's h of its (token,
    expert) pair, bit for bit on >= 99.9 % (the fp32 SiLU near bf16 rounding
    boundaries aside)."""
    T, E, k, H, I = 16, 16, 2, 256, 128
    d = _stream_case(3, T, E, k, H, I)
    wd = [t(d[n]) for n in WN]
    ws = torch.empty(mx.grouped_expert_mlp_workspace_size(T, H, I, k, E), dtype=torch.uint8, device="cuda")
    y = mx.grouped_expert_mlp(bf16_t(d["x"]), t(d["ids"]), t(d["w"]), *wd, workspace=ws)
    torch.cuda.synchronize()
    assert_mlp_close(bits(y), _oracle_grouped(d))
    eo, rt, h = _stream_ws_h(ws, T, H, I, k, E)
    counts = np.bincount(d["ids"].ravel(), minlength=E)
    assert np.array_equal(np.diff(eo), counts) and counts[0] > 16 and counts[E - 1] == 0
    hb, rb = [], []
    for e in range(E):
        if counts[e] == 0:
            continue
        rows = np.arange(eo[e], eo[e + 1])
        _, inter = O.expert_mlp(d["x"][rt[rows]], *(d[n][e] for n in WN), intermediates=True)
        hb.append(h[rows])
        rb.append(inter["h"])
    hb, rb = np.concatenate(hb), np.concatenate(rb)
    hv, rv = bf16_f64(hb), bf16_f64(rb)
    big = np.abs(rv) >= H_TINY
    assert np.mean(hb[big] == rb[big]) >= 0.999
    assert np.all(np.abs(hv - rv) <= np.abs(rv) * 2.0 ** -7 + H_TINY)


def test_grouped_stream_permutation_and_foreign_ids(mx):
    d = _stream_case(4)
    y = _run_grouped(mx, d)
    perm = np.random.default_rng(2).permutation(16)
    dp = dict(d, x=d["x"][perm], ids=d["ids"][perm], w=d["w"][perm])
    assert np.array_equal(_run_grouped(mx, dp), y[perm])
    d2 = dict(d, ids=d["ids"].copy())
    d2["ids"][::2, 1] = -1
    d2["ids"][1::4, 1] = 16
    assert_mlp_close(_run_grouped(mx, d2), _oracle_grouped(d2))


def test_grouped_stream_single_expert_equals_shared(mx):
    """E = 1, k = 1, w = 1 over 2 tokens: the routed weight-streaming kernels
    against the dense few-token kernels, which sum in the same order."""
    d = W.shared_expert(2, seed=6, hidden=512, inter=256)
    g = {n: d[n][None] for n in WN}
    g.update(x=d["x"], ids=np.zeros((2, 1), np.int32), w=np.ones((2, 1), np.float32))
    yg = _run_grouped(mx, g)
    yd, _ = _run_dense(mx, d, 2, 512, 256)
    assert np.array_equal(yg, yd)
    assert_mlp_close(yg, _oracle_grouped(g))


@pytest.mark.parametrize("requant,T", [("mxfp4", 12), ("mxfp4", 13), ("nvfp4", 48), ("nvfp4", 49)])
def test_grouped_stream_threshold(mx, requant, T):
    """T * k = mean_rows * E runs the weight-streaming kernels, one token more the GEMMs."""
    d = W.grouped(tokens=T, n_experts=4, k=2, seed=8, hidden=384, inter=256)
    assert (T * 2 <= STREAM_MEAN_ROWS[requant] * 4) == (T in (12, 48))
    g = 0.0
    if requant == "nvfp4":
        h = [O.expert_mlp(d["x"], *(d[n][e] for n in WN), intermediates=True)[1]["h"] for e in range(4)]
        g = float(O.nvfp4_warmup_global(np.concatenate(h)))
    ref = O.grouped_expert_mlp(d["x"], d["ids"], d["w"], *(d[n] for n in WN), requant=requant, nv_global=g)
    assert_mlp_close(_run_grouped(mx, d, packed=True, requant=requant, g=g), ref)


@pytest.mark.parametrize("requant", ["mxfp4", "nvfp4"])
def test_grouped_stream_max_experts(mx, requant):
    """The largest expert count (512) with two tokens: a grid of 512 experts,
    almost all without rows."""
    d = W.grouped(tokens=2, n_experts=512, k=8, seed=12, hidden=128, inter=128)
    g = 0.0
    if requant == "nvfp4":
        h = [O.expert_mlp(d["x"], *(d[n][e] for n in WN), intermediates=True)[1]["h"] for e in np.unique(d["ids"])]
        g = float(O.nvfp4_warmup_global(np.concatenate(h)))
    ref = O.grouped_expert_mlp(d["x"], d["ids"], d["w"], *(d[n] for n in WN), requant=requant, nv_global=g)
    assert_mlp_close(_run_grouped(mx, d, requant=requant, g=g), ref)


def test_grouped_stream_decode_real_shape(mx):
    """8 tokens of the uniformly routed 48-expert batch at the real shape."""
    d = W.grouped(tokens=4096, n_experts=48, k=8, seed=0)
    tail = dict(d, x=d["x"][:8], ids=d["ids"][:8], w=d["w"][:8])
    assert_mlp_close(_run_grouped(mx, tail, packed=True), _oracle_grouped(tail))


@pytest.mark.parametrize("requant", ["mxfp4", "nvfp4"])
def test_grouped_stream_packed_codes(mx, requant):
    """The routed weight-streaming kernels read the tile-major codes when given:
    bit-identical output, on the 16-row-chunk case (expert 0 with two chunks, the
    last expert empty) and on 8 tokens of the real-shape batch."""
    g = 0.05 if requant == "nvfp4" else 0.0
    d = _stream_case(21)
    assert np.array_equal(_run_grouped(mx, d, requant=requant, g=g),
                          _run_grouped(mx, d, packed="all", requant=requant, g=g))
    full = W.grouped(tokens=4096, n_experts=48, k=8, seed=0)
    tail = dict(full, x=full["x"][:8], ids=full["ids"][:8], w=full["w"][:8])
    y1 = _run_grouped(mx, tail, packed="all", requant=requant, g=g)
    assert np.array_equal(_run_grouped(mx, tail, requant=requant, g=g), y1)
    if requant == "mxfp4":
        assert_mlp_close(y1, _oracle_grouped(tail))


@pytest.mark.parametrize("E,H,I", [(3, 384, 256), (2, 512, 384), (1, 7168, 3072)])
def test_pack_weight_scales_layout(mx, E, H, I):
    """mx_pack_weight_scales moves bytes only: compare with the layout written out in numpy
    (rows past the end repeat the last row; bytes past a row's end are zero)."""
    rng = np.random.default_rng(E * 1000 + H + I)
    w1s = rng.integers(0, 256, (E, I, H // 32), dtype=np.uint8)
    w3s = rng.integers(0, 256, (E, I, H // 32), dtype=np.uint8)
    w2s = rng.integers(0, 256, (E, H, I // 32), dtype=np.uint8)
    pk = mx.pack_weight_scales(t(w1s), t(w3s), t(w2s))
    assert pk.numel() == mx.packed_weight_scales_size(H, I, E)
    assert np.array_equal(pk.cpu().numpy(), pack_weight_scales_ref(w1s, w3s, w2s))


@pytest.mark.parametrize("E,H,I", [(3, 384, 256), (2, 512, 384), (1, 7168, 3072)])
def test_pack_weight_codes_layout(mx, E, H, I):
    """mx_pack_weight_codes moves bytes only: compare with the layout written out
    in numpy (the GEMM's LDS image of each tile's half stage)."""
    rng = np.random.default_rng(E * 1000 + H + I + 1)
    w1 = rng.integers(0, 256, (E, I, H // 2), dtype=np.uint8)
    w3 = rng.integers(0, 256, (E, I, H // 2), dtype=np.uint8)
    w2 = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    pc = mx.pack_weight_codes(t(w1), t(w3), t(w2))
    assert pc.numel() == mx.packed_weight_codes_size(H, I, E)
    assert np.array_equal(pc.cpu().numpy(), pack_weight_codes_ref(w1, w3, w2))


@pytest.mark.parametrize("M,H,I", [(16, 256, 128), (300, 384, 384), (700, 1024, 640), (1, 7168, 3072),
                                   (8, 7168, 3072), (40, 7168, 3072), (128, 7168, 3072), (200, 7168, 3072),
                                   (130, 8320, 384), (4096, 7168, 3072)])
def test_packed_codes_same_result_dense(mx, M, H, I):
    """The tile-major weight codes feed the same MFMAs the same bytes: output
    bit-identical to the row-major weights', on every path: the few-token
    kernels (1, 8), the weight-streaming kernels (16, 40: a partial last chunk
    of a 4-chunk launch; 128; 200: two token groups), the split-K L1 (130 at
    hidden 8320, each split starting mid-matrix) and the tiled GEMMs."""
    d = W.tiny_mlp(0) if H == 256 else W.shared_expert(M, seed=12, hidden=H, inter=I)
    d["x"] = d["x"][:M]
    y0, _ = _run_dense(mx, d, M, H, I)
    y1, _ = _run_dense(mx, d, M, H, I, packed="all")
    assert np.array_equal(y0, y1)


@pytest.mark.parametrize("requant", ["mxfp4", "nvfp4"])
def test_packed_codes_same_result_grouped(mx, requant):
    d = W.grouped(tokens=600, n_experts=8, k=4, seed=6, hidden=640, inter=384)
    g = 0.05 if requant == "nvfp4" else 0.0
    y0 = _run_grouped(mx, d, requant=requant, g=g)
    y1 = _run_grouped(mx, d, packed="all", requant=requant, g=g)
    assert np.array_equal(y0, y1)
    if requant == "mxfp4":
        assert_mlp_close(y1, _oracle_grouped(d))


@pytest.mark.parametrize("M,H,I", [(16, 256, 128), (300, 384, 384), (128, 7168, 3072)])
def test_packed_scales_same_result_dense(mx, M, H, I):
    """The tile-major weight scales feed the same MFMAs the same bytes: bit-identical output."""
    d = W.tiny_mlp(0) if H == 256 else W.shared_expert(M, seed=11, hidden=H, inter=I)
    d["x"] = d["x"][:M]
    y0, _ = _run_dense(mx, d, M, H, I)
    y1, _ = _run_dense(mx, d, M, H, I, packed=True)
    assert np.array_equal(y0, y1)
    ref = O.expert_mlp(d["x"], *(d[n] for n in WN))
    assert_mlp_close(y1, ref)


@pytest.mark.parametrize("requant", ["mxfp4", "nvfp4"])
def test_packed_scales_same_result_grouped(mx, requant):
    d = W.grouped(tokens=600, n_experts=8, k=4, seed=5, hidden=512, inter=256)
    g = 0.05 if requant == "nvfp4" else 0.0
    y0 = _run_grouped(mx, d, requant=requant, g=g)
    y1 = _run_grouped(mx, d, packed=True, requant=requant, g=g)
    assert np.array_equal(y0, y1)
    if requant == "mxfp4":
        assert_mlp_close(y1, _oracle_grouped(d))
