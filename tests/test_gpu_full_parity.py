"""Full-size parity of the hot path with the oracle: every output of the routed
48-expert batch (4096 tokens, top-8, hidden 7168, intermediate 3072) and the
re-quantised intermediate of every one of its 32768 (token, expert) pairs; all
4096 rows of the shared expert's prefill; the skewed 16384-token batch's heaviest
expert and an expert whose last m-tile is partial, pair by pair, in both
re-quantisation formats; a routed batch at hidden 1024 (more K stages than the
copy prologue) with experts of more than 256 rows, compared in full; the
most tokens the routed weight-streaming kernels take with NVFP4 re-quantisation
at the real shape, compared in full.

The pages ask for a standalone test of the pipeline against a reference before
anything else (page "Current Bug: vLLM produces empty/garbage output", section
"Revised Plan", Phase 1); the formats are those of "2026-05-08 DeepSeek V4 Pro
NVFP4 Quantization", "FP4 (E2M1) expert weight format confirmed"."""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import (assert_mlp_close, assert_nvfp4_requant_close, assert_requant_close, bf16_f64, bf16_t, bits,
                      routed_ws_slices, t)

pytestmark = pytest.mark.gpu
WN = ("w1", "w1s", "w3", "w3s", "w2", "w2s")


@pytest.fixture(scope="module")
def mx():
    import mxfp4_block_scaled_e2m1_amd as m
    return m


def _routed(mx, d, requant="mxfp4", g=None, packed=True):
    T, H = d["x"].shape
    k = d["ids"].shape[1]
    E, I = d["w1"].shape[0], d["w1"].shape[1]
    wd = [t(d[n]) for n in WN]
    pk = mx.pack_weight_scales(wd[1], wd[3], wd[5]) if packed else None
    pc = mx.pack_weight_codes(wd[0], wd[2], wd[4]) if packed else None
    ws = torch.empty(mx.grouped_expert_mlp_workspace_size(T, H, I, k, E, requant), dtype=torch.uint8, device="cuda")
    y = mx.grouped_expert_mlp(bf16_t(d["x"]), t(d["ids"]), t(d["w"]), *wd, requant=requant, requant_global=g,
                              workspace=ws, packed_scales=pk, packed_codes=pc)
    torch.cuda.synchronize()
    return bits(y), routed_ws_slices(ws, T, H, I, k, E, requant)


def _sorted_rows(d, sl, e):
    """The sorted rows of expert e and their (token, slot): the route keeps the
    row-major (t, j) order of topk_ids within an expert, as np.nonzero does."""
    eo = sl["expert_off"]
    rows = np.arange(eo[e], eo[e + 1])
    tok, slot = sl["row_token"][rows], sl["row_slot"][rows]
    k = d["ids"].shape[1]
    return rows, tok, slot, slot - tok * k


def _check_route(d, sl):
    E = d["w1"].shape[0]
    counts = np.bincount(d["ids"].ravel()[(d["ids"].ravel() >= 0) & (d["ids"].ravel() < E)], minlength=E)
    assert np.array_equal(np.diff(sl["expert_off"]), counts)
    for e in range(E):
        _, tok, _, j = _sorted_rows(d, sl, e)
        t_idx, k_idx = np.nonzero(d["ids"] == e)
        assert np.array_equal(tok, t_idx) and np.array_equal(j, k_idx), e


def _check_requant_all_pairs(d, sl, inter, requant="mxfp4", g=None):
    gq, gs, rq, rs = [], [], [], []
    for e, it in inter.items():
        rows, _, _, _ = _sorted_rows(d, sl, e)
        gq.append(sl["hq"][rows])
        gs.append(sl["hs"][rows])
        rq.append(it["hq"])
        rs.append(it["hs"])
    gq, gs, rq, rs = (np.concatenate(v) for v in (gq, gs, rq, rs))
    if requant == "nvfp4":
        return assert_nvfp4_requant_close(gq, gs, rq, rs, g)
    return assert_requant_close(gq, gs, rq, rs)


@pytest.mark.timeout(600)
def test_headline_every_output_and_every_pair_requant(mx):
    """48 experts x 4096 tokens, top-8: all 4096 x 7168 outputs against the
    oracle, the route against np.nonzero, and the re-quantised h of all 32768
    pairs (read from the workspace in sorted order) against the oracle's codes."""
    d = W.grouped(tokens=4096, n_experts=48, k=8, seed=0)
    y, sl = _routed(mx, d)
    _check_route(d, sl)
    ref, inter = O.grouped_expert_mlp(d["x"], d["ids"], d["w"], *(d[n] for n in WN), intermediates=True)
    assert sum(len(v["t_idx"]) for v in inter.values()) == 32768
    assert_mlp_close(y, ref)
    frac = _check_requant_all_pairs(d, sl, inter)
    assert frac >= 0.999


@pytest.mark.timeout(600)
def test_shared_expert_prefill_every_row(mx):
    M, H, I = 4096, 7168, 3072
    d = W.shared_expert(M, seed=0)
    wd = [t(d[n]) for n in WN]
    pk = mx.pack_weight_scales(wd[1], wd[3], wd[5])
    pc = mx.pack_weight_codes(wd[0], wd[2], wd[4])
    y = bits(mx.expert_mlp(bf16_t(d["x"]), *wd, packed_scales=pk, packed_codes=pc))
    ref = O.expert_mlp(d["x"], *(d[n] for n in WN))
    assert_mlp_close(y, ref)


def _warmup_pairs(d, tokens):
    """g = f32(max |h| / (6 * 448)) over the (token, expert) pairs of `tokens` (the
    oracle's reading of the pages' warm-up global)."""
    ids = d["ids"][tokens]
    hs = []
    for e in np.unique(ids[(ids >= 0) & (ids < d["w1"].shape[0])]):
        tt = np.nonzero((ids == e).any(axis=1))[0]
        _, it = O.expert_mlp(d["x"][tokens][tt], *(d[n][e] for n in WN), intermediates=True)
        hs.append(it["h"])
    return float(O.nvfp4_warmup_global(np.concatenate(hs)))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("requant", ["mxfp4", "nvfp4"])
def test_skewed_heaviest_and_partial_tile_experts_pair_by_pair(mx, requant):
    """16384 tokens, Zipf(1.2) routing: the per-pair rows the L2 GEMM writes (gate
    weight applied, bf16, slot order) for every pair of the heaviest expert and of
    an expert whose last m-tile is partial, against the oracle's single-expert
    pipeline on the same tokens; their re-quantised h too."""
    d = W.skewed(tokens=16384, seed=0)
    E = d["w1"].shape[0]
    counts = np.bincount(d["ids"].ravel(), minlength=E)
    assert (counts == 0).sum() >= 1 and counts.max() > 4 * counts.mean()
    g = _warmup_pairs(d, np.arange(16)) if requant == "nvfp4" else None
    y, sl = _routed(mx, d, requant=requant, g=g)
    _check_route(d, sl)
    heavy = int(np.argmax(counts))
    partial = [e for e in np.argsort(counts)[::-1] if counts[e] % 256 not in (0,) and e != heavy]
    for e in (heavy, int(partial[0])):
        rows, tok, slot, j = _sorted_rows(d, sl, e)
        ref_y, it = O.expert_mlp(d["x"][tok], *(d[n][e] for n in WN), requant=requant, nv_global=g,
                                 intermediates=True)
        wgt = d["w"][tok, j].astype(np.float32).astype(np.float64)
        ref_o = O.f64_to_bf16(wgt[:, None] * it["y64"])
        assert_mlp_close(sl["o"][slot], ref_o)
        if requant == "nvfp4":
            assert_nvfp4_requant_close(sl["hq"][rows], sl["hs"][rows], it["hq"], it["hs"], g)
        else:
            assert_requant_close(sl["hq"][rows], sl["hs"][rows], it["hq"], it["hs"])
    assert np.all(np.isfinite(bf16_f64(y)))


@pytest.mark.parametrize("requant", ["mxfp4", "nvfp4"])
def test_routed_hidden_1024_full(mx, requant):
    """Hidden 1024 (four K stages, so the L1 runs its steady copy loop) with
    experts of 500-700 rows (three m-tiles, the last partial, so every row
    position of a tile is used): the whole output and every pair's h re-quant."""
    d = W.grouped(tokens=1200, n_experts=4, k=2, seed=21, hidden=1024, inter=512)
    counts = np.bincount(d["ids"].ravel(), minlength=4)
    assert counts.min() > 256 and np.any(counts % 256 != 0)
    g = None
    if requant == "nvfp4":
        g = _warmup_pairs(d, np.arange(1200))
    y, sl = _routed(mx, d, requant=requant, g=g)
    _check_route(d, sl)
    ref, inter = O.grouped_expert_mlp(d["x"], d["ids"], d["w"], *(d[n] for n in WN), requant=requant, nv_global=g,
                                      intermediates=True)
    assert_mlp_close(y, ref)
    _check_requant_all_pairs(d, sl, inter, requant, g)


@pytest.mark.timeout(600)
def test_routed_stream_nvfp4_most_tokens_real_shape(mx):
    """The most tokens the routed weight-streaming kernels take with NVFP4
    re-quantisation (T k = 24 E: 144 tokens of the uniform 48-expert batch,
    top-8, hidden 7168, intermediate 3072), with expert 0 given 40+ rows (three
    16-row chunks); the whole output against the oracle."""
    full = W.grouped(tokens=4096, n_experts=48, k=8, seed=0)
    T, E, k = 144, 48, 8
    d = dict(full, x=full["x"][:T], ids=full["ids"][:T].copy(), w=full["w"][:T])
    for i in range(48):
        if not (d["ids"][i] == 0).any():
            d["ids"][i, k - 1] = 0
    counts = np.bincount(d["ids"].ravel(), minlength=E)
    assert T * k == 24 * E and counts[0] > 32
    g = _warmup_pairs(d, np.arange(T))
    wd = [t(d[n]) for n in WN]
    pk = mx.pack_weight_scales(wd[1], wd[3], wd[5])
    pc = mx.pack_weight_codes(wd[0], wd[2], wd[4])
    H, I = d["x"].shape[1], d["w1"].shape[1]
    ws = torch.empty(mx.grouped_expert_mlp_workspace_size(T, H, I, k, E, "nvfp4"), dtype=torch.uint8, device="cuda")
    y = mx.grouped_expert_mlp(bf16_t(d["x"]), t(d["ids"]), t(d["w"]), *wd, requant="nvfp4", requant_global=g,
                              workspace=ws, packed_scales=pk, packed_codes=pc)
    torch.cuda.synchronize()
    ref = O.grouped_expert_mlp(d["x"], d["ids"], d["w"], *(d[n] for n in WN), requant="nvfp4", nv_global=g)
    assert_mlp_close(bits(y), ref)
