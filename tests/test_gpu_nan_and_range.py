"""Edge cases of the hot path on the GPU: NaN codes in the weights travel to
exactly the outputs they feed, non-finite activation blocks get the NaN scale,
and the scaled-MFMA GEMM holds its 1e-5 bar with E8M0 scale bytes across the
whole finite range (0, 1, ..., 253, 254) wherever the fp32 result is
representable.

The pages' debugging history is about exactly these failure classes: a block
scale that must carry the real value ("2026-05-11 - DeepSeek V4 NVFP4 vLLM
Serving: Full End-to-End", "What We Fixed" item 5) and sign or scale-order
mistakes in the E2M1 unpack ("Outstanding Issues"). E8M0 byte 0xFF and E4M3
byte 0x7F are the NaN encodings of the formats the pages name (e8m0fnu,
e4m3fn)."""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import bf16_f64, bf16_t, bits, t

pytestmark = pytest.mark.gpu
WN = ("w1", "w1s", "w3", "w3s", "w2", "w2s")


@pytest.fixture(scope="module")
def mx():
    import mxfp4_block_scaled_e2m1_amd as m
    return m


def _nan(y):
    return np.isnan(bf16_f64(y))


def _dense(mx, d, **kw):
    y = mx.expert_mlp(bf16_t(d["x"]), *(t(d[n]) for n in WN), **kw)
    torch.cuda.synchronize()
    return bits(y)


# ---------------------------------------------------------------- quantisers
@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8", "nvfp4"])
def test_quantize_nonfinite_blocks(mx, fmt):
    """Blocks holding +inf, -inf or NaN get the NaN scale byte; every other block
    is bit-identical to the oracle's."""
    x = W.activations(3, 64, 512)
    poison = [(0, 5, 0x7F80), (1, 300, 0xFF80), (2, 33, 0x7FC0), (63, 511, 0xFFC1)]
    for r, c, v in poison:
        x[r, c] = v
    g = np.float32(0.01)
    if fmt == "mxfp4":
        rc, rs = O.mxfp4_quantize(x)
        per, nan_byte, bpb = 32, 0xFF, 16
        gc, gs = mx.quantize_act("mxfp4", bf16_t(x))
    elif fmt == "mxfp8":
        rc, rs = O.mxfp8_quantize(x)
        per, nan_byte, bpb = 32, 0xFF, 32
        gc, gs = mx.quantize_act("mxfp8", bf16_t(x))
    else:
        rc, rs = O.nvfp4_quantize(x, g)
        per, nan_byte, bpb = 16, 0x7F, 8
        gc, gs = mx.quantize_act("nvfp4", bf16_t(x), global_scale=float(g))
    gc, gs = gc.cpu().numpy(), gs.cpu().numpy()
    hit = np.zeros(rs.shape, bool)
    for r, c, _ in poison:
        hit[r, c // per] = True
    assert np.all(gs[hit] == nan_byte) and np.all(rs[hit] == nan_byte)
    assert np.array_equal(gs[~hit], rs[~hit])
    codes_ok = np.repeat(~hit, bpb, axis=1)
    assert np.array_equal(gc[codes_ok], rc[codes_ok])


# ---------------------------------------------------------------- shared expert
@pytest.mark.parametrize("M", [4, 40, 300])
def test_shared_expert_nan_weights(mx, M):
    """A NaN down-projection scale byte: exactly that output column is NaN for
    every token, the rest bit-identical to the clean run. A NaN gate scale byte:
    h is NaN in one block of every token, re-quantised with the NaN scale, so
    every output is NaN. M = 4 runs the few-token kernels, 40 the
    weight-streaming pair, 300 the tiled GEMMs."""
    d = W.shared_expert(M, seed=13, hidden=1024, inter=512)
    y0 = _dense(mx, d)
    assert not _nan(y0).any()
    d2 = dict(d, w2s=d["w2s"].copy())
    d2["w2s"][333, 7] = 0xFF
    y2 = _dense(mx, d2)
    assert _nan(y2)[:, 333].all()
    assert np.array_equal(np.delete(y2, 333, axis=1), np.delete(y0, 333, axis=1))
    d1 = dict(d, w1s=d["w1s"].copy())
    d1["w1s"][100, 3] = 0xFF
    assert _nan(_dense(mx, d1)).all()
    # the oracle agrees on the pattern
    assert _nan(O.expert_mlp(d2["x"][:2], *(d2[n] for n in WN)))[:, 333].all()


def test_shared_expert_nan_nvfp4_requant(mx):
    """With NVFP4 re-quantisation a NaN gate scale makes every output NaN too
    (the block of h gets the E4M3 NaN scale)."""
    d = W.shared_expert(300, seed=13, hidden=1024, inter=512)
    d1 = dict(d, w1s=d["w1s"].copy())
    d1["w1s"][100, 3] = 0xFF
    y = _dense(mx, d1, requant="nvfp4", requant_global=2.0 ** -6)
    assert _nan(y).all()


# ---------------------------------------------------------------- routed experts
@pytest.mark.parametrize("T", [300, 4])
def test_routed_nan_weights_touch_only_their_tokens(mx, T):
    """Expert 2's NaN down scale byte: y[t, n] is NaN exactly for the tokens routed
    to expert 2 at that column n; its NaN gate scale byte: every output of
    exactly those tokens. All else is bit-identical to the clean run. T = 300 is
    the tiled path, T = 4 the weight-streaming one."""
    d = W.grouped(tokens=T, n_experts=6, k=3, seed=9, hidden=512, inter=256)
    run = lambda dd: bits(mx.grouped_expert_mlp(bf16_t(dd["x"]), t(dd["ids"]), t(dd["w"]),
                                                *(t(dd[n]) for n in WN)))
    y0 = run(d)
    assert not _nan(y0).any()
    to2 = (d["ids"] == 2).any(axis=1)
    assert to2.any() and not to2.all()
    d2 = dict(d, w2s=d["w2s"].copy())
    d2["w2s"][2, 77, 1] = 0xFF
    y2 = run(d2)
    want = np.zeros_like(y2, bool)
    want[to2, 77] = True
    assert np.array_equal(_nan(y2), want)
    assert np.array_equal(y2[~want], y0[~want])
    d1 = dict(d, w1s=d["w1s"].copy())
    d1["w1s"][2, 40, 2] = 0xFF
    y1 = run(d1)
    assert _nan(y1)[to2].all() and not _nan(y1)[~to2].any()
    assert np.array_equal(y1[~to2], y0[~to2])


# ---------------------------------------------------------------- FP8 and NVFP4 weights
def test_fp8_linear_nan_codes(mx):
    """FP8 linear: an E4M3 NaN code makes its output column NaN; an E8M0 NaN block
    scale makes the 128 output columns of its block NaN; the rest unchanged."""
    d = W.fp8_linear(64, 384, 512, seed=4)
    run = lambda w, ws: bits(mx.fp8_block_linear(bf16_t(d["x"]), t(w), t(ws)))
    y0 = run(d["w"], d["ws"])
    w = d["w"].copy()
    w[200, 37] = 0x7F
    y1 = run(w, d["ws"])
    assert _nan(y1)[:, 200].all()
    assert np.array_equal(np.delete(y1, 200, axis=1), np.delete(y0, 200, axis=1))
    ws = d["ws"].copy()
    ws[1, 2] = 0xFF
    y2 = run(d["w"], ws)
    assert _nan(y2)[:, 128:256].all()
    keep = np.r_[0:128, 256:384]
    assert np.array_equal(y2[:, keep], y0[:, keep])


def test_nvfp4_linear_nan_scale(mx):
    """NVFP4-weight linear: an E4M3 NaN block scale makes its output column NaN."""
    d = W.nvfp4_linear(32, 256, 512, seed=2)
    run = lambda ws: bits(mx.nvfp4_linear(bf16_t(d["x"]), t(d["w"]), t(ws), float(d["wg"]), float(d["xg"])))
    y0 = run(d["ws"])
    ws = d["ws"].copy()
    ws[99, 5] = 0x7F
    y1 = run(ws)
    assert _nan(y1)[:, 99].all()
    assert np.array_equal(np.delete(y1, 99, axis=1), np.delete(y0, 99, axis=1))


# ---------------------------------------------------------------- extreme exponents
@pytest.mark.parametrize("M,N,K", [(64, 256, 2048), (300, 384, 7168)])
def test_debug_gemm_extreme_scale_bytes(mx, M, N, K):
    """Scale bytes over the whole finite E8M0 range in both operands (0, 1, 253
    and 254 included), paired per K block so that every product scale 2^(sa +
    sb - 254) stays within a few binades of 1 and the fp32 result is
    representable: the 1e-5 relative Frobenius bar of the GEMM still holds.
    Each block's A scales are one random byte per block shifted by +-2 per row,
    B's the complement 254 - byte shifted by +-2."""
    rng = np.random.default_rng(M + N + K)
    nb = K // 32
    base = rng.integers(0, 255, nb)
    base[:4] = [0, 1, 253, 254]
    a = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    b = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    a_s = np.clip(base[None, :] + rng.integers(-2, 3, (M, nb)), 0, 254).astype(np.uint8)
    b_s = np.clip(254 - base[None, :] + rng.integers(-2, 3, (N, nb)), 0, 254).astype(np.uint8)
    assert a_s.min() == 0 and a_s.max() == 254 and b_s.min() == 0 and b_s.max() == 254
    c = mx.debug_gemm_f32(t(a), t(a_s), t(b), t(b_s)).cpu().numpy().astype(np.float64)
    ref = O.gemm_f64(O.mxfp4_dequant_f64(a, a_s), O.mxfp4_dequant_f64(b, b_s))
    assert np.all(np.isfinite(ref))
    err = np.linalg.norm(c - ref) / np.linalg.norm(ref)
    assert err <= 1e-5, err
