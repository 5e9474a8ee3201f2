"""Parity of the FP8 block-scaled linear (MXFP8 activations x FP8 E4M3 weights
with 128 x 128 E8M0 block scales) and of its activation quantiser with the oracle."""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import bf16_f64, bf16_t, bits, t

pytestmark = pytest.mark.gpu

H_TINY = 1e-30   # fp32 exp(-g) overflows for g < -88.7: silu(g) * u below ~1e-36 flushes to +-0


@pytest.fixture(scope="module")
def mx():
    import mxfp4_block_scaled_e2m1_amd as m
    return m


def _spread_blocks(rng, R, C):
    """bf16 rows whose 32-blocks span many binades, with zero, subnormal, tiny and
    saturating blocks mixed in."""
    x = rng.standard_normal((R, C)) * np.exp2(rng.integers(-40, 40, (R, C // 32))).repeat(32, axis=1)
    x = x.astype(np.float32)
    x[0, :32] = 0.0
    x[0, 32:64] = -0.0
    x[1, :32] = np.float32(2.0 ** -130) * rng.integers(-8, 9, 32)      # bf16 subnormals
    x[1, 32:64] = np.float32(1.9375)                                     # 496 under the scale: saturates
    x[1, 64] = np.float32(1.0)
    x[1, 65:96] = np.float32(-2.0 ** -20)                                # below half the subnormal step
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    return b


def test_mxfp8_quantize_bitexact(mx):
    rng = np.random.default_rng(61)
    xb = _spread_blocks(rng, 64, 1024)
    codes, scales = mx.quantize_act("mxfp8", bf16_t(xb))
    rc, rs = O.mxfp8_quantize(xb)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_mxfp8_quantize_every_bf16(mx):
    """Every finite bf16 pattern, in blocks anchored at every binade."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = allbits[((allbits >> 7) & 0xFF) != 0xFF]
    rng = np.random.default_rng(67)
    rows = []
    for ea in range(0, 255, 2):
        cand = rng.permutation(fin)[:31 * 64].reshape(64, 31)
        anchor = np.full((64, 1), (ea << 7) | 0x7F, np.uint16)
        rows.append(np.concatenate([anchor, cand], axis=1))
    xb = np.concatenate(rows).reshape(-1, 1024)
    codes, scales = mx.quantize_act("mxfp8", bf16_t(xb))
    rc, rs = O.mxfp8_quantize(xb)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def _exact_and_magnitude(x_bits, w, ws):
    """fp64 product of the quantised operands, and the sum of its terms' magnitudes."""
    xq, xs = O.mxfp8_quantize(x_bits)
    a = O.mxfp8_dequant_f64(xq, xs)
    b = O.fp8_block_dequant_f64(w, ws)
    return O.gemm_f64(a, b), O.gemm_f64(np.abs(a), np.abs(b))


def _check_linear(y_bits, ref_bits, exact, mag):
    """Same quantised operands on both sides. The FP8 scaled MFMA does not sum
    its products exactly in fp32: measured on the device, its error stays
    below 2^-15.8 of the sum of the products' magnitudes (S). The bar is that
    bound with margin, 2^-12 S, plus the bf16 rounding of the output (2^-9,
    taken as 2^-8); most outputs equal the oracle's correctly rounded value."""
    yv, rv = bf16_f64(y_bits), bf16_f64(ref_bits)
    assert np.all(np.isfinite(yv))
    same = np.mean(y_bits == ref_bits)
    assert same >= 0.9, same
    bad = np.abs(yv - exact) > np.abs(exact) * 2.0 ** -8 + mag * 2.0 ** -12
    assert not bad.any(), (np.argwhere(bad)[:5], yv[bad][:5], exact[bad][:5])
    err = np.linalg.norm(yv - exact) / np.linalg.norm(exact)
    assert err <= 4e-3, err


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (37, 384, 256), (300, 640, 1152), (257, 256, 8192),
                                   (16, 7168, 1536)])
def test_fp8_linear_matches_oracle(mx, M, N, K):
    d = W.fp8_linear(M, N, K, seed=M + N + K)
    y = mx.fp8_block_linear(bf16_t(d["x"]), t(d["w"]), t(d["ws"]))
    torch.cuda.synchronize()
    ref = O.fp8_block_linear(d["x"], d["w"], d["ws"])
    _check_linear(bits(y), ref, *_exact_and_magnitude(d["x"], d["w"], d["ws"]))


def test_fp8_linear_real_shape_sampled_rows(mx):
    """4096 tokens through the pages' FP8 matrix [7168, 1536]; rows sampled
    from every m-tile for the oracle (rows are independent)."""
    d = W.fp8_linear(4096, seed=0)
    ws = torch.empty(mx.fp8_block_linear_workspace_size(4096, 1536), dtype=torch.uint8, device="cuda")
    y = bits(mx.fp8_block_linear(bf16_t(d["x"]), t(d["w"]), t(d["ws"]), workspace=ws))
    rows = np.array([0, 255, 256, 1000, 2047, 3333, 4095])
    ref = O.fp8_block_linear(d["x"][rows], d["w"], d["ws"])
    _check_linear(y[rows], ref, *_exact_and_magnitude(d["x"][rows], d["w"], d["ws"]))
    # the quantised activations in the workspace, bit for bit
    xq = ws[:4096 * 1536].cpu().numpy().reshape(4096, 1536)
    rq, _ = O.mxfp8_quantize(d["x"][rows])
    assert np.array_equal(xq[rows], rq)


def test_fp8_linear_unit_rows_give_dequant_columns(mx):
    """x = e_k: y = the FP8 block dequant of W's column k (the dequant kernel's
    output, itself bit-exact with the oracle)."""
    d = W.fp8_linear(1, 384, 512, seed=3)
    ks = np.array([0, 1, 127, 128, 300, 511])
    x = np.zeros((len(ks), 512), np.uint16)
    x[np.arange(len(ks)), ks] = 0x3F80
    y = bits(mx.fp8_block_linear(bf16_t(x), t(d["w"]), t(d["ws"])))
    deq = bits(mx.dequant("fp8_b128", t(d["w"]), t(d["ws"]), 384, 512))
    assert np.array_equal(bf16_f64(y), bf16_f64(np.ascontiguousarray(deq[:, ks].T)))


def test_fp8_linear_empty(mx):
    d = W.fp8_linear(1, 128, 128)
    y = mx.fp8_block_linear(bf16_t(d["x"][:0]), t(d["w"]), t(d["ws"]))
    torch.cuda.synchronize()
    assert y.shape == (0, 128)


# ---------------------------------------------------------------- FP8 shared expert
FP8_WN = ("w1", "w1s", "w3", "w3s", "w2", "w2s")


@pytest.mark.parametrize("M,H,I", [(5, 256, 128), (300, 512, 384), (64, 7168, 3072)])
def test_fp8_expert_mlp_matches_oracle(mx, M, H, I):
    """Every stage against the oracle applied to the GPU's own input of that
    stage: g and u (the plain FP8 linear on the GPU: the same quantiser and K
    loop as the gate/up GEMM, whose epilogue rounds them the same way) to the
    FP8 linear's bar; h (from the workspace) bit-equal to bf16(silu(g) * u)
    except near bf16 rounding boundaries (fp32 SiLU); the MXFP8 codes of h
    bit-exact; y to the linear's bar given h. End to end the cosine stays >=
    0.9999; the largest error is allowed 5e-2 of max |y|, since a one-step
    difference in g or u (the FP8 MFMA's own summation error) can move an
    element of h across an E4M3 rounding boundary, a step of up to 2^-3 of
    that element."""
    from gpu_util import assert_mlp_close, bf16_f64
    d = W.fp8_expert(M, H, I, seed=M + H)
    ws = torch.empty(mx.fp8_expert_mlp_workspace_size(M, H, I), dtype=torch.uint8, device="cuda")
    x = bf16_t(d["x"])
    y = bits(mx.fp8_expert_mlp(x, *(t(d[n]) for n in FP8_WN), workspace=ws))
    torch.cuda.synchronize()
    al = lambda n: (n + 255) // 256 * 256
    sizes = [M * H, M * H // 32, M * I * 2, M * I, M * I // 32]
    off, sl = 0, []
    for n in sizes:
        sl.append(ws[off:off + n].cpu().numpy())
        off += al(n)
    assert off == mx.fp8_expert_mlp_workspace_size(M, H, I)
    g = bits(mx.fp8_block_linear(x, t(d["w1"]), t(d["w1s"])))
    u = bits(mx.fp8_block_linear(x, t(d["w3"]), t(d["w3s"])))
    h = sl[2].view(np.uint16).reshape(M, I)
    hq, hs = sl[3].reshape(M, I), sl[4].reshape(M, I // 32)
    _check_linear(g, O.fp8_block_linear(d["x"], d["w1"], d["w1s"]), *_exact_and_magnitude(d["x"], d["w1"], d["w1s"]))
    _check_linear(u, O.fp8_block_linear(d["x"], d["w3"], d["w3s"]), *_exact_and_magnitude(d["x"], d["w3"], d["w3s"]))
    # h: the GPU's fp32 SiLU (hardware exp2 and reciprocal, a few tens of fp32
    # ulps at worst for large |g|) may round the other way only where the exact
    # value lies within 2^-16 of a bf16 rounding midpoint (bf16 g and u often
    # make g * u an exact midpoint); values below 1e-30 flush in fp32 (e^-g
    # overflows for g < -88.7) and are not compared
    gv, uv = bf16_f64(g), bf16_f64(u)
    rh = O.silu_mul_bf16(gv, uv)
    with np.errstate(over="ignore"):
        exact = gv / (1.0 + np.exp(-gv)) * uv
    diff = (h != rh) & (np.abs(exact) >= H_TINY)
    assert np.mean(diff) <= 0.01
    mid = (bf16_f64(h) + bf16_f64(rh)) / 2
    assert np.all(np.abs(exact[diff] - mid[diff]) <= np.abs(exact[diff]) * 2.0 ** -16)
    rq, rs = O.mxfp8_quantize(h)
    assert np.array_equal(hq, rq) and np.array_equal(hs, rs)
    _check_linear(y, O.fp8_block_linear(h, d["w2"], d["w2s"]), *_exact_and_magnitude(h, d["w2"], d["w2s"]))
    assert_mlp_close(y, O.fp8_expert_mlp(d["x"], *(d[n] for n in FP8_WN)), rel_max=5e-2)

