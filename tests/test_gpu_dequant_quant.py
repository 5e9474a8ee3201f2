"""Bit-exact parity of the GPU dequant and quantise kernels with the oracle."""

import numpy as np
import pytest

import oracle as O
import pins
import workloads as W
from gpu_util import bf16_t, bits, t

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    import mxfp4_block_scaled_e2m1_amd as m
    return m


def test_mxfp4_dequant_every_byte_every_scale(mx):
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))          # row s: all bytes
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 16, 1)  # row s: scale byte s
    out = mx.dequant("mxfp4", t(codes), t(scales), 256, 512)
    assert np.array_equal(bits(out), O.mxfp4_dequant_bf16(codes, scales))


@pytest.mark.parametrize("name", ["w1", "w2"])
def test_mxfp4_dequant_real_shapes(mx, name):
    d = W.dequant_inputs(0)
    c, s = d[name], d[name + "s"]
    rows, cols = c.shape[0], 2 * c.shape[1]
    out = mx.dequant("mxfp4", t(c), t(s), rows, cols)
    assert out.shape == (rows, cols)
    assert np.array_equal(bits(out), O.mxfp4_dequant_bf16(c, s))


def test_fp8_dequant_every_code_every_scale(mx):
    q = np.tile(np.arange(256, dtype=np.uint8), (2048, 8))               # [2048, 2048]
    s = np.arange(256, dtype=np.uint8).reshape(16, 16)
    out = mx.dequant("fp8_b128", t(q), t(s), 2048, 2048)
    assert np.array_equal(bits(out), O.fp8_block_dequant_bf16(q, s))


def test_fp8_dequant_real_and_ragged(mx):
    d = W.dequant_inputs(0)
    out = mx.dequant("fp8_b128", t(d["fp8"]), t(d["fp8s"]), 7168, 1536)
    assert np.array_equal(bits(out), O.fp8_block_dequant_bf16(d["fp8"], d["fp8s"]))
    rng = np.random.default_rng(4)
    q = W.e4m3_finite_codes(rng, (200, 304))
    s = rng.integers(118, 135, (2, 3)).astype(np.uint8)
    out = mx.dequant("fp8_b128", t(q), t(s), 200, 304)
    assert np.array_equal(bits(out), O.fp8_block_dequant_bf16(q, s))


def test_nvfp4_dequant(mx):
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 256, (96, 256), dtype=np.uint8)
    scales = W.e4m3_finite_codes(rng, (96, 32))
    scales[scales >= 0x80] &= 0x7F                     # E4M3 block scales are positive
    g = np.float32(0.0123)
    out = mx.dequant("nvfp4", t(codes), t(scales), 96, 512, global_scale=float(g))
    with np.errstate(invalid="ignore"):
        want = O.f64_to_bf16(O.nvfp4_dequant_f64(codes, scales, g))
    assert np.array_equal(bits(out), want)


def _sweep_blocks():
    """Blocks [anchor, 31 candidates] covering every finite bf16 pattern at every anchor binade."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = allbits[((allbits >> 7) & 0xFF) != 0xFF]
    mags = finite & 0x7FFF
    rows = []

    def add(anchor, cand):
        pad = (-len(cand)) % 31
        cb = np.concatenate([cand, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        rows.append(np.concatenate([np.full((cb.shape[0], 1), anchor, np.uint16), cb], axis=1))
    add(np.uint16(0x7F7F), finite)
    add(np.uint16(0x007F), finite[mags <= 0x007F])
    add(np.uint16(0x0000), np.zeros(31, np.uint16) | np.uint16(0x8000))
    for ea in range(1, 255):
        ab = (ea << 7) | 0x7F
        add(np.uint16(ab), finite[(mags <= ab) & (mags >= (max(ea - 12, 0) << 7))])
    x = np.concatenate(rows)                       # [nblocks, 32]
    n = x.shape[0] - x.shape[0] % 8
    return x[:n].reshape(-1, 256)                  # 8 blocks per row


def test_mxfp4_quantize_exhaustive_sweep(mx):
    x = _sweep_blocks()
    codes, scales = mx.quantize_act("mxfp4", bf16_t(x))
    rc, rs = O.mxfp4_quantize(x)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("rows,cols", [(4096, 7168), (1, 7168), (3, 96), (0, 64)])
def test_mxfp4_quantize_activations(mx, rows, cols):
    x = W.bf16_normal(np.random.default_rng(rows + cols), (rows, cols))
    codes, scales = mx.quantize_act("mxfp4", bf16_t(x))
    if rows == 0:
        return
    rc, rs = O.mxfp4_quantize(x)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_nvfp4_quantize(mx):
    rng = np.random.default_rng(8)
    x = W.bf16_normal(rng, (512, 1024))
    # widen the dynamic range so that E4M3 scales span subnormals and saturation
    xv = O.bf16_to_f64(x) * np.ldexp(1.0, rng.integers(-20, 8, (512, 1))).astype(np.float64)
    x = O.f64_to_bf16(xv)
    g = O.nvfp4_warmup_global(x[:64])
    codes, scales = mx.quantize_act("nvfp4", bf16_t(x), global_scale=float(g))
    rc, rs = O.nvfp4_quantize(x, g)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)
