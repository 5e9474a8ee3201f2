"""Plant plausible mistakes in the oracle (CPU only) and require a pin to catch each.

The mistakes mirror the failures the pages report (nibble order and sign
handling of the E2M1 unpack, a block scale left at 1.0, dividing by the scale,
no width doubling) and generic ones (a dropped term, a wrong sign, a wrong
index, a transposed operand).
"""

import numpy as np
import pytest

import oracle.mx_oracle as O
import pins

_orig = {name: getattr(O, name) for name in dir(O) if not name.startswith("__")}


def _unpack_hi_first(codes):
    c = np.asarray(codes).view(np.uint8) if np.asarray(codes).dtype == np.int8 else np.asarray(codes)
    out = np.empty(c.shape[:-1] + (2 * c.shape[-1],), np.uint8)
    out[..., 0::2] = (c >> 4) & 15
    out[..., 1::2] = c & 15
    return out


def _unpack_sign_extended(codes):
    c = np.asarray(codes)
    s = c.view(np.int8) if c.dtype == np.uint8 else c
    out = np.empty(c.shape[:-1] + (2 * c.shape[-1],), np.uint8)
    out[..., 0::2] = s.view(np.uint8) & 15
    out[..., 1::2] = (s >> 4).astype(np.uint8)        # arithmetic shift, no mask
    return out


def _unpack_no_doubling(codes):
    c = np.asarray(codes).view(np.uint8) if np.asarray(codes).dtype == np.int8 else np.asarray(codes)
    return (c & 15).astype(np.uint8)


def _e8m0_ones(b):
    return np.ones(np.asarray(b).shape)


def _e8m0_divide(b):
    b = np.asarray(b).astype(np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, 127 - b))


def _e4m3_bias8(b):
    b = np.asarray(b).astype(np.int64) & 0xFF
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -7, (1.0 + m / 8.0) * np.ldexp(1.0, e - 8))
    v = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, v)


def _f64_to_bf16_via_f32(x):
    x32 = np.asarray(x, np.float64).astype(np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(np.isnan(x32), np.uint16(0x7FC0), r)


def _code_ties_away(a):
    a = np.asarray(a, np.float64)
    return np.select([a < 0.25, a < 0.75, a < 1.25, a < 1.75, a < 2.5, a < 3.5, a < 5.0],
                     [0, 1, 2, 3, 4, 5, 6], 7).astype(np.uint8)


def _quantize_flush_neg_zero(x_bits):
    codes, sc = _orig["mxfp4_quantize"](x_bits)
    lo, hi = codes & 15, codes >> 4
    lo = np.where(lo == 8, 0, lo)
    hi = np.where(hi == 8, 0, hi)
    return (lo | (hi << 4)).astype(np.uint8), sc


def _quantize_emax1(x_bits):
    # shared exponent floor(log2 amax) - 1 instead of - 2: largest codes saturate
    x = O.bf16_to_f64(x_bits)
    R, C = x.shape
    blk = x.reshape(R, C // 32, 32)
    amax = np.abs(blk).max(axis=2)
    _, e = np.frexp(amax)
    b = np.where(amax == 0, 0, np.clip(e - 1 - 1 + 127, 0, 254)).astype(np.int64)
    v = blk / np.ldexp(1.0, b - 127)[..., None]
    nib = O.e2m1_code_rne_sat(np.abs(v)) | (np.signbit(blk).astype(np.uint8) << 3)
    nib = nib.reshape(R, C)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8), b.astype(np.uint8)


def _gemm_drop_last_block(a, b):
    return np.asarray(a)[:, :-32] @ np.asarray(b)[:, :-32].T


def _gemm_transposed_b(a, b):
    # B [N, K] read as if it were stored [K, N]
    b = np.asarray(b, np.float64)
    return np.asarray(a, np.float64) @ b.reshape(b.shape[1], b.shape[0])


def _silu_wrong_sign(g, u):
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return _orig["f64_to_bf16"](g / (1.0 + np.exp(g)) * np.asarray(u, np.float64))


def _silu_no_up(g, u):
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return _orig["f64_to_bf16"](g / (1.0 + np.exp(-g)))


def _requant_skipped(h_bits, requant, nv_global):
    hq, hs = _orig["mxfp4_quantize"](h_bits)
    return hq, hs, O.bf16_to_f64(h_bits)


def _grouped_ignore_weights(x_bits, topk_ids, topk_w, *a, **k):
    return _orig["grouped_expert_mlp"](x_bits, topk_ids, np.ones_like(np.asarray(topk_w)), *a, **k)


def _fp8_divide(q, s, block=128):
    q = np.asarray(q)
    R, C = q.shape
    full = np.repeat(np.repeat(_e8m0_divide(s), block, 0), block, 1)[:R, :C]
    return O.e4m3_decode(q) * full


def _fp8_scale_transposed_index(q, s, block=128):
    q = np.asarray(q)
    R, C = q.shape
    sv = O.e8m0_decode(s).ravel()
    gr, gc = np.asarray(s).shape
    i = np.arange(R)[:, None] // block
    j = np.arange(C)[None, :] // block
    return O.e4m3_decode(q) * sv[(j * gr + i) % sv.size]


def _mxfp8_emax7(x_bits):
    # shared exponent floor(log2 amax) - 7: the largest values leave the E4M3 range
    x = O.bf16_to_f64(x_bits)
    R, C = x.shape
    blk = x.reshape(R, C // 32, 32)
    amax = np.abs(blk).max(axis=2)
    _, e = np.frexp(amax)
    b = np.where(amax == 0, 0, np.clip(e - 1 - 7 + 127, 0, 254)).astype(np.int64)
    v = blk / np.ldexp(1.0, b - 127)[..., None]
    mag, _ = O.e4m3_rne_satfinite(np.abs(v))
    return ((mag & 0x7F) | (np.signbit(blk).astype(np.uint8) << 7)).reshape(R, C).astype(np.uint8), b.astype(np.uint8)


def _mxfp8_no_saturation(x_bits):
    # values above 448 become the NaN code instead of saturating
    codes, sc = _orig["mxfp8_quantize"](x_bits)
    x = O.bf16_to_f64(x_bits)
    R, C = x.shape
    v = np.abs(x) / np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)
    return np.where(v > 448, codes | 0x7F, codes).astype(np.uint8), sc


def _fp8_linear_scale_per_row(x_bits, w, w_s, block=128):
    # weight scale indexed [n // 128] only (first K block's scale for every K)
    ws = np.asarray(w_s)
    flat = np.repeat(ws[:, :1], ws.shape[1], axis=1)
    return _orig["fp8_block_linear"](x_bits, w, flat, block)


def _fp8_linear_drop_last_k_block(x_bits, w, w_s, block=128):
    # the last 128 columns of K left out of the product (a dropped term)
    x = np.asarray(x_bits).copy()
    x[:, -block:] = 0
    return _orig["fp8_block_linear"](x, w, w_s, block)


def _nvfp4_linear_drop_last_k_block(x_bits, w, w_s, w_global, x_global):
    x = np.asarray(x_bits).copy()
    x[:, -16:] = 0
    return _orig["nvfp4_linear"](x, w, w_s, w_global, x_global)


def _nvfp4_quantize_exact_6g(x_bits, g):
    # the block scale from amax / (6 g) in fp64 (no fp32 rounding of 6 g)
    codes, sc = _orig["nvfp4_quantize"](x_bits, g)
    x = O.bf16_to_f64(x_bits)
    blk = np.abs(x.reshape(x.shape[0], -1, 16)).max(axis=2)
    byte = pins.e4m3_bruteforce(blk / (6.0 * float(g)))     # nearest E4M3 of the fp64 quotient
    return codes, np.asarray(byte, np.uint8)


def _quantize_nan_block_finite_scale(x_bits):
    # a block holding inf or NaN keeps a finite scale byte (254)
    x = O.bf16_to_f64(x_bits)
    xf = np.where(np.isfinite(x), x, 0.0)
    bits = O.f64_to_bf16(xf)
    codes, sc = _orig["mxfp4_quantize"](bits)
    bad = ~np.isfinite(x.reshape(x.shape[0], -1, 32)).all(axis=2)
    return codes, np.where(bad, 254, sc).astype(np.uint8)


LUT_POS_ZERO = np.array([0.0, 0.5, 1, 1.5, 2, 3, 4, 6, 0.0, -0.5, -1, -1.5, -2, -3, -4, -6])

MUTATIONS = [
    ("nibble order swapped", "mxfp4_unpack", _unpack_hi_first, pins.check_dequant_examples),
    ("high nibble sign-extended", "mxfp4_unpack", _unpack_sign_extended, pins.check_dequant_examples),
    ("no width doubling", "mxfp4_unpack", _unpack_no_doubling, pins.check_format_shapes),
    ("scale left at one", "e8m0_decode", _e8m0_ones, pins.check_dequant_examples),
    ("divide by scale", "e8m0_decode", _e8m0_divide, pins.check_dequant_all_bytes),
    ("nibble 8 is +0", "E2M1_LUT", LUT_POS_ZERO, pins.check_nibble8_negative_zero),
    ("e4m3 bias 8", "e4m3_decode", _e4m3_bias8, pins.check_fp8_examples),
    ("fp8 divide by scale", "fp8_block_dequant_f64", _fp8_divide, pins.check_fp8_examples),
    ("fp8 scale grid index", "fp8_block_dequant_f64", _fp8_scale_transposed_index,
     pins.check_fp8_block_bruteforce),
    ("bf16 through fp32", "f64_to_bf16", _f64_to_bf16_via_f32, pins.check_no_double_rounding),
    ("ties away from zero", "e2m1_code_rne_sat", _code_ties_away, pins.check_quantize_exhaustive),
    ("-0 flushed to +0", "mxfp4_quantize", _quantize_flush_neg_zero, pins.check_nibble_balance),
    ("shared exponent off by one", "mxfp4_quantize", _quantize_emax1, pins.check_quantize_examples),
    ("GEMM drops a K block", "gemm_f64", _gemm_drop_last_block, pins.check_gemm_bruteforce),
    ("GEMM operand transposed", "gemm_f64", _gemm_transposed_b, pins.check_gemm_integer),
    ("SiLU sign", "silu_mul_bf16", _silu_wrong_sign, pins.check_silu),
    ("up projection dropped", "silu_mul_bf16", _silu_no_up, pins.check_mlp_bruteforce),
    ("re-quant skipped", "_requant", _requant_skipped, pins.check_mlp_bruteforce),
    ("gate weights ignored", "grouped_expert_mlp", _grouped_ignore_weights,
     pins.check_grouped_reductions),
    ("MXFP8 shared exponent off by one", "mxfp8_quantize", _mxfp8_emax7, pins.check_mxfp8_examples),
    ("MXFP8 without saturation", "mxfp8_quantize", _mxfp8_no_saturation, pins.check_mxfp8_quantize_exhaustive),
    ("FP8 linear weight scale per row block only", "fp8_block_linear", _fp8_linear_scale_per_row,
     pins.check_fp8_linear_unit_rows),
    # the composition pins recompose the MLPs from the oracle's own linears, so a
    # fault inside the linear escapes them; the Fraction brute force does not
    ("FP8 expert over a linear that drops a K block", "fp8_block_linear", _fp8_linear_drop_last_k_block,
     pins.check_fp8_mlp_fraction_bruteforce),
    ("NVFP4 expert over a linear that drops a K block", "nvfp4_linear", _nvfp4_linear_drop_last_k_block,
     pins.check_nvfp4_mlp_fraction_bruteforce),
    ("NVFP4 scale without the fp32 rounding of 6 g", "nvfp4_quantize", _nvfp4_quantize_exact_6g,
     pins.check_nvfp4_golden_block),
    ("non-finite block keeps a finite scale", "mxfp4_quantize", _quantize_nan_block_finite_scale,
     pins.check_quantizers_nonfinite_blocks),
]


@pytest.mark.parametrize("name,attr,mutant,check", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, attr, mutant, check):
    check(O)                              # passes on the real oracle
    monkeypatch.setattr(O, attr, mutant)
    with pytest.raises(Exception):
        check(O)
