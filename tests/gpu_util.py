"""Helpers for the GPU parity tests: host <-> device tensors and the comparison metrics."""

import numpy as np
import torch

import pins


def dev():
    return torch.device("cuda:0")


def t(a):
    """numpy -> device tensor (same dtype)."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_t(bits):
    """numpy uint16 bf16 bit patterns -> device bf16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def bits(x):
    """device bf16 tensor -> numpy uint16 bit patterns."""
    return x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_f64(b):
    return ((b.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)


def cosine(y_bits, r_bits):
    y, r = bf16_f64(y_bits).ravel(), bf16_f64(r_bits).ravel()
    return float(y @ r / (np.linalg.norm(y) * np.linalg.norm(r)))


def max_rel(y_bits, r_bits):
    y, r = bf16_f64(y_bits), bf16_f64(r_bits)
    return float(np.abs(y - r).max() / np.abs(r).max())


def assert_mlp_close(y_bits, r_bits, cos_min=0.9999, rel_max=1e-2):
    """Final-output bar: fp64 cosine over the flattened output and max error over max |ref|."""
    assert np.all(np.isfinite(bf16_f64(y_bits)))
    c, m = cosine(y_bits, r_bits), max_rel(y_bits, r_bits)
    assert c >= cos_min and m <= rel_max, (c, m)
    return c, m


def nibbles(codes):
    c = np.asarray(codes, np.uint8)
    n = np.empty(c.shape[:-1] + (2 * c.shape[-1],), np.uint8)
    n[..., 0::2] = c & 15
    n[..., 1::2] = c >> 4
    return n


def assert_requant_close(gpu_codes, gpu_scales, ref_codes, ref_scales, min_equal=0.999):
    """Re-quantised codes: >= 99.9 % equal (+0 == -0); each mismatch within one E2M1
    grid step at the larger of the two block scales."""
    g, r = nibbles(gpu_codes), nibbles(ref_codes)
    grid = np.array(pins.E2M1_GRID + [-v for v in pins.E2M1_GRID])
    gv, rv = grid[g], grid[r]
    same = gv == rv
    frac = same.mean()
    assert frac >= min_equal, frac
    sg = np.repeat(gpu_scales.astype(np.int64), 32, axis=-1)
    sr = np.repeat(ref_scales.astype(np.int64), 32, axis=-1)
    ga = gv * np.ldexp(1.0, sg - 127)
    ra = rv * np.ldexp(1.0, sr - 127)
    step = 2.0 * np.ldexp(1.0, np.maximum(sg, sr) - 127)     # widest E2M1 step (4 -> 6)
    assert np.all(np.abs(ga - ra) <= step), np.abs(ga - ra).max()
    return frac


def assert_nvfp4_requant_close(gpu_codes, gpu_scales, ref_codes, ref_scales, g, min_equal=0.999):
    """NVFP4 re-quantised h: >= 99.9 % equal codes (+0 == -0) and E4M3 block
    scales; each code mismatch within one E2M1 grid step at the larger of the two
    dequantised block scales s * g."""
    gn, rn = nibbles(gpu_codes), nibbles(ref_codes)
    grid = np.array(pins.E2M1_GRID + [-v for v in pins.E2M1_GRID])
    gv, rv = grid[gn], grid[rn]
    frac = (gv == rv).mean()
    assert frac >= min_equal, frac
    assert (np.asarray(gpu_scales) == np.asarray(ref_scales)).mean() >= min_equal
    sg = np.repeat(pins.e4m3_values()[np.asarray(gpu_scales, np.int64)], 16, axis=-1) * g
    sr = np.repeat(pins.e4m3_values()[np.asarray(ref_scales, np.int64)], 16, axis=-1) * g
    step = 2.0 * np.maximum(sg, sr)
    assert np.all(np.abs(gv * sg - rv * sr) <= step), np.abs(gv * sg - rv * sr).max()
    return frac
