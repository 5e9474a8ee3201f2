"""Plain, slow, obviously correct CPU oracle of the block-scaled FP4 expert MLP.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark, never by the GPU library. It shares no code,
tables or helpers with the HIP path; only the seeded input generators
(``workloads``) feed both.

Arithmetic is fp64 (NumPy) except where a step is defined as a sequence of
fp32 operations (the NVFP4 quantiser). Every function names the passage it
follows. The pages are cited by title and section:

* [Q0508] "2026-05-08 DeepSeek V4 Pro NVFP4 Quantization": sections "Script
  update" (the complete dequant script: FP8 128x128 block dequant and FP4
  E2M1 expert-weight dequant) and "FP4 (E2M1) expert weight format confirmed".
* [BUG0518] "Current Bug: vLLM produces empty/garbage output": sections
  "Revised Plan: Our Own NVFP4 Kernels" (Phase 1: the shared-expert pipeline,
  Phase 3: where BF16 stays), "What we know" and "Config values".
* [SRV0511] "2026-05-11 - DeepSeek V4 NVFP4 vLLM Serving: Full End-to-End":
  "What We Fixed" item 5 (the block scale must carry the real value) and
  "Outstanding Issues" (sign handling in the E2M1 unpack, scale ordering).

Readings taken where the pages are silent are listed in the docstrings
("Reading:") and collected in the design notes of the repository.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "E2M1_LUT", "e2m1_decode", "e8m0_decode", "e4m3_decode",
    "bf16_to_f64", "bf16_to_f32", "f64_to_bf16",
    "mxfp4_unpack", "mxfp4_dequant_f64", "mxfp4_dequant_bf16",
    "fp8_block_dequant_f64", "fp8_block_dequant_bf16",
    "e2m1_code_rne_sat", "mxfp4_quantize",
    "e4m3_rne_satfinite", "e4m3_encode_exact", "nvfp4_quantize", "nvfp4_dequant_f64",
    "gemm_f64", "silu_mul_bf16", "expert_mlp", "grouped_expert_mlp",
    "nvfp4_warmup_global", "mxfp8_quantize", "mxfp8_dequant_f64", "fp8_block_linear", "fp8_expert_mlp",
    "nvfp4_linear", "nvfp4_expert_mlp", "grouped_nvfp4_expert_mlp",
]

# ---------------------------------------------------------------------------
# Element and scale formats
# ---------------------------------------------------------------------------

#: E2M1 magnitudes for codes 0..7; codes 8..15 are the same with the sign bit
#: (bit 3) set, so code 8 is negative zero. [Q0508] "Script update" item 2 says
#: the expert weights decode through an E2M1 look-up table; "FP4 (E2M1) expert
#: weight format confirmed" identifies code 8 as -0.0 (it is as frequent as
#: code 0 in real weights, which rules out INT4).
E2M1_LUT = np.array(
    [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
     -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=np.float64)


def e2m1_decode(nibbles):
    """Value of 4-bit E2M1 codes (fp64). [Q0508] "Script update" item 2."""
    n = np.asarray(nibbles).astype(np.int64)
    if n.size and (n.min() < 0 or n.max() > 15):
        raise ValueError("E2M1 codes are 4-bit")
    return E2M1_LUT[n]


def e8m0_decode(b):
    """E8M0 (float8_e8m0fnu) scale byte -> 2**(b-127); byte 255 is NaN.

    [Q0508] "Script update" items 1-2 and "FP4 (E2M1) expert weight format
    confirmed" (the scales are float8_e8m0fnu). Reading: the NaN code 0xFF
    comes from the format name (finite, no infinities, NaN = all ones).
    """
    b = np.asarray(b).view(np.uint8) if np.asarray(b).dtype == np.int8 else np.asarray(b)
    b = b.astype(np.int64)
    if b.size and (b.min() < 0 or b.max() > 255):
        raise ValueError("E8M0 scales are bytes")
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def e4m3_decode(b):
    """float8_e4m3fn byte -> fp64 value.

    [Q0508] "Script update" item 1 (FP8 weights are float8_e4m3fn). Reading of
    the format name: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0
    is subnormal (m/8 * 2**-6); S.1111.111 is NaN; there is no infinity.
    """
    b = np.asarray(b).astype(np.int64) & 0xFF
    s = b >> 7
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


# ---------------------------------------------------------------------------
# bf16 <-> fp64
# ---------------------------------------------------------------------------

def bf16_to_f64(bits):
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def bf16_to_f32(bits):
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def f64_to_bf16(x):
    """Round fp64 to bf16 bits once, round-to-nearest-even, no fp32 step.

    Rounding through fp32 first would round twice. Here the bf16 quantum at
    the value's binade (2**(e-8) with frexp's e, floored at the subnormal
    quantum 2**-133) is applied to the exact fp64 value. Results that round
    to 2**128 or beyond become infinity; NaN becomes the quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(a)
        q_exp = np.maximum(e, -125) - 8
        r = np.rint(np.ldexp(a, -q_exp))
        val = np.ldexp(r, q_exp)
        inf = ~(val < 2.0 ** 128)
        val = np.where(inf, 0.0, val)
        bits = (val.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(inf, np.uint16(0x7F80), bits)
    bits = bits | (np.signbit(x).astype(np.uint16) << 15)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


# ---------------------------------------------------------------------------
# Dequantisation
# ---------------------------------------------------------------------------

def mxfp4_unpack(codes):
    """Packed bytes [..., K/2] -> E2M1 nibbles [..., K].

    [Q0508] "Script update" item 2: two FP4 values per byte, lower nibble
    first, so logical element 2j is byte j & 0xF and element 2j+1 is
    byte j >> 4. The checkpoint stores the bytes as int8, so they are
    reinterpreted as unsigned before shifting: an arithmetic shift of a
    negative int8 would drag the sign bit into the high nibble (the sign
    handling trap named in [SRV0511] "Outstanding Issues").
    """
    c = np.asarray(codes)
    if c.dtype == np.int8:
        c = c.view(np.uint8)
    c = c.astype(np.uint8)
    out = np.empty(c.shape[:-1] + (2 * c.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = c & 0x0F
    out[..., 1::2] = (c >> 4) & 0x0F
    return out


def mxfp4_dequant_f64(codes, scales):
    """MXFP4 weight [R, K/2] bytes + E8M0 [R, K/32] -> fp64 [R, K].

    [Q0508] "Script update" item 2 and "FP4 (E2M1) expert weight format
    confirmed": value = E2M1(nibble) * 2**(scale-127), one scale per row per
    32 logical columns; the logical width is twice the stored bytes (224*32 =
    7168 for w1/w3, 96*32 = 3072 for w2). The scale multiplies ([SRV0511]
    "What We Fixed" item 5 shows what a scale of 1.0 in its place does).
    """
    n = mxfp4_unpack(codes)
    R, K = n.shape[-2], n.shape[-1]
    s = np.asarray(scales)
    if K % 32 != 0 or s.shape[-2:] != (R, K // 32):
        raise ValueError(f"scale shape {s.shape} does not match [{R}, {K // 32}]")
    return E2M1_LUT[n] * np.repeat(e8m0_decode(s), 32, axis=-1)


def mxfp4_dequant_bf16(codes, scales):
    """MXFP4 -> bf16 bits, one RNE rounding of the exact product."""
    with np.errstate(invalid="ignore"):
        return f64_to_bf16(mxfp4_dequant_f64(codes, scales))


def fp8_block_dequant_f64(q, s, block=128):
    """FP8 E4M3 [R, C] with one E8M0 scale per 128x128 tile -> fp64 [R, C].

    [Q0508] "What needs to happen" item 1 and "Script update" item 1: block-
    wise 128x128 dequant, weight times block scale. Reading: the scale grid is
    row-major [ceil(R/128), ceil(C/128)] and multiplies (not divides).
    """
    q = np.asarray(q)
    R, C = q.shape
    s = np.asarray(s)
    gr, gc = -(-R // block), -(-C // block)
    if s.shape != (gr, gc):
        raise ValueError(f"scale grid {s.shape} != [{gr}, {gc}]")
    full = np.repeat(np.repeat(e8m0_decode(s), block, axis=0), block, axis=1)[:R, :C]
    return e4m3_decode(q) * full


def fp8_block_dequant_bf16(q, s, block=128):
    with np.errstate(invalid="ignore"):
        return f64_to_bf16(fp8_block_dequant_f64(q, s, block))


# ---------------------------------------------------------------------------
# Quantisation
# ---------------------------------------------------------------------------

def e2m1_code_rne_sat(a):
    """|v| (fp64, >= 0) -> E2M1 magnitude code 0..7.

    Round to the nearest grid value {0, .5, 1, 1.5, 2, 3, 4, 6}; a value
    exactly half-way goes to the even code; anything above 5 saturates to 6.
    Reading: the OCP MX rule (round to nearest even, saturate) as named for
    the activation quantiser; the pages only say "MXFP4 microscaling".
    """
    a = np.asarray(a, dtype=np.float64)
    return np.select(
        [a <= 0.25, a < 0.75, a <= 1.25, a < 1.75, a <= 2.5, a < 3.5, a <= 5.0],
        [0, 1, 2, 3, 4, 5, 6], 7).astype(np.uint8)


def _pack_nibbles(nib):
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def mxfp4_quantize(x_bits):
    """bf16 [R, C] -> (codes uint8 [R, C/2], E8M0 uint8 [R, C/32]).

    Per row and 32-column block: amax = max |x|; shared exponent
    E = floor(log2 amax) (read from frexp, not a log); scale byte =
    clamp(E - 2 + 127, 0, 254), 2 being the largest E2M1 exponent; each
    element x / 2**(byte-127) is rounded by ``e2m1_code_rne_sat``; the sign
    bit is x's sign bit, so a negative value that rounds to zero is code 8.
    A block of zeros gets scale byte 0. Packing is low nibble first as in
    [Q0508] "Script update" item 2.

    Reading (the pages give no quantiser): the OCP MX v1.0 shared-exponent
    rule. Keeping -0 is supported by [Q0508] "FP4 (E2M1) expert weight format
    confirmed": -0 is about as common as +0 in real weights, which a producer
    that flushed -0 to +0 would not give.

    A block holding an infinity or a NaN has no finite shared exponent: it gets
    the E8M0 NaN byte 0xFF, so that it dequantises to NaN and the NaN travels on
    (reading: 0xFF is the NaN of the format named ``e8m0fnu`` on the pages);
    the oracle writes zero codes for such a block (the codes do not matter).
    """
    x = bf16_to_f64(x_bits)
    if x.ndim != 2 or x.shape[1] % 32 != 0:
        raise ValueError("mxfp4_quantize wants [R, C] with C % 32 == 0")
    R, C = x.shape
    blk = x.reshape(R, C // 32, 32)
    bad = ~np.isfinite(blk).all(axis=2)
    blk = np.where(bad[..., None], 0.0, blk)
    amax = np.abs(blk).max(axis=2)
    _, e = np.frexp(amax)
    biased = np.clip((e - 1) - 2 + 127, 0, 254)
    biased = np.where(amax == 0, 0, biased).astype(np.int64)
    v = blk / np.ldexp(1.0, biased - 127)[..., None]
    nib = e2m1_code_rne_sat(np.abs(v)) | (np.signbit(blk).astype(np.uint8) << 3)
    nib = np.where(bad[..., None], 0, nib).astype(np.uint8)
    biased = np.where(bad, 255, biased)
    return _pack_nibbles(nib.reshape(R, C)), biased.astype(np.uint8)


def e4m3_encode_exact(val):
    """Exact E4M3 value (fp64, finite, |v| <= 448) -> byte."""
    v = np.asarray(val, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)
    E = e - 1
    normal = a >= 2.0 ** -6
    with np.errstate(invalid="ignore", divide="ignore"):
        mant_n = np.rint(a / np.ldexp(1.0, E) * 8.0 - 8.0)
        ef = np.where(normal, E + 7, 0)
        mf = np.where(normal, mant_n, np.rint(a / 2.0 ** -9))
    if np.any(np.abs(np.where(normal, (1 + mf / 8) * np.ldexp(1.0, ef - 7), mf * 2.0 ** -9) - a) > 0):
        raise ValueError("value is not exactly representable in E4M3")
    return ((np.signbit(v).astype(np.int64) << 7) | (ef.astype(np.int64) << 3)
            | mf.astype(np.int64)).astype(np.uint8)


def e4m3_rne_satfinite(r):
    """fp32 r >= 0 -> (E4M3 byte, its value fp64): nearest, ties to even, clamp to 448.

    Reading (NVFP4 is never defined on the pages; see ``nvfp4_quantize``;
    the MXFP8 activation quantiser uses it too): round-to-nearest-even on the
    E4M3 grid (quantum 2**(E-3) in binade E,
    2**-9 below 2**-6), and any result above 448 saturates to 448.
    """
    r = np.asarray(r, dtype=np.float32).astype(np.float64)
    if np.any(~np.isfinite(r)) or np.any(r < 0):
        raise ValueError("e4m3_rne_satfinite wants finite r >= 0")
    _, e = np.frexp(r)
    q_exp = np.maximum(e - 1, -6) - 3
    val = np.minimum(np.rint(np.ldexp(r, -q_exp)) * np.ldexp(1.0, q_exp), 448.0)
    return e4m3_encode_exact(val), val


def mxfp8_quantize(x_bits):
    """bf16 [R, C] -> (E4M3 codes uint8 [R, C], E8M0 uint8 [R, C/32]).

    The activation side of the FP8 block-scaled linear (``fp8_block_linear``).
    Per row and 32-column block: amax = max |x|; shared exponent
    E = floor(log2 amax) (from frexp); scale byte = clamp(E - 8 + 127, 0, 254),
    8 being the largest E4M3 exponent; each element x / 2**(byte-127) (exact)
    is rounded to the nearest E4M3 value, ties to the even code, magnitudes
    above 448 saturating to 448 (they reach up to 512 under this scale); the
    sign bit is x's, so a negative value that rounds to zero is byte 0x80. A
    block of zeros gets scale byte 0.

    Reading: the pages name the FP8 linear of the shared expert but never its
    activation quantiser. The plainest one that the rest supports is the rule
    already taken for the MXFP4 activations (OCP shared exponent, round to
    nearest even, saturate) with E4M3 elements and 32-column E8M0 blocks.
    A block holding an infinity or a NaN gets scale byte 0xFF (NaN) and zero
    codes, as in ``mxfp4_quantize``.
    """
    x = bf16_to_f64(x_bits)
    if x.ndim != 2 or x.shape[1] % 32 != 0:
        raise ValueError("mxfp8_quantize wants [R, C] with C % 32 == 0")
    R, C = x.shape
    blk = x.reshape(R, C // 32, 32)
    bad = ~np.isfinite(blk).all(axis=2)
    blk = np.where(bad[..., None], 0.0, blk)
    amax = np.abs(blk).max(axis=2)
    _, e = np.frexp(amax)
    biased = np.clip((e - 1) - 8 + 127, 0, 254)
    biased = np.where(amax == 0, 0, biased).astype(np.int64)
    v = blk / np.ldexp(1.0, biased - 127)[..., None]
    mag, _ = e4m3_rne_satfinite(np.abs(v))
    codes = (mag & 0x7F) | (np.signbit(blk).astype(np.uint8) << 7)
    codes = np.where(bad[..., None], 0, codes)
    biased = np.where(bad, 255, biased)
    return codes.reshape(R, C).astype(np.uint8), biased.astype(np.uint8)


def mxfp8_dequant_f64(codes, scales):
    """E4M3 codes [R, C] with one E8M0 byte per 32 columns -> fp64 [R, C]."""
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    if scales.shape != (codes.shape[0], codes.shape[1] // 32):
        raise ValueError(f"scales {scales.shape} do not match codes {codes.shape}")
    return e4m3_decode(codes) * np.repeat(e8m0_decode(scales), 32, axis=1)


def nvfp4_quantize(x_bits, g):
    """bf16 [R, C] + fp32 global g -> (codes [R, C/2], E4M3 scales [R, C/16]).

    The pages run NVFP4 (global scales named weight_scale_2 / input_scale,
    a warm-up global "gs": [BUG0518] "Revised Plan", Phase 1 and Phase 2) but
    never define it. Reading: 16-element blocks, an E4M3 block scale and an
    fp32 global scale g, every step an IEEE fp32 round-to-nearest-even op:
        t = f32(6 * g); r = f32(amax / t); s = E4M3_RNE_satfinite(r)
        s == 0 -> all codes +-0
        d = f32(s * g); v = f32(x / d); code = E2M1_RNE_sat(|v|), sign of x
    Dequant is code * s * g. A block holding an infinity or a NaN gets the
    E4M3 NaN byte 0x7F and zero codes, so that it dequantises to NaN.
    """
    g = np.float32(g)
    if not (np.isfinite(g) and g > 0 and g >= np.finfo(np.float32).tiny * 2 ** 9):
        raise ValueError("NVFP4 global scale must be finite, positive and normal")
    x = bf16_to_f32(x_bits)
    if x.ndim != 2 or x.shape[1] % 16 != 0:
        raise ValueError("nvfp4_quantize wants [R, C] with C % 16 == 0")
    R, C = x.shape
    blk = x.reshape(R, C // 16, 16)
    bad = ~np.isfinite(blk).all(axis=2)
    blk = np.where(bad[..., None], np.float32(0.0), blk).astype(np.float32)
    amax = np.abs(blk).max(axis=2)
    t = np.float32(np.float32(6.0) * g)
    r = (amax / t).astype(np.float32)
    sbyte, sval = e4m3_rne_satfinite(r)
    d = (sval.astype(np.float32) * g).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (blk / d[..., None]).astype(np.float32)
    mag = e2m1_code_rne_sat(np.abs(v.astype(np.float64)))
    mag = np.where((sval == 0)[..., None], 0, mag).astype(np.uint8)
    nib = mag | (np.signbit(blk).astype(np.uint8) << 3)
    nib = np.where(bad[..., None], 0, nib).astype(np.uint8)
    sbyte = np.where(bad, 0x7F, sbyte).astype(np.uint8)
    return _pack_nibbles(nib.reshape(R, C)), sbyte


def nvfp4_dequant_f64(codes, scales, g):
    """NVFP4 codes [R, C/2] + E4M3 [R, C/16] + g -> fp64 code * s * g."""
    n = mxfp4_unpack(codes)
    R, C = n.shape
    s = np.asarray(scales)
    if s.shape != (R, C // 16):
        raise ValueError("NVFP4 scale shape mismatch")
    return E2M1_LUT[n] * np.repeat(e4m3_decode(s), 16, axis=1) * np.float64(np.float32(g))


def nvfp4_warmup_global(h_bits):
    """Global scale from a warm-up pass: f32(max |h| / (6 * 448)).

    [BUG0518] "Revised Plan", Phase 1 plans a warm-up based global scale for
    the shared-expert runner. Reading: the usual choice that maps the tensor
    amax onto the largest E2M1 value times the largest E4M3 scale.
    """
    a = np.abs(bf16_to_f64(h_bits)).max()
    return np.float32(a / (6.0 * 448.0)) if a > 0 else np.float32(1.0)


# ---------------------------------------------------------------------------
# The expert MLP
# ---------------------------------------------------------------------------

def gemm_f64(a, b):
    """C = A @ B^T in fp64 (BLAS dgemm). A [M, K], B [N, K]."""
    return np.asarray(a, np.float64) @ np.asarray(b, np.float64).T


def fp8_block_linear(x_bits, w, w_s, block=128):
    """y = bf16(MXFP8(x) . W^T): the FP8 linear of the original checkpoint's shared expert.

    W is FP8 E4M3 [N, K] with one E8M0 scale per 128 x 128 tile
    (``fp8_block_dequant_f64``), as the checkpoint stores the shared experts
    ([Q0508] "Status": FP8 float8_e4m3fn with float8_e8m0fnu scales) and as
    the serving stack runs them through an FP8 block-scaled GEMM ([SRV0511]
    "Architecture Map": shared expert on the FP8 linear; "What We Fixed"
    item 1: 128 x 128 blocks with E8M0 scales). x is quantised by
    ``mxfp8_quantize`` (reading there), the product is fp64 (BLAS dgemm),
    the result rounded once to bf16.
    """
    xq, xs = mxfp8_quantize(x_bits)
    a = mxfp8_dequant_f64(xq, xs)
    b = fp8_block_dequant_f64(w, w_s, block)
    return f64_to_bf16(gemm_f64(a, b))


def silu_mul_bf16(g, u):
    """h = bf16_RNE(silu(g) * u), silu(g) = g / (1 + exp(-g)), all fp64.

    [BUG0518] "Revised Plan", Phase 1: the pipeline is L1 GEMM -> SiLU ->
    re-quant -> L2 GEMM; Phase 3 keeps the SiLU activation in BF16.
    Reading: g and u are not rounded before the SiLU; h is rounded to bf16
    once.
    """
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return f64_to_bf16(g / (1.0 + np.exp(-g)) * np.asarray(u, np.float64))


def _requant(h_bits, requant, nv_global):
    if requant == "mxfp4":
        hq, hs = mxfp4_quantize(h_bits)
        return hq, hs, mxfp4_dequant_f64(hq, hs)
    if requant == "nvfp4":
        hq, hs = nvfp4_quantize(h_bits, nv_global)
        return hq, hs, nvfp4_dequant_f64(hq, hs, nv_global)
    raise ValueError(requant)


def expert_mlp(x_bits, w1, w1s, w3, w3s, w2, w2s, requant="mxfp4", nv_global=None,
               intermediates=False):
    """One expert (the shared expert): y = bf16(L2(requant(bf16(silu(x W1^T) * (x W3^T))))).

    [BUG0518] "Revised Plan", Phase 1: the shared expert is the MoE expert
    pipeline with one expert and no routing: L1 gate/up GEMM, SiLU, re-quant,
    L2 down GEMM. The activations are quantised to MXFP4 before L1 (the
    per-32 E8M0 shared-exponent rule of ``mxfp4_quantize``). Weights are the
    MXFP4 layout of [Q0508] "FP4 (E2M1) expert weight format confirmed":
    w1, w3 [I, H/2] + [I, H/32]; w2 [H, I/2] + [H, I/32].
    Returns y as bf16 bits [M, H]; with ``intermediates`` also a dict holding
    the quantised x, g, u (fp64), h (bf16 bits), its re-quantised codes and
    scales and the unrounded fp64 L2 output.
    """
    xq, xs = mxfp4_quantize(x_bits)
    a = mxfp4_dequant_f64(xq, xs)
    g = gemm_f64(a, mxfp4_dequant_f64(w1, w1s))
    u = gemm_f64(a, mxfp4_dequant_f64(w3, w3s))
    h = silu_mul_bf16(g, u)
    hq, hs, hd = _requant(h, requant, nv_global)
    y64 = gemm_f64(hd, mxfp4_dequant_f64(w2, w2s))
    y = f64_to_bf16(y64)
    if intermediates:
        return y, dict(xq=xq, xs=xs, g=g, u=u, h=h, hq=hq, hs=hs, y64=y64)
    return y


def grouped_expert_mlp(x_bits, topk_ids, topk_w, w1, w1s, w3, w3s, w2, w2s,
                       requant="mxfp4", nv_global=None, tokens=None, intermediates=False):
    """Routed experts: y[t] = bf16(sum_k w[t,k] * expert_{ids[t,k]}(x[t])).

    x is quantised once per token. Each (token, slot) pair whose id lies in
    [0, E) runs the single-expert pipeline (``expert_mlp`` without its final
    rounding); the weighted sum is fp64 and rounded to bf16 once. Ids outside
    [0, E) are skipped (the expert lives elsewhere). The routed MoE runs the
    same L1 -> SiLU -> re-quant -> L2 pipeline as the shared expert with
    routing, top-k and scatter added ([BUG0518] "Revised Plan", Phase 1;
    48 experts per rank in "Config values"). Router and top-k selection are
    inputs. ``tokens`` restricts the work to a subset of token indices
    (rows of the result are in that order). With ``intermediates`` also a dict
    per expert with pairs: the (token, slot) indices of its pairs in row-major
    order of ``topk_ids`` and their re-quantised h (codes and scales).
    """
    x_bits = np.asarray(x_bits)
    ids = np.asarray(topk_ids).astype(np.int64)
    wts = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        x_bits, ids, wts = x_bits[tokens], ids[tokens], wts[tokens]
    T, k = ids.shape
    E = w1.shape[0]
    H = x_bits.shape[1]
    xq, xs = mxfp4_quantize(x_bits)
    a = mxfp4_dequant_f64(xq, xs)
    acc = np.zeros((T, H), dtype=np.float64)
    inter = {}
    for e in range(E):
        t_idx, k_idx = np.nonzero(ids == e)
        if t_idx.size == 0:
            continue
        ae = a[t_idx]
        g = gemm_f64(ae, mxfp4_dequant_f64(w1[e], w1s[e]))
        u = gemm_f64(ae, mxfp4_dequant_f64(w3[e], w3s[e]))
        h = silu_mul_bf16(g, u)
        hq, hs, hd = _requant(h, requant, nv_global)
        y_pair = gemm_f64(hd, mxfp4_dequant_f64(w2[e], w2s[e]))
        np.add.at(acc, t_idx, wts[t_idx, k_idx][:, None] * y_pair)
        if intermediates:
            inter[e] = dict(t_idx=t_idx, k_idx=k_idx, hq=hq, hs=hs)
    y = f64_to_bf16(acc)
    return (y, inter) if intermediates else y


def fp8_expert_mlp(x_bits, w1, w1s, w3, w3s, w2, w2s):
    """The shared expert in the original checkpoint's FP8 format: three FP8 block-
    scaled linears around SiLU * up.

    g = fp8_block_linear(x, W1), u = fp8_block_linear(x, W3) (bf16 outputs),
    h = bf16(silu(g) * u) evaluated in fp64 from those bf16 values, and
    y = fp8_block_linear(h, W2). W1, W3 [inter, hidden] and W2 [hidden, inter]
    are FP8 E4M3 with 128 x 128 E8M0 block scales ([Q0508] "Status": the
    shared experts are FP8; [SRV0511] "Architecture Map": they run on the FP8
    linear). The MLP steps are those of [BUG0518] "Revised Plan", Phase 1.
    Reading: each linear rounds its output to bf16, as a standalone FP8 linear
    does, so g and u are bf16 before the SiLU here (unlike the fused MXFP4
    epilogue); h is re-quantised by the linear's MXFP8 activation quantiser.
    """
    g = fp8_block_linear(x_bits, w1, w1s)
    u = fp8_block_linear(x_bits, w3, w3s)
    h = silu_mul_bf16(bf16_to_f64(g), bf16_to_f64(u))
    return fp8_block_linear(h, w2, w2s)


def nvfp4_linear(x_bits, w, w_s, w_global, x_global):
    """y = bf16(NVFP4(x) . W^T) for NVFP4 weights: the GEMM of the routed experts
    as the pages run them on B200 (MoE w13/w2 in NVFP4: [SRV0511] "Architecture
    Map"; per-matrix global scales weight_scale_2 and the activations' input
    scale: [BUG0518] "Revised Plan", Phase 2).

    W: E2M1 codes [N, K/2] (low nibble first) with one E4M3 scale per 16
    columns [N, K/16] and the fp32 global w_global; x is quantised by
    ``nvfp4_quantize`` with the fp32 global x_global. Reading: the weight
    format is the NVFP4 reading of ``nvfp4_quantize`` (R7) applied to the
    weights, value = code * s * w_global. Product in fp64, rounded once to bf16.
    """
    xq, xs = nvfp4_quantize(x_bits, x_global)
    a = nvfp4_dequant_f64(xq, xs, x_global)
    b = nvfp4_dequant_f64(w, w_s, w_global)
    return f64_to_bf16(gemm_f64(a, b))


def nvfp4_expert_mlp(x_bits, w1, w1s, g1, w3, w3s, g3, w2, w2s, g2, x_global, h_global):
    """One expert with NVFP4 weights: gate and up NVFP4 linears with their own
    weight globals g1, g3 (the pages' dual gate/up weight_scale_2, [BUG0518]
    "Revised Plan", Phase 2) over x quantised with x_global, h = bf16(silu(g) *
    u) from their bf16 outputs, h quantised to NVFP4 with h_global, and the down
    NVFP4 linear with g2. Reading: as for ``fp8_expert_mlp``, each linear
    rounds its output to bf16."""
    g = nvfp4_linear(x_bits, w1, w1s, g1, x_global)
    u = nvfp4_linear(x_bits, w3, w3s, g3, x_global)
    h = silu_mul_bf16(bf16_to_f64(g), bf16_to_f64(u))
    return nvfp4_linear(h, w2, w2s, g2, h_global)


def grouped_nvfp4_expert_mlp(x_bits, topk_ids, topk_w, w1, w1s, g1, w3, w3s, g3, w2, w2s, g2, x_global,
                             h_global, tokens=None):
    """Routed experts with NVFP4 weights, as the pages run the MoE on B200 (w13/w2
    in NVFP4 with per-expert weight_scale_2: [SRV0511] "Architecture Map",
    [BUG0518] "Revised Plan", Phase 2): y[t] = bf16(sum_k w[t,k] *
    expert_{ids[t,k]}(x[t])). Each pair runs the steps of ``nvfp4_expert_mlp``
    with its expert's globals g1[e], g3[e], g2[e] (arrays of E fp32); the
    down product is kept in fp64 and the weighted sum rounded to bf16 once, as
    in ``grouped_expert_mlp``. Ids outside [0, E) are skipped; ``tokens``
    restricts the work to those token indices."""
    x_bits = np.asarray(x_bits)
    ids = np.asarray(topk_ids).astype(np.int64)
    wts = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        x_bits, ids, wts = x_bits[tokens], ids[tokens], wts[tokens]
    T, k = ids.shape
    E = w1.shape[0]
    H = x_bits.shape[1]
    acc = np.zeros((T, H), dtype=np.float64)
    for e in range(E):
        t_idx, k_idx = np.nonzero(ids == e)
        if t_idx.size == 0:
            continue
        xe = x_bits[t_idx]
        g = nvfp4_linear(xe, w1[e], w1s[e], g1[e], x_global)
        u = nvfp4_linear(xe, w3[e], w3s[e], g3[e], x_global)
        h = silu_mul_bf16(bf16_to_f64(g), bf16_to_f64(u))
        hq, hs = nvfp4_quantize(h, h_global)
        y_pair = gemm_f64(nvfp4_dequant_f64(hq, hs, h_global), nvfp4_dequant_f64(w2[e], w2s[e], g2[e]))
        np.add.at(acc, t_idx, wts[t_idx, k_idx][:, None] * y_pair)
    return f64_to_bf16(acc)

