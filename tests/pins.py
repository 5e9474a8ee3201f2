"""Checks that pin the oracle to facts outside itself.

Each ``check_*`` function takes the oracle module (so the mutation tests can
hand it a deliberately broken copy) and raises AssertionError on a mismatch.
The expected values come from the pages (golden fixtures under
``tests/golden``, each citing its passage), from closed forms, from brute
force over tiny inputs, or from independent library routines; none of them
re-types the oracle's own formula.
"""

from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln.split()


def _same(a, b):
    """Equal as floats, with -0 != +0 and nan == nan."""
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def bf16_value(bits):
    """bf16 bits -> Python float via struct (independent of the oracle)."""
    import struct
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


# ---------------------------------------------------------------------------
# Element formats
# ---------------------------------------------------------------------------

def check_e2m1_formula(O):
    """The table equals the general minifloat formula for (s, e, m) = (1, 2, 1), bias 1."""
    for n in range(16):
        s, e, m = n >> 3, (n >> 1) & 3, n & 1
        mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        want = -mag if s else mag
        got = float(O.e2m1_decode(np.array([n]))[0])
        assert _same(got, want), (n, got, want)


def check_nibble8_negative_zero(O):
    v = float(O.e2m1_decode(np.array([8]))[0])
    assert v == 0.0 and math.copysign(1.0, v) < 0, v
    v0 = float(O.e2m1_decode(np.array([0]))[0])
    assert v0 == 0.0 and math.copysign(1.0, v0) > 0, v0


def check_e8m0(O):
    b = np.arange(256)
    got = O.e8m0_decode(b.astype(np.uint8))
    for i in range(255):
        assert got[i] == math.ldexp(1.0, i - 127), i
    assert math.isnan(got[255])
    assert got[127] == 1.0


def _e4m3_fraction(b):
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    if e == 15 and m == 7:
        return None
    mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if s else mag


def e4m3_values():
    """The 256 E4M3fn code values from the bit-field definition (NaN for 0x7F, 0xFF)."""
    return np.array([float("nan") if _e4m3_fraction(b) is None else float(_e4m3_fraction(b))
                     for b in range(256)])


def check_e4m3(O):
    got = O.e4m3_decode(np.arange(256).astype(np.uint8))
    finite = 0
    for b in range(256):
        want = _e4m3_fraction(b)
        if want is None:
            assert math.isnan(got[b]), b
            continue
        finite += 1
        assert Fraction(float(got[b])) == want, (b, got[b], want)
        if want == 0:
            assert math.copysign(1.0, got[b]) == (-1.0 if b & 0x80 else 1.0)
    assert finite == 254
    assert np.nanmax(got) == 448.0
    assert got[1] == 2.0 ** -9


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

def _bf16_table():
    """All finite non-negative bf16 values, sorted, with their bit patterns."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    return vals, bits


def bf16_rne_reference(x):
    """Nearest bf16 by table search over all values (ties to even pattern)."""
    vals, bits = _bf16_table()
    out = np.empty(len(x), dtype=np.uint16)
    max_fin = vals[-1]
    half_ulp_top = (vals[-1] - vals[-2]) / 2
    for i, xv in enumerate(x):
        if math.isnan(xv):
            out[i] = 0x7FC0
            continue
        a = abs(xv)
        sign = 0x8000 if math.copysign(1.0, xv) < 0 else 0
        if a >= max_fin + half_ulp_top:
            out[i] = sign | 0x7F80
            continue
        j = int(np.searchsorted(vals, a))
        cands = [c for c in (j - 1, j) if 0 <= c < len(vals)]
        d = [abs(Fraction(vals[c]) - Fraction(a)) for c in cands]
        best = min(d)
        win = [c for c, dd in zip(cands, d) if dd == best]
        c = win[0] if len(win) == 1 else [w for w in win if bits[w] % 2 == 0][0]
        out[i] = sign | int(bits[c])
    return out


def check_bf16_roundtrip(O):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    back = O.f64_to_bf16(O.bf16_to_f64(bits))
    e = (bits.astype(np.int64) >> 7) & 0xFF
    m = bits.astype(np.int64) & 0x7F
    isnan = (e == 0xFF) & (m != 0)
    assert np.array_equal(back[~isnan], bits[~isnan])
    assert np.all(back[isnan] == 0x7FC0)


def check_bf16_rounding_random(O, n=4000, seed=5):
    rng = np.random.default_rng(seed)
    x = np.concatenate([
        rng.standard_normal(n // 4) * 10.0 ** rng.integers(-40, 39, n // 4),
        # exact half-way points and their neighbours in fp64
        _midpoints(rng, n // 4),
        rng.standard_normal(n // 4) * 2.0 ** -130,                 # subnormal range
        rng.uniform(3.0e38, 3.5e38, n // 4) * rng.choice([-1, 1], n // 4),  # overflow edge
    ])
    got = O.f64_to_bf16(x)
    want = bf16_rne_reference(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(x[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def _midpoints(rng, n):
    b = rng.integers(0, 0x7F7F, n).astype(np.uint32)
    lo = (b << 16).view(np.float32).astype(np.float64)
    hi = ((b + 1) << 16).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2
    nudge = rng.choice([-1, 0, 1], n)
    return np.where(nudge == 0, mid, np.nextafter(mid, mid + nudge)) * rng.choice([-1, 1], n)


def check_no_double_rounding(O):
    """A value just above a bf16 midpoint must round up even though fp32 would hit the midpoint."""
    lo = 1.0
    ulp = 2.0 ** -7
    x = lo + ulp / 2 + 2.0 ** -40          # fp32(x) == 1 + ulp/2 exactly, a tie -> even (down)
    assert float(np.float32(x)) == lo + ulp / 2
    got = int(O.f64_to_bf16(np.array([x]))[0])
    assert got == 0x3F81, hex(got)


# ---------------------------------------------------------------------------
# Dequantisation
# ---------------------------------------------------------------------------

def check_format_shapes(O):
    """Logical width = 2 x stored bytes; one scale per 32 columns (the pages' shapes)."""
    rows_used = 2
    for parts in _lines("mxfp4_format_facts.txt"):
        if parts[0].startswith("nibble"):
            continue
        name, pr, pc, sr, sc, lr, lc = parts
        pc, sc, lc = int(pc), int(sc), int(lc)
        assert int(pr) == int(sr) == int(lr)
        codes = np.zeros((rows_used, pc), np.int8)
        scales = np.full((rows_used, sc), 127, np.uint8)
        out = O.mxfp4_dequant_bf16(codes, scales)
        assert out.shape == (rows_used, lc), (name, out.shape, lc)
        assert sc * 32 == lc


def check_dequant_examples(O):
    for hb, sb, v0, v1 in _lines("mxfp4_dequant_examples.txt"):
        byte, scale = int(hb, 16), int(sb)
        codes = np.full((1, 16), 0, np.uint8)
        codes[0, 3] = byte
        scales = np.full((1, 1), scale, np.uint8)
        out = O.mxfp4_dequant_bf16(codes, scales)
        got = (bf16_value(out[0, 6]), bf16_value(out[0, 7]))
        assert _same(got[0], float(v0)) and _same(got[1], float(v1)), (hb, sb, got, v0, v1)
        # int8 storage of the same byte (what the checkpoint holds)
        out8 = O.mxfp4_dequant_bf16(codes.view(np.int8), scales)
        assert np.array_equal(out8, out), hb


def check_dequant_scale_columns(O):
    """Scale j covers logical columns 32j..32j+31 of its own row."""
    codes = np.full((2, 64), 0x22, np.uint8)        # every element 1.0
    scales = np.array([[127, 129, 126, 130], [128, 120, 127, 127]], np.uint8)
    out = O.mxfp4_dequant_f64(codes, scales)
    for r in range(2):
        for c in range(128):
            assert out[r, c] == 2.0 ** (int(scales[r, c // 32]) - 127), (r, c)


def check_dequant_all_bytes(O):
    """Every byte at several scales, against per-element Python arithmetic."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    codes = np.arange(256, dtype=np.uint8).reshape(16, 16)
    for s in (1, 60, 120, 127, 133, 200, 253):
        scales = np.full((16, 1), s, np.uint8)
        out = O.mxfp4_dequant_f64(codes, scales)
        for b in range(256):
            lo, hi = b & 15, b >> 4
            for nib, col in ((lo, 2 * (b % 16)), (hi, 2 * (b % 16) + 1)):
                mag = grid[nib & 7]
                want = math.ldexp(-mag if nib & 8 else mag, s - 127)
                assert _same(float(out[b // 16, col]), want), (b, s, nib)


def check_fp8_examples(O):
    for hc, sb, v in _lines("fp8_block_dequant_examples.txt"):
        q = np.zeros((1, 1), np.uint8)
        q[0, 0] = int(hc, 16)
        s = np.full((1, 1), int(sb), np.uint8)
        got = bf16_value(O.fp8_block_dequant_bf16(q, s)[0, 0])
        assert _same(got, float(v)), (hc, sb, got, v)


def check_fp8_block_bruteforce(O, R=200, C=300, seed=3):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, (R, C)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38
    s = rng.integers(118, 135, (2, 3)).astype(np.uint8)
    out = O.fp8_block_dequant_f64(q, s)
    for i in range(0, R, 7):
        for j in range(0, C, 5):
            want = _e4m3_fraction(int(q[i, j])) * Fraction(2) ** (int(s[i // 128, j // 128]) - 127)
            assert Fraction(float(out[i, j])) == want, (i, j)


# ---------------------------------------------------------------------------
# Quantisation
# ---------------------------------------------------------------------------

def e2m1_bruteforce(a):
    """Nearest grid index for |v| values; ties -> even index; beyond 6 -> 7."""
    a = np.asarray(a, np.float64)
    g = np.array(E2M1_GRID)
    d = np.abs(a[:, None] - g[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    pick_even = even.any(axis=1) & (cand.sum(axis=1) > 1)
    first = cand.argmax(axis=1)
    first_even = even.argmax(axis=1)
    return np.where(pick_even, first_even, first)


def check_quantize_examples(O):
    blocks, scales = {}, {}
    for parts in _lines("mxfp4_quantize_examples.txt"):
        if parts[0] == "scale":
            scales[int(parts[1])] = int(parts[2])
        else:
            blocks.setdefault(int(parts[0]), []).append((float(parts[1]), int(parts[2])))
    for bid, items in blocks.items():
        vals = [v for v, _ in items] + [0.0] * (32 - len(items))
        x = np.array(vals, np.float32).reshape(1, 32)
        bits = (x.view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), x)
        codes, sc = O.mxfp4_quantize(bits)
        assert int(sc[0, 0]) == scales[bid], (bid, int(sc[0, 0]))
        nib = np.empty(32, np.int64)
        nib[0::2] = codes[0] & 15
        nib[1::2] = codes[0] >> 4
        for i, (_, want) in enumerate(items):
            assert nib[i] == want, (bid, i, items[i], nib[i])


def _quantize_sweep(O, anchor_bits, cand_bits):
    """Blocks [anchor, 31 candidates]; compare codes with brute force."""
    anchor = bf16_value(anchor_bits)
    n = len(cand_bits)
    pad = (-n) % 31
    cb = np.concatenate([cand_bits, np.zeros(pad, np.uint16)])
    blocks = cb.reshape(-1, 31)
    x = np.concatenate([np.full((blocks.shape[0], 1), anchor_bits, np.uint16), blocks], axis=1)
    codes, sc = O.mxfp4_quantize(x)
    # independent scale: floor(log2 anchor) from math.frexp, minus 2, biased, clamped
    if anchor == 0:
        want_byte = 0
    else:
        _, ex = math.frexp(abs(anchor))
        want_byte = min(max(ex - 1 - 2 + 127, 0), 254)
    assert np.all(sc == want_byte), (anchor, np.unique(sc), want_byte)
    X = math.ldexp(1.0, want_byte - 127)
    vals = ((x.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
    want = e2m1_bruteforce(np.abs(vals.ravel()) / X).reshape(x.shape)
    want = want | (np.signbit(vals).astype(np.int64) << 3)
    nib = np.empty(x.shape, np.int64)
    nib[:, 0::2] = codes & 15
    nib[:, 1::2] = codes >> 4
    bad = np.argwhere(nib != want)
    assert bad.size == 0, [(vals[i, j], nib[i, j], want[i, j], want_byte) for i, j in bad[:5]]


def check_quantize_exhaustive(O):
    """Every finite bf16 pattern as a block element, at every binade of the block amax."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    e = (allbits >> 7) & 0xFF
    finite = allbits[e != 0xFF]
    mags = finite & 0x7FFF
    # full sweep at the largest anchor and at a subnormal anchor (scale byte 0)
    _quantize_sweep(O, np.uint16(0x7F7F), finite)
    _quantize_sweep(O, np.uint16(0x007F), finite[mags <= 0x007F])
    # every binade of the anchor, candidates within 2**-12 of the anchor
    for ea in range(1, 255):
        abits = np.uint16((ea << 7) | 0x7F)
        lo = max(ea - 12, 0) << 7
        sel = finite[(mags <= int(abits)) & (mags >= lo)]
        _quantize_sweep(O, abits, sel)


def check_quantize_roundtrip(O, seed=11):
    rng = np.random.default_rng(seed)
    R, C = 64, 256
    codes = rng.integers(0, 256, (R, C // 2)).astype(np.uint8)
    # force every block's max |code| into {4, 6}: set one element per block
    nib = np.empty((R, C), np.uint8)
    nib[:, 0::2] = codes & 15
    nib[:, 1::2] = codes >> 4
    nb = nib.reshape(R, C // 32, 32)
    nb[:, :, 0] = rng.choice([6, 7, 14, 15], size=(R, C // 32))
    nib = nb.reshape(R, C)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(3, 250, (R, C // 32)).astype(np.uint8)
    deq = O.mxfp4_dequant_bf16(codes, scales)
    q2, s2 = O.mxfp4_quantize(deq)
    assert np.array_equal(s2, scales)
    assert np.array_equal(q2, codes)
    # any codes: dequant(quant(dequant)) == dequant
    anyc = rng.integers(0, 256, (R, C // 2)).astype(np.uint8)
    d1 = O.mxfp4_dequant_bf16(anyc, scales)
    q3, s3 = O.mxfp4_quantize(d1)
    assert np.array_equal(O.mxfp4_dequant_bf16(q3, s3), d1)


def check_nibble_balance(O, seed=13):
    """Symmetric data gives as many -0 codes as +0 codes (the pages' 0.996 ratio)."""
    ratio_pages = None
    for parts in _lines("mxfp4_format_facts.txt"):
        if parts[0] == "nibble0_to_nibble8_ratio":
            ratio_pages = float(parts[1])
    assert ratio_pages is not None
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((512, 1024)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)   # truncation: sign-symmetric
    codes, _ = O.mxfp4_quantize(bits)
    lo, hi = codes & 15, codes >> 4
    n0 = int((lo == 0).sum() + (hi == 0).sum())
    n8 = int((lo == 8).sum() + (hi == 8).sum())
    assert n8 > 0
    ratio = n0 / n8
    assert abs(ratio - 1.0) < 0.05 and abs(ratio - ratio_pages) < 0.05, ratio


def check_e4m3_rne(O, seed=17):
    vals = sorted({_e4m3_fraction(b) for b in range(128) if _e4m3_fraction(b) is not None})
    rng = np.random.default_rng(seed)
    mids = [float((vals[i] + vals[i + 1]) / 2) for i in range(len(vals) - 1)]
    r = np.concatenate([
        np.array([float(v) for v in vals]), np.array(mids),
        rng.uniform(0, 500, 2000), rng.uniform(0, 2.0 ** -6, 500), np.array([464.0, 480.0, 1e30]),
    ]).astype(np.float32)
    byte, val = O.e4m3_rne_satfinite(r)
    for ri, bi, vi in zip(r, byte, val):
        rf = Fraction(float(ri))
        if rf >= 448:
            want = Fraction(448)
        else:
            d = [abs(v - rf) for v in vals]
            best = min(d)
            win = [i for i, dd in enumerate(d) if dd == best]
            if len(win) == 1:
                want = vals[win[0]]
            else:
                # ties: the even mantissa (even byte, since values ascend with the byte)
                bytes_ = [b for b in range(128) if _e4m3_fraction(b) in [vals[w] for w in win]]
                want = _e4m3_fraction([b for b in bytes_ if b % 2 == 0][0])
        assert Fraction(float(vi)) == want, (float(ri), float(vi), float(want))
        assert _e4m3_fraction(int(bi)) == want


def e4m3_bruteforce(a):
    """|v| values -> nearest non-negative E4M3 byte; ties to the even byte; above 448 -> 448.

    The grid comes from the bit-field definition (``_e4m3_fraction``)."""
    bytes_ = np.array([b for b in range(127)])
    grid = np.array([float(_e4m3_fraction(int(b))) for b in bytes_])
    a = np.asarray(a, np.float64)
    out = np.empty(a.shape, np.int64)
    for i0 in range(0, a.size, 4096):
        aa = a.ravel()[i0:i0 + 4096]
        d = np.abs(aa[:, None] - grid[None, :])
        best = d.min(axis=1, keepdims=True)
        cand = d == best
        even = cand & (bytes_[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1) & (cand.sum(axis=1) > 1), even.argmax(axis=1), cand.argmax(axis=1))
        pick = np.where(aa > 448.0, 126, pick)
        out.ravel()[i0:i0 + 4096] = bytes_[pick]
    return out


def _mxfp8_sweep(O, anchor_bits, cand_bits):
    """Blocks [anchor, 31 candidates]: scale byte and E4M3 codes against brute force."""
    anchor = bf16_value(anchor_bits)
    n = len(cand_bits)
    cb = np.concatenate([cand_bits, np.zeros((-n) % 31, np.uint16)])
    blocks = cb.reshape(-1, 31)
    x = np.concatenate([np.full((blocks.shape[0], 1), anchor_bits, np.uint16), blocks], axis=1)
    codes, sc = O.mxfp8_quantize(x)
    if anchor == 0:
        want_byte = 0
    else:
        _, ex = math.frexp(abs(anchor))
        want_byte = min(max(ex - 1 - 8 + 127, 0), 254)       # 8: largest E4M3 exponent
    assert np.all(sc == want_byte), (anchor, np.unique(sc), want_byte)
    X = math.ldexp(1.0, want_byte - 127)
    vals = ((x.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
    want = e4m3_bruteforce(np.abs(vals.ravel()) / X).reshape(x.shape)
    want = want | (np.signbit(vals).astype(np.int64) << 7)
    bad = np.argwhere(codes.astype(np.int64) != want)
    assert bad.size == 0, [(vals[i, j], codes[i, j], want[i, j], want_byte) for i, j in bad[:5]]


def check_mxfp8_quantize_exhaustive(O):
    """Every finite bf16 pattern as a block element of an MXFP8 block, for anchors
    in every binade (candidates within 2**-12 of the anchor, the rest round to 0)."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    e = (allbits >> 7) & 0xFF
    finite = allbits[e != 0xFF]
    mags = finite & 0x7FFF
    _mxfp8_sweep(O, np.uint16(0x7F7F), finite)
    _mxfp8_sweep(O, np.uint16(0x007F), finite[mags <= 0x007F])
    for ea in range(1, 255, 3):
        abits = np.uint16((ea << 7) | 0x55)
        lo = max(ea - 12, 0) << 7
        _mxfp8_sweep(O, abits, finite[(mags <= int(abits)) & (mags >= lo)])


def check_mxfp8_examples(O):
    """Hand-worked blocks: scale 2**(floor(log2 amax) - 8), saturation, kept sign of zero."""
    def q(vals):
        x = np.array(list(vals) + [0.0] * (32 - len(vals)), np.float32).reshape(1, 32)
        return O.mxfp8_quantize((x.view(np.uint32) >> 16).astype(np.uint16))
    c, s = q([1.0])                     # amax 1: X = 2**-8, 1 / X = 256 = 2**8 -> e 15, m 0
    assert int(s[0, 0]) == 119 and int(c[0, 0]) == 0x78 and int(c[0, 1]) == 0
    c, s = q([1.75, -1.0])              # 448 exactly; -256
    assert int(s[0, 0]) == 119 and int(c[0, 0]) == 0x7E and int(c[0, 1]) == 0xF8
    c, s = q([1.9375, 1.8125])          # 496 and 464 saturate to 448 (no NaN code)
    assert int(c[0, 0]) == 0x7E and int(c[0, 1]) == 0x7E
    c, s = q([1.0, -2.0 ** -20])        # -2**-12 under the scale: below half the subnormal step
    assert int(c[0, 1]) == 0x80
    c, s = q([1.0, 2.0 ** -16])         # 2**-8 = 2 * 2**-9: subnormal byte 2
    assert int(c[0, 1]) == 0x02
    c, s = q([0.0, -0.0])               # zero block: scale byte 0, signs kept
    assert int(s[0, 0]) == 0 and int(c[0, 0]) == 0 and int(c[0, 1]) == 0x80


def check_mxfp8_roundtrip(O, seed=47):
    """quant(dequant(c, s)) == (c, s) when a block's largest code lies in [256, 448];
    dequant(quant(dequant)) == dequant for any finite codes."""
    rng = np.random.default_rng(seed)
    R, C = 32, 256
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    codes = rng.choice(finite, size=(R, C)).astype(np.uint8)
    cb = codes.reshape(R, C // 32, 32)
    top = np.arange(0x78, 0x7F, dtype=np.uint8)
    cb[:, :, 0] = rng.choice(top, size=(R, C // 32)) | (rng.integers(0, 2, (R, C // 32)) << 7).astype(np.uint8)
    codes = cb.reshape(R, C)
    # the largest code must be the one forced into [256, 448]
    mag = codes.reshape(R, C // 32, 32) & 0x7F
    mag[:, :, 1:] = np.minimum(mag[:, :, 1:], mag[:, :, :1])
    codes = (mag.reshape(R, C) | (codes & 0x80)).astype(np.uint8)
    scales = rng.integers(20, 230, (R, C // 32)).astype(np.uint8)
    vals = np.array([float("nan") if _e4m3_fraction(b) is None else float(_e4m3_fraction(b)) for b in range(256)])
    deq = vals[codes] * np.ldexp(1.0, np.repeat(scales.astype(np.int64), 32, axis=1) - 127)
    bits = (deq.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(((bits.astype(np.uint32) << 16).view(np.float32)).astype(np.float64), deq)
    q2, s2 = O.mxfp8_quantize(bits)
    assert np.array_equal(s2, scales)
    nz = (codes & 0x7F) != 0
    assert np.array_equal(q2[nz], codes[nz])
    d2 = O.mxfp8_dequant_f64(q2, s2)
    assert np.array_equal(d2, deq)


def check_fp8_linear_bruteforce(O, seed=53):
    """FP8 linear on a ragged tiny shape (two 128-row scale blocks, the second
    partial; two K blocks) against exact Fractions from the bit fields, rounded
    by the table-search bf16 reference."""
    rng = np.random.default_rng(seed)
    M, N, K = 2, 130, 256
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    w = rng.choice(finite, size=(N, K)).astype(np.uint8)
    ws = rng.integers(118, 135, (2, 2)).astype(np.uint8)
    x = rng.standard_normal((M, K)).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    y = O.fp8_block_linear(xb, w, ws)
    xq, xs = O.mxfp8_quantize(xb)          # pinned by the MXFP8 checks
    P2 = [Fraction(2) ** (e - 127) for e in range(256)]
    wf = [[_e4m3_fraction(int(w[n, k])) * P2[int(ws[n // 128, k // 128])] for k in range(K)] for n in range(N)]
    want = []
    for m in range(M):
        xf = [_e4m3_fraction(int(xq[m, k])) * P2[int(xs[m, k // 32])] for k in range(K)]
        for n in range(N):
            want.append(float(sum(a * b for a, b in zip(xf, wf[n]))))
    ref = bf16_rne_reference(np.array(want)).reshape(M, N)
    assert np.array_equal(y, ref)


def check_fp8_linear_unit_rows(O):
    """x = unit rows e_k (exact in MXFP8): y = the bf16 FP8-block dequant of W's columns k."""
    rng = np.random.default_rng(59)
    N, K = 256, 384
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    w = rng.choice(finite, size=(N, K)).astype(np.uint8)
    ws = rng.integers(118, 135, (2, 3)).astype(np.uint8)
    ks = np.array([0, 5, 127, 128, 200, 383])
    x = np.zeros((len(ks), K), np.uint16)
    x[np.arange(len(ks)), ks] = 0x3F80                  # bf16 1.0
    y = O.fp8_block_linear(x, w, ws)
    deq = O.fp8_block_dequant_bf16(w, ws)               # pinned by the FP8 block checks
    # as values: a -0 weight times 1 plus the +0 products of the other columns is +0
    tof = lambda b: ((b.astype(np.uint32) << 16).view(np.float32))
    assert np.array_equal(tof(y), tof(np.ascontiguousarray(deq[:, ks].T)))


def check_nvfp4_grid(O, seed=19):
    """Exhaustive bf16 magnitudes against brute-force nearest grid at fixed (s, g)."""
    g = np.float32(0.0123)
    allbits = np.arange(0x7F80, dtype=np.uint32).astype(np.uint16)
    vals = (allbits.astype(np.uint32) << 16).view(np.float32)
    anchor_val = np.float32(5.75)                      # amax of every block
    anchor_bits = (np.array([anchor_val]).view(np.uint32) >> 16).astype(np.uint16)[0]
    keep = allbits[vals <= anchor_val]
    pad = (-len(keep)) % 15
    cand = np.concatenate([keep, np.zeros(pad, np.uint16)]).reshape(-1, 15)
    x = np.concatenate([np.full((cand.shape[0], 1), anchor_bits, np.uint16), cand], axis=1)
    codes, sbytes = O.nvfp4_quantize(x, g)
    # expected scale: E4M3 RNE of f32(5.75 / f32(6 g)) -- via the brute-force E4M3 table
    r = np.float32(anchor_val / np.float32(np.float32(6.0) * g))
    vals_e4 = sorted({_e4m3_fraction(b) for b in range(127)})
    rf = Fraction(float(r))
    s_want = min(vals_e4, key=lambda v: (abs(v - rf), 0))
    assert np.all(sbytes == sbytes[0, 0]) and Fraction(float(O.e4m3_decode(sbytes[:1, :1])[0, 0])) == s_want
    d = np.float32(np.float32(float(s_want)) * g)
    v = ((x.astype(np.uint32) << 16).view(np.float32) / d).astype(np.float32).astype(np.float64)
    want = e2m1_bruteforce(np.abs(v.ravel())).reshape(x.shape)
    nib = np.empty(x.shape, np.int64)
    nib[:, 0::2] = codes & 15
    nib[:, 1::2] = codes >> 4
    assert np.array_equal(nib, want)


def _f32_nearest(q):
    """The fp32 number nearest to the rational q > 0 (ties to the even
    significand), by exact comparison with Fractions."""
    v = np.float32(float(q))
    best = None
    for c in (np.nextafter(v, np.float32(0)), v, np.nextafter(v, np.float32(np.inf))):
        key = (abs(Fraction(float(c)) - q), int(np.array([c]).view(np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def check_nvfp4_warmup_global(O):
    """Warm-up global g = f32(max |h| / (6 * 448)): against the exact quotient
    rounded once to fp32, for every positive finite bf16 value as the maximum
    (signs and smaller entries must not matter), and g = 1 for all-zero h. The
    same values also equal an fp32 IEEE division of the bf16 value by 2688, the
    one-rounding form a device computes."""
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    for i in range(0, len(bits), 97):                   # a spread of maxima, exact
        b = int(bits[i])
        h = np.array([[b | 0x8000, b >> 1, 0, 0x8000]], np.uint16)   # -a, a smaller value, +0, -0
        assert O.nvfp4_warmup_global(h) == _f32_nearest(Fraction(float(vals[i])) / 2688), hex(b)
    ones = np.array([O.nvfp4_warmup_global(np.array([[b]], np.uint16)) for b in bits], np.float32)
    assert np.array_equal(ones, vals / np.float32(2688.0))
    assert O.nvfp4_warmup_global(np.zeros((3, 16), np.uint16)) == np.float32(1.0)
    assert O.nvfp4_warmup_global(np.full((2, 16), 0x8000, np.uint16)) == np.float32(1.0)


def check_nvfp4_error_bound(O, seed=23):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((64, 256)).astype(np.float32) * np.float32(3.0)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    xf = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g = np.float32(np.abs(xf).max() / (6 * 448))
    codes, sc = O.nvfp4_quantize(bits, g)
    deq = O.nvfp4_dequant_f64(codes, sc, g)
    s = np.repeat(O.e4m3_decode(sc), 16, axis=1) * float(g)
    # half of the widest grid step (2 at the top of the grid) in units of s*g,
    # plus the saturation overshoot when the E4M3 scale rounded down (<= 1/16 rel.)
    amax = np.repeat(np.abs(xf.reshape(64, -1, 16)).max(axis=2), 16, axis=1)
    bound = 1.0 * s + amax * (1 / 16) + 1e-30
    assert np.all(np.abs(deq - xf) <= bound)
    # relative RMS error is that of 4-bit floats (well under 10 %)
    rel = np.linalg.norm(deq - xf) / np.linalg.norm(xf)
    assert rel < 0.1, rel


# ---------------------------------------------------------------------------
# GEMM, SiLU, MLP
# ---------------------------------------------------------------------------

def check_gemm_integer(O, seed=29):
    """All scales 127: 2*E2M1 values are integers, so the fp64 GEMM equals int64 matmul / 4."""
    rng = np.random.default_rng(seed)
    M, N, K = 24, 40, 512
    a = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    b = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    s_a = np.full((M, K // 32), 127, np.uint8)
    s_b = np.full((N, K // 32), 127, np.uint8)
    C = O.gemm_f64(O.mxfp4_dequant_f64(a, s_a), O.mxfp4_dequant_f64(b, s_b))
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)

    def ints(c):
        n = np.empty((c.shape[0], 2 * c.shape[1]), np.int64)
        n[:, 0::2] = twice[c & 15]
        n[:, 1::2] = twice[c >> 4]
        return n
    Ci = ints(a) @ ints(b).T
    assert np.array_equal(C * 4, Ci.astype(np.float64))


def check_gemm_bruteforce(O, seed=31):
    rng = np.random.default_rng(seed)
    M, N, K = 4, 8, 64
    a = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    b = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sa = rng.integers(120, 131, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(120, 131, (N, K // 32)).astype(np.uint8)
    C = O.gemm_f64(O.mxfp4_dequant_f64(a, sa), O.mxfp4_dequant_f64(b, sb))

    def elem(c, s, r, k):
        byte = int(c[r, k // 2])
        nib = (byte >> 4) if k % 2 else (byte & 15)
        mag = E2M1_GRID[nib & 7]
        return Fraction(-mag if nib & 8 else mag) * Fraction(2) ** (int(s[r, k // 32]) - 127)
    for m in range(M):
        for n in range(N):
            want = sum(elem(a, sa, m, k) * elem(b, sb, n, k) for k in range(K))
            assert Fraction(float(C[m, n])) == want, (m, n)


def check_silu(O, seed=37):
    from scipy.special import expit
    rng = np.random.default_rng(seed)
    g = np.concatenate([rng.standard_normal(3000) * 4, [0.0, -0.0, 40.0, 80.0, -40.0, -800.0]])
    u = rng.standard_normal(g.size) * 3
    got = O.silu_mul_bf16(g, u)
    want = O.f64_to_bf16(expit(g) * g * u)
    # fp64 results agree to ~1 ulp, so the bf16 roundings agree except at exact ties
    assert np.mean(got == want) > 0.999
    gv = np.array([bf16_value(b) for b in got])
    wv = np.array([bf16_value(b) for b in want])
    assert np.all(np.abs(gv - wv) <= np.abs(wv) * 2.0 ** -7 + 1e-300)
    one = O.silu_mul_bf16(np.array([0.0, 50.0, -40.0]), np.array([1.0, 1.0, 1.0]))
    assert bf16_value(one[0]) == 0.0
    assert bf16_value(one[1]) == 50.0
    assert -1e-15 < bf16_value(one[2]) <= 0.0


def mlp_bruteforce(x_bits, w1, w1s, w3, w3s, w2, w2s):
    """Pure-Python tiny expert MLP: brute-force quantiser, exact sums, bf16 by table."""
    M, H = x_bits.shape
    I = w1.shape[0]

    def deq_row(c, s, r):
        out = []
        for k in range(2 * c.shape[1]):
            byte = int(c[r, k // 2])
            nib = (byte >> 4) if k % 2 else (byte & 15)
            mag = E2M1_GRID[nib & 7]
            out.append(Fraction(-mag if nib & 8 else mag) * Fraction(2) ** (int(s[r, k // 32]) - 127))
        return out

    def quant_row(vals):
        codes, out = [], []
        for j in range(0, len(vals), 32):
            blk = vals[j:j + 32]
            amax = max(abs(v) for v in blk)
            if amax == 0:
                byte = 0
            else:
                e = 0
                while Fraction(2) ** (e + 1) <= amax:
                    e += 1
                while Fraction(2) ** e > amax:
                    e -= 1
                byte = min(max(e - 2 + 127, 0), 254)
            X = Fraction(2) ** (byte - 127)
            for v in blk:
                idx = int(e2m1_bruteforce(np.array([float(abs(v) / X)]))[0])
                out.append(Fraction(E2M1_GRID[idx]) * X * (-1 if v < 0 else 1))
        return out

    def to_bf16(vals):
        return bf16_rne_reference(np.array([float(v) for v in vals]))

    W1 = [deq_row(w1, w1s, i) for i in range(I)]
    W3 = [deq_row(w3, w3s, i) for i in range(I)]
    W2 = [deq_row(w2, w2s, n) for n in range(H)]
    ys = []
    for m in range(M):
        xr = [Fraction(bf16_value(b)) for b in x_bits[m]]
        a = quant_row(xr)
        h = []
        for i in range(I):
            g = sum(p * q for p, q in zip(a, W1[i]))
            u = sum(p * q for p, q in zip(a, W3[i]))
            gf = float(g)
            silu = gf / (1.0 + math.exp(-gf)) if gf > -700 else 0.0 * gf
            h.append(silu * float(u))
        hb = to_bf16(h)
        hq = quant_row([Fraction(bf16_value(b)) for b in hb])
        y = [sum(p * q for p, q in zip(hq, W2[n])) for n in range(H)]
        ys.append(to_bf16(y))
    return np.array(ys, np.uint16)


def check_mlp_bruteforce(O, seed=41):
    rng = np.random.default_rng(seed)
    H, I, M = 64, 32, 3
    w1 = rng.integers(0, 256, (I, H // 2)).astype(np.uint8)
    w3 = rng.integers(0, 256, (I, H // 2)).astype(np.uint8)
    w2 = rng.integers(0, 256, (H, I // 2)).astype(np.uint8)
    w1s = rng.integers(122, 129, (I, H // 32)).astype(np.uint8)
    w3s = rng.integers(122, 129, (I, H // 32)).astype(np.uint8)
    w2s = rng.integers(122, 129, (H, I // 32)).astype(np.uint8)
    x = rng.standard_normal((M, H)).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    got = O.expert_mlp(xb, w1, w1s, w3, w3s, w2, w2s)
    want = mlp_bruteforce(xb, w1, w1s, w3, w3s, w2, w2s)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


def _tiny_grouped(seed, E=3, T=5, k=2, H=64, I=32):
    rng = np.random.default_rng(seed)
    w = dict(
        w1=rng.integers(0, 256, (E, I, H // 2)).astype(np.uint8),
        w1s=rng.integers(122, 129, (E, I, H // 32)).astype(np.uint8),
        w3=rng.integers(0, 256, (E, I, H // 2)).astype(np.uint8),
        w3s=rng.integers(122, 129, (E, I, H // 32)).astype(np.uint8),
        w2=rng.integers(0, 256, (E, H, I // 2)).astype(np.uint8),
        w2s=rng.integers(122, 129, (E, H, I // 32)).astype(np.uint8),
    )
    x = (rng.standard_normal((T, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    wts = rng.random((T, k)).astype(np.float32)
    return x, ids, wts, w


def check_grouped_reductions(O, seed=43):
    x, ids, wts, w = _tiny_grouped(seed)
    E, T, k = w["w1"].shape[0], ids.shape[0], ids.shape[1]
    y = O.grouped_expert_mlp(x, ids, wts, **w)
    # brute force: explicit loop over pairs with the single-expert pipeline
    acc = np.zeros((T, x.shape[1]))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            _, inter = O.expert_mlp(x[t:t + 1], w["w1"][e], w["w1s"][e], w["w3"][e], w["w3s"][e],
                                    w["w2"][e], w["w2s"][e], intermediates=True)
            acc[t] += float(wts[t, j]) * inter["y64"][0]
    assert np.array_equal(y, O.f64_to_bf16(acc))
    # E = 1, k = 1, weight 1 is the shared expert
    one = {kk: v[:1] for kk, v in w.items()}
    y1 = O.grouped_expert_mlp(x, np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32), **one)
    ys = O.expert_mlp(x, *(one[n][0] for n in ("w1", "w1s", "w3", "w3s", "w2", "w2s")))
    assert np.array_equal(y1, ys)
    # permuting tokens permutes the output
    perm = np.random.default_rng(seed).permutation(T)
    yp = O.grouped_expert_mlp(x[perm], ids[perm], wts[perm], **w)
    assert np.array_equal(yp, y[perm])
    # ids outside [0, E) contribute nothing; unused experts do not matter
    ids2 = ids.copy()
    ids2[:, -1] = -1
    ids3 = ids.copy()
    ids3[:, -1] = E
    y2 = O.grouped_expert_mlp(x, ids2, wts, **w)
    y3 = O.grouped_expert_mlp(x, ids3, wts, **w)
    assert np.array_equal(y2, y3)
    w_only = wts.copy()
    w_only[:, -1] = 0
    y4 = O.grouped_expert_mlp(x, ids, w_only, **w)
    assert np.array_equal(y4, y2)
    # subset of tokens equals the same rows of the full result
    ysub = O.grouped_expert_mlp(x, ids, wts, tokens=[3, 1], **w)
    assert np.array_equal(ysub, y[[3, 1]])


def check_fp8_mlp_bruteforce(O, seed=71):
    """The FP8 shared-expert MLP on a tiny shape: every step by hand from pinned
    pieces (the FP8 linear, SiLU) and the table-search bf16 rounding, plus the
    composition of the oracle's own pinned linears."""
    rng = np.random.default_rng(seed)
    M, H, I = 3, 256, 128
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    w1 = rng.choice(finite, size=(I, H)).astype(np.uint8)
    w3 = rng.choice(finite, size=(I, H)).astype(np.uint8)
    w2 = rng.choice(finite, size=(H, I)).astype(np.uint8)
    s1 = rng.integers(110, 118, (1, 2)).astype(np.uint8)
    s3 = rng.integers(110, 118, (1, 2)).astype(np.uint8)
    s2 = rng.integers(110, 118, (2, 1)).astype(np.uint8)
    x = (rng.standard_normal((M, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = O.fp8_expert_mlp(x, w1, s1, w3, s3, w2, s2)
    g = O.fp8_block_linear(x, w1, s1)
    u = O.fp8_block_linear(x, w3, s3)
    gv = np.array([bf16_value(b) for b in g.ravel()])
    uv = np.array([bf16_value(b) for b in u.ravel()])
    hv = [float(Fraction(a) / (1 + Fraction(math.exp(-a))) * Fraction(b)) for a, b in zip(gv, uv)]
    h = bf16_rne_reference(np.array(hv)).reshape(M, I)
    assert np.array_equal(O.fp8_block_linear(h, w2, s2), y)
    assert y.shape == (M, H) and np.all(np.isfinite(((y.astype(np.uint32) << 16).view(np.float32))))


def check_nvfp4_linear_bruteforce(O, seed=73):
    """NVFP4-weight linear on a tiny shape against exact Fractions from the bit
    fields (E2M1 grid, E4M3 bit fields, the fp32 globals), rounded by the
    table-search bf16 reference; x's NVFP4 codes come from the pinned quantiser."""
    rng = np.random.default_rng(seed)
    M, N, K = 2, 24, 64
    w = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    finite = np.array([b for b in range(127) if b != 0], np.uint8)
    ws = rng.choice(finite, size=(N, K // 16)).astype(np.uint8)
    gw, gx = np.float32(0.0123), np.float32(0.75)
    x = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = O.nvfp4_linear(x, w, ws, gw, gx)
    xq, xs = O.nvfp4_quantize(x, gx)

    def val(codes, scales, g, r, k):
        byte = int(codes[r, k // 2])
        nib = (byte >> 4) if k % 2 else (byte & 15)
        mag = Fraction(E2M1_GRID[nib & 7])
        return (-mag if nib & 8 else mag) * _e4m3_fraction(int(scales[r, k // 16])) * Fraction(float(g))
    want = [float(sum(val(xq, xs, gx, m, k) * val(w, ws, gw, n, k) for k in range(K)))
            for m in range(M) for n in range(N)]
    assert np.array_equal(y, bf16_rne_reference(np.array(want)).reshape(M, N))


def check_nvfp4_mlp_composition(O, seed=79):
    """The NVFP4-weight expert on a tiny shape: gate and up use their own
    globals (swapping them changes the result), and the steps compose from the
    pinned linear, SiLU and quantiser."""
    rng = np.random.default_rng(seed)
    M, H, I = 3, 128, 128
    w = {n: rng.integers(0, 256, (r, c // 2)).astype(np.uint8) for n, (r, c) in
         (("w1", (I, H)), ("w3", (I, H)), ("w2", (H, I)))}
    sc = {n: rng.integers(0x20, 0x58, (r, c // 16)).astype(np.uint8) for n, (r, c) in
          (("w1", (I, H)), ("w3", (I, H)), ("w2", (H, I)))}
    g1, g3, g2, gx, gh = (np.float32(v) for v in (2.0 ** -6, 2.0 ** -4, 2.0 ** -5, 2.0 ** -9, 2.0 ** -3))
    x = (rng.standard_normal((M, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = O.nvfp4_expert_mlp(x, w["w1"], sc["w1"], g1, w["w3"], sc["w3"], g3, w["w2"], sc["w2"], g2, gx, gh)
    g = O.nvfp4_linear(x, w["w1"], sc["w1"], g1, gx)
    u = O.nvfp4_linear(x, w["w3"], sc["w3"], g3, gx)
    gv = np.array([bf16_value(b) for b in g.ravel()])
    uv = np.array([bf16_value(b) for b in u.ravel()])
    hv = [float(Fraction(a) / (1 + Fraction(math.exp(-a))) * Fraction(b)) for a, b in zip(gv, uv)]
    h = bf16_rne_reference(np.array(hv)).reshape(M, I)
    assert np.array_equal(O.nvfp4_linear(h, w["w2"], sc["w2"], g2, gh), y)
    swapped = O.nvfp4_expert_mlp(x, w["w1"], sc["w1"], g3, w["w3"], sc["w3"], g1, w["w2"], sc["w2"], g2, gx, gh)
    assert not np.array_equal(swapped, y)


def check_grouped_nvfp4_reductions(O, seed=83):
    """Routed NVFP4-weight experts: one expert with k = 1 and w = 1 reduces to the
    single NVFP4-weight expert; the result is linear in the gate weights;
    foreign ids contribute nothing; each expert's own globals are used."""
    rng = np.random.default_rng(seed)
    E, T, k, H, I = 3, 5, 2, 128, 128
    w = {n: rng.integers(0, 256, (E, r, c // 2)).astype(np.uint8) for n, (r, c) in
         (("w1", (I, H)), ("w3", (I, H)), ("w2", (H, I)))}
    sc = {n: rng.integers(0x20, 0x58, (E, r, c // 16)).astype(np.uint8) for n, (r, c) in
          (("w1", (I, H)), ("w3", (I, H)), ("w2", (H, I)))}
    g1 = np.array([2.0 ** -6, 2.0 ** -5, 2.0 ** -7], np.float32)
    g3 = np.array([2.0 ** -5, 2.0 ** -6, 2.0 ** -6], np.float32)
    g2 = np.array([2.0 ** -6, 2.0 ** -4, 2.0 ** -5], np.float32)
    gx, gh = np.float32(2.0 ** -9), np.float32(1.0)
    x = (rng.standard_normal((T, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    args = lambda gg1: (w["w1"], sc["w1"], gg1, w["w3"], sc["w3"], g3, w["w2"], sc["w2"], g2, gx, gh)
    ids = np.array([[0, 1], [2, 0], [1, 2], [0, 0], [2, 1]], np.int32)
    wt = rng.random((T, k)).astype(np.float32)
    y = O.grouped_nvfp4_expert_mlp(x, ids, wt, *args(g1))
    # single expert: ids all e, k = 1, w = 1
    for e in range(E):
        one = O.grouped_nvfp4_expert_mlp(x, np.full((T, 1), e, np.int32), np.ones((T, 1), np.float32), *args(g1))
        single = O.nvfp4_expert_mlp(x, w["w1"][e], sc["w1"][e], g1[e], w["w3"][e], sc["w3"][e], g3[e],
                                    w["w2"][e], sc["w2"][e], g2[e], gx, gh)
        assert np.max(np.abs(bf16_to_f64_local(one) - bf16_to_f64_local(single))
                      / (np.abs(bf16_to_f64_local(single)) + 1e-30)) <= 2.0 ** -7
    # linear in the weights; foreign ids skipped
    y2 = O.grouped_nvfp4_expert_mlp(x, ids, 2 * wt, *args(g1))
    assert np.allclose(bf16_to_f64_local(y2), 2 * bf16_to_f64_local(y), rtol=2.0 ** -7, atol=0)
    ids_f = ids.copy()
    ids_f[:, 1] = -1
    yf = O.grouped_nvfp4_expert_mlp(x, ids_f, wt, *args(g1))
    yk = O.grouped_nvfp4_expert_mlp(x, ids[:, :1], wt[:, :1], *args(g1))
    assert np.array_equal(yf, yk)
    # per-expert globals matter: change expert 1's gate global
    g1b = g1.copy()
    g1b[1] *= 2
    assert not np.array_equal(O.grouped_nvfp4_expert_mlp(x, ids, wt, *args(g1b)), y)


def bf16_to_f64_local(bits):
    return ((np.asarray(bits).astype(np.uint32) << 16).view(np.float32)).astype(np.float64)



def check_quantizers_nonfinite_blocks(O, seed=89):
    """A block holding +inf, -inf or a NaN has no finite shared exponent: the
    quantisers give it the format's NaN scale byte (E8M0 0xFF for MXFP4 and
    MXFP8, E4M3 0x7F for NVFP4: the NaN encodings of the format names
    e8m0fnu / e4m3fn) and zero codes, so it dequantises to NaN; every other
    block is quantised exactly as on its own."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((3, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bad = x.copy()
    poison = {0: (5, 0x7F80), 1: (40, 0xFF80), 2: (33, 0x7FC0)}    # +inf, -inf, NaN
    for r, (col, v) in poison.items():
        bad[r, col] = v
    for quant, per, nan_byte, bpb in (
            (O.mxfp4_quantize, 32, 0xFF, 16), (O.mxfp8_quantize, 32, 0xFF, 32),
            (lambda v: O.nvfp4_quantize(v, np.float32(0.01)), 16, 0x7F, 8)):
        c0, s0 = quant(x)
        c1, s1 = quant(bad)
        for r in range(3):
            for b in range(64 // per):
                cb = slice(b * bpb, (b + 1) * bpb)
                if b == poison[r][0] // per:
                    assert int(s1[r, b]) == nan_byte
                    assert np.all(c1[r, cb] == 0)
                else:
                    assert s1[r, b] == s0[r, b]
                    assert np.array_equal(c1[r, cb], c0[r, cb])
    # dequantised, the NaN block is NaN and nothing else is
    c, s = O.mxfp4_quantize(bad)
    dq = O.mxfp4_dequant_f64(c, s)
    assert np.isnan(dq[0, :32]).all() and np.isnan(dq[1, 32:]).all() and np.isnan(dq[2, 32:]).all()
    assert np.isfinite(dq[0, 32:]).all() and np.isfinite(dq[1, :32]).all() and np.isfinite(dq[2, :32]).all()


def check_mlp_nan_propagation(O, seed=97):
    """NaN in the weights: the E8M0 NaN byte in one down-projection scale makes
    exactly that output column NaN for every token (the others are unchanged);
    in a gate scale it makes h NaN in one block of every token, which the
    re-quantisation carries on as a NaN scale, so every output is NaN. Routed:
    only the tokens routed to the poisoned expert are affected."""
    rng = np.random.default_rng(seed)
    H, I, M = 64, 64, 3
    w = dict(w1=rng.integers(0, 256, (I, H // 2)), w3=rng.integers(0, 256, (I, H // 2)),
             w2=rng.integers(0, 256, (H, I // 2)), w1s=rng.integers(122, 129, (I, H // 32)),
             w3s=rng.integers(122, 129, (I, H // 32)), w2s=rng.integers(122, 129, (H, I // 32)))
    w = {k: v.astype(np.uint8) for k, v in w.items()}
    x = (rng.standard_normal((M, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    order = ("w1", "w1s", "w3", "w3s", "w2", "w2s")
    nan = lambda y: np.isnan(bf16_to_f64_local(y))
    y0 = O.expert_mlp(x, *(w[n] for n in order))
    assert not nan(y0).any()
    w2 = dict(w, w2s=w["w2s"].copy())
    w2["w2s"][17, 1] = 0xFF
    y2 = O.expert_mlp(x, *(w2[n] for n in order))
    assert nan(y2)[:, 17].all() and not np.delete(nan(y2), 17, axis=1).any()
    assert np.array_equal(np.delete(y2, 17, axis=1), np.delete(y0, 17, axis=1))
    w1 = dict(w, w1s=w["w1s"].copy())
    w1["w1s"][5, 0] = 0xFF
    assert nan(O.expert_mlp(x, *(w1[n] for n in order))).all()
    # routed: expert 1 poisoned in its gate scales
    E, T, k = 3, 6, 2
    we = {n: np.stack([v] * E) for n, v in w.items()}
    we["w1s"] = we["w1s"].copy()
    we["w1s"][1, 5, 0] = 0xFF
    xt = (rng.standard_normal((T, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ids = np.array([[0, 2], [1, 0], [2, 0], [1, 2], [0, 2], [2, 1]], np.int32)
    wt = rng.random((T, k)).astype(np.float32)
    yr = O.grouped_expert_mlp(xt, ids, wt, *(we[n] for n in order))
    routed1 = (ids == 1).any(axis=1)
    assert nan(yr)[routed1].all() and not nan(yr)[~routed1].any()


def check_nvfp4_golden_block(O):
    """The hand-worked NVFP4 block of tests/golden/nvfp4_quantize_example.txt:
    the fp32 rounding of 6 g decides the block scale (0x3A, not 0x39) and the
    division by the fp32 product s g decides one code (0.5, not 1.0)."""
    g, sbyte, rows = None, None, []
    for parts in _lines("nvfp4_quantize_example.txt"):
        if parts[0] == "global":
            g = np.array([int(parts[1], 16)], np.uint32).view(np.float32)[0]
        elif parts[0] == "scale":
            sbyte = int(parts[1], 16)
        else:
            rows.append((int(parts[0], 16), float(parts[1]), int(parts[2])))
    assert len(rows) == 16 and g == np.float32(1.0 / 3.0)
    bits = np.array([b for b, _, _ in rows], np.uint16)
    for b, v, _ in rows:
        assert _same(bf16_value(b), v)
    codes, sc = O.nvfp4_quantize(bits[None, :], g)
    assert int(sc[0, 0]) == sbyte
    nib = np.empty(16, np.int64)
    nib[0::2] = codes[0] & 15
    nib[1::2] = codes[0] >> 4
    assert [int(n) for n in nib] == [c for _, _, c in rows]


def _silu_mul_fraction(gv, uv):
    """bf16(silu(g) * u) of bf16 values g, u: silu from an exact quotient with
    math.exp, rounded once by the table-search bf16 reference."""
    hv = [float(Fraction(a) / (1 + Fraction(math.exp(-a))) * Fraction(b)) if a > -700 else 0.0 * a * b
          for a, b in zip(gv, uv)]
    return bf16_rne_reference(np.array(hv))


def check_fp8_mlp_fraction_bruteforce(O, seed=101):
    """The FP8 shared expert from first principles on a tiny shape: weights from
    the E4M3 bit fields times their 128 x 128 block's 2^(s-127), exact Fraction
    sums for the three linears, each rounded to bf16 by table search, SiLU * up by
    an exact quotient; only the MXFP8 activation quantiser is the oracle's
    (pinned on its own). Independent of the oracle's linear and composition."""
    rng = np.random.default_rng(seed)
    M, H, I = 2, 256, 128
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    w1 = rng.choice(finite, size=(I, H)).astype(np.uint8)
    w3 = rng.choice(finite, size=(I, H)).astype(np.uint8)
    w2 = rng.choice(finite, size=(H, I)).astype(np.uint8)
    s1 = rng.integers(110, 118, (1, 2)).astype(np.uint8)
    s3 = rng.integers(110, 118, (1, 2)).astype(np.uint8)
    s2 = rng.integers(110, 118, (2, 1)).astype(np.uint8)
    x = (rng.standard_normal((M, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    P2 = [Fraction(2) ** (e - 127) for e in range(256)]

    def wmat(w, s):
        return [[_e4m3_fraction(int(w[n, k])) * P2[int(s[n // 128, k // 128])] for k in range(w.shape[1])]
                for n in range(w.shape[0])]

    def act(bits):
        q, sc = O.mxfp8_quantize(bits)
        return [[_e4m3_fraction(int(q[m, k])) * P2[int(sc[m, k // 32])] for k in range(bits.shape[1])]
                for m in range(bits.shape[0])]

    def linear(a, wf):
        v = [float(sum(p * q for p, q in zip(r, wr))) for r in a for wr in wf]
        return bf16_rne_reference(np.array(v)).reshape(len(a), len(wf))

    a = act(x)
    g = linear(a, wmat(w1, s1))
    u = linear(a, wmat(w3, s3))
    h = _silu_mul_fraction([bf16_value(b) for b in g.ravel()], [bf16_value(b) for b in u.ravel()]).reshape(M, I)
    want = linear(act(h), wmat(w2, s2))
    assert np.array_equal(O.fp8_expert_mlp(x, w1, s1, w3, s3, w2, s2), want)


def check_nvfp4_mlp_fraction_bruteforce(O, seed=103):
    """The expert with NVFP4 weights from first principles on a tiny shape: weight
    and activation values code * E4M3(s) * g as exact Fractions from the bit
    fields, exact sums for the three linears, each rounded to bf16 by table
    search, SiLU * up by an exact quotient; only the NVFP4 quantiser is the
    oracle's (pinned by the grid checks and the hand-worked block). Gate and up
    carry different globals. Independent of the oracle's linear and
    composition."""
    rng = np.random.default_rng(seed)
    M, H, I = 2, 128, 64
    w = {n: rng.integers(0, 256, (r, c // 2)).astype(np.uint8) for n, (r, c) in
         (("w1", (I, H)), ("w3", (I, H)), ("w2", (H, I)))}
    sc = {n: rng.integers(0x20, 0x58, (r, c // 16)).astype(np.uint8) for n, (r, c) in
          (("w1", (I, H)), ("w3", (I, H)), ("w2", (H, I)))}
    g1, g3, g2, gx, gh = (np.float32(v) for v in (2.0 ** -6, 3 * 2.0 ** -6, 2.0 ** -5, 2.0 ** -9, 0.75))
    x = (rng.standard_normal((M, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)

    def vals(codes, scales, g):
        G = Fraction(float(g))
        out = []
        for r in range(codes.shape[0]):
            row = []
            for k in range(2 * codes.shape[1]):
                byte = int(codes[r, k // 2])
                nib = (byte >> 4) if k % 2 else (byte & 15)
                mag = Fraction(E2M1_GRID[nib & 7])
                row.append((-mag if nib & 8 else mag) * _e4m3_fraction(int(scales[r, k // 16])) * G)
            out.append(row)
        return out

    def linear(a, wf):
        v = [float(sum(p * q for p, q in zip(r, wr))) for r in a for wr in wf]
        return bf16_rne_reference(np.array(v)).reshape(len(a), len(wf))

    a = vals(*O.nvfp4_quantize(x, gx), gx)
    g = linear(a, vals(w["w1"], sc["w1"], g1))
    u = linear(a, vals(w["w3"], sc["w3"], g3))
    h = _silu_mul_fraction([bf16_value(b) for b in g.ravel()], [bf16_value(b) for b in u.ravel()]).reshape(M, I)
    want = linear(vals(*O.nvfp4_quantize(h, gh), gh), vals(w["w2"], sc["w2"], g2))
    got = O.nvfp4_expert_mlp(x, w["w1"], sc["w1"], g1, w["w3"], sc["w3"], g3, w["w2"], sc["w2"], g2, gx, gh)
    assert np.array_equal(got, want)
