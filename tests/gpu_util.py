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


def as_np(a):
    """device tensor or numpy array -> numpy array."""
    return a.cpu().numpy() if isinstance(a, torch.Tensor) else np.asarray(a)


# Tile-major scale layout of the GEMM (the library's pack.hip): per tile of 256
# rows and per 256-wide K stage, 8 scale bytes of each row, contiguous.
def packed_scale_bytes(tiles, k):
    return tiles * ((k + 255) // 256) * 2048


def packed_code_bytes(tiles, k):
    return tiles * (k // 128) * 16384


def unpack_tile_codes(buf, tiles, k):
    """Tile-major codes [tiles][k/128][256 rows][64 bytes], 16-byte chunk c of row
    R at slot c ^ ((R >> 2) & 3) -> row-major [tiles * 256, k/2]."""
    nh = k // 128
    a = np.asarray(buf, np.uint8)[:tiles * nh * 16384].reshape(tiles, nh, 256, 4, 16)
    R = np.arange(256)
    out = np.empty((tiles, 256, nh, 4, 16), np.uint8)
    for c in range(4):
        out[:, :, :, c] = a[:, :, R, c ^ ((R >> 2) & 3)].transpose(0, 2, 1, 3)
    return out.reshape(tiles * 256, k // 2)


STREAM_WAVES = 8   # waves of the weight-streaming kernels; the chunked scales follow their K split


def stream_wave_runs(ksteps, waves=STREAM_WAVES):
    """The kernels' balanced split of ksteps K steps over the waves: (first step,
    count) per wave, the first ksteps % waves waves taking one more."""
    base, extra = divmod(ksteps, waves)
    runs, s = [], 0
    for w in range(waves):
        n = base + (1 if w < extra else 0)
        runs.append((s, n))
        s += n
    return runs


def chunked_scale_bytes(rows):
    return (rows + 15) // 16 * STREAM_WAVES * 64 * 8


def unpack_chunked(codes, scales, rows, k):
    """Chunked token operand of the weight-streaming kernels -> row-major codes
    [rows, k/2] and scales [rows, k/32]. Codes: per 16-row chunk c and 128-wide
    K step s a 1 KB block whose 16 bytes at lane l = 16 q + r are columns
    128 s + 32 q .. +31 of row 16 c + r. Scales: per chunk c, wave w and lane l
    8 bytes, byte j the scale of lane l's 32 columns in step s0(w) + j of the
    wave's run."""
    ks, nck = k // 128, (rows + 15) // 16
    c = np.asarray(codes, np.uint8)[:nck * ks * 1024].reshape(nck, ks, 4, 16, 16)
    c = c.transpose(0, 3, 1, 2, 4).reshape(nck * 16, k // 2)
    a = np.asarray(scales, np.uint8)[:chunked_scale_bytes(rows)].reshape(nck, STREAM_WAVES, 4, 16, 8)
    s = np.zeros((nck, 16, ks, 4), np.uint8)
    for w, (s0, n) in enumerate(stream_wave_runs(ks)):
        s[:, :, s0:s0 + n, :] = a[:, w, :, :, :n].transpose(0, 2, 3, 1)
    return c[:rows], s.reshape(nck * 16, k // 32)[:rows]


def unpack_tile_major(buf, rows, k):
    """Tile-major bytes of row tiles [tiles][stage][256][8] -> row-major [rows, k/32]."""
    nst, ks = (k + 255) // 256, k // 32
    tiles = (rows + 255) // 256
    a = np.asarray(buf, np.uint8)[:tiles * nst * 2048].reshape(tiles, nst, 256, 8)
    full = a.transpose(0, 2, 1, 3).reshape(tiles * 256, nst * 8)
    return full[:rows, :ks]


def pack_weight_scales_ref(w1s, w3s, w2s):
    """Expected output of mx_pack_weight_scales (layout only: byte moves) for
    stacked scales w1s/w3s [E, I, H/32], w2s [E, H, I/32]."""
    E, I, hs = w1s.shape
    H = 32 * hs

    # L1 tiles: 128 j per tile; tile row r -> gate (w1) rows for (r/32)%4 < 2, else up (w3)
    nst1, ks1 = (H + 255) // 256, H // 32
    g = np.zeros((E, I, nst1 * 8), np.uint8)
    g[:, :, :ks1] = w1s
    u = np.zeros((E, I, nst1 * 8), np.uint8)
    u[:, :, :ks1] = w3s
    nt1 = (I + 127) // 128
    l1 = np.zeros((E, nt1, nst1, 256, 8), np.uint8)
    for nt in range(nt1):
        for r in range(256):
            f = (r >> 5) & 3
            row = min(nt * 128 + (r >> 7) * 64 + (f & 1) * 32 + (r & 31), I - 1)
            src = g if f < 2 else u
            l1[:, nt, :, r, :] = src[:, row].reshape(E, nst1, 8)
    nst2, ks2 = (I + 255) // 256, I // 32
    d = np.zeros((E, H, nst2 * 8), np.uint8)
    d[:, :, :ks2] = w2s
    nt2 = (H + 255) // 256
    l2 = np.zeros((E, nt2, nst2, 256, 8), np.uint8)
    for nt in range(nt2):
        for r in range(256):
            row = min(nt * 256 + r, H - 1)
            l2[:, nt, :, r, :] = d[:, row].reshape(E, nst2, 8)
    return np.concatenate([l1.reshape(-1), l2.reshape(-1)])


def _align256(n):
    return (n + 255) // 256 * 256


def pack_weight_codes_ref(w1, w3, w2):
    """Expected output of mx_pack_weight_codes (layout only: byte moves) for
    stacked codes w1/w3 [E, I, H/2], w2 [E, H, I/2]: per expert, tile and
    128-wide half stage, 256 rows x 64 bytes, row R at R*64 with its 16-byte
    chunk c at (c ^ ((R >> 2) & 3)) * 16; L1 tiles interleave gate and up rows
    as the scale layout does; rows past the end repeat the last row."""
    E, I, hb = w1.shape
    H = 2 * hb

    def blocks(rows_of, mats, nrows, kb, ntiles):
        nh = kb // 64
        out = np.zeros((E, ntiles, nh, 256, 4, 16), np.uint8)
        for nt in range(ntiles):
            for r in range(256):
                mat, row = rows_of(nt, r)
                row = min(row, nrows - 1)
                src = mats[mat][:, row].reshape(E, nh, 4, 16)
                for c in range(4):
                    out[:, nt, :, r, c ^ ((r >> 2) & 3)] = src[:, :, c]
        return out.reshape(E, -1)

    def l1_rows(nt, r):
        f = (r >> 5) & 3
        return (0 if f < 2 else 1), nt * 128 + (r >> 7) * 64 + (f & 1) * 32 + (r & 31)

    l1 = blocks(l1_rows, (w1, w3), I, hb, (I + 127) // 128)
    l2 = blocks(lambda nt, r: (0, nt * 256 + r), (w2,), H, I // 2, (H + 255) // 256)
    return np.concatenate([l1.ravel(), l2.ravel()])


def routed_ws_slices(ws, T, H, I, k, E, requant="mxfp4"):
    """The routed GEMM-path workspace of mx_grouped_expert_mlp (each region
    256-byte aligned): xq, xs, block counts, expert offsets, tile bases,
    row_token, row_slot, row_weight, hq, hs (tile-major over the m-tiles for
    MXFP4, row-major E4M3 per 16 for NVFP4), o (bf16 per-pair rows in slot order
    t*k + j), xs_pk. Returns a dict of numpy views of the regions the tests read."""
    P = T * k
    mt = (P + E * 255) // 256
    hs_bytes = P * I // 16 if requant == "nvfp4" else packed_scale_bytes(mt, I)
    hq_bytes = P * I // 2 if requant == "nvfp4" else packed_code_bytes(mt, I)
    names = ["xq", "xs", "block_counts", "expert_off", "tile_base", "row_token", "row_slot", "row_weight", "hq",
             "hs", "o"]
    sizes = [T * H // 2, T * H // 32, -(-P // 1024) * E * 4, (E + 1) * 4, (E + 1) * 4, P * 4, P * 4, P * 4,
             hq_bytes, hs_bytes, P * H * 2]
    off, out = 0, {}
    host = ws.cpu().numpy()
    for n, s in zip(names, sizes):
        out[n] = host[off:off + s]
        off += _align256(s)
    for n in ("expert_off", "tile_base", "row_token", "row_slot"):
        out[n] = out[n].view(np.int32)
    out["o"] = out["o"].view(np.uint16).reshape(P, H)
    if requant == "nvfp4":
        out["hq"] = out["hq"].reshape(P, I // 2)
        out["hs"] = out["hs"].reshape(P, I // 16)
    else:
        # codes: m-tile tile_base[e] + i, tile row q holds sorted row expert_off[e] + 256 i + q
        tc = unpack_tile_codes(out["hq"], mt, I)
        hq = np.zeros((P, I // 2), np.uint8)
        eo, tb = out["expert_off"], out["tile_base"]
        for e in range(E):
            for i in range(tb[e + 1] - tb[e]):
                r0 = eo[e] + 256 * i
                n = min(256, eo[e + 1] - r0)
                hq[r0:r0 + n] = tc[(tb[e] + i) * 256:(tb[e] + i) * 256 + n]
        out["hq"] = hq
        # m-tile tile_base[e] + i holds the sorted rows expert_off[e] + 256 i ...
        nst = (I + 255) // 256
        tm = out["hs"][:mt * nst * 2048].reshape(mt, nst, 256, 8)
        rowmaj = np.zeros((P, nst * 8), np.uint8)
        eo, tb = out["expert_off"], out["tile_base"]
        for e in range(E):
            for i in range(tb[e + 1] - tb[e]):
                r0 = eo[e] + 256 * i
                n = min(256, eo[e + 1] - r0)
                rowmaj[r0:r0 + n] = tm[tb[e] + i].transpose(1, 0, 2).reshape(256, nst * 8)[:n]
        out["hs"] = rowmaj[:, :I // 32]
    return out
