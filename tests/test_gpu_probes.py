"""The measurement probes compute what they claim, so that the rates taken from
them rest on work that was done: the MFMA loop's sums against their closed
form, the register and LDS reads' XOR checksums against the buffer's, and the
copy byte for byte."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    import mxfp4_block_scaled_e2m1_amd as m
    return m


@pytest.mark.parametrize("a_code,b_code,prod", [(2, 2, 1.0), (3, 4, 3.0), (7, 9, -3.0)])
def test_probe_mfma_closed_form(mx, a_code, b_code, prod):
    """Every A code a_code and every B code b_code (E2M1: 2 = 1.0, 3 = 1.5, 4 = 2,
    7 = 6, 9 = -0.5): each output of one 32x32x64 step is 64 * prod, a lane holds
    16 outputs of each of 4 accumulators, so a lane's sum after `iters` steps is
    64 * 64 * prod * iters, exact in fp32."""
    ops = np.zeros((512, 16), np.uint32)
    ops[:, :8] = int("".join([f"{a_code:x}"] * 8), 16)
    ops[:, 8:] = int("".join([f"{b_code:x}"] * 8), 16)
    d = torch.from_numpy(ops.view(np.int32)).cuda()
    for iters, wgs in ((1, 1), (5, 3), (37, 17)):
        out = mx.probe_mfma_fp4(d, iters, wgs)
        torch.cuda.synchronize()
        assert out.shape == (wgs, 512)
        assert torch.all(out == 4096.0 * prod * iters).item(), (iters, wgs)


E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def _lane_codes(words):
    """The 32 E2M1 values of a lane's 4 operand words, element j = nibble j % 8 of
    word j // 8 (low nibble first)."""
    nib = (words[:, :4, None] >> (4 * np.arange(8, dtype=np.uint32))) & 0xF
    return E2M1[nib.reshape(words.shape[0], 32)]


def mfma_probe_lane_sums(ops, iters):
    """Independent model of the probe, from the 32x32x64 operand layout: in each
    wave, lane l holds K values 32 * (l // 32) .. +32 of A row l % 32 and of B
    row l % 32; D = A . B^T (32 x 32); lane l's 16 accumulator values are
    D[8 (v // 4) + 4 (l // 32) + v % 4][l % 32], v = 0..15. The probe sums them
    over its 4 accumulators, each after `iters` steps."""
    out = np.zeros(512)
    for w in range(8):
        lanes = np.arange(64)
        a = _lane_codes(ops[64 * w + lanes, :8])
        b = _lane_codes(ops[64 * w + lanes, 8:])
        A = np.zeros((32, 64))
        Bm = np.zeros((32, 64))
        for l in range(64):
            A[l % 32, 32 * (l // 32):32 * (l // 32) + 32] = a[l]
            Bm[l % 32, 32 * (l // 32):32 * (l // 32) + 32] = b[l]
        D = A @ Bm.T
        for l in range(64):
            v = np.arange(16)
            out[64 * w + l] = D[8 * (v // 4) + 4 * (l // 32) + v % 4, l % 32].sum() * 4 * iters
    return out


def test_probe_mfma_random_operands_match_the_layout_model(mx):
    """Random codes in every operand word: every workgroup's lane sums equal the
    model's exactly (FP4 products are multiples of 1/4 and the sums stay far
    below 2^22, so fp32 holds them exactly in any order)."""
    rng = np.random.default_rng(11)
    ops = rng.integers(0, 2**32, (512, 16), dtype=np.uint64).astype(np.uint32)
    d = torch.from_numpy(ops.view(np.int32)).cuda()
    for iters, wgs in ((1, 2), (7, 9)):
        out = mx.probe_mfma_fp4(d, iters, wgs).cpu().numpy().astype(np.float64)
        want = mfma_probe_lane_sums(ops, iters)
        assert np.array_equal(out, np.broadcast_to(want, out.shape)), (iters, wgs)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("lpw", [8, 32])
@pytest.mark.parametrize("wgs", [1, 7, 256])
def test_probe_read_checksum(mx, mode, lpw, wgs):
    rng = np.random.default_rng(mode * 100 + lpw + wgs)
    n = 3 * (1 << 20) // 4   # 3 MiB of int32 words
    host = rng.integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(host).cuda()
    out = mx.probe_read(src, mode, lpw, wgs)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host.view(np.uint32))


def test_probe_copy(mx):
    rng = np.random.default_rng(5)
    for nbytes in (16, 4096 + 48, (1 << 22) + 16 * 7):
        host = rng.integers(0, 256, nbytes, dtype=np.uint8)
        src = torch.from_numpy(host).cuda()
        dst = torch.zeros_like(src)
        mx.probe_copy(src, dst)
        torch.cuda.synchronize()
        assert np.array_equal(dst.cpu().numpy(), host)
