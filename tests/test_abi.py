"""The C-ABI library loads, exports every symbol include/mxfp4.h declares, and
its host-side validation rejects bad arguments before touching the GPU (CPU only)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp4.h")


def _declared():
    text = open(HEADER).read()
    return re.findall(r"MX_API\s+[\w\s\*]+?\b(mx_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def L():
    from mxfp4_block_scaled_e2m1_amd import binding, build
    if not os.path.exists(binding.LIB_PATH):
        build.build()
    return binding.lib()


def test_header_declares_the_boundary():
    names = set(_declared())
    for n in ("mx_dequant", "mx_quantize_act", "mx_expert_mlp", "mx_grouped_expert_mlp"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    from mxfp4_block_scaled_e2m1_amd import binding
    for name in _declared():
        assert hasattr(L, name), name
        assert name in binding.SIGNATURES, name


def _err(L):
    return L.mx_last_error().decode()


def test_status_strings(L):
    assert L.mx_status_string(0) == b"ok"
    assert L.mx_status_string(5) == b"workspace too small"


def test_dequant_validation(L):
    P = ctypes.c_void_p
    assert L.mx_dequant(0, None, None, None, 4, 33, None, None) == 2 and "32" in _err(L)
    assert L.mx_dequant(0, None, None, None, 4, 64, None, None) == 1 and "codes" in _err(L)
    assert L.mx_dequant(9, None, None, None, 4, 64, None, None) == 4
    assert L.mx_dequant(-1, None, None, None, 4, 64, None, None) == 4   # any int32 is a checked format
    assert L.mx_dequant(1, None, None, None, 4, 24, None, None) == 2
    assert L.mx_dequant(0, None, None, None, -1, 64, None, None) == 2
    assert L.mx_dequant(0, None, None, None, 0, 64, None, None) == 0      # empty: nothing to do
    # misaligned output pointer (never dereferenced: validation fails first)
    assert L.mx_dequant(0, P(16), P(16), None, 1, 64, P(8), None) == 3
    # NVFP4: the global scale is a device pointer, required and 4-byte aligned
    assert L.mx_dequant(2, P(16), P(16), None, 1, 64, P(16), None) == 1 and "global" in _err(L)
    assert L.mx_dequant(2, P(16), P(16), P(18), 1, 64, P(16), None) == 3


def test_quantize_validation(L):
    P = ctypes.c_void_p
    assert L.mx_quantize_act(1, None, 4, 64, None, None, None, None) == 4        # FP8 is dequant-only
    assert L.mx_quantize_act(0, None, 4, 48, None, None, None, None) == 2
    assert L.mx_quantize_act(2, None, 4, 64, None, None, None, None) == 1        # NVFP4 needs its global
    assert L.mx_quantize_act(2, None, 4, 64, P(258), None, None, None) == 3     # ... 4-byte aligned
    assert L.mx_quantize_act(0, None, 4, 64, None, None, None, None) == 1


def test_mlp_validation(L):
    P = ctypes.c_void_p
    z = [P(256)] * 6
    # hidden not a multiple of 128
    assert L.mx_expert_mlp(P(256), 4, 200, 128, *z, None, None, 0, None, P(256), P(256), 1 << 30, None) == 2
    assert L.mx_expert_mlp(P(256), 4, 256, 96, *z, None, None, 0, None, P(256), P(256), 1 << 30, None) == 2
    # NVFP4 re-quant needs its global scale (a device pointer); FP8 is not a re-quant format
    assert L.mx_expert_mlp(P(256), 4, 256, 128, *z, None, None, 2, None, P(256), P(256), 1 << 30, None) == 1
    assert L.mx_expert_mlp(P(256), 4, 256, 128, *z, None, None, 2, P(257), P(256), P(256), 1 << 30, None) == 3
    assert L.mx_expert_mlp(P(256), 4, 256, 128, *z, None, None, 1, None, P(256), P(256), 1 << 30, None) == 4
    # NVFP4 keeps one E4M3 byte per 16 columns of h: a larger workspace than MXFP4
    assert L.mx_expert_mlp_workspace_size(4096, 7168, 3072, 2) > L.mx_expert_mlp_workspace_size(4096, 7168, 3072, 0)
    # workspace too small
    need = L.mx_expert_mlp_workspace_size(4, 256, 128, 0)
    assert need > 0
    assert L.mx_expert_mlp(P(256), 4, 256, 128, *z, None, None, 0, None, P(256), P(256), need - 1, None) == 5
    # misaligned workspace, null weights
    assert L.mx_expert_mlp(P(256), 4, 256, 128, *z, None, None, 0, None, P(256), P(128), need, None) == 3
    assert L.mx_expert_mlp(P(256), 4, 256, 128, None, *z[1:], None, None, 0, None, P(256), P(256), need, None) == 1
    # zero tokens is a no-op
    assert L.mx_expert_mlp(None, 0, 256, 128, *([None] * 8), 0, None, None, None, 0, None) == 0
    # packed weight scales and codes must be 256-byte aligned (NULL selects the row-major ones)
    assert L.mx_expert_mlp(P(256), 4, 256, 128, *z, P(128), None, 0, None, P(256), P(256), need, None) == 3
    assert L.mx_expert_mlp(P(256), 4, 256, 128, *z, None, P(128), 0, None, P(256), P(256), need, None) == 3
    assert "packed_codes" in _err(L)


def test_pack_weight_scales_validation(L):
    P = ctypes.c_void_p
    need = L.mx_packed_weight_scales_size(256, 128, 4)
    # per expert: L1 one tile of 128 j x 1 stage, L2 one tile of 256 rows x 1 stage, 2 KB each
    assert need == 4 * (2048 + 2048)
    assert L.mx_packed_weight_scales_size(7168, 3072, 48) == 48 * (24 * 28 + 28 * 12) * 2048
    assert L.mx_pack_weight_scales(P(256), P(256), P(256), 200, 128, 4, P(256), need, None) == 2
    assert L.mx_pack_weight_scales(P(256), P(256), P(256), 256, 128, 0, P(256), need, None) == 2
    assert L.mx_pack_weight_scales(None, P(256), P(256), 256, 128, 4, P(256), need, None) == 1
    assert L.mx_pack_weight_scales(P(256), P(256), P(256), 256, 128, 4, P(128), need, None) == 3
    assert L.mx_pack_weight_scales(P(256), P(256), P(256), 256, 128, 4, P(256), need - 1, None) == 5


def test_pack_weight_codes_validation(L):
    P = ctypes.c_void_p
    need = L.mx_packed_weight_codes_size(256, 128, 4)
    # per expert: L1 one tile of 128 j x 2 half stages, L2 one tile of 256 rows x 1 half stage, 16 KB each
    assert need == 4 * (2 + 1) * 16384
    # the headline's 48 experts: as large as the code tensors (whole tiles)
    assert L.mx_packed_weight_codes_size(7168, 3072, 48) == 48 * (24 * 56 + 28 * 24) * 16384 == 48 * 3 * 3072 * 3584
    assert L.mx_packed_weight_codes_size(200, 128, 4) == 0
    assert L.mx_pack_weight_codes(P(256), P(256), P(256), 200, 128, 4, P(256), need, None) == 2
    assert L.mx_pack_weight_codes(P(256), P(256), P(256), 256, 128, 0, P(256), need, None) == 2
    assert L.mx_pack_weight_codes(None, P(256), P(256), 256, 128, 4, P(256), need, None) == 1
    assert L.mx_pack_weight_codes(P(264), P(256), P(256), 256, 128, 4, P(256), need, None) == 3
    assert L.mx_pack_weight_codes(P(256), P(256), P(256), 256, 128, 4, P(128), need, None) == 3
    assert L.mx_pack_weight_codes(P(256), P(256), P(256), 256, 128, 4, P(256), need - 1, None) == 5


def test_grouped_validation(L):
    P = ctypes.c_void_p
    z = [P(256)] * 6
    args = lambda k, E, ws: (P(256), 8, 256, 128, P(256), P(256), k, E, *z, None, None, 0, None, P(256), P(256), ws, None)
    assert L.mx_grouped_expert_mlp(*args(0, 4, 1 << 30)) == 2
    assert L.mx_grouped_expert_mlp(*args(5, 4, 1 << 30)) == 2
    assert L.mx_grouped_expert_mlp(*args(2, 2000, 1 << 30)) == 2
    need = L.mx_grouped_expert_mlp_workspace_size(8, 256, 128, 2, 4, 0)
    assert L.mx_grouped_expert_mlp(*args(2, 4, need - 1)) == 5
    nv = lambda g: (P(256), 8, 256, 128, P(256), P(256), 2, 4, *z, None, None, 2, g, P(256), P(256), 1 << 30, None)
    assert L.mx_grouped_expert_mlp(*nv(None)) == 1                  # NVFP4 without its global
    assert L.mx_grouped_expert_mlp(*nv(P(258))) == 3
    # workspace grows with tokens and with k
    a = L.mx_grouped_expert_mlp_workspace_size(64, 256, 128, 2, 4, 0)
    b = L.mx_grouped_expert_mlp_workspace_size(128, 256, 128, 2, 4, 0)
    c = L.mx_grouped_expert_mlp_workspace_size(64, 256, 128, 4, 4, 0)
    assert b > a and c > a


def test_nvfp4_global_warmup_validation(L):
    P = ctypes.c_void_p
    z = [P(256)] * 4

    def call(ids, k, E, g, ws):
        return L.mx_nvfp4_global_warmup(P(256), 8, 256, 128, ids, P(256), k, E, *z, None, g, P(256), ws, None)
    need_dense = L.mx_nvfp4_global_warmup_workspace_size(8, 256, 128, 0, 1)
    need_routed = L.mx_nvfp4_global_warmup_workspace_size(8, 256, 128, 2, 4)
    assert 0 < need_dense < need_routed
    assert call(None, 2, 4, P(256), 1 << 30) == 2           # one expert takes k = 0
    assert call(P(256), 0, 4, P(256), 1 << 30) == 2         # routed: 1 <= k <= E
    assert call(P(256), 5, 4, P(256), 1 << 30) == 2
    assert call(None, 0, 1, None, 1 << 30) == 1             # no output word
    assert call(None, 0, 1, P(258), 1 << 30) == 3           # misaligned output word
    assert call(None, 0, 1, P(256), need_dense - 1) == 5
    assert call(P(256), 2, 4, P(256), need_routed - 1) == 5
    assert "workspace" in _err(L)


def test_debug_gemm_validation(L):
    P = ctypes.c_void_p
    assert L.mx_debug_gemm_f32(P(256), P(256), P(256), P(256), 4, 6, 256, P(256), None) == 2
    assert L.mx_debug_gemm_f32(P(256), P(256), P(256), P(256), 4, 8, 64, P(256), None) == 2
    assert L.mx_debug_gemm_f32(None, P(256), P(256), P(256), 4, 8, 256, P(256), None) == 1
    assert L.mx_debug_gemm_f32(P(257), P(256), P(256), P(256), 4, 8, 256, P(256), None) == 3


def test_fp8_linear_validation(L):
    P = ctypes.c_void_p

    def call(M, K, N, ws, x=P(256), w=P(256), y=P(256)):
        return L.mx_fp8_block_linear(x, M, K, w, P(256), N, y, P(256), ws, None)
    need = L.mx_fp8_block_linear_workspace_size(8, 256)
    assert need >= 8 * 256 + 8 * 8
    assert call(8, 200, 128, 1 << 30) == 2            # K % 128
    assert call(8, 256, 100, 1 << 30) == 2            # N % 128
    assert call(8, 8320, 128, 1 << 30) == 2           # K above 8192
    assert call(0, 256, 128, 0) == 0                  # nothing to do
    assert call(8, 256, 128, 1 << 30, x=None) == 1
    assert call(8, 256, 128, 1 << 30, w=P(264)) == 3
    assert call(8, 256, 128, need - 1) == 5
    assert "workspace" in _err(L)


def test_quantize_mxfp8_validation(L):
    P = ctypes.c_void_p
    assert L.mx_quantize_act(3, P(256), 4, 48, None, P(256), P(256), None) == 2     # cols % 32
    assert L.mx_quantize_act(3, P(256), 4, 64, None, P(264), P(256), None) == 3     # codes alignment
    assert L.mx_quantize_act(9, P(256), 4, 64, None, P(256), P(256), None) == 4     # unknown format


def test_runner_validation(L):
    P = ctypes.c_void_p
    z = [P(256)] * 6
    out = P()

    def create(T, k, E, x=P(256), o=True):
        return L.mx_moe_runner_create(x, T, 256, 128, P(256), P(256), k, E, *z, None, None, 0, None, P(256),
                                      ctypes.byref(out) if o else None)
    assert create(8, 2, 4, o=False) == 1
    assert create(0, 2, 4) == 2 and out.value is None
    assert create(8, 5, 4) == 2
    assert L.mx_moe_runner_replay(None, None) == 1
    assert L.mx_moe_runner_destroy(None) == 0


def test_fp8_expert_mlp_validation(L):
    P = ctypes.c_void_p
    z = [P(256)] * 6

    def call(M, H, I, ws, x=P(256)):
        return L.mx_fp8_expert_mlp(x, M, H, I, *z, P(256), P(256), ws, None)
    need = L.mx_fp8_expert_mlp_workspace_size(8, 256, 128)
    assert need > 0
    assert call(8, 200, 128, 1 << 30) == 2
    assert call(8, 256, 8320, 1 << 30) == 2
    assert call(0, 256, 128, 0) == 0
    assert call(8, 256, 128, 1 << 30, x=None) == 1
    assert call(8, 256, 128, need - 1) == 5


def test_nvfp4_linear_validation(L):
    P = ctypes.c_void_p

    def call(M, K, N, wg, xg, ws, x=P(256), wsc=P(256)):
        return L.mx_nvfp4_linear(x, M, K, P(256), wsc, wg, N, xg, P(256), P(256), ws, None)
    need = L.mx_nvfp4_linear_workspace_size(8, 256)
    assert need >= 8 * 128 + 8 * 16
    assert call(8, 200, 128, 1.0, 1.0, 1 << 30) == 2
    assert call(8, 256, 100, 1.0, 1.0, 1 << 30) == 2
    assert call(8, 256, 128, 1.0, 0.0, 1 << 30) == 7          # activation global
    assert call(8, 256, 128, float("inf"), 1.0, 1 << 30) == 7  # weight global
    assert call(0, 256, 128, 1.0, 1.0, 0) == 0
    assert call(8, 256, 128, 1.0, 1.0, 1 << 30, x=None) == 1
    assert call(8, 256, 128, 1.0, 1.0, 1 << 30, wsc=P(257)) == 3
    assert call(8, 256, 128, 1.0, 1.0, need - 1) == 5


def test_nvfp4_expert_mlp_validation(L):
    P = ctypes.c_void_p

    def call(M, H, I, ws, wg=1.0, hg=1.0, x=P(256), s3=P(256)):
        return L.mx_nvfp4_expert_mlp(x, M, H, I, P(256), P(256), wg, P(256), s3, 1.0, P(256), P(256), 1.0,
                                     1.0, hg, P(256), P(256), ws, None)
    need = L.mx_nvfp4_expert_mlp_workspace_size(8, 256, 128)
    assert need > 0
    assert call(8, 200, 128, 1 << 30) == 2
    assert call(8, 256, 128, 1 << 30, wg=0.0) == 7
    assert call(8, 256, 128, 1 << 30, hg=float("nan")) == 7
    assert call(0, 256, 128, 0) == 0
    assert call(8, 256, 128, 1 << 30, x=None) == 1
    assert call(8, 256, 128, 1 << 30, s3=P(257)) == 3
    assert call(8, 256, 128, need - 1) == 5


def test_grouped_nvfp4_validation(L):
    P = ctypes.c_void_p

    def call(k, E, ws, xg=1.0, g1=P(256), s1=P(256)):
        return L.mx_grouped_nvfp4_expert_mlp(P(256), 8, 256, 128, P(256), P(256), k, E, P(256), s1, g1, P(256),
                                             P(256), P(256), P(256), P(256), P(256), xg, 1.0, P(256), P(256), ws,
                                             None)
    need = L.mx_grouped_nvfp4_expert_mlp_workspace_size(8, 256, 128, 2, 4)
    assert need > 0
    assert call(0, 4, 1 << 30) == 2
    assert call(5, 4, 1 << 30) == 2
    assert call(2, 4, 1 << 30, xg=0.0) == 7
    assert call(2, 4, 1 << 30, g1=None) == 1
    assert call(2, 4, 1 << 30, s1=P(257)) == 3
    assert call(2, 4, need - 1) == 5



def test_noalloc_validation(L):
    """The no-allocation shared expert checks its arguments like mx_expert_mlp and
    refuses sizes whose workspace exceeds its fixed scratch, before touching the GPU."""
    P = ctypes.c_void_p
    z = [P(256)] * 6
    limit = L.mx_expert_mlp_noalloc_max_bytes()
    assert limit == 64 << 20
    assert L.mx_expert_mlp_noalloc(P(256), 4, 200, 128, *z, None, None, 0, None, P(256), None) == 2
    assert L.mx_expert_mlp_noalloc(P(256), 4, 256, 128, *z, None, None, 2, None, P(256), None) == 1
    assert L.mx_expert_mlp_noalloc(None, 0, 256, 128, *([None] * 8), 0, None, None, None) == 0
    big = 1
    while L.mx_expert_mlp_workspace_size(big, 7168, 3072, 0) <= limit:
        big *= 2
    assert L.mx_expert_mlp_noalloc(P(256), big, 7168, 3072, *z, None, None, 0, None, P(256), None) == 5
    assert "no-allocation" in _err(L)


def test_probe_validation(L):
    """The measurement probes reject bad sizes, modes and pointers on the host."""
    P = ctypes.c_void_p
    assert L.mx_probe_mfma_fp4(P(256), 0, 4, P(256), None) == 7
    assert L.mx_probe_mfma_fp4(P(256), (1 << 20) + 1, 4, P(256), None) == 7
    assert L.mx_probe_mfma_fp4(P(256), 8, 0, P(256), None) == 7
    assert L.mx_probe_mfma_fp4(None, 8, 4, P(256), None) == 1
    assert L.mx_probe_mfma_fp4(P(264), 8, 4, P(256), None) == 3
    assert L.mx_probe_read(2, 8, 4, P(256), 8192, P(256), None) == 7
    assert L.mx_probe_read(0, 16, 4, P(256), 8192, P(256), None) == 7
    assert L.mx_probe_read(0, 8, 4, P(256), 8192 + 1024, P(256), None) == 2
    assert L.mx_probe_read(1, 32, 4, P(256), 8192, P(256), None) == 2
    assert L.mx_probe_read(0, 8, 4, P(256), 0, P(256), None) == 2
    assert L.mx_probe_read(0, 8, 4, None, 8192, P(256), None) == 1
    assert L.mx_probe_read(0, 8, 4, P(264), 8192, P(256), None) == 3
    assert L.mx_probe_copy(P(256), P(4096), 24, None) == 2
    assert L.mx_probe_copy(P(256), P(512), 512, None) == 7 and "overlap" in _err(L)
    assert L.mx_probe_copy(P(256), P(4096), 0, None) == 0
    assert L.mx_probe_copy(P(264), P(4096), 512, None) == 3


def test_status_strings_every_value(L):
    names = [L.mx_status_string(s).decode() for s in range(8)]
    assert len(set(names)) == 8 and "unknown status" not in names
    for s in (8, 99, -1, 2**31 - 1):
        assert L.mx_status_string(s) == b"unknown status"


def test_size_queries_over_shapes(L):
    """Every workspace and packing size query over a grid of shapes: positive for
    valid sizes, 0 for invalid ones (the host carving code, also under the
    sanitizers)."""
    for M in (1, 8, 9, 96, 97, 128, 300, 4096):
        for H, I in ((256, 128), (640, 384), (7168, 3072)):
            for rq in (0, 2):
                assert L.mx_expert_mlp_workspace_size(M, H, I, rq) > 0
            assert L.mx_nvfp4_expert_mlp_workspace_size(M, H, I) > 0
            assert L.mx_fp8_expert_mlp_workspace_size(M, H, I) > 0
            assert L.mx_fp8_block_linear_workspace_size(M, H) > 0
            assert L.mx_nvfp4_linear_workspace_size(M, H) > 0
            assert L.mx_nvfp4_global_warmup_workspace_size(M, H, I, 0, 1) > 0
            for k, E in ((1, 1), (2, 8), (8, 48)):
                for rq in (0, 2):
                    assert L.mx_grouped_expert_mlp_workspace_size(M, H, I, k, E, rq) > 0
                assert L.mx_grouped_nvfp4_expert_mlp_workspace_size(M, H, I, k, E) > 0
                assert L.mx_nvfp4_global_warmup_workspace_size(M, H, I, k, E) > 0
                assert L.mx_packed_weight_scales_size(H, I, E) > 0
                assert L.mx_packed_weight_codes_size(H, I, E) > 0
    assert L.mx_expert_mlp_workspace_size(-1, 256, 128, 0) == 0
    assert L.mx_grouped_expert_mlp_workspace_size(8, 256, 128, 0, 4, 0) == 0
    assert L.mx_packed_weight_codes_size(256, 128, 0) == 0


def test_profiler_toggle_without_launches(L):
    from mxfp4_block_scaled_e2m1_amd import binding
    n = ctypes.c_int32(-1)
    buf = (binding.PhaseStat * 4)()
    assert L.mx_profile_start() == 0
    assert L.mx_profile_stop(buf, 4, ctypes.byref(n)) == 0 and n.value == 0
    assert L.mx_profile_stop(None, 0, ctypes.byref(n)) == 0 and n.value == 0


def test_runner_create_reaches_allocation(L):
    """Arguments that pass the checks reach the runner's allocation: on a machine
    without a GPU that fails with MX_ERR_HIP and the partly built runner is
    released (host paths only)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("needs a machine without a GPU")
    P = ctypes.c_void_p
    out = P()
    st = L.mx_moe_runner_create(P(256), 8, 256, 128, P(256), P(256), 2, 4, *([P(256)] * 6), None, None, 0, None,
                                P(256), ctypes.byref(out))
    assert st == 6 and out.value is None and _err(L)
