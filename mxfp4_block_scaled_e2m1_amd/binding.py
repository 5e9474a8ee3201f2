"""Thin ctypes binding of libmxfp4 (include/mxfp4.h): argument marshalling only.

Every step of the path runs in the HIP library; this module only turns torch
device tensors into pointers and the current torch stream into a hipStream_t,
and raises MxError when the library reports a failure. There is no fallback:
if the library is missing, calls raise.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# MXFP4_LIB selects another build of the same library (the host-sanitized copy
# the CPU tests load); by default the in-tree libmxfp4.so.
LIB_PATH = os.environ.get("MXFP4_LIB") or os.path.join(HERE, "libmxfp4.so")

MX_FMT = {"mxfp4": 0, "fp8_b128": 1, "nvfp4": 2, "mxfp8": 3}
STATUS = {0: "MX_OK", 1: "MX_ERR_NULL", 2: "MX_ERR_SHAPE", 3: "MX_ERR_ALIGN", 4: "MX_ERR_FORMAT",
          5: "MX_ERR_WORKSPACE", 6: "MX_ERR_HIP", 7: "MX_ERR_VALUE"}

#: name -> (restype, argtypes) for every symbol declared in include/mxfp4.h
_P, _I64, _I32, _F, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t


class PhaseStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("total_ms", ctypes.c_double), ("launches", ctypes.c_int64)]


SIGNATURES = {
    "mx_dequant": (_I32, [_I32, _P, _P, _P, _I64, _I64, _P, _P]),
    "mx_quantize_act": (_I32, [_I32, _P, _I64, _I64, _P, _P, _P, _P]),
    "mx_expert_mlp": (_I32, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _SZ, _P]),
    "mx_nvfp4_global_warmup": (_I32, [_P, _I64, _I64, _I64, _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                      _P]),
    "mx_nvfp4_global_warmup_workspace_size": (_SZ, [_I64, _I64, _I64, _I32, _I32]),
    "mx_expert_mlp_workspace_size": (_SZ, [_I64, _I64, _I64, _I32]),
    "mx_expert_mlp_noalloc": (_I32, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P]),
    "mx_expert_mlp_noalloc_max_bytes": (_SZ, []),
    "mx_grouped_expert_mlp": (_I32, [_P, _I64, _I64, _I64, _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _P,
                                     _P, _P, _I32, _P, _P, _P, _SZ, _P]),
    "mx_grouped_expert_mlp_workspace_size": (_SZ, [_I64, _I64, _I64, _I32, _I32, _I32]),
    "mx_pack_weight_scales": (_I32, [_P, _P, _P, _I64, _I64, _I32, _P, _SZ, _P]),
    "mx_packed_weight_scales_size": (_SZ, [_I64, _I64, _I32]),
    "mx_pack_weight_codes": (_I32, [_P, _P, _P, _I64, _I64, _I32, _P, _SZ, _P]),
    "mx_packed_weight_codes_size": (_SZ, [_I64, _I64, _I32]),
    "mx_debug_gemm_f32": (_I32, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "mx_fp8_block_linear": (_I32, [_P, _I64, _I64, _P, _P, _I64, _P, _P, _SZ, _P]),
    "mx_fp8_block_linear_workspace_size": (_SZ, [_I64, _I64]),
    "mx_nvfp4_linear": (_I32, [_P, _I64, _I64, _P, _P, _F, _I64, _F, _P, _P, _SZ, _P]),
    "mx_nvfp4_linear_workspace_size": (_SZ, [_I64, _I64]),
    "mx_nvfp4_expert_mlp": (_I32, [_P, _I64, _I64, _I64, _P, _P, _F, _P, _P, _F, _P, _P, _F, _F, _F, _P, _P, _SZ,
                                   _P]),
    "mx_nvfp4_expert_mlp_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "mx_grouped_nvfp4_expert_mlp": (_I32, [_P, _I64, _I64, _I64, _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _F, _F, _P, _P, _SZ, _P]),
    "mx_grouped_nvfp4_expert_mlp_workspace_size": (_SZ, [_I64, _I64, _I64, _I32, _I32]),
    "mx_fp8_expert_mlp": (_I32, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "mx_fp8_expert_mlp_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "mx_moe_runner_create": (_I32, [_P, _I64, _I64, _I64, _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _I32, _P, _P, ctypes.POINTER(_P)]),
    "mx_moe_runner_replay": (_I32, [_P, _P]),
    "mx_moe_runner_destroy": (_I32, [_P]),
    "mx_status_string": (ctypes.c_char_p, [_I32]),
    "mx_last_error": (ctypes.c_char_p, []),
    "mx_profile_start": (_I32, []),
    "mx_profile_stop": (_I32, [ctypes.POINTER(PhaseStat), _I32, ctypes.POINTER(_I32)]),
    "mx_probe_mfma_fp4": (_I32, [_P, _I64, _I32, _P, _P]),
    "mx_probe_read": (_I32, [_I32, _I32, _I32, _P, _I64, _P, _P]),
    "mx_probe_copy": (_I32, [_P, _P, _I64, _P]),
}

_lib = None


class MxError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


def lib():
    """Load libmxfp4.so (built in-tree). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mxfp4_block_scaled_e2m1_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise MxError(status, lib().mx_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmxfp4 takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmxfp4 takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _fmt(f) -> int:
    return MX_FMT[f] if isinstance(f, str) else int(f)


def _global(g, device):
    """An NVFP4 global scale as the library takes it: a one-element fp32 device
    tensor (passed through), a Python float (copied into a new device tensor),
    or None. Returns the tensor, which the caller keeps alive until the call
    that reads it has run (stream order makes a temporary safe)."""
    if g is None:
        return None
    if isinstance(g, torch.Tensor):
        if g.dtype != torch.float32 or g.numel() != 1:
            raise ValueError("a global scale tensor must hold one fp32 value")
        return g
    return torch.tensor([float(g)], dtype=torch.float32, device=device)


# ---------------------------------------------------------------------------

def dequant(fmt, codes, scales, rows: int, cols: int, global_scale=None, out=None, stream=None):
    """mx_dequant -> bf16 tensor [rows, cols]. global_scale (NVFP4): float or
    one-element fp32 device tensor."""
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=codes.device)
    g = _global(global_scale, codes.device)
    _check(lib().mx_dequant(_fmt(fmt), _ptr(codes), _ptr(scales), _ptr(g), rows, cols,
                            _ptr(out), _stream(stream)))
    return out


def quantize_act(fmt, x, global_scale=None, codes=None, scales=None, stream=None):
    """mx_quantize_act: bf16 x [rows, cols] -> (codes [rows, cols/2], or [rows, cols]
    for MXFP8, scales). global_scale (NVFP4): float or one-element fp32 device tensor."""
    rows, cols = x.shape
    f = _fmt(fmt)
    per = 16 if f == MX_FMT["nvfp4"] else 32
    if codes is None:
        width = cols if f == MX_FMT["mxfp8"] else cols // 2
        codes = torch.empty((rows, width), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // per), dtype=torch.uint8, device=x.device)
    g = _global(global_scale, x.device)
    _check(lib().mx_quantize_act(f, _ptr(x), rows, cols, _ptr(g), _ptr(codes), _ptr(scales),
                                 _stream(stream)))
    return codes, scales


def expert_mlp_workspace_size(M, hidden, inter, requant="mxfp4") -> int:
    return int(lib().mx_expert_mlp_workspace_size(M, hidden, inter, _fmt(requant)))


def grouped_expert_mlp_workspace_size(T, hidden, inter, k, E, requant="mxfp4") -> int:
    return int(lib().mx_grouped_expert_mlp_workspace_size(T, hidden, inter, k, E, _fmt(requant)))


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def packed_weight_scales_size(hidden, inter, E=1) -> int:
    return int(lib().mx_packed_weight_scales_size(hidden, inter, E))


def pack_weight_scales(w1s, w3s, w2s, out=None, stream=None):
    """mx_pack_weight_scales: tile-major copy of the weight scales of one expert
    (w1s [inter, hidden/32]) or of E stacked experts (w1s [E, inter, hidden/32])."""
    E = w1s.shape[0] if w1s.dim() == 3 else 1
    inter, hidden = w1s.shape[-2], 32 * w1s.shape[-1]
    nbytes = packed_weight_scales_size(hidden, inter, E)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w1s.device)
    _check(lib().mx_pack_weight_scales(_ptr(w1s), _ptr(w3s), _ptr(w2s), hidden, inter, E, _ptr(out),
                                       out.numel(), _stream(stream)))
    return out


def packed_weight_codes_size(hidden, inter, E=1) -> int:
    return int(lib().mx_packed_weight_codes_size(hidden, inter, E))


def pack_weight_codes(w1, w3, w2, out=None, stream=None):
    """mx_pack_weight_codes: tile-major copy of the weight codes of one expert
    (w1 [inter, hidden/2]) or of E stacked experts (w1 [E, inter, hidden/2])."""
    E = w1.shape[0] if w1.dim() == 3 else 1
    inter, hidden = w1.shape[-2], 2 * w1.shape[-1]
    nbytes = packed_weight_codes_size(hidden, inter, E)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w1.device)
    _check(lib().mx_pack_weight_codes(_ptr(w1), _ptr(w3), _ptr(w2), hidden, inter, E, _ptr(out), out.numel(),
                                      _stream(stream)))
    return out


def expert_mlp(x, w1, w1s, w3, w3s, w2, w2s, requant="mxfp4", requant_global=None,
               out=None, workspace=None, stream=None, packed_scales=None, packed_codes=None):
    """mx_expert_mlp: the shared expert on bf16 x [M, hidden] -> bf16 y [M, hidden].
    requant_global (NVFP4): float or one-element fp32 device tensor."""
    M, hidden = x.shape
    inter = w1.shape[0]
    if out is None:
        out = torch.empty((M, hidden), dtype=torch.bfloat16, device=x.device)
    nbytes = expert_mlp_workspace_size(M, hidden, inter, requant)
    ws = _workspace(nbytes, x.device, workspace)
    g = _global(requant_global, x.device)
    _check(lib().mx_expert_mlp(_ptr(x), M, hidden, inter, _ptr(w1), _ptr(w1s), _ptr(w3), _ptr(w3s),
                               _ptr(w2), _ptr(w2s), _ptr(packed_scales), _ptr(packed_codes), _fmt(requant),
                               _ptr(g), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def expert_mlp_noalloc(x, w1, w1s, w3, w3s, w2, w2s, requant="mxfp4", requant_global=None, out=None,
                       stream=None, packed_scales=None, packed_codes=None):
    """mx_expert_mlp_noalloc: mx_expert_mlp on the library's fixed device scratch
    (no workspace argument; calls on one GPU must not overlap)."""
    M, hidden = x.shape
    inter = w1.shape[0]
    if out is None:
        out = torch.empty((M, hidden), dtype=torch.bfloat16, device=x.device)
    g = _global(requant_global, x.device)
    _check(lib().mx_expert_mlp_noalloc(_ptr(x), M, hidden, inter, _ptr(w1), _ptr(w1s), _ptr(w3), _ptr(w3s),
                                       _ptr(w2), _ptr(w2s), _ptr(packed_scales), _ptr(packed_codes),
                                       _fmt(requant), _ptr(g), _ptr(out), _stream(stream)))
    return out


def grouped_expert_mlp(x, topk_ids, topk_w, w1, w1s, w3, w3s, w2, w2s, requant="mxfp4",
                       requant_global=None, out=None, workspace=None, stream=None, packed_scales=None,
                       packed_codes=None):
    """mx_grouped_expert_mlp: routed experts, stacked weights [E, ...]. requant_global
    (NVFP4): float or one-element fp32 device tensor."""
    T, hidden = x.shape
    k = topk_ids.shape[1]
    E, inter = w1.shape[0], w1.shape[1]
    if out is None:
        out = torch.empty((T, hidden), dtype=torch.bfloat16, device=x.device)
    nbytes = grouped_expert_mlp_workspace_size(T, hidden, inter, k, E, requant)
    ws = _workspace(nbytes, x.device, workspace)
    g = _global(requant_global, x.device)
    _check(lib().mx_grouped_expert_mlp(_ptr(x), T, hidden, inter, _ptr(topk_ids), _ptr(topk_w), k, E,
                                       _ptr(w1), _ptr(w1s), _ptr(w3), _ptr(w3s), _ptr(w2), _ptr(w2s),
                                       _ptr(packed_scales), _ptr(packed_codes), _fmt(requant), _ptr(g),
                                       _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def nvfp4_global_warmup(x, w1, w1s, w3, w3s, topk_ids=None, topk_w=None, packed_scales=None, out=None,
                        workspace=None, stream=None):
    """mx_nvfp4_global_warmup: g = f32(max |h| / (6 * 448)) of a warm-up batch, as a
    one-element fp32 device tensor. One expert (w1 [inter, hidden/2]) when
    topk_ids is None, else routed over stacked weights [E, ...]."""
    T, hidden = x.shape
    routed = topk_ids is not None
    inter = w1.shape[-2]
    k = topk_ids.shape[1] if routed else 0
    E = w1.shape[0] if routed else 1
    if out is None:
        out = torch.empty((1,), dtype=torch.float32, device=x.device)
    nbytes = int(lib().mx_nvfp4_global_warmup_workspace_size(T, hidden, inter, k, E))
    ws = _workspace(nbytes, x.device, workspace)
    _check(lib().mx_nvfp4_global_warmup(_ptr(x), T, hidden, inter, _ptr(topk_ids), _ptr(topk_w), k, E,
                                        _ptr(w1), _ptr(w1s), _ptr(w3), _ptr(w3s), _ptr(packed_scales), _ptr(out),
                                        _ptr(ws), ws.numel(), _stream(stream)))
    return out


def debug_gemm_f32(a, a_s, b, b_s, out=None, stream=None):
    """mx_debug_gemm_f32: C [M, N] = A . B^T for MXFP4 A [M, K/2] and B [N, K/2]."""
    M, N, K = a.shape[0], b.shape[0], 2 * a.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    _check(lib().mx_debug_gemm_f32(_ptr(a), _ptr(a_s), _ptr(b), _ptr(b_s), M, N, K, _ptr(out),
                                   _stream(stream)))
    return out


def profile_start():
    _check(lib().mx_profile_start())


def profile_stop():
    """Returns {kernel name: (total_ms, launches)} for launches since profile_start()."""
    buf = (PhaseStat * 64)()
    n = _I32(0)
    _check(lib().mx_profile_stop(buf, 64, ctypes.byref(n)))
    return {buf[i].name.decode(): (buf[i].total_ms, int(buf[i].launches)) for i in range(min(n.value, 64))}


def probe_mfma_fp4(operands, iters: int, workgroups: int, out=None, stream=None):
    """mx_probe_mfma_fp4: operands uint32 [512, 16] (device); returns float32 [workgroups, 512]."""
    if out is None:
        out = torch.empty((workgroups, 512), dtype=torch.float32, device=operands.device)
    _check(lib().mx_probe_mfma_fp4(_ptr(operands), iters, workgroups, _ptr(out), _stream(stream)))
    return out


def probe_read(src, mode: int, loads_per_wave: int, workgroups: int, out=None, stream=None):
    """mx_probe_read over all bytes of src; returns the per-wave XOR words (int32 [workgroups * 4])."""
    if out is None:
        out = torch.empty(workgroups * 4, dtype=torch.int32, device=src.device)
    nbytes = src.numel() * src.element_size()
    _check(lib().mx_probe_read(mode, loads_per_wave, workgroups, _ptr(src), nbytes, _ptr(out), _stream(stream)))
    return out


def probe_copy(src, dst, stream=None):
    """mx_probe_copy: dst = src (same byte size)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    _check(lib().mx_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))
    return dst


def fp8_block_linear_workspace_size(M, K) -> int:
    return int(lib().mx_fp8_block_linear_workspace_size(M, K))


def fp8_block_linear(x, w, w_s, out=None, workspace=None, stream=None):
    """mx_fp8_block_linear: bf16 x [M, K], E4M3 w [N, K], E8M0 w_s [N/128, K/128] -> bf16 y [M, N]."""
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    ws = _workspace(fp8_block_linear_workspace_size(M, K), x.device, workspace)
    _check(lib().mx_fp8_block_linear(_ptr(x), M, K, _ptr(w), _ptr(w_s), N, _ptr(out), _ptr(ws), ws.numel(),
                                     _stream(stream)))
    return out


def nvfp4_linear_workspace_size(M, K) -> int:
    return int(lib().mx_nvfp4_linear_workspace_size(M, K))


def nvfp4_linear(x, w, w_s, w_global: float, x_global: float, out=None, workspace=None, stream=None):
    """mx_nvfp4_linear: bf16 x [M, K], NVFP4 w [N, K/2] + E4M3 w_s [N, K/16] + w_global -> bf16 y [M, N]."""
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    ws = _workspace(nvfp4_linear_workspace_size(M, K), x.device, workspace)
    _check(lib().mx_nvfp4_linear(_ptr(x), M, K, _ptr(w), _ptr(w_s), float(w_global), N, float(x_global), _ptr(out),
                                 _ptr(ws), ws.numel(), _stream(stream)))
    return out


def nvfp4_expert_mlp_workspace_size(M, hidden, inter) -> int:
    return int(lib().mx_nvfp4_expert_mlp_workspace_size(M, hidden, inter))


def nvfp4_expert_mlp(x, w1, w1s, w1g, w3, w3s, w3g, w2, w2s, w2g, x_global, h_global, out=None, workspace=None,
                     stream=None):
    """mx_nvfp4_expert_mlp: one expert with NVFP4 weights on bf16 x [M, hidden] -> bf16 y [M, hidden]."""
    M, hidden = x.shape
    inter = w1.shape[0]
    if out is None:
        out = torch.empty((M, hidden), dtype=torch.bfloat16, device=x.device)
    ws = _workspace(nvfp4_expert_mlp_workspace_size(M, hidden, inter), x.device, workspace)
    _check(lib().mx_nvfp4_expert_mlp(_ptr(x), M, hidden, inter, _ptr(w1), _ptr(w1s), float(w1g), _ptr(w3),
                                     _ptr(w3s), float(w3g), _ptr(w2), _ptr(w2s), float(w2g), float(x_global),
                                     float(h_global), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def grouped_nvfp4_expert_mlp_workspace_size(T, hidden, inter, k, E) -> int:
    return int(lib().mx_grouped_nvfp4_expert_mlp_workspace_size(T, hidden, inter, k, E))


def grouped_nvfp4_expert_mlp(x, topk_ids, topk_w, w1, w1s, w1g, w3, w3s, w3g, w2, w2s, w2g, x_global, h_global,
                             out=None, workspace=None, stream=None):
    """mx_grouped_nvfp4_expert_mlp: routed experts with NVFP4 weights; w*g are device fp32 [E] tensors."""
    T, hidden = x.shape
    k = topk_ids.shape[1]
    E, inter = w1.shape[0], w1.shape[1]
    if out is None:
        out = torch.empty((T, hidden), dtype=torch.bfloat16, device=x.device)
    ws = _workspace(grouped_nvfp4_expert_mlp_workspace_size(T, hidden, inter, k, E), x.device, workspace)
    _check(lib().mx_grouped_nvfp4_expert_mlp(_ptr(x), T, hidden, inter, _ptr(topk_ids), _ptr(topk_w), k, E,
                                             _ptr(w1), _ptr(w1s), _ptr(w1g), _ptr(w3), _ptr(w3s), _ptr(w3g),
                                             _ptr(w2), _ptr(w2s), _ptr(w2g), float(x_global), float(h_global),
                                             _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def fp8_expert_mlp_workspace_size(M, hidden, inter) -> int:
    return int(lib().mx_fp8_expert_mlp_workspace_size(M, hidden, inter))


def fp8_expert_mlp(x, w1, w1s, w3, w3s, w2, w2s, out=None, workspace=None, stream=None):
    """mx_fp8_expert_mlp: the FP8 shared expert on bf16 x [M, hidden] -> bf16 y [M, hidden]."""
    M, hidden = x.shape
    inter = w1.shape[0]
    if out is None:
        out = torch.empty((M, hidden), dtype=torch.bfloat16, device=x.device)
    ws = _workspace(fp8_expert_mlp_workspace_size(M, hidden, inter), x.device, workspace)
    _check(lib().mx_fp8_expert_mlp(_ptr(x), M, hidden, inter, _ptr(w1), _ptr(w1s), _ptr(w3), _ptr(w3s), _ptr(w2),
                                   _ptr(w2s), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


class MoeRunner:
    """mx_moe_runner: the routed experts over fixed device buffers, captured once
    into a hipGraph. Refresh x, topk_ids, topk_w (and the NVFP4 global tensor) in
    place, then replay()."""

    def __init__(self, x, topk_ids, topk_w, w1, w1s, w3, w3s, w2, w2s, requant="mxfp4",
                 requant_global=None, out=None, packed_scales=None, packed_codes=None):
        T, hidden = x.shape
        k = topk_ids.shape[1]
        E, inter = w1.shape[0], w1.shape[1]
        self.out = out if out is not None else torch.empty((T, hidden), dtype=torch.bfloat16, device=x.device)
        g = _global(requant_global, x.device)
        # keep the bound tensors alive as long as the runner
        self._bound = (x, topk_ids, topk_w, w1, w1s, w3, w3s, w2, w2s, packed_scales, packed_codes, self.out, g)
        h = _P()
        _check(lib().mx_moe_runner_create(_ptr(x), T, hidden, inter, _ptr(topk_ids), _ptr(topk_w), k, E,
                                          _ptr(w1), _ptr(w1s), _ptr(w3), _ptr(w3s), _ptr(w2), _ptr(w2s),
                                          _ptr(packed_scales), _ptr(packed_codes), _fmt(requant), _ptr(g),
                                          _ptr(self.out), ctypes.byref(h)))
        self._h = h

    def replay(self, stream=None):
        _check(lib().mx_moe_runner_replay(self._h, _stream(stream)))
        return self.out

    def close(self):
        if self._h is not None and self._h.value is not None:
            _check(lib().mx_moe_runner_destroy(self._h))
        self._h = None

