"""mx_expert_mlp_noalloc (the shared expert on the library's fixed device scratch,
for callers that cannot allocate) against mx_expert_mlp with a caller workspace:
the same kernels, so the outputs must be bit-identical. Two calls in a row on the
one scratch array, the second smaller, and the limit's error path."""

import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import bf16_t, bits, t

pytestmark = pytest.mark.gpu

NAMES = ("w1", "w1s", "w3", "w3s", "w2", "w2s")


@pytest.fixture(scope="module")
def mx():
    import mxfp4_block_scaled_e2m1_amd as m
    return m


def _noalloc_abi(mx, x, w, y, requant=0, g=None, pk=None):
    """mx_expert_mlp_noalloc straight through the C ABI (ctypes)."""
    L = mx.lib()
    P = lambda a: ctypes.c_void_p(a.data_ptr()) if a is not None else None
    M, H = x.shape
    I = w["w1"].shape[0]
    st = L.mx_expert_mlp_noalloc(P(x), M, H, I, *(P(w[n]) for n in NAMES), P(pk), None, requant, P(g), P(y),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, L.mx_last_error().decode()


@pytest.mark.parametrize("requant", ["mxfp4", "nvfp4"])
def test_noalloc_matches_workspace_entry_point(mx, requant):
    H, I = W.HIDDEN, W.INTER
    d = W.expert_weights(0)
    w = {n: t(d[n]) for n in NAMES}
    pk = mx.pack_weight_scales(w["w1s"], w["w3s"], w["w2s"])
    rq = {"mxfp4": 0, "nvfp4": 2}[requant]
    g = torch.tensor([2.0 ** -6], dtype=torch.float32, device="cuda") if requant == "nvfp4" else None
    # first call: 1024 tokens (tiled GEMMs); second, smaller: 8 tokens (few-token kernels with
    # MXFP4 re-quantisation, the GEMMs with NVFP4), on the scratch the first call left behind
    for M in (1024, 8):
        x = bf16_t(W.activations(5 + M, M))
        ref = mx.expert_mlp(x, *(w[n] for n in NAMES), requant=requant, requant_global=g, packed_scales=pk)
        y = torch.full((M, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        st, err = _noalloc_abi(mx, x, w, y, rq, g, pk)
        assert st == 0, err
        torch.cuda.synchronize()
        assert np.array_equal(bits(y), bits(ref)), (requant, M)


def test_noalloc_routes_through_the_binding_and_rejects_sizes_above_the_limit(mx):
    d = W.shared_expert(40, seed=3, hidden=1024, inter=512)
    w = {n: t(d[n]) for n in NAMES}
    x = bf16_t(d["x"])
    ref = mx.expert_mlp(x, *(w[n] for n in NAMES))
    y = mx.expert_mlp_noalloc(x, *(w[n] for n in NAMES))
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(ref))
    # 20000 tokens at the real shape need more than the 64 MiB scratch: refused, nothing enqueued
    L = mx.lib()
    limit = L.mx_expert_mlp_noalloc_max_bytes()
    assert limit == 64 << 20
    assert L.mx_expert_mlp_workspace_size(20000, W.HIDDEN, W.INTER, 0) > limit
    P = ctypes.c_void_p
    z = [P(256)] * 6
    st = L.mx_expert_mlp_noalloc(P(256), 20000, W.HIDDEN, W.INTER, *z, None, None, 0, None, P(256), None)
    assert st == 5 and "no-allocation" in L.mx_last_error().decode()
