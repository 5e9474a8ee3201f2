"""Block-scaled FP4 (MXFP4: E2M1 x E8M0) expert MLP for AMD MI355X (gfx950).

The compute path is the HIP library ``libmxfp4.so`` (C ABI in
``include/mxfp4.h``); ``binding`` marshals torch device tensors into it.
"""

from .binding import (  # noqa: F401
    MoeRunner, MxError, debug_gemm_f32, dequant, expert_mlp, expert_mlp_noalloc, expert_mlp_workspace_size,
    fp8_block_linear,
    fp8_block_linear_workspace_size, fp8_expert_mlp, fp8_expert_mlp_workspace_size, grouped_expert_mlp,
    grouped_expert_mlp_workspace_size, grouped_nvfp4_expert_mlp, grouped_nvfp4_expert_mlp_workspace_size, lib, nvfp4_global_warmup, nvfp4_linear, nvfp4_linear_workspace_size,
    nvfp4_expert_mlp, nvfp4_expert_mlp_workspace_size, pack_weight_codes, pack_weight_scales,
    packed_weight_codes_size, packed_weight_scales_size, probe_copy, probe_mfma_fp4, probe_read, profile_start, profile_stop, quantize_act,
)

__all__ = [
    "MoeRunner", "MxError", "debug_gemm_f32", "dequant", "expert_mlp", "expert_mlp_noalloc", "expert_mlp_workspace_size",
    "fp8_block_linear",
    "fp8_block_linear_workspace_size", "fp8_expert_mlp", "fp8_expert_mlp_workspace_size",
    "grouped_expert_mlp", "grouped_expert_mlp_workspace_size",
    "grouped_nvfp4_expert_mlp", "grouped_nvfp4_expert_mlp_workspace_size", "lib", "nvfp4_global_warmup", "nvfp4_linear", "nvfp4_linear_workspace_size",
    "nvfp4_expert_mlp", "nvfp4_expert_mlp_workspace_size", "pack_weight_codes", "pack_weight_scales",
    "packed_weight_codes_size", "packed_weight_scales_size", "probe_copy", "probe_mfma_fp4", "probe_read", "profile_start", "profile_stop",
    "quantize_act",
]
