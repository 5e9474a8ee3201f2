"""The oracle against what the pages and the mathematics fix (CPU only)."""

import pytest

import oracle.mx_oracle as O
import pins

CHECKS = [
    pins.check_e2m1_formula,
    pins.check_nibble8_negative_zero,
    pins.check_e8m0,
    pins.check_e4m3,
    pins.check_bf16_roundtrip,
    pins.check_bf16_rounding_random,
    pins.check_no_double_rounding,
    pins.check_format_shapes,
    pins.check_dequant_examples,
    pins.check_dequant_scale_columns,
    pins.check_dequant_all_bytes,
    pins.check_fp8_examples,
    pins.check_fp8_block_bruteforce,
    pins.check_quantize_examples,
    pins.check_quantize_exhaustive,
    pins.check_quantize_roundtrip,
    pins.check_nibble_balance,
    pins.check_e4m3_rne,
    pins.check_nvfp4_grid,
    pins.check_nvfp4_error_bound,
    pins.check_nvfp4_warmup_global,
    pins.check_gemm_integer,
    pins.check_gemm_bruteforce,
    pins.check_silu,
    pins.check_mlp_bruteforce,
    pins.check_grouped_reductions,
    pins.check_mxfp8_examples,
    pins.check_mxfp8_quantize_exhaustive,
    pins.check_mxfp8_roundtrip,
    pins.check_fp8_linear_bruteforce,
    pins.check_fp8_linear_unit_rows,
    pins.check_fp8_mlp_bruteforce,
    pins.check_nvfp4_linear_bruteforce,
    pins.check_nvfp4_mlp_composition,
    pins.check_grouped_nvfp4_reductions,
    pins.check_quantizers_nonfinite_blocks,
    pins.check_mlp_nan_propagation,
    pins.check_nvfp4_golden_block,
    pins.check_fp8_mlp_fraction_bruteforce,
    pins.check_nvfp4_mlp_fraction_bruteforce,
]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_pin(check):
    check(O)
