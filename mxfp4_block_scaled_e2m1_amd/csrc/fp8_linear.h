// Gate/up FP8 linear with SiLU * up fused (fp8_linear.hip): h [M, I] =
// bf16(silu(g) * u) with g = bf16(MXFP8(x) . w1^T) and u = bf16(MXFP8(x) . w3^T)
// rounded as the plain FP8 linear rounds its output, so h equals that of two
// launch_fp8_gemm calls and launch_silu_mul_bf16 bit for bit. xq, xs: the
// MXFP8 activations [M, K] and [M, K/32]; w1, w3 [I, K] E4M3 with w1s, w3s
// [I/128, K/128] E8M0. I % 128 == 0, K within fp8_linear_fits.
#pragma once

#include "mx_internal.h"

namespace mx {

hipError_t launch_fp8_swiglu(const uint8_t* xq, const uint8_t* xs, const uint8_t* w1, const uint8_t* w1s,
                             const uint8_t* w3, const uint8_t* w3s, int M, int I, int K, uint16_t* h,
                             hipStream_t s);

}  // namespace mx
