// The bf16-MFMA GEMM of gemm_nv.hip with NVFP4 weights (E2M1 codes, E4M3 per
// 16 columns in wa_s [n_rows, k/16]) and NVFP4 token rows (x codes, x_s E4M3
// [rows, k/16]): out_bf16 = bf16(nv_global * sum (code s)(code s)), nv_global
// the product of the two fp32 global scales. Dense or routed tile lists as
// for launch_gemm_nv_l2.
#pragma once

#include "mx_internal.h"

namespace mx {

hipError_t launch_gemm_nv_w(const GemmArgs& a, int max_tiles, hipStream_t s);

}  // namespace mx
