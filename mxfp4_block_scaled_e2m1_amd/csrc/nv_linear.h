// The bf16-MFMA GEMM of gemm_nv.hip with NVFP4 weights (E2M1 codes, E4M3 per
// 16 columns in wa_s [n_rows, k/16]) and NVFP4 token rows (x codes, x_s E4M3
// [rows, k/16]): out_bf16 = bf16(nv_global * sum (code s)(code s)), nv_global
// the product of the two fp32 global scales. Dense or routed tile lists as
// for launch_gemm_nv_l2.
#pragma once

#include "mx_internal.h"

namespace mx {

hipError_t launch_gemm_nv_w(const GemmArgs& a, int max_tiles, hipStream_t s);

// The fused gate/up L1 of the NVFP4-weight expert MLP on the same kernel: gate
// rows wa/wa_s and up rows wb/wb_s (n_rows = inter each, tiles of 128 j,
// n_tiles = ceil(inter / 128)); h = bf16(silu(bf16(gate * sg)) * bf16(up * su))
// with sg = nv_global (* e_global[e]) and su = nv_global2 (* e_global2[e]),
// re-quantised to NVFP4 with h_nv_global into h_codes [rows, inter/2] and
// h_scales [rows, inter/16] (row-major, sorted rows for routed tiles).
hipError_t launch_gemm_nv_w_swiglu(const GemmArgs& a, int max_tiles, hipStream_t s);

}  // namespace mx
