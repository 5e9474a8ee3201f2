// Device helpers shared by the gfx950 kernels of libmxfp4.
//
// Formats (page "2026-05-08 DeepSeek V4 Pro NVFP4 Quantization", sections
// "Script update" and "FP4 (E2M1) expert weight format confirmed"):
//   * E2M1 element: 4 bits, sign in bit 3, magnitudes 0 .5 1 1.5 2 3 4 6; code 8 is -0.
//   * Packed MXFP4 row: two elements per byte, element 2j in the low nibble.
//   * E8M0 scale byte b: 2^(b-127), one per row per 32 logical columns; 0xFF is NaN.
//
// The gfx950 scaled conversions used here were checked bit for bit on the
// device against the CPU oracle: V_CVT_SCALEF32_PK_BF16_FP4 for every byte
// and every finite scale byte, and V_CVT_SCALEF32_PK_FP4_{F32,BF16} on every
// bf16 magnitude below 8x the scale (round to nearest even, ties to the even
// code, saturation at 6, sign kept so that small negatives give code 8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

// E8M0 byte -> fp32 value 2^(b-127). Byte 0 is the fp32 subnormal 2^-127
// (fp32 denormals are kept by these kernels). Byte 255 maps to +inf; callers
// that can see 255 turn it into NaN themselves.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return __uint_as_float(b == 0 ? 0x00400000u : (b << 23));
}

// fp32 -> bf16 bits, round to nearest even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two fp32 -> two bf16 in a dword (lo in the low half), round to nearest even,
// with the gfx950 conversion instruction (one instruction instead of five per
// value). Finite values round exactly as f32_to_bf16_rne; a NaN stays a NaN
// but keeps the sign and payload bits the hardware gives it, where
// f32_to_bf16_rne returns 0x7FC0 (the dequant kernels, whose NaN output is
// compared bit for bit, use that one).
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Two E2M1 codes (byte `sel` of `src`) times 2^(sb-127) -> two bf16 packed in a dword.
template <int SEL>
__device__ __forceinline__ uint32_t dequant_pair(uint32_t src, float scale) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scale, SEL);
  return __builtin_bit_cast(uint32_t, r);
}

// Quantise a bf16 pair (packed dword) by the power-of-two scale `x`, writing
// the two codes into byte SEL of `old`. Valid for scale bytes 1..254.
template <int SEL>
__device__ __forceinline__ uint32_t quant_pair_bf16(uint32_t old, uint32_t pair, float x) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, __builtin_bit_cast(bf16x2, pair), x, SEL);
}

// Quantise two fp32 values already divided by their scale (|v| <= 8 or
// clamped), into byte SEL of `old`.
template <int SEL>
__device__ __forceinline__ uint32_t quant_pair_f32_unit(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Quantise a bf16 pair for E8M0 scale byte sb (any value 0..254). Byte 0
// (blocks whose amax is below 2^-124) pre-multiplies by 2^127, which is exact
// for such small inputs, and converts at unit scale.
template <int SEL>
__device__ __forceinline__ uint32_t quant_pair_e8m0(uint32_t old, uint32_t pair, uint32_t sb) {
  if (sb != 0) return quant_pair_bf16<SEL>(old, pair, __uint_as_float(sb << 23));
  const float up = 0x1p127f;
  return quant_pair_f32_unit<SEL>(old, bf16_to_f32(pair & 0xFFFFu) * up, bf16_to_f32(pair >> 16) * up);
}

// Quantise N bf16 pairs (N a multiple of 4) sharing the E8M0 scale byte sb
// into N/4 code dwords, as quant_pair_e8m0 per pair but with one branch for
// the whole group instead of one per pair (a divergent branch per pair costs
// more than the conversions it guards).
template <int N>
__device__ __forceinline__ void quant_pairs_e8m0(const uint32_t* p, uint32_t sb, uint32_t* out) {
  static_assert(N % 4 == 0, "whole code dwords");
  if (sb != 0) {
    const float x = __uint_as_float(sb << 23);
#pragma unroll
    for (int d = 0; d < N / 4; ++d) {
      uint32_t v = 0;
      v = quant_pair_bf16<0>(v, p[4 * d], x);
      v = quant_pair_bf16<1>(v, p[4 * d + 1], x);
      v = quant_pair_bf16<2>(v, p[4 * d + 2], x);
      v = quant_pair_bf16<3>(v, p[4 * d + 3], x);
      out[d] = v;
    }
  } else {
#pragma unroll
    for (int d = 0; d < N / 4; ++d) {
      uint32_t v = 0;
      v = quant_pair_e8m0<0>(v, p[4 * d], 0u);
      v = quant_pair_e8m0<1>(v, p[4 * d + 1], 0u);
      v = quant_pair_e8m0<2>(v, p[4 * d + 2], 0u);
      v = quant_pair_e8m0<3>(v, p[4 * d + 3], 0u);
      out[d] = v;
    }
  }
}

// MXFP4 shared-exponent scale byte from the bf16 bit pattern of the block's
// largest magnitude: floor(log2 amax) - 2 + 127, clamped at 0. For a bf16
// amax with exponent field ef this is max(ef - 2, 0); zero and subnormal
// maxima give 0. A block holding an infinity or a NaN (ef = 255: those bit
// patterns are the largest magnitudes) has no finite shared exponent and gets
// the E8M0 NaN byte 0xFF, so that the NaN travels on; its codes are then
// unspecified.
__device__ __forceinline__ uint32_t mx_scale_from_amax_bits(uint32_t amax_bits) {
  int ef = (int)((amax_bits >> 7) & 0xFFu);
  if (ef == 0xFF) return 0xFFu;
  return (uint32_t)(ef > 2 ? ef - 2 : 0);
}

// Max of the bf16 magnitudes held in a dword (two bf16), as bit patterns.
__device__ __forceinline__ uint32_t amax2(uint32_t w) {
  uint32_t a = w & 0x7FFFu, b = (w >> 16) & 0x7FFFu;
  return a > b ? a : b;
}

// E4M3 (e4m3fn) of r >= 0 (finite fp32), nearest with ties to even, results
// above 448 clamped to 448. Returns the byte.
__device__ __forceinline__ uint32_t e4m3_rne_satfinite(float r) {
  if (r >= 448.0f) return 0x7Eu;
  if (r < 0x1p-6f) {
    // subnormal range: quantum 2^-9; rintf rounds half to even; 8 -> 0x08 (2^-6)
    return (uint32_t)rintf(r * 512.0f);
  }
  uint32_t u = __float_as_uint(r);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  uint32_t e = (u >> 23) - 120u;   // biased e4m3 exponent (bias 7)
  uint32_t code = (e << 3) | ((u >> 20) & 7u);
  return code > 0x7Eu ? 0x7Eu : code;
}

// E4M3 (e4m3fn) byte -> fp32, exact; 0x7F and 0xFF give the NaN 0x7FC00000.
// Selects only (no branches), so that it can be scheduled among MFMAs.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float sub = (float)m * 0x1p-9f;
  const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  const float mag = e == 0u ? sub : nrm;
  const float v = (b & 0x80u) ? -mag : mag;
  return (e == 15u && m == 7u) ? __uint_as_float(0x7FC00000u) : v;
}

// silu(g) * u = g / (1 + e^-g) * u in fp32 with the hardware exp2 and
// reciprocal (a few ulp of fp32): the result is rounded to bf16 afterwards, so
// only values within a few fp32 ulp of a bf16 rounding boundary can round
// differently from the exact value. For g < -88.7 e^-g overflows and the
// product flushes to +-0 (the exact value is below 1e-36 there).
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

}  // namespace mx
