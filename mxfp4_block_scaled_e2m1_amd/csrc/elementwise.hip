// Streaming dequant / quantise kernels (HBM-bound): 16-byte loads, VALU decode,
// 16-byte stores, grid-stride loops over blocks.
//
// * MXFP4 dequant: page "2026-05-08 DeepSeek V4 Pro NVFP4 Quantization", section
//   "Script update", item 2 (E2M1 codes two per byte, low nibble first, times the
//   E8M0 scale of each 32 columns; the output is twice as wide as the bytes).
// * FP8 block dequant: same page and section, item 1 (float8_e4m3fn times the
//   E8M0 scale of its 128 x 128 block).
// * MXFP4 quantise: shared exponent floor(log2 amax) - 2 per 32 elements, E2M1
//   round to nearest even with saturation (the OCP MX rule the activation
//   quantiser is named by; the pages only name "MXFP4 microscaling").
// * NVFP4 quantise/dequant: E2M1 with an E4M3 scale per 16 elements and an fp32
//   global scale (the pages run NVFP4 with a warm-up global scale, page
//   "Current Bug: vLLM produces empty/garbage output", "Revised Plan" Phase 1,
//   but never define it; the fp32 operation order below is the reading taken).
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

namespace {

constexpr int EW_THREADS = 256;

inline int ew_grid(int64_t work) {
  int64_t g = (work + EW_THREADS - 1) / EW_THREADS;
  if (g > 8192) g = 8192;
  return (int)(g < 1 ? 1 : g);
}

// One thread per 32-element block: 16 code bytes + 1 scale byte -> 64 output bytes.
__global__ __launch_bounds__(EW_THREADS) void k_dequant_mxfp4(const uint4* __restrict__ codes,
                                                              const uint8_t* __restrict__ scales,
                                                              uint4* __restrict__ out, int64_t nblk) {
  const int64_t stride = (int64_t)gridDim.x * EW_THREADS;
  for (int64_t b = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x; b < nblk; b += stride) {
    const uint4 c = codes[b];
    const uint32_t sb = scales[b];
    uint4 o[4];
    if (sb == 255u) {
      const uint4 nan4 = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
      o[0] = o[1] = o[2] = o[3] = nan4;
    } else {
      const float sc = e8m0_to_f32(sb);
      const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = make_uint4(dequant_pair<0>(w[i], sc), dequant_pair<1>(w[i], sc),
                          dequant_pair<2>(w[i], sc), dequant_pair<3>(w[i], sc));
    }
    uint4* dst = out + b * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = o[i];
  }
}

// e4m3 x 2^(sb-127) -> bf16, exact in fp32 (fp32 denormals kept) then one RNE.
__device__ __forceinline__ uint32_t fp8_to_bf16(uint32_t byte, float sc) {
  return f32_to_bf16_rne(e4m3_to_f32(byte) * sc);
}

// One thread per 16 elements (one 16-byte load) of a row; cols % 16 == 0.
__global__ __launch_bounds__(EW_THREADS) void k_dequant_fp8_block(const uint4* __restrict__ q,
                                                                  const uint8_t* __restrict__ scales,
                                                                  int64_t cols, int64_t gcols,
                                                                  uint4* __restrict__ out, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * EW_THREADS;
  const int64_t per_row = cols >> 4;
  for (int64_t i = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x; i < n16; i += stride) {
    const int64_t r = i / per_row;
    const int64_t c0 = (i - r * per_row) << 4;
    const uint32_t sb = scales[(r >> 7) * gcols + (c0 >> 7)];
    const uint4 v = q[i];
    uint4 o0, o1;
    if (sb == 255u) {
      o0 = o1 = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
    } else {
      const float sc = e8m0_to_f32(sb);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t p[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        p[2 * k] = fp8_to_bf16(w[k] & 0xFFu, sc) | (fp8_to_bf16((w[k] >> 8) & 0xFFu, sc) << 16);
        p[2 * k + 1] = fp8_to_bf16((w[k] >> 16) & 0xFFu, sc) | (fp8_to_bf16(w[k] >> 24, sc) << 16);
      }
      o0 = make_uint4(p[0], p[1], p[2], p[3]);
      o1 = make_uint4(p[4], p[5], p[6], p[7]);
    }
    out[2 * i] = o0;
    out[2 * i + 1] = o1;
  }
}

// fp64 -> bf16 with a single rounding: fp64 -> fp32 rounded to odd, then RNE to
// bf16 (fp32 keeps 16 more bits than bf16, so the two steps equal one RNE).
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double d) {
  float f = (float)d;   // RNE
  if ((double)f != d && !__builtin_isnan(d) && !__builtin_isinf(f)) {
    uint32_t u = __float_as_uint(f);
    if (fabs((double)f) > fabs(d)) u -= 1;   // step toward zero: truncation
    u |= 1u;                                 // sticky: odd
    f = __uint_as_float(u);
  }
  return f32_to_bf16_rne(f);
}

// NVFP4 dequant: one thread per 16 elements (8 code bytes, 1 E4M3 scale byte).
__global__ __launch_bounds__(EW_THREADS) void k_dequant_nvfp4(const uint2* __restrict__ codes,
                                                              const uint8_t* __restrict__ scales,
                                                              float global, uint4* __restrict__ out,
                                                              int64_t nblk) {
  const int64_t stride = (int64_t)gridDim.x * EW_THREADS;
  const double g = (double)global;
  for (int64_t b = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x; b < nblk; b += stride) {
    const uint2 c = codes[b];
    const double s = (double)e4m3_to_f32(scales[b]) * g;   // exact: 4 x 24 significant bits
    const uint32_t w[2] = {c.x, c.y};
    uint32_t p[8];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t byte = (w[k] >> (8 * j)) & 0xFFu;
        const uint32_t lo = f64_to_bf16_rne((double)bf16_to_f32(dequant_pair<0>(byte, 1.0f) & 0xFFFFu) * s);
        const uint32_t hi = f64_to_bf16_rne((double)bf16_to_f32(dequant_pair<0>(byte, 1.0f) >> 16) * s);
        p[4 * k + j] = lo | (hi << 16);
      }
    }
    out[2 * b] = make_uint4(p[0], p[1], p[2], p[3]);
    out[2 * b + 1] = make_uint4(p[4], p[5], p[6], p[7]);
  }
}

// MXFP4 quantise: one thread per 32 elements (64 bytes of bf16 in, 16 code bytes
// and one scale byte out).
__global__ __launch_bounds__(EW_THREADS) void k_quant_mxfp4(const uint4* __restrict__ x,
                                                            uint4* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, int64_t nblk) {
  const int64_t stride = (int64_t)gridDim.x * EW_THREADS;
  for (int64_t b = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x; b < nblk; b += stride) {
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = x[b * 4 + i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = max(am, amax2(w[i]));
    const uint32_t sb = mx_scale_from_amax_bits(am);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t r = 0;
      r = quant_pair_e8m0<0>(r, w[4 * i], sb);
      r = quant_pair_e8m0<1>(r, w[4 * i + 1], sb);
      r = quant_pair_e8m0<2>(r, w[4 * i + 2], sb);
      r = quant_pair_e8m0<3>(r, w[4 * i + 3], sb);
      o[i] = r;
    }
    codes[b] = make_uint4(o[0], o[1], o[2], o[3]);
    scales[b] = (uint8_t)sb;
  }
}

// NVFP4 quantise: one thread per 16 elements (32 bytes in, 8 code bytes + one
// E4M3 byte out). fp32 steps: t = 6 g; r = amax / t; s = E4M3(r); d = s g;
// v = x / d; code = E2M1(v) (|v| clamped to 6, which is what saturation gives).
__global__ __launch_bounds__(EW_THREADS) void k_quant_nvfp4(const uint4* __restrict__ x, float g,
                                                            uint2* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, int64_t nblk) {
  const int64_t stride = (int64_t)gridDim.x * EW_THREADS;
  const float t6 = 6.0f * g;
  for (int64_t b = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x; b < nblk; b += stride) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 v = x[b * 2 + i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = max(am, amax2(w[i]));
    const uint32_t sbyte = e4m3_rne_satfinite(bf16_to_f32(am) / t6);
    const float d = e4m3_to_f32(sbyte) * g;
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v0 = bf16_to_f32(w[i] & 0xFFFFu), v1 = bf16_to_f32(w[i] >> 16);
      if (sbyte == 0u) { v0 *= 0.0f; v1 *= 0.0f; }
      else {
        v0 = fminf(fmaxf(v0 / d, -6.0f), 6.0f);
        v1 = fminf(fmaxf(v1 / d, -6.0f), 6.0f);
      }
      uint32_t& r = o[i >> 2];
      switch (i & 3) {
        case 0: r = quant_pair_f32_unit<0>(r, v0, v1); break;
        case 1: r = quant_pair_f32_unit<1>(r, v0, v1); break;
        case 2: r = quant_pair_f32_unit<2>(r, v0, v1); break;
        default: r = quant_pair_f32_unit<3>(r, v0, v1); break;
      }
    }
    codes[b] = make_uint2(o[0], o[1]);
    scales[b] = (uint8_t)sbyte;
  }
}

}  // namespace

hipError_t launch_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                int64_t cols, uint16_t* out, hipStream_t s) {
  const int64_t nblk = rows * (cols / 32);
  if (nblk == 0) return hipSuccess;
  k_dequant_mxfp4<<<ew_grid(nblk), EW_THREADS, 0, s>>>((const uint4*)codes, scales, (uint4*)out, nblk);
  return hipGetLastError();
}

hipError_t launch_dequant_fp8_block(const uint8_t* q, const uint8_t* scales, int64_t rows,
                                    int64_t cols, uint16_t* out, hipStream_t s) {
  const int64_t n16 = rows * (cols / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t gcols = (cols + 127) / 128;
  k_dequant_fp8_block<<<ew_grid(n16), EW_THREADS, 0, s>>>((const uint4*)q, scales, cols, gcols,
                                                          (uint4*)out, n16);
  return hipGetLastError();
}

hipError_t launch_dequant_nvfp4(const uint8_t* codes, const uint8_t* scales, float global,
                                int64_t rows, int64_t cols, uint16_t* out, hipStream_t s) {
  const int64_t nblk = rows * (cols / 16);
  if (nblk == 0) return hipSuccess;
  k_dequant_nvfp4<<<ew_grid(nblk), EW_THREADS, 0, s>>>((const uint2*)codes, scales, global,
                                                       (uint4*)out, nblk);
  return hipGetLastError();
}

hipError_t launch_quant_mxfp4(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes,
                              uint8_t* scales, hipStream_t s) {
  const int64_t nblk = rows * (cols / 32);
  if (nblk == 0) return hipSuccess;
  k_quant_mxfp4<<<ew_grid(nblk), EW_THREADS, 0, s>>>((const uint4*)x, (uint4*)codes, scales, nblk);
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4(const uint16_t* x, int64_t rows, int64_t cols, float global,
                              uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t nblk = rows * (cols / 16);
  if (nblk == 0) return hipSuccess;
  k_quant_nvfp4<<<ew_grid(nblk), EW_THREADS, 0, s>>>((const uint4*)x, global, (uint2*)codes, scales,
                                                     nblk);
  return hipGetLastError();
}

}  // namespace mx
