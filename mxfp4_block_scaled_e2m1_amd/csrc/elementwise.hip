// Streaming dequant / quantise kernels (HBM-bound): VALU decode between loads
// and stores that are contiguous across the lanes of each wave instruction.
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

// Streaming store of 16 bytes: the outputs of the dequant kernels are written
// once and not read again by the same kernel, so they bypass the caches
// (measured on the w1 dequant, 3072 x 7168: 14.0 -> 9.7 us per call).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_stream16(uint4* p, const uint4& v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), (u32x4_t*)p);
}
constexpr int EW_UNROLL = 4;   // units per thread per pass: all loads of a pass are in flight together

inline int ew_grid(int64_t work) {
  int64_t g = (work + EW_THREADS - 1) / EW_THREADS;
  if (g > 8192) g = 8192;
  return (int)(g < 1 ? 1 : g);
}

// Grid for the unit kernels below: a workgroup pass covers EW_THREADS * u units.
inline int ew_grid_units(int64_t units, int u = EW_UNROLL) {
  const int64_t per = (int64_t)EW_THREADS * u;
  int64_t g = (units + per - 1) / per;
  if (g > 4096) g = 4096;
  return (int)(g < 1 ? 1 : g);
}

// Units per thread of the chunked quantiser. Its inputs are small (at most 512
// token rows), where one unit per thread on four times the workgroups ends
// sooner: measured on the shared expert (7168 x 3072, two quantiser calls per
// call): 18.9 -> 17.8 us at 16 tokens, 23.0 -> 20.7 at 64, 27.3 -> 25.1 at
// 128, 56.5 -> 55.0 at 512 (two units per thread: 18.2, 21.6, 25.9, 56.0).
constexpr int EW_UNROLL_CHUNKED = 1;

// The unit kernels walk units u = pass base + j * EW_THREADS + tid (j < EW_UNROLL),
// so every wave instruction touches one contiguous span: loads of 64 lanes x
// 4..16 bytes and stores of 64 lanes x 4..16 bytes. Loads are unconditional
// (clamped to the last unit) and only the stores test the bound.
#define EW_FOR_PASSES_U(units, U)                                                    \
  for (int64_t base = (int64_t)blockIdx.x * EW_THREADS * (U); base < (units);     \
       base += (int64_t)gridDim.x * EW_THREADS * (U))
#define EW_FOR_PASSES(units) EW_FOR_PASSES_U(units, EW_UNROLL)

// MXFP4 dequant. Unit u = code dword u: elements 8u .. 8u+7 -> 16 output bytes;
// its scale is byte u / 4 (a 32-block is 4 dwords; rows hold whole blocks).
__global__ __launch_bounds__(EW_THREADS) void k_dequant_mxfp4(const uint32_t* __restrict__ codes,
                                                              const uint8_t* __restrict__ scales,
                                                              uint4* __restrict__ out, int64_t units) {
  EW_FOR_PASSES(units) {
    uint32_t c[EW_UNROLL], sb[EW_UNROLL];
#pragma unroll
    for (int j = 0; j < EW_UNROLL; ++j) {
      const int64_t u = min(base + j * EW_THREADS + (int64_t)threadIdx.x, units - 1);
      c[j] = codes[u];
      sb[j] = scales[u >> 2];
    }
#pragma unroll
    for (int j = 0; j < EW_UNROLL; ++j) {
      const int64_t u = base + j * EW_THREADS + (int64_t)threadIdx.x;
      uint4 o = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);   // scale byte 255: NaN
      if (sb[j] != 255u) {
        const float sc = e8m0_to_f32(sb[j]);
        o = make_uint4(dequant_pair<0>(c[j], sc), dequant_pair<1>(c[j], sc), dequant_pair<2>(c[j], sc),
                       dequant_pair<3>(c[j], sc));
      }
      if (u < units) store_stream16(&out[u], o);
    }
  }
}

// Two E4M3 codes (low or high 16 bits of `w`) times the scale sc = 2^(sb-127)
// -> a bf16 pair, rounded to nearest even (V_CVT_SCALEF32_PK_BF16_FP8). The NaN
// codes (0x7F, 0xFF) give the canonical quiet NaN 0x7FC0 whatever their sign.
template <bool HI>
__device__ __forceinline__ uint32_t fp8_pair_to_bf16(uint32_t w, float sc) {
  uint32_t r = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, HI));
  const uint32_t c = HI ? (w >> 16) : w;
  if ((c & 0x7Fu) == 0x7Fu) r = (r & 0xFFFF0000u) | 0x7FC0u;
  if (((c >> 8) & 0x7Fu) == 0x7Fu) r = (r & 0x0000FFFFu) | 0x7FC00000u;
  return r;
}

// FP8 block dequant. Unit u = 8 codes (elements 8u .. 8u+7 of the row-major
// matrix, one row and one 128-column block since cols % 16 == 0) -> 16 bytes.
// (Units of 16 codes, one 16-byte load and two stores per thread, measured
// slower on the [7168, 1536] matrix: 8.9 against 6.6 us.)
template <typename Idx>
__global__ __launch_bounds__(EW_THREADS) void k_dequant_fp8_block(const uint2* __restrict__ q,
                                                                  const uint8_t* __restrict__ scales,
                                                                  Idx cols, Idx gcols, uint4* __restrict__ out,
                                                                  int64_t units) {
  EW_FOR_PASSES(units) {
    uint2 v[EW_UNROLL];
    uint32_t sb[EW_UNROLL];
#pragma unroll
    for (int j = 0; j < EW_UNROLL; ++j) {
      const int64_t u = min(base + j * EW_THREADS + (int64_t)threadIdx.x, units - 1);
      const Idx e = (Idx)u * 8;
      const Idx r = e / cols, c = e - r * cols;
      v[j] = q[u];
      sb[j] = scales[(r >> 7) * gcols + (c >> 7)];
    }
#pragma unroll
    for (int j = 0; j < EW_UNROLL; ++j) {
      const int64_t u = base + j * EW_THREADS + (int64_t)threadIdx.x;
      uint4 o = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);   // scale byte 255: NaN
      if (sb[j] != 255u) {
        // hardware convert of two E4M3 codes times a power-of-two scale to bf16
        const float sc = e8m0_to_f32(sb[j]);
        o = make_uint4(fp8_pair_to_bf16<false>(v[j].x, sc), fp8_pair_to_bf16<true>(v[j].x, sc),
                       fp8_pair_to_bf16<false>(v[j].y, sc), fp8_pair_to_bf16<true>(v[j].y, sc));
      }
      if (u < units) store_stream16(&out[u], o);
    }
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
                                                              float global, const float* __restrict__ gptr,
                                                              uint4* __restrict__ out, int64_t nblk) {
  const int64_t stride = (int64_t)gridDim.x * EW_THREADS;
  const double g = (double)(gptr != nullptr ? *gptr : global);
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
    store_stream16(&out[2 * b], make_uint4(p[0], p[1], p[2], p[3]));
    store_stream16(&out[2 * b + 1], make_uint4(p[4], p[5], p[6], p[7]));
  }
}

// MXFP4 quantise. Unit u = 8 elements (16 bytes of bf16 in, one code dword
// out); the 4 units of a 32-block are 4 consecutive lanes, which combine their
// amax with two lane exchanges. The first lane of the four writes the scale.
// CHUNKED writes the layout the weight-streaming kernels read their token
// operand in (launch_quant_mxfp4_chunked): rows in chunks of 16, per chunk and
// 128-wide K step one 1 KB block of codes, and per chunk, wave of the reading
// kernel and lane 8 scale bytes, one per step of that wave's run, so that a
// lane loads its scales for a chunk at once. Rows past the input (up to a
// multiple of 16) are written as zero codes with scale byte 0.
template <bool CHUNKED>
__global__ __launch_bounds__(EW_THREADS) void k_quant_mxfp4(const uint4* __restrict__ x,
                                                            uint32_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, int64_t in_units,
                                                            int64_t units, uint32_t row_units, uint32_t ksteps) {
  constexpr int U = CHUNKED ? EW_UNROLL_CHUNKED : EW_UNROLL;
  EW_FOR_PASSES_U(units, U) {
    uint4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t u = base + j * EW_THREADS + (int64_t)threadIdx.x;
      v[j] = x[min(u, in_units - 1)];
      if (CHUNKED && u >= in_units) v[j] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t u = base + j * EW_THREADS + (int64_t)threadIdx.x;
      const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      uint32_t am = max(max(amax2(w[0]), amax2(w[1])), max(amax2(w[2]), amax2(w[3])));
      am = max(am, (uint32_t)__shfl_xor((int)am, 1));
      am = max(am, (uint32_t)__shfl_xor((int)am, 2));
      const uint32_t sb = mx_scale_from_amax_bits(am);
      uint32_t r;
      quant_pairs_e8m0<4>(w, sb, &r);
      if (u < units) {
        if constexpr (CHUNKED) {
          // u < 2^32: the chunked layout serves at most 512 rows
          const uint32_t row = (uint32_t)u / row_units, i = (uint32_t)u - row * row_units;
          const uint32_t s = i >> 4, lane = ((i >> 2) & 3) * 16 + (row & 15);
          codes[(((row >> 4) * ksteps + s) * 64 + lane) * 4 + (i & 3)] = r;
          if ((i & 3) == 0) {
            // step s -> (wave w, place k in its run) of the balanced split
            const uint32_t base = ksteps / STREAM_WAVES, extra = ksteps - base * STREAM_WAVES;
            uint32_t w, k;
            if (s < extra * (base + 1)) {
              w = s / (base + 1);
              k = s - w * (base + 1);
            } else {
              const uint32_t t = s - extra * (base + 1);
              w = extra + t / base;
              k = t - (w - extra) * base;
            }
            scales[(((row >> 4) * STREAM_WAVES + w) * 64 + lane) * 8 + k] = (uint8_t)sb;
          }
        } else {
          codes[u] = r;
          if ((threadIdx.x & 3) == 0) scales[u >> 2] = (uint8_t)sb;
        }
      }
    }
  }
}

// NVFP4 quantise: one thread per 16 elements (32 bytes in, 8 code bytes + one
// E4M3 byte out). fp32 steps: t = 6 g; r = amax / t; s = E4M3(r); d = s g;
// v = x / d; code = E2M1(v) (|v| clamped to 6, which is what saturation gives).
__global__ __launch_bounds__(EW_THREADS) void k_quant_nvfp4(const uint4* __restrict__ x, float gval,
                                                            const float* __restrict__ gptr,
                                                            uint2* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, int64_t nblk) {
  const int64_t stride = (int64_t)gridDim.x * EW_THREADS;
  const float g = gptr != nullptr ? *gptr : gval;
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
    // a block holding an infinity or a NaN gets the E4M3 NaN byte 0x7F
    const uint32_t sbyte = am >= 0x7F80u ? 0x7Fu : e4m3_rne_satfinite(bf16_to_f32(am) / t6);
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

// NVFP4 warm-up: the running max of |h| (bf16 magnitude bits, so that an
// unsigned max orders them as values) starts at zero ...
__global__ void k_amax_clear(uint32_t* amax) {
  if (threadIdx.x == 0) *amax = 0u;
}

// ... and becomes g = f32(max |h| / (6 * 448)) (IEEE fp32 division), or 1 when
// h is all zero.
__global__ void k_nvfp4_global(const uint32_t* amax, float* g) {
  if (threadIdx.x == 0) {
    const uint32_t a = *amax;
    *g = a != 0u ? bf16_to_f32(a) / (6.0f * 448.0f) : 1.0f;
  }
}

}  // namespace

hipError_t launch_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                int64_t cols, uint16_t* out, hipStream_t s) {
  const int64_t units = rows * (cols / 8);
  if (units == 0) return hipSuccess;
  k_dequant_mxfp4<<<ew_grid_units(units), EW_THREADS, 0, s>>>((const uint32_t*)codes, scales, (uint4*)out,
                                                              units);
  return hipGetLastError();
}

hipError_t launch_dequant_fp8_block(const uint8_t* q, const uint8_t* scales, int64_t rows,
                                    int64_t cols, uint16_t* out, hipStream_t s) {
  const int64_t units = rows * (cols / 8);
  if (units == 0) return hipSuccess;
  const int64_t gcols = (cols + 127) / 128;
  if (rows * cols < ((int64_t)1 << 32))   // 32-bit element indexes: cheaper division
    k_dequant_fp8_block<uint32_t><<<ew_grid_units(units), EW_THREADS, 0, s>>>(
        (const uint2*)q, scales, (uint32_t)cols, (uint32_t)gcols, (uint4*)out, units);
  else
    k_dequant_fp8_block<uint64_t><<<ew_grid_units(units), EW_THREADS, 0, s>>>(
        (const uint2*)q, scales, (uint64_t)cols, (uint64_t)gcols, (uint4*)out, units);
  return hipGetLastError();
}

hipError_t launch_dequant_nvfp4(const uint8_t* codes, const uint8_t* scales, float global, const float* gptr,
                                int64_t rows, int64_t cols, uint16_t* out, hipStream_t s) {
  const int64_t nblk = rows * (cols / 16);
  if (nblk == 0) return hipSuccess;
  k_dequant_nvfp4<<<ew_grid(nblk), EW_THREADS, 0, s>>>((const uint2*)codes, scales, global, gptr,
                                                       (uint4*)out, nblk);
  return hipGetLastError();
}

hipError_t launch_quant_mxfp4(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes,
                              uint8_t* scales, hipStream_t s) {
  const int64_t units = rows * (cols / 8);
  if (units == 0) return hipSuccess;
  k_quant_mxfp4<false><<<ew_grid_units(units), EW_THREADS, 0, s>>>((const uint4*)x, (uint32_t*)codes,
                                                                             scales, units, units, 0u, 0u);
  return hipGetLastError();
}

hipError_t launch_quant_mxfp4_chunked(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes,
                                      uint8_t* scales, hipStream_t s) {
  const int64_t in_units = rows * (cols / 8);
  const int64_t units = (rows + 15) / 16 * 16 * (cols / 8);
  if (in_units == 0) return hipSuccess;
  k_quant_mxfp4<true><<<ew_grid_units(units, EW_UNROLL_CHUNKED), EW_THREADS, 0, s>>>(
      (const uint4*)x, (uint32_t*)codes, scales, in_units, units, (uint32_t)(cols / 8), (uint32_t)(cols / 128));
  return hipGetLastError();
}

hipError_t launch_amax_clear(uint32_t* amax, hipStream_t s) {
  k_amax_clear<<<1, 64, 0, s>>>(amax);
  return hipGetLastError();
}

hipError_t launch_nvfp4_global(const uint32_t* amax, float* g, hipStream_t s) {
  k_nvfp4_global<<<1, 64, 0, s>>>(amax, g);
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4(const uint16_t* x, int64_t rows, int64_t cols, float global, const float* gptr,
                              uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t nblk = rows * (cols / 16);
  if (nblk == 0) return hipSuccess;
  k_quant_nvfp4<<<ew_grid(nblk), EW_THREADS, 0, s>>>((const uint4*)x, global, gptr, (uint2*)codes, scales,
                                                     nblk);
  return hipGetLastError();
}

}  // namespace mx
