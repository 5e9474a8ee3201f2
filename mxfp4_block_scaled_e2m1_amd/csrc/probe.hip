// Measurement probes: kernels whose rates are the measured ceilings that the
// roofline figures of the expert MLP can be read against, beside MI355X's
// published peaks (10.1 PFLOP/s dense FP4 matrix math, 8 TB/s HBM3E). They
// compute nothing of the method; each has a result the caller can check, so
// that a rate is never taken from work the compiler removed.
//  * k_probe_mfma: back-to-back V_MFMA_SCALE_F32_32X32X64_F8F6F4 with FP4
//    operands held in registers (four independent accumulators per wave), the
//    instruction the tiled GEMMs are built on.
//  * k_probe_read: a read-only stream, either into registers
//    (GLOBAL_LOAD_DWORDX4) or into LDS (GLOBAL_LOAD_LDS_DWORDX4, the copies of
//    the tiled GEMMs), folded into an XOR checksum per wave.
//  * k_probe_copy: a plain device copy (16-byte loads and stores).
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

namespace {

constexpr int PROBE_THREADS = 256;   // read and copy probes: 4 waves
constexpr int MFMA_THREADS = 512;    // MFMA probe: 8 waves

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// A global -> LDS copy of 16 bytes per lane: lane i writes LDS [m0 + 16 i, +16).
__device__ __forceinline__ void probe_lds_dma16(const void* src, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_off)
               : "memory", "m0");
}

// Thread tid's operands are words [16 tid, 16 tid + 8) (A) and [16 tid + 8,
// 16 tid + 16) (B) of the same 512 x 16 words for every workgroup; an FP4
// operand of this instruction is 4 words (32 E2M1 codes), so the instruction
// reads the first 4 of each. Scale byte 127 (2^0) on both sides.
// out[wg * 512 + tid] = the sum of the lane's 64 accumulator values.
__global__ __launch_bounds__(MFMA_THREADS) void k_probe_mfma(const uint32_t* __restrict__ operands, int64_t iters,
                                                             float* __restrict__ out) {
  const uint32_t* op = operands + 16 * threadIdx.x;
  i32x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (int)op[i];
    b[i] = (int)op[8 + i];
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int64_t it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 4, 4, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 4, 4, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 4, 4, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 4, 4, 0, 127, 0, 127);
  }
  float s = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += (c0[v] + c1[v]) + (c2[v] + c3[v]);
  out[(int64_t)blockIdx.x * MFMA_THREADS + threadIdx.x] = s;
}

// Wave w of the grid reads chunks w, w + waves, ... of U * 1 KB each (U 16-byte
// loads per lane, all in flight together), then XORs the words it read.
// out[wave of the grid] = the XOR over everything that wave read.
template <int U, bool LDS>
__global__ __launch_bounds__(PROBE_THREADS) void k_probe_read(const uint4* __restrict__ src, int64_t chunks,
                                                              uint32_t* __restrict__ out) {
  __shared__ uint4 stage[LDS ? 4 * U * 64 : 1];
  // the wave index is uniform: kept in a scalar register, as the LDS base in m0 must be
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t waves = (int64_t)gridDim.x * 4;
  uint32_t x = 0;
  for (int64_t c = (int64_t)blockIdx.x * 4 + wave; c < chunks; c += waves) {
    const uint4* p = src + c * (U * 64) + lane;
    if constexpr (LDS) {
      const uint32_t base = lds_addr_of(stage) + wave * U * 1024;
#pragma unroll
      for (int j = 0; j < U; ++j) probe_lds_dma16(p + j * 64, base + j * 1024);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const uint4 v = stage[(wave * U + j) * 64 + lane];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
      }
      // the next chunk's copies overwrite this wave's region
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    } else {
      uint4 v[U];
#pragma unroll
      for (int j = 0; j < U; ++j) v[j] = p[j * 64];
#pragma unroll
      for (int j = 0; j < U; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
  if (lane == 0) out[(int64_t)blockIdx.x * 4 + wave] = x;
}

__global__ __launch_bounds__(PROBE_THREADS) void k_probe_copy(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                              int64_t n16) {
  constexpr int U = 4;
  const int64_t stride = (int64_t)gridDim.x * PROBE_THREADS * U;
  for (int64_t base = (int64_t)blockIdx.x * PROBE_THREADS * U + threadIdx.x; base < n16; base += stride) {
    uint4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t i = base + j * PROBE_THREADS;
      if (i < n16) v[j] = src[i];
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t i = base + j * PROBE_THREADS;
      if (i < n16) dst[i] = v[j];
    }
  }
}

}  // namespace

hipError_t launch_probe_mfma(const uint32_t* operands, int64_t iters, int workgroups, float* out, hipStream_t s) {
  k_probe_mfma<<<workgroups, MFMA_THREADS, 0, s>>>(operands, iters, out);
  return hipGetLastError();
}

hipError_t launch_probe_read(int mode, int loads_per_wave, int workgroups, const void* src, int64_t bytes,
                             uint32_t* out, hipStream_t s) {
  const int64_t chunks = bytes / ((int64_t)loads_per_wave * 1024);
  const uint4* p = (const uint4*)src;
  if (loads_per_wave == 8) {
    if (mode == 1) k_probe_read<8, true><<<workgroups, PROBE_THREADS, 0, s>>>(p, chunks, out);
    else k_probe_read<8, false><<<workgroups, PROBE_THREADS, 0, s>>>(p, chunks, out);
  } else {
    if (mode == 1) k_probe_read<32, true><<<workgroups, PROBE_THREADS, 0, s>>>(p, chunks, out);
    else k_probe_read<32, false><<<workgroups, PROBE_THREADS, 0, s>>>(p, chunks, out);
  }
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  int64_t g = (n16 + PROBE_THREADS * 4 - 1) / (PROBE_THREADS * 4);
  if (g > 8192) g = 8192;
  k_probe_copy<<<(int)g, PROBE_THREADS, 0, s>>>((const uint4*)src, (uint4*)dst, n16);
  return hipGetLastError();
}

}  // namespace mx
