// FP8 block-scaled linear: y = bf16(MXFP8(x) . W^T) with W in FP8 E4M3 and
// one E8M0 scale per 128 x 128 tile.
//
// The original checkpoint stores the shared experts in FP8 E4M3 with E8M0
// block scales (page "2026-05-08 DeepSeek V4 Pro NVFP4 Quantization", section
// "Status") and the serving stack runs them through an FP8 block-scaled GEMM
// (page "2026-05-11 - DeepSeek V4 NVFP4 vLLM Serving: Full End-to-End",
// sections "Architecture Map" and "What We Fixed" item 1: 128 x 128 blocks,
// E8M0 scales). The pages leave the activation side open; x is quantised to
// MXFP8: per row and 32 columns an E8M0 byte clamp(floor(log2 amax) - 8 + 127,
// 0, 254) and E4M3 elements rounded to nearest even, saturating at 448, the
// sign kept (the OCP shared-exponent rule with E4M3 elements).
//
// Both operands are then what gfx950's scaled MFMA takes natively: FP8 codes
// with one E8M0 byte per 32 K values. A weight row's byte for a 32-wide K
// chunk is its 128 x 128 tile's byte, so W is used as stored.
//
// GEMM design:
//  * 512-thread workgroups on 256 (weight rows) x 256 (token rows) tiles,
//    K stage 128 (one weight-scale column); 8 waves of 128 x 64, each 4 x 2
//    blocks of V_MFMA_SCALE_F32_32X32X64_F8F6F4 (FP8 E4M3 A and B).
//  * Each stage is 2 x 32 KB of codes in LDS, two slots. The copies of the
//    next stage go straight from global memory into the other slot
//    (GLOBAL_LOAD_LDS_DWORDX4) while the current stage's MFMAs run; one
//    barrier per stage. Rows are 128 bytes, 16-byte chunk c of row r stored
//    at chunk c ^ ((r / 2) % 8), so the 16 rows a quarter-wave reads spread
//    over all banks.
//  * The tile's weight scales (2 block rows x K/128 bytes) sit in LDS for the
//    whole K loop; a wave's 128 weight rows share one byte per stage. Token
//    scales: one dword (4 chunks) per row and stage, loaded a stage ahead.
//  * Tiles: m fastest, cut into 8 contiguous ranges, workgroup b on XCD b % 8
//    taking range b % 8, so the workgroups of one XCD share weight tiles.
#include "mx_device.h"
#include "mx_internal.h"
#include "fp8_linear.h"

namespace mx {

namespace {

constexpr int F8_THREADS = 512;
constexpr int F8_BN = 256;            // weight rows per tile
constexpr int F8_BM = 256;            // token rows per tile
constexpr int F8_BK = 128;            // K per stage (bytes per row)
constexpr int F8_OPND = 256 * F8_BK;  // 32 KB per operand and stage
constexpr int F8_SLOT = 2 * F8_OPND;  // weights + tokens
constexpr int F8_MAX_KB = 64;         // K / 128 <= 64: weight-scale rows in LDS
// The bf16 output tile is staged in the K loop's LDS before it is stored:
// 256 token rows of 512 bytes, pitch 520 so that the 32 rows a wave writes at
// one column fall in distinct banks (130 dwords = 2 mod 64).
constexpr int F8_YPITCH = F8_BN * 2 + 8;
constexpr int F8_SMEM = (2 * F8_SLOT > F8_BM * F8_YPITCH) ? 2 * F8_SLOT : F8_BM * F8_YPITCH;

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ quantiser
// One thread per 32-element block: 64 bytes in, 32 code bytes and a scale out.
__global__ __launch_bounds__(256) void k_quant_mxfp8(const uint4* __restrict__ x, uint4* __restrict__ codes,
                                                     uint8_t* __restrict__ scales, int64_t nblk) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblk; b += stride) {
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = x[4 * b + i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = max(am, amax2(w[i]));
    // floor(log2 amax) - 8 + 127 from the bf16 exponent field ef: ef - 8, at
    // least 0; a block holding an infinity or a NaN (ef = 255) gets the NaN
    // byte 0xFF (and zero codes)
    const int ef = (int)((am >> 7) & 0xFFu);
    const uint32_t sb = ef == 0xFF ? 0xFFu : (uint32_t)(ef > 8 ? ef - 8 : 0);
    const float inv = sb == 0xFFu ? 0.0f : __uint_as_float((254u - sb) << 23);   // 2^(127 - sb), exact multiply
    uint32_t q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t d = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t e = (w[2 * i + (j >> 1)] >> (16 * (j & 1))) & 0xFFFFu;
        const float v = bf16_to_f32(e & 0x7FFFu) * inv;
        const uint32_t c = e4m3_rne_satfinite(v) | ((e >> 8) & 0x80u);
        d |= c << (8 * j);
      }
      q[i] = d;
    }
    codes[2 * b] = make_uint4(q[0], q[1], q[2], q[3]);
    codes[2 * b + 1] = make_uint4(q[4], q[5], q[6], q[7]);
    scales[b] = (uint8_t)sb;
  }
}

// ------------------------------------------------------------------ SiLU * up
// h = bf16(silu(g) * u) from bf16 g and u, 8 elements per thread: the step
// between the FP8 gate/up linears and the down linear of the FP8 shared expert
// (page "Current Bug: vLLM produces empty/garbage output", section "Revised
// Plan", Phase 1). silu_mul is the fused MXFP4 epilogue's fp32 evaluation.
__global__ __launch_bounds__(256) void k_silu_mul_bf16(const uint4* __restrict__ g, const uint4* __restrict__ u,
                                                       uint4* __restrict__ h, int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
    const uint4 a = g[i], b = u[i];
    const uint32_t ga[4] = {a.x, a.y, a.z, a.w}, ub[4] = {b.x, b.y, b.z, b.w};
    uint32_t r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      r[q] = bf16x2_rne(silu_mul(bf16_to_f32(ga[q] & 0xFFFFu), bf16_to_f32(ub[q] & 0xFFFFu)),
                        silu_mul(bf16_to_f32(ga[q] >> 16), bf16_to_f32(ub[q] >> 16)));
    h[i] = make_uint4(r[0], r[1], r[2], r[3]);
  }
}

// ------------------------------------------------------------------ GEMM
struct F8Args {
  const uint8_t* w;      // [N, K] E4M3 (SwiGLU: w1 [N, K])
  const uint8_t* ws;     // [N/128, K/128] E8M0
  const uint8_t* w3;     // SwiGLU: w3 [N, K] and its scales
  const uint8_t* w3s;
  const uint8_t* xq;     // [M, K] E4M3
  const uint8_t* xs;     // [M, K/32] E8M0
  uint16_t* y;           // [M, N] bf16
  int M, N, K;
  int tiles_n, tiles_m, per_xcd;
};

// Global -> LDS copy of 16 bytes per lane: lane i writes LDS bytes
// [m0 + 16 i, +16). Issued as inline asm so that the compiler does not wait
// for it before every LDS read; the K loop waits for it explicitly.
__device__ __forceinline__ void f8_dma16(const void* src, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_off) : "memory", "m0");
}

// LDS byte offset of 16-byte chunk c of row r in an operand tile: the chunk
// index is XORed with (r / 2) % 8, so the 16 rows that a quarter-wave reads at
// one chunk fall in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int f8_off(int r, int c) { return r * F8_BK + ((c ^ ((r >> 1) & 7)) << 4); }

// SWIGLU: the tile's 256 weight rows are 128 rows j0 .. j0 + 127 of w1 (gate,
// tile rows 0..127, waves with wn = 0) and the same rows of w3 (up, tile rows
// 128..255), j0 = 128 * (n-tile). The epilogue rounds g and u to bf16 in the
// staged tile, exactly as the plain GEMM stores them, and writes
// h = bf16(silu(g) * u) with the arithmetic of k_silu_mul_bf16, so the result
// is that of the two GEMMs and the elementwise kernel, bit for bit, without
// the g and u round trip through memory.
template <bool SWIGLU>
__global__ __launch_bounds__(F8_THREADS, 1) void k_fp8_gemm(const F8Args a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[F8_SMEM];
  __shared__ uint8_t wsc[2][F8_MAX_KB];
  const int b = blockIdx.x;
  const int L = (b & 7) * a.per_xcd + (b >> 3);
  if (L >= a.tiles_n * a.tiles_m) return;
  const int nt = L / a.tiles_m, mt = L - nt * a.tiles_m;
  const int n0 = nt * (SWIGLU ? 128 : F8_BN), m0 = mt * F8_BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int K = a.K, kb128 = K / F8_BK, nst = kb128;

  // weight scales of the tile's two 128-row blocks (the second clamped at the
  // end of W; SwiGLU: w1's and w3's block of rows n0 .. n0 + 127)
  for (int i = tid; i < 2 * kb128; i += F8_THREADS) {
    const int blk = i / kb128, col = i - blk * kb128;
    if constexpr (SWIGLU) {
      wsc[blk][col] = (blk ? a.w3s : a.ws)[(int64_t)(n0 / 128) * kb128 + col];
    } else {
      const int br = min(n0 / 128 + blk, a.N / 128 - 1);
      wsc[blk][col] = a.ws[(int64_t)br * kb128 + col];
    }
  }

  // Global -> LDS copies (GLOBAL_LOAD_LDS_DWORDX4): wave instruction c of wave
  // w writes 16-byte chunks p = (4 w + c) * 64 + lane of an operand tile, which
  // is stored chunk position p % 8 of row p / 8, i.e. logical chunk
  // (p % 8) ^ (row % 8) of that row. Eight lanes cover one 128-byte row.
  // Rows past the end of W or x re-read the last row.
  // (SwiGLU: the copies of waves 0..3 are tile rows 0..127, from w1, those of
  // waves 4..7 rows 128..255, from w3.)
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const uint8_t* __restrict__ wbase =
      SWIGLU ? (wu < 4 ? a.w : a.w3) + (int64_t)n0 * K : a.w + (int64_t)n0 * K;
  const uint8_t* __restrict__ xbase = a.xq + (int64_t)m0 * K;
  uint32_t woff[4], xoff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int p = (wave * 4 + c) * 64 + lane;
    const int r = p >> 3, lc = (p & 7) ^ ((r >> 1) & 7);
    woff[c] = (uint32_t)((SWIGLU ? (r & 127) : min(n0 + r, a.N - 1) - n0) * K + lc * 16);
    xoff[c] = (uint32_t)((min(m0 + r, a.M - 1) - m0) * K + lc * 16);
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)smem;
  auto issue = [&](int st) {
    const uint32_t sb = lds0 + (st & 1) * F8_SLOT + wu * 4 * 1024;
#pragma unroll
    for (int c = 0; c < 4; ++c) f8_dma16(wbase + woff[c] + st * F8_BK, sb + c * 1024);
#pragma unroll
    for (int c = 0; c < 4; ++c) f8_dma16(xbase + xoff[c] + st * F8_BK, sb + F8_OPND + c * 1024);
  };
  // token scales of this lane's two 32-row blocks: one dword per row and stage
  const int r32 = lane & 31, half = lane >> 5;
  const uint32_t* xsrow[2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
    xsrow[g] = (const uint32_t*)a.xs + (int64_t)min(m0 + wm * 64 + g * 32 + r32, a.M - 1) * (K / 128);
  uint32_t xsd[2], xsn[2];

  f32x16 acc[4][2];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[f][g][v] = 0.f;

  issue(0);
#pragma unroll
  for (int g = 0; g < 2; ++g) xsn[g] = xsrow[g][0];

  for (int st = 0; st < nst; ++st) {
    // stage st is in LDS (all waves' copies), and every wave's reads of the
    // other slot (stage st - 1) are done: refill it with stage st + 1
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    xsd[0] = xsn[0];
    xsd[1] = xsn[1];
    if (st + 1 < nst) {
      issue(st + 1);
#pragma unroll
      for (int g = 0; g < 2; ++g) xsn[g] = xsrow[g][st + 1];
    }
    const uint8_t* sw = smem + (st & 1) * F8_SLOT;
    const uint8_t* sx = sw + F8_OPND;
    const int sa = wsc[wn][st];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // FP8 operand layout of the 32x32x64 scaled MFMA (checked on the device):
      // lane (row, h) holds K = 16 h .. 16 h + 15 in its first 16 bytes and
      // K = 32 + 16 h .. 32 + 16 h + 15 in the next 16, and supplies the scale
      // byte of the 32-wide block h. So this lane reads 16-byte chunks 4 ks + h
      // and 4 ks + 2 + h of the stage, and passes the scale of chunk pair 2 ks + h.
      const int c0 = ks * 4 + half, c1 = c0 + 2;
      i32x8_t B[2];
      int sb[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int r = wm * 64 + g * 32 + r32;
        const uint4 lo = *(const uint4*)(sx + f8_off(r, c0));
        const uint4 hi = *(const uint4*)(sx + f8_off(r, c1));
        B[g] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sb[g] = (int)((xsd[g] >> (8 * (2 * ks + half))) & 0xFFu);
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int r = wn * 128 + f * 32 + r32;
        const uint4 lo = *(const uint4*)(sw + f8_off(r, c0));
        const uint4 hi = *(const uint4*)(sw + f8_off(r, c1));
        const i32x8_t A = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                  (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
        for (int g = 0; g < 2; ++g)
          acc[f][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B[g], acc[f][g], 0, 0, 0, sa, 0, sb[g]);
      }
    }
  }

  // lane holds token m = 64 wm + 32 g + lane%32 of the tile and weight rows
  // n = 128 wn + 32 f + 8 (v/4) + 4 (lane/32) + v%4: into LDS as the bf16
  // tile [m][n], then out in whole rows (a wave stores two 512-byte rows per
  // instruction instead of 16 bytes in each of 32 rows).
  __syncthreads();   // every wave's last fragment reads are done
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    uint8_t* yl = smem + (wm * 64 + g * 32 + r32) * F8_YPITCH;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = wn * 128 + f * 32 + 8 * q + 4 * half;
        const uint32_t p0 = bf16x2_rne(acc[f][g][4 * q], acc[f][g][4 * q + 1]);
        const uint32_t p1 = bf16x2_rne(acc[f][g][4 * q + 2], acc[f][g][4 * q + 3]);
        *(uint2*)(yl + n * 2) = make_uint2(p0, p1);
      }
  }
  __syncthreads();
  if constexpr (SWIGLU) {
    // 16-byte chunk i of h: row i / 16, columns 8 (i % 16) .. + 7, from g at
    // those tile columns and u 128 columns further
#pragma unroll 4
    for (int i = tid; i < F8_BM * 16; i += F8_THREADS) {
      const int r = i >> 4, c = (i & 15) * 8;
      const int m = m0 + r;
      if (m >= a.M) continue;
      const uint4 gv = *(const uint4*)(smem + r * F8_YPITCH + c * 2);
      const uint4 uv = *(const uint4*)(smem + r * F8_YPITCH + (128 + c) * 2);
      const uint32_t ga[4] = {gv.x, gv.y, gv.z, gv.w}, ub[4] = {uv.x, uv.y, uv.z, uv.w};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = bf16x2_rne(silu_mul(bf16_to_f32(ga[q] & 0xFFFFu), bf16_to_f32(ub[q] & 0xFFFFu)),
                          silu_mul(bf16_to_f32(ga[q] >> 16), bf16_to_f32(ub[q] >> 16)));
      *(uint4*)(a.y + (int64_t)m * a.N + n0 + c) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  } else {
    // 16-byte chunk i of the tile: row i / 32, columns 8 (i % 32) .. + 7
#pragma unroll 4
    for (int i = tid; i < F8_BM * 32; i += F8_THREADS) {
      const int r = i >> 5, c = (i & 31) * 8;
      const int m = m0 + r, n = n0 + c;
      if (m < a.M && n < a.N) *(uint4*)(a.y + (int64_t)m * a.N + n) = *(const uint4*)(smem + r * F8_YPITCH + c * 2);
    }
  }
}

}  // namespace

hipError_t launch_quant_mxfp8(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
  const int64_t nblk = rows * (cols / 32);
  if (nblk == 0) return hipSuccess;
  int64_t g = (nblk + 255) / 256;
  if (g > 8192) g = 8192;
  k_quant_mxfp8<<<(int)g, 256, 0, s>>>((const uint4*)x, (uint4*)codes, scales, nblk);
  return hipGetLastError();
}

hipError_t launch_fp8_gemm(const uint8_t* xq, const uint8_t* xs, const uint8_t* w, const uint8_t* ws, int M, int N,
                           int K, uint16_t* y, hipStream_t s) {
  if (M == 0) return hipSuccess;
  F8Args a;
  a.w = w; a.ws = ws; a.w3 = nullptr; a.w3s = nullptr; a.xq = xq; a.xs = xs; a.y = y;
  a.M = M; a.N = N; a.K = K;
  a.tiles_n = (N + F8_BN - 1) / F8_BN;
  a.tiles_m = (M + F8_BM - 1) / F8_BM;
  const int total = a.tiles_n * a.tiles_m;
  a.per_xcd = (total + 7) / 8;
  k_fp8_gemm<false><<<8 * a.per_xcd, F8_THREADS, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_fp8_swiglu(const uint8_t* xq, const uint8_t* xs, const uint8_t* w1, const uint8_t* w1s,
                             const uint8_t* w3, const uint8_t* w3s, int M, int I, int K, uint16_t* h,
                             hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (I % 128 != 0) return hipErrorInvalidValue;
  F8Args a;
  a.w = w1; a.ws = w1s; a.w3 = w3; a.w3s = w3s; a.xq = xq; a.xs = xs; a.y = h;
  a.M = M; a.N = I; a.K = K;
  a.tiles_n = I / 128;
  a.tiles_m = (M + F8_BM - 1) / F8_BM;
  const int total = a.tiles_n * a.tiles_m;
  a.per_xcd = (total + 7) / 8;
  k_fp8_gemm<true><<<8 * a.per_xcd, F8_THREADS, 0, s>>>(a);
  return hipGetLastError();
}

bool fp8_linear_fits(int64_t K) { return K / F8_BK <= F8_MAX_KB; }

hipError_t launch_silu_mul_bf16(const uint16_t* g, const uint16_t* u, int64_t n, uint16_t* h, hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  int64_t grid = (n8 + 255) / 256;
  if (grid > 8192) grid = 8192;
  k_silu_mul_bf16<<<(int)grid, 256, 0, s>>>((const uint4*)g, (const uint4*)u, (uint4*)h, n8);
  return hipGetLastError();
}

}  // namespace mx
