// Expert MLP for a few tokens (M <= 8): the weight stream from HBM is the cost.
//
// Same arithmetic as the prefill path (page "Current Bug: vLLM produces
// empty/garbage output", section "Revised Plan", Phase 1: L1 GEMM, SiLU,
// re-quant, L2 GEMM; MXFP4 formats of page "2026-05-08 DeepSeek V4 Pro NVFP4
// Quantization", sections "Script update" and "FP4 (E2M1) expert weight format
// confirmed"), arranged for bandwidth instead of MFMA rate. Two kernels, each a
// single pass over its weights:
//  * L1: one workgroup per 8 intermediate columns j. Its 16 weight rows (8 of
//    w1, 8 of w3) form one 16-row MFMA tile over the whole K = hidden, so the
//    gate and the up value of a column meet in the same workgroup and SiLU(g)*u
//    needs no second pass. 3072 / 8 = 384 workgroups.
//  * L2: one workgroup per 16 output columns (16 rows of w2), 448 workgroups.
//  * 8 waves; wave w owns a contiguous run of the 128-wide K steps and keeps
//    that run's weight codes in registers (16 bytes per lane per step).
//  * Every thread issues its loads in a fixed order: the activation blocks it
//    will quantise, then its share of the rows' scales, then its weight codes.
//    Memory loads of a wave complete in issue order, so the quantisation of the
//    activations (x for L1, h for L2, with the conversions of the standalone
//    MXFP4 quantiser) and the scale staging wait only for those first loads and
//    run while the weight codes are still in flight.
//  * V_MFMA_SCALE_F32_16X16X128_F8F6F4: weight rows are the 16-row A operand,
//    tokens the 16 columns of B (columns >= M are zero operands). The 8 waves'
//    partial sums meet in LDS, in wave order, and wave 0 writes the result:
//    h = bf16(silu(g) * u) for L1, y = bf16(acc) for L2.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

namespace {

constexpr int DT = 512;             // threads per workgroup
constexpr int DW = DT / 64;         // waves
static_assert(DW == STREAM_WAVES, "the chunked token scales are laid out per wave of these kernels");
constexpr int MAX_STEPS = 8;        // K steps of 128 per wave held in registers
constexpr int MAX_TOK = 8;          // tokens per call on this path

__device__ __forceinline__ i32x8 opnd(const uint4& v) {
  return i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

// The thread's activation blocks (32 bf16 each): block b = tid + DT * r of the
// row-major list of m * cols/32 blocks.
template <int XR>
struct XBlocks {
  uint4 v[XR][4];
};

// Loads are unconditional (a thread past the end re-reads the last block):
// the compiler counts outstanding loads exactly only when none is skipped by a
// branch, and an exact count is what lets the later waits ignore the weights.
template <int XR>
__device__ __forceinline__ void load_x(const uint16_t* __restrict__ src, int m, int cols, XBlocks<XR>& xb) {
  const int bpr = cols >> 5, nb = m * bpr;
#pragma unroll
  for (int r = 0; r < XR; ++r) {
    const int b = min((int)threadIdx.x + DT * r, nb - 1);
    const int row = b / bpr, c = b - row * bpr;
    const uint4* p = (const uint4*)(src + (int64_t)row * cols + c * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) xb.v[r][i] = p[i];
  }
}

// MXFP4-quantise the loaded blocks into LDS: codes at row * cstride + c * 16,
// scale bytes at row * (cols/32) + c. Every thread converts its blocks (those
// past the end are re-read copies) and only the stores are conditional, so the
// compiler has no branch to sink the loads into.
template <int XR>
__device__ __forceinline__ void quant_x_to_lds(const XBlocks<XR>& xb, int m, int cols, uint8_t* codes,
                                               int cstride, uint8_t* scales) {
  const int bpr = cols >> 5, nb = m * bpr;
#pragma unroll
  for (int r = 0; r < XR; ++r) {
    const int b = threadIdx.x + DT * r;
    {
      const int row = b / bpr, c = b - row * bpr;
      uint32_t w[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[4 * i] = xb.v[r][i].x; w[4 * i + 1] = xb.v[r][i].y;
        w[4 * i + 2] = xb.v[r][i].z; w[4 * i + 3] = xb.v[r][i].w;
      }
      uint32_t am = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) am = max(am, amax2(w[i]));
      const uint32_t sb = mx_scale_from_amax_bits(am);
      uint32_t q[4];
      quant_pairs_e8m0<16>(w, sb, q);
      if (b < nb) {
        *(uint4*)(codes + row * cstride + c * 16) = make_uint4(q[0], q[1], q[2], q[3]);
        scales[row * bpr + c] = (uint8_t)sb;
      }
    }
  }
}

// Balanced split of `ksteps` K steps over the DW waves: wave w takes [s0, s0 + n).
__device__ __forceinline__ void wave_steps(int ksteps, int& s0, int& n) {
  const int wave = threadIdx.x >> 6;
  const int base = ksteps / DW, extra = ksteps - base * DW;
  n = base + (wave < extra ? 1 : 0);
  s0 = wave * base + min(wave, extra);
}

// The 16 rows of a weight tile: rows 0..7 start at lo + r * stride, rows 8..15
// at hi + (r - 8) * stride (the same matrix continued, or a second matrix).
struct RowPair {
  const uint8_t* lo;
  const uint8_t* hi;
  __device__ __forceinline__ const uint8_t* row(int r, int stride) const {
    return (r < 8 ? lo : hi) + (int64_t)(r & 7) * stride;
  }
};

// Where the code bytes of a 16-row weight tile are: lane (row r16, quarter q)
// of K step s (128 columns) reads the 16 bytes of columns 128 s + 32 q .. +31
// of tile row r16 at at(r16, s, q).
//  * Row-major codes [rows, K/2]: rows 0..7 at lo + r * kb, rows 8..15 at
//    hi + (r - 8) * kb, step s 64 bytes further per step.
//  * The GEMM's tile-major copy (mx_pack_weight_codes): per GEMM tile and step
//    a 16 KB block with row R at R * 64 and its 16-byte chunk c at slot
//    c ^ ((R / 4) % 4); blocks of consecutive steps 16 KB apart. lo and hi point
//    at the places of the first row of each half in the step-0 block, sw_lo and
//    sw_hi are those rows' R / 4. Each half of a tile is then 512 consecutive
//    bytes per step (a 16-row group of a GEMM tile 1 KB), where the row-major
//    layout gives 16 separate 64-byte pieces.
struct WTile {
  const uint8_t* lo;
  const uint8_t* hi;
  int row_stride;    // kb (row-major) or 64 (tile-major)
  int step_stride;   // 64 (row-major) or 16384 (tile-major)
  int sw_lo, sw_hi;  // tile-major: R / 4 of the first row of each half; -1: row-major
  __device__ __forceinline__ const uint8_t* at(int r16, int s, int q) const {
    const int i = r16 & 7, sw = r16 < 8 ? sw_lo : sw_hi;
    const int slot = sw < 0 ? q : (q ^ ((sw + (i >> 2)) & 3));
    return (r16 < 8 ? lo : hi) + (int64_t)i * row_stride + (int64_t)s * step_stride + slot * 16;
  }
};

__device__ __forceinline__ WTile wtile_rows(const uint8_t* lo, const uint8_t* hi, int kb) {
  return WTile{lo, hi, kb, 64, -1, -1};
}

// Row R of its GEMM tile, and that tile, of L1 weight row j of the gate (up =
// false) or up matrix: the L1 tile order (128 intermediate columns per tile;
// per 64 of them 32 gate rows, 32 more gate rows, then the 64 up rows).
__device__ __forceinline__ int l1_tile_row(int j, bool up) {
  const int jj = j & (L1_J_PER_TILE - 1);
  return (jj >> 6) * 128 + (up ? 64 : 0) + (jj & 63);
}

// Tile-major halves: L1 rows (j_lo, up_lo) .. +7 and (j_hi, up_hi) .. +7 (both
// in one GEMM tile), of the expert's L1 blocks at pk; K = hidden.
__device__ __forceinline__ WTile wtile_l1_packed(const uint8_t* pk, int K, int j_lo, bool up_lo, int j_hi,
                                                 bool up_hi) {
  const uint8_t* blk = pk + (int64_t)(j_lo / L1_J_PER_TILE) * (K / 128) * CODE_BLOCK_BYTES;
  const int rl = l1_tile_row(j_lo, up_lo), rh = l1_tile_row(j_hi, up_hi);
  return WTile{blk + rl * 64, blk + rh * 64, 64, CODE_BLOCK_BYTES, rl >> 2, rh >> 2};
}

// Tile-major L2 rows n0 .. n0+15 (n0 % 16 == 0) of the expert's L2 blocks at
// pk; K = intermediate.
__device__ __forceinline__ WTile wtile_l2_packed(const uint8_t* pk, int K, int n0) {
  const uint8_t* blk = pk + (int64_t)(n0 / BN) * (K / 128) * CODE_BLOCK_BYTES;
  const int r = n0 & (BN - 1);
  return WTile{blk + r * 64, blk + (r + 8) * 64, 64, CODE_BLOCK_BYTES, r >> 2, (r + 8) >> 2};
}

// The tile rows' scale bytes (ks per row), two dwords per thread at most
// (16 * ks <= 4 KB).
struct ScaleRegs {
  uint32_t v[2];
};

__device__ __forceinline__ void load_wscales(const RowPair& sp, int ks, ScaleRegs& sr) {
  const int per_row = ks >> 2;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = min((int)threadIdx.x + DT * r, 16 * per_row - 1);   // unconditional, as load_x
    const int row = i / per_row, c = i - row * per_row;
    sr.v[r] = *(const uint32_t*)(sp.row(row, ks) + c * 4);
  }
}

__device__ __forceinline__ void store_wscales(const ScaleRegs& sr, int ks, uint8_t* dst) {
  const int per_row = ks >> 2;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = threadIdx.x + DT * r;
    if (i < 16 * per_row) *(uint32_t*)(dst + i * 4) = sr.v[r];
  }
}

// Workgroup barrier that does not wait for outstanding global loads (the
// weight codes stay in flight); LDS writes are complete before it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Shared body of both kernels: the wave's K-step run of one 16-row weight tile
// (codes `wp`, scales `sp`) times the m tokens of `act` [m, K] bf16, quantised
// into LDS. Wave 0 returns the workgroup's total for lane (token lane%16, tile
// rows 4*(lane/16) + v).
template <int XR, int NS>
__device__ __forceinline__ f32x4 tile_times_tokens(const uint16_t* __restrict__ act, int m, int K, WTile wp,
                                                   RowPair sp, uint8_t* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int kb = K / 2, ks = K / 32, ksteps = K / 128;
  const int xstride = kb + 16;   // pad: consecutive tokens start 4 banks apart
  uint8_t* xq = lds;
  uint8_t* xs = xq + MAX_TOK * xstride;
  uint8_t* wsl = xs + ((MAX_TOK * ks + 15) & ~15);
  f32x4* red = (f32x4*)(wsl + ((16 * ks + 15) & ~15));

  // Loads, in completion order: activations, scales, weight codes.
  XBlocks<XR> xb;
  load_x<XR>(act, m, K, xb);
  ScaleRegs sr;
  load_wscales(sp, ks, sr);
  __builtin_amdgcn_sched_barrier(0);
  int s0, n;
  wave_steps(ksteps, s0, n);
  // NS >= n steps per wave; steps past the wave's run re-read a valid step
  // (unconditional loads, as load_x) and are not multiplied.
  uint4 wa[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) wa[k] = *(const uint4*)wp.at(r16, min(s0 + k, ksteps - 1), q);
  __builtin_amdgcn_sched_barrier(0);

  quant_x_to_lds<XR>(xb, m, K, xq, xstride, xs);
  store_wscales(sr, ks, wsl);
  lds_barrier();

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool tok_ok = r16 < m;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    if (k < n) {
      const int s = s0 + k;
      uint4 b = make_uint4(0u, 0u, 0u, 0u);
      int sb = 0;
      if (tok_ok) {
        b = *(const uint4*)(xq + r16 * xstride + s * 64 + q * 16);
        sb = xs[r16 * ks + s * 4 + q];
      }
      const int sa = wsl[r16 * ks + s * 4 + q];
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(opnd(wa[k]), opnd(b), acc, 4, 4, 0, sa, 0, sb);
    }
  }
  if (wave > 0) red[(wave - 1) * 64 + lane] = acc;
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < DW - 1; ++w) {
      const f32x4 o = red[w * 64 + lane];
      acc[0] += o[0]; acc[1] += o[1]; acc[2] += o[2]; acc[3] += o[3];
    }
  }
  return acc;
}

// L1 for 8 intermediate columns j0 .. j0+7: tile rows 0..7 are w1 (gate), rows
// 8..15 are w3 (up). h[m][j] = bf16(silu(g) * u).
template <int XR, int NS>
__global__ __launch_bounds__(DT, 1) void k_decode_l1(const uint16_t* __restrict__ x, int m, int H, int I,
                                                     const uint8_t* __restrict__ w1, const uint8_t* __restrict__ w1s,
                                                     const uint8_t* __restrict__ w3, const uint8_t* __restrict__ w3s,
                                                     const uint8_t* __restrict__ pk, uint16_t* __restrict__ h) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int j0 = blockIdx.x * 8;
  const int kb = H / 2, ks = H / 32;
  const WTile wp = pk != nullptr ? wtile_l1_packed(pk, H, j0, false, j0, true)
                                 : wtile_rows(w1 + (int64_t)j0 * kb, w3 + (int64_t)j0 * kb, kb);
  const RowPair sp{w1s + (int64_t)j0 * ks, w3s + (int64_t)j0 * ks};
  f32x4 acc = tile_times_tokens<XR, NS>(x, m, H, wp, sp, lds);
  const int lane = threadIdx.x & 63;
  // lane (token t, q): rows 4q + v; q = 0, 1 hold the gate of j = j0 + 4q + v
  // and lane ^ 32 (q + 2) holds the up value of the same j.
  float up[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) up[v] = __shfl_xor(acc[v], 32);
  const int t = lane & 15, q = lane >> 4;
  if ((threadIdx.x >> 6) == 0 && q < 2 && t < m) {
    const uint32_t p0 = bf16x2_rne(silu_mul(acc[0], up[0]), silu_mul(acc[1], up[1]));
    const uint32_t p1 = bf16x2_rne(silu_mul(acc[2], up[2]), silu_mul(acc[3], up[3]));
    *(uint2*)(h + (int64_t)t * I + j0 + 4 * q) = make_uint2(p0, p1);
  }
}

// L2 for 16 output columns n0 .. n0+15: y[m][n] = bf16(MXFP4(h) . w2[n]).
template <int XR, int NS>
__global__ __launch_bounds__(DT, 1) void k_decode_l2(const uint16_t* __restrict__ h, int m, int H, int I,
                                                     const uint8_t* __restrict__ w2, const uint8_t* __restrict__ w2s,
                                                     const uint8_t* __restrict__ pk, uint16_t* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int n0 = blockIdx.x * 16;
  const int kb = I / 2, ks = I / 32;
  const WTile wp = pk != nullptr ? wtile_l2_packed(pk, I, n0)
                                 : wtile_rows(w2 + (int64_t)n0 * kb, w2 + (int64_t)(n0 + 8) * kb, kb);
  const RowPair sp{w2s + (int64_t)n0 * ks, w2s + (int64_t)(n0 + 8) * ks};
  f32x4 acc = tile_times_tokens<XR, NS>(h, m, I, wp, sp, lds);
  const int lane = threadIdx.x & 63;
  const int t = lane & 15, q = lane >> 4;
  if ((threadIdx.x >> 6) == 0 && t < m) {
    const uint32_t p0 = bf16x2_rne(acc[0], acc[1]);
    const uint32_t p1 = bf16x2_rne(acc[2], acc[3]);
    *(uint2*)(y + (int64_t)t * H + n0 + 4 * q) = make_uint2(p0, p1);
  }
}

// ---------------------------------------------------------------- 9 <= M <= 512
// Same weight stream, with the activations quantised beforehand into the
// chunked layout (launch_quant_mxfp4_chunked): the token operand of a wave's
// load instruction is one 1 KB block of codes per 16-token chunk and K step,
// read straight from memory (the token rows are small and stay in the L2), and
// one 8-byte load per lane and chunk brings its scales for the wave's whole K
// run. Row-major token rows would make each code load 16 separate 64-byte
// pieces 3.5 KB apart (measured nearly twice as slow at 64..128 tokens), and a
// scale byte per step costs the address unit as much as a code load. A workgroup holds MT 16-row weight tiles; a wave keeps its
// K run of every tile in registers and walks the NC token chunks, the loads of
// the next two chunks (three for runs of up to 3 K steps, whose registers
// allow it) in flight during the MFMAs of chunk c (one chunk ahead measured
// 2-5 % slower from 128 tokens on), each chunk's token operands
// feeding the MT tiles' MFMAs. The 8 waves' partial sums meet in LDS and wave
// c finishes chunk c. Every workgroup reads all m token rows, so MT = 2 halves
// the token bytes per weight byte (and the workgroups: one round over the CUs
// instead of two).
constexpr int SK_MAX_CHUNKS = 8;     // chunks of 16 tokens per group (registers of the accumulators)

// LDS sized by the chunk count: a launch of few chunks leaves room for more
// workgroups per CU (the weight stream needs many loads in flight per CU).
template <int MT, int NC>
struct SkinnyLds {
  uint8_t wscale[MT][16 * 256];                    // the tiles' E8M0 bytes, K <= 8192
  f32x4 red[DW][NC][MT][64];                       // partial sums per wave, chunk, tile, lane
};

template <int MT>
struct TileSums {
  f32x4 v[MT];
};

// wtile(t) / srows(t): where tile t's codes and scale rows are, by value (an
// array of them would be a private array, which the compiler places in LDS).
// aq / as: the m token rows' codes and scales in the chunked layout, which
// holds ceil(m / 16) chunks; chunks c of the launch's NC beyond those re-read
// the last one (their rows are not written out).
template <int MT, int NC, int NS, class WTiles, class SRows, class Emit>
__device__ __forceinline__ void tiles_times_qtokens(const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as,
                                                    int m, int K, WTiles wtile, SRows srows, SkinnyLds<MT, NC>& L,
                                                    Emit&& emit) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int ks = K / 32, ksteps = K / 128;

  ScaleRegs sr[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) load_wscales(srows(t), ks, sr[t]);
  int s0, n;
  wave_steps(ksteps, s0, n);
  uint4 wa[MT][NS];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const WTile w = wtile(t);
#pragma unroll
    for (int k = 0; k < NS; ++k) wa[t][k] = *(const uint4*)w.at(r16, min(s0 + k, ksteps - 1), q);
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) store_wscales(sr[t], ks, L.wscale[t]);
  lds_barrier();

  // token operands of chunk c: the lane's 16 bytes of each (chunk, step) code
  // block (the padding rows of the last chunk hold zero codes) and its 8 scale
  // bytes of the wave's run, step k in byte k
  constexpr int PD = NS <= 3 ? 3 : 2;   // chunks in flight ahead of the MFMAs
  uint4 b[PD + 1][NS];
  uint2 bsc[PD + 1];
  const int nchunks = (m + 15) / 16, last_chunk = nchunks - 1;
  // this lane's weight scale bytes (row r16, quarter q of each step of the
  // run) are the same for every token chunk: read from LDS once into registers
  // when they fit (up to 16: two tiles of up to 8 steps), else per chunk
  constexpr bool HOIST = MT * NS <= 16;
  auto wsc_byte = [&](int t, int k) { return (int)L.wscale[t][r16 * ks + min(s0 + k, ksteps - 1) * 4 + q]; };
  int sar[HOIST ? MT : 1][HOIST ? NS : 1];
  if constexpr (HOIST) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int k = 0; k < NS; ++k) sar[t][k] = wsc_byte(t, k);
  }
  auto load_chunk = [&](int c, uint4 (&bb)[NS], uint2& ss) {
    const int cc = min(c, last_chunk);
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int64_t blk = (int64_t)cc * ksteps + min(s0 + k, ksteps - 1);
      bb[k] = *(const uint4*)(aq + blk * 1024 + lane * 16);
    }
    ss = *(const uint2*)(as + (((int64_t)cc * DW + wave) * 64 + lane) * 8);
  };
  // groups of NC chunks (more than one only past 16 * NC tokens): the weight
  // runs stay in registers, the partial sums' LDS is reused per group
  for (int c0 = 0; c0 < nchunks; c0 += NC) {
    f32x4 acc[NC][MT];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < PD; ++c)
      if (c < NC) load_chunk(c0 + c, b[c], bsc[c]);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c + PD < NC) load_chunk(c0 + c + PD, b[(c + PD) % (PD + 1)], bsc[(c + PD) % (PD + 1)]);
      // steps past the wave's run (k >= n) multiply zero codes: no branch around
      // the MFMAs, which would make the compiler copy the accumulators; their
      // token scale bytes are not written by the quantiser, so 2^0 stands in
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        const int sb = k < n ? (int)((k < 4 ? bsc[c % (PD + 1)].x : bsc[c % (PD + 1)].y) >> (8 * (k & 3))) : 0x7F;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const uint4 az = k < n ? wa[t][k] : z;
          acc[c][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(opnd(az), opnd(b[c % (PD + 1)][k]), acc[c][t], 4, 4,
                                                                       0, HOIST ? sar[HOIST ? t : 0][HOIST ? k : 0] : wsc_byte(t, k), 0, sb);
        }
      }
      // keep the loads of later chunks where they are written (PD chunks ahead):
      // hoisting them all would hold every chunk's operands in registers
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int t = 0; t < MT; ++t) L.red[wave][c][t][lane] = acc[c][t];
    __syncthreads();
    TileSums<MT> tot;
#pragma unroll
    for (int t = 0; t < MT; ++t) tot.v[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (wave < NC) {
#pragma unroll
      for (int w = 0; w < DW; ++w)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const f32x4 o = L.red[w][wave][t][lane];
          tot.v[t][0] += o[0]; tot.v[t][1] += o[1]; tot.v[t][2] += o[2]; tot.v[t][3] += o[3];
        }
    }
    // lane (token c0 * 16 + 16 * wave + lane % 16, tile rows 4 * (lane / 16) + v)
    // in waves < NC
    emit(c0 * 16 + wave * 16 + r16, tot);
    if (c0 + NC < nchunks) __syncthreads();   // the next group rewrites L.red
  }
}

// L1: chunk `wave` of each token group -> h for 16 * P intermediate columns j0 ..
// per workgroup: tiles 2p and 2p + 1 hold the gate (w1) and up (w3) rows of
// columns j0 + 16p .. +15, so a lane holds g and u of the same (token, j) and
// forms h = bf16(silu(g) * u) in place. pk: the tile-major L1 codes, or null.
//  * RQ = false: h is written in bf16, row-major [m, I].
//  * RQ = true (P = 2): a token's 32 columns j0 .. j0+31 are one MXFP4 block,
//    held by its 4 lanes (8 values each), so the workgroup re-quantises h
//    itself with the MXFP4 quantiser's steps (block max over the 4 lanes,
//    the same scale and code rounding) into the chunked layout the L2 reads:
//    hq codes and hs scales of K = I, rows up to the last whole chunk (rows
//    past m as zero codes with scale byte 0, as the quantiser writes them).
template <int P, int NC, int NS, bool RQ>
__global__ __launch_bounds__(DT, 1) void k_skinny_l1(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                                                     int m, int H, int I, const uint8_t* __restrict__ w1,
                                                     const uint8_t* __restrict__ w1s, const uint8_t* __restrict__ w3,
                                                     const uint8_t* __restrict__ w3s,
                                                     const uint8_t* __restrict__ pk, uint16_t* __restrict__ h,
                                                     uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  static_assert(!RQ || P == 2, "a 32-column MXFP4 block needs two gate/up pairs");
  __shared__ SkinnyLds<2 * P, NC> L;
  const int j0 = blockIdx.x * 16 * P;
  const int kb = H / 2, ks = H / 32;
  auto wtile = [=](int t) {
    const int j = j0 + 16 * (t >> 1);
    if (pk != nullptr) return wtile_l1_packed(pk, H, j, (t & 1) == 1, j + 8, (t & 1) == 1);
    const uint8_t* w = (t & 1) == 0 ? w1 : w3;
    return wtile_rows(w + (int64_t)j * kb, w + (int64_t)(j + 8) * kb, kb);
  };
  auto srows = [=](int t) {
    const int j = j0 + 16 * (t >> 1);
    const uint8_t* s = (t & 1) == 0 ? w1s : w3s;
    return RowPair{s + (int64_t)j * ks, s + (int64_t)(j + 8) * ks};
  };
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane >> 4;
  const int mrows = (m + 15) / 16 * 16;   // rows of the chunked layout
  tiles_times_qtokens<2 * P, NC, NS>(xq, xs, m, H, wtile, srows, L, [&](int tk, const TileSums<2 * P>& acc) {
    // lane (token, q): rows 4q + v of every tile, j = j0 + 16p + 4q + v
    uint32_t hp[2 * P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const f32x4& g = acc.v[2 * p];
      const f32x4& u = acc.v[2 * p + 1];
      hp[2 * p] = bf16x2_rne(silu_mul(g[0], u[0]), silu_mul(g[1], u[1]));
      hp[2 * p + 1] = bf16x2_rne(silu_mul(g[2], u[2]), silu_mul(g[3], u[3]));
    }
    if constexpr (!RQ) {
      if (wave < NC && tk < m) {
#pragma unroll
        for (int p = 0; p < P; ++p)
          *(uint2*)(h + (int64_t)tk * I + j0 + 16 * p + 4 * q) = make_uint2(hp[2 * p], hp[2 * p + 1]);
      }
    } else {
      if (tk >= m) hp[0] = hp[1] = hp[2] = hp[3] = 0u;   // padding rows of the last chunk
      uint32_t am = max(max(amax2(hp[0]), amax2(hp[1])), max(amax2(hp[2]), amax2(hp[3])));
      am = max(am, (uint32_t)__shfl_xor((int)am, 16));
      am = max(am, (uint32_t)__shfl_xor((int)am, 32));
      const uint32_t sb = mx_scale_from_amax_bits(am);
      uint32_t w;
      quant_pairs_e8m0<4>(hp, sb, &w);   // codes of j0 + 4q .. +3 (bytes 0, 1), j0 + 16 + 4q .. +3 (2, 3)
      if (wave < NC && tk < mrows) {
        // the L2's K step s = j0 / 128 and lane quarter (j0 / 32) % 4
        const int ksteps = I / 128, s = j0 >> 7, lq = (j0 >> 5) & 3, r = tk & 15, c = tk >> 4;
        uint8_t* blk = hq + (((int64_t)c * ksteps + s) * 64 + lq * 16 + r) * 16;
        *(uint16_t*)(blk + 2 * q) = (uint16_t)(w & 0xFFFFu);
        *(uint16_t*)(blk + 8 + 2 * q) = (uint16_t)(w >> 16);
        if (q == 0) {
          // step s -> (wave w2, place k2 in its run) of the L2's balanced split
          const int base = ksteps / DW, extra = ksteps - base * DW;
          int w2, k2;
          if (s < extra * (base + 1)) {
            w2 = s / (base + 1);
            k2 = s - w2 * (base + 1);
          } else {
            const int e = s - extra * (base + 1);
            w2 = extra + e / base;
            k2 = e - (w2 - extra) * base;
          }
          hs[(((int64_t)c * DW + w2) * 64 + lq * 16 + r) * 8 + k2] = (uint8_t)sb;
        }
      }
    }
  });
}

// L2: chunk `wave` of each token group -> y (bf16), 16 * MT output columns per
// workgroup (tile t: w2 rows n0 + 16t .. +15). pk: the tile-major L2 codes, or
// null.
template <int MT, int NC, int NS>
__global__ __launch_bounds__(DT, 1) void k_skinny_l2(const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs,
                                                     int m, int H, int I, const uint8_t* __restrict__ w2,
                                                     const uint8_t* __restrict__ w2s,
                                                     const uint8_t* __restrict__ pk, uint16_t* __restrict__ y) {
  __shared__ SkinnyLds<MT, NC> L;
  const int n0 = blockIdx.x * 16 * MT;
  const int kb = I / 2, ks = I / 32;
  auto wtile = [=](int t) {
    const int n = n0 + 16 * t;
    if (pk != nullptr) return wtile_l2_packed(pk, I, n);
    return wtile_rows(w2 + (int64_t)n * kb, w2 + (int64_t)(n + 8) * kb, kb);
  };
  auto srows = [=](int t) { return RowPair{w2s + (int64_t)(n0 + 16 * t) * ks, w2s + (int64_t)(n0 + 16 * t + 8) * ks}; };
  const int wave = threadIdx.x >> 6, q = (threadIdx.x & 63) >> 4;
  tiles_times_qtokens<MT, NC, NS>(hq, hs, m, I, wtile, srows, L, [&](int tk, const TileSums<MT>& acc) {
    if (wave < NC && tk < m) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const uint32_t p0 = bf16x2_rne(acc.v[t][0], acc.v[t][1]);
        const uint32_t p1 = bf16x2_rne(acc.v[t][2], acc.v[t][3]);
        *(uint2*)(y + (int64_t)tk * H + n0 + 16 * t + 4 * q) = make_uint2(p0, p1);
      }
    }
  });
}

// ---------------------------------------------------------------- routed, few tokens
// Routed experts with few rows each (a decode step, or the tail of a batch):
// the tiled GEMM would give each (expert, weight tile) a 256-row token tile
// holding a handful of rows and wait out one copy latency per K stage, so the
// weights are streamed once instead, as on the dense few-token path. The rows
// of expert e are the sorted pair rows expert_off[e] .. expert_off[e+1] of the
// route kernels. Grid: (groups of RT_TILES 16-row weight tiles) x (experts);
// the workgroups of experts without rows leave at once. A workgroup keeps its
// weight tiles in registers (each wave a run of K steps) and multiplies them
// by the expert's rows 16 at a time; the 8 waves' partial sums meet in LDS and
// wave t adds those of tile t in wave order.
//  * L1 gathers the MXFP4 token rows by row_token and writes h (bf16) in
//    sorted row order.
//  * L2 reads re-quantised h rows in sorted order: MXFP4 codes through the
//    scaled FP4 MFMA, or (NVFP4 re-quantisation, whose E4M3 per-16 scale an
//    E8M0 MFMA scale cannot carry) NVFP4 codes and E4M3 scales converted in
//    registers to code * s in bf16 (exact: at most 6 significant bits), with
//    the weight codes converted exactly to bf16 too, through
//    V_MFMA_F32_16X16X32_BF16. The output row of pair p is o[row_slot[p]] =
//    bf16(acc * (scale * row_weight[p])), scale 1 or the NVFP4 global g, as in
//    the GEMM's epilogue.
enum RoutedOperand { RT_FP4 = 0, RT_NV = 1 };

// MT tiles of 16 weight rows per workgroup; the partial sums of one chunk of
// 16 token rows at a time.
template <int MT>
struct RoutedLds {
  uint8_t wscale[MT][16 * 256];   // the tiles' E8M0 bytes, K <= 8192
  f32x4 red[DW][MT][64];          // partial sums per wave, tile, lane
};

__device__ __forceinline__ uint4 dequant16_bf16(uint32_t codes, float scale) {
  return make_uint4(dequant_pair<0>(codes, scale), dequant_pair<1>(codes, scale), dequant_pair<2>(codes, scale),
                    dequant_pair<3>(codes, scale));
}

// Eight NVFP4 codes (one dword) times their E4M3 block scale s -> eight bf16,
// exact: code * s has at most 2 + 4 significant bits.
__device__ __forceinline__ uint4 nv8_bf16(uint32_t d, float s) {
  const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
  const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
  const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
  const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
  return make_uint4(bf16x2_rne(v0[0] * s, v0[1] * s), bf16x2_rne(v1[0] * s, v1[1] * s),
                    bf16x2_rne(v2[0] * s, v2[1] * s), bf16x2_rne(v3[0] * s, v3[1] * s));
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// The expert's `rows` token rows times MT 16-row weight tiles, tile t's codes
// at wtile(t) and scale rows at srows(t) (by value, as on the dense path).
// Token row i of the expert is row gather[base + i] (gather != nullptr) or
// base + i of the operand: FP4 codes `aq` [.., K/2] with E8M0 scales `as`
// [.., K/32] (RT_FP4) or E4M3 scales `as` [.., K/16] (RT_NV). A lane's token
// operand of a step is loaded (and, for RT_NV, converted to bf16) once and
// serves all MT tiles. `emit(c0, t, tot)` runs in wave t (MT <= DW) for every
// chunk of 16 rows starting at c0, with lane (row c0 + lane%16, rows
// 4*(lane/16) + v of tile t). EVEN: K / 128 = DW NS, every wave's run is NS
// steps (no step to zero).
template <int OP, int NS, int MT, bool EVEN, class WTiles, class SRows, class Emit>
__device__ __forceinline__ void routed_tile_rows(const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as,
                                                 const int32_t* __restrict__ gather,
                                                 int base, int rows, int K, WTiles wtile, SRows srows,
                                                 RoutedLds<MT>& L, Emit&& emit) {
  static_assert(MT <= DW, "one wave per tile reduces the partial sums");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int kb = K / 2, ks = K / 32, ksteps = K / 128;

  ScaleRegs sr[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) load_wscales(srows(t), ks, sr[t]);
  int s0, n;
  wave_steps(ksteps, s0, n);
  uint4 wa[MT][NS];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const WTile w = wtile(t);
#pragma unroll
    for (int k = 0; k < NS; ++k) wa[t][k] = *(const uint4*)w.at(r16, min(s0 + k, ksteps - 1), q);
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) store_wscales(sr[t], ks, L.wscale[t]);
  lds_barrier();
  int sa[MT][NS];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int k = 0; k < NS; ++k) sa[t][k] = L.wscale[t][r16 * ks + min(s0 + k, ksteps - 1) * 4 + q];

  for (int c0 = 0; c0 < rows; c0 += 16) {
    const int i = min(c0 + r16, rows - 1);
    // rows past the expert's (the last chunk's padding) re-read its last row:
    // they feed only their own output columns, which emit does not write
    const int64_t tok = gather != nullptr ? (int64_t)gather[base + i] : (int64_t)(base + i);
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (OP == RT_FP4) {
      uint4 b[NS];
      int sb[NS];
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const int s = min(s0 + k, ksteps - 1);
        b[k] = *(const uint4*)(aq + tok * kb + s * 64 + q * 16);
        sb[k] = as[tok * ks + s * 4 + q];
      }
      // steps past the wave's run (k >= n) multiply zero codes: no branch
      // around the MFMAs
#pragma unroll
      for (int k = 0; k < NS; ++k) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const uint4 az = EVEN || k < n ? wa[t][k] : z;
          acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(opnd(az), opnd(b[k]), acc[t], 4, 4, 0, sa[t][k],
                                                                     0, sb[k]);
        }
      }
    } else {
      // A lane's 32 K values of a step (K = 128 s + 32 q + 0..31, code dwords
      // j = 0..3 of 8 values each, NVFP4 blocks j / 2) feed four 16x16x32
      // MFMAs per tile, dword j in the j-th; the token row uses the same
      // order, so each MFMA contracts matching K.
      uint4 b[NS];
      uint32_t bs[NS];
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const int s = min(s0 + k, ksteps - 1);
        b[k] = *(const uint4*)(aq + tok * kb + s * 64 + q * 16);
        bs[k] = *(const uint16_t*)(as + tok * (K / 16) + s * 8 + q * 2);
      }
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const uint32_t hv[4] = {b[k].x, b[k].y, b[k].z, b[k].w};
        const float hs0 = e4m3_to_f32(bs[k] & 0xFFu), hs1 = e4m3_to_f32(bs[k] >> 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 bv = nv8_bf16(hv[j], j < 2 ? hs0 : hs1);
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const uint32_t wv[4] = {wa[t][k].x, wa[t][k].y, wa[t][k].z, wa[t][k].w};
            const uint4 av = EVEN || k < n ? dequant16_bf16(wv[j], e8m0_to_f32((uint32_t)sa[t][k])) : z;
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                             __builtin_bit_cast(bf16x8_t, bv), acc[t], 0, 0, 0);
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) L.red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave < MT) {
      f32x4 tot = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < DW; ++w) {
        const f32x4 o = L.red[w][wave][lane];
        tot[0] += o[0]; tot[1] += o[1]; tot[2] += o[2]; tot[3] += o[3];
      }
      emit(c0, wave, tot);
    }
    // the next chunk overwrites the partial sums
    if (c0 + 16 < rows) __syncthreads();
  }
}

// L1 of expert blockIdx.y for 8 MT intermediate columns from j0 (tile t: rows
// 0..7 of w1 and 8..15 of w3 for columns j0 + 8 t ..): h[r][j] =
// bf16(silu(g) * u) for its sorted rows r.
template <int NS, int MT, bool EVEN>
__global__ __launch_bounds__(DT, 1) void k_routed_l1(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                                                     const int32_t* __restrict__ row_token,
                                                     const int32_t* __restrict__ expert_off, int H, int I,
                                                     const uint8_t* __restrict__ w1, const uint8_t* __restrict__ w1s,
                                                     const uint8_t* __restrict__ w3, const uint8_t* __restrict__ w3s,
                                                     const uint8_t* __restrict__ pk, int64_t pk_estride,
                                                     uint16_t* __restrict__ h) {
  __shared__ RoutedLds<MT> L;
  const int e = blockIdx.y;
  const int base = expert_off[e], rows = expert_off[e + 1] - base;
  if (rows <= 0) return;
  const int j0 = blockIdx.x * 8 * MT;
  const int64_t kb = H / 2, ks = H / 32;
  const int64_t we = (int64_t)e * I * kb, se = (int64_t)e * I * ks;
  auto wtile = [&](int t) {
    const int j = j0 + 8 * t;
    return pk != nullptr ? wtile_l1_packed(pk + e * pk_estride, H, j, false, j, true)
                         : wtile_rows(w1 + we + j * kb, w3 + we + j * kb, kb);
  };
  auto srows = [&](int t) {
    const int j = j0 + 8 * t;
    return RowPair{w1s + se + j * ks, w3s + se + j * ks};
  };
  routed_tile_rows<RT_FP4, NS, MT, EVEN>(xq, xs, row_token, base, rows, H, wtile, srows, L,
                                   [&](int c0, int tile, const f32x4& acc) {
    const int lane = threadIdx.x & 63, t = lane & 15, q = lane >> 4;
    float up[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) up[v] = __shfl_xor(acc[v], 32);
    if (q < 2 && c0 + t < rows) {
      const uint32_t p0 = bf16x2_rne(silu_mul(acc[0], up[0]), silu_mul(acc[1], up[1]));
      const uint32_t p1 = bf16x2_rne(silu_mul(acc[2], up[2]), silu_mul(acc[3], up[3]));
      *(uint2*)(h + (int64_t)(base + c0 + t) * I + j0 + 8 * tile + 4 * q) = make_uint2(p0, p1);
    }
  });
}

// L2 of expert blockIdx.y for 16 MT output columns from n0 (tile t: n0 + 16 t
// ..), from the re-quantised h rows (FP4 codes + E8M0 or E4M3 scales):
// o[row_slot[r]][n] = bf16(acc * (scale * row_weight[r])).
template <int OP, int NS, int MT, bool EVEN>
__global__ __launch_bounds__(DT, 1) void k_routed_l2(const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs,
                                                     const int32_t* __restrict__ expert_off,
                                                     const int32_t* __restrict__ row_slot,
                                                     const float* __restrict__ row_weight, float scale_val,
                                                     const float* __restrict__ scale_ptr, int H, int I,
                                                     const uint8_t* __restrict__ w2, const uint8_t* __restrict__ w2s,
                                                     const uint8_t* __restrict__ pk, int64_t pk_estride,
                                                     uint16_t* __restrict__ o) {
  __shared__ RoutedLds<MT> L;
  const int e = blockIdx.y;
  const int base = expert_off[e], rows = expert_off[e + 1] - base;
  if (rows <= 0) return;
  const float scale = scale_ptr != nullptr ? *scale_ptr : scale_val;
  const int n0 = blockIdx.x * 16 * MT;
  const int64_t kb = I / 2, ks = I / 32;
  const int64_t we = (int64_t)e * H * kb, se = (int64_t)e * H * ks;
  auto wtile = [&](int t) {
    const int n = n0 + 16 * t;
    return pk != nullptr ? wtile_l2_packed(pk + e * pk_estride, I, n)
                         : wtile_rows(w2 + we + n * kb, w2 + we + (n + 8) * kb, kb);
  };
  auto srows = [&](int t) {
    const int n = n0 + 16 * t;
    return RowPair{w2s + se + n * ks, w2s + se + (n + 8) * ks};
  };
  routed_tile_rows<OP, NS, MT, EVEN>(hq, hs, nullptr, base, rows, I, wtile, srows, L,
                               [&](int c0, int tile, const f32x4& acc) {
    const int lane = threadIdx.x & 63, t = lane & 15, q = lane >> 4;
    if (c0 + t < rows) {
      const int r = base + c0 + t;
      const float wgt = scale * row_weight[r];
      const uint32_t p0 = bf16x2_rne(acc[0] * wgt, acc[1] * wgt);
      const uint32_t p1 = bf16x2_rne(acc[2] * wgt, acc[3] * wgt);
      *(uint2*)(o + (int64_t)row_slot[r] * H + n0 + 16 * tile + 4 * q) = make_uint2(p0, p1);
    }
  });
}

size_t decode_lds(int cols) {
  const size_t kb = cols / 2, ks = cols / 32;
  return MAX_TOK * (kb + 16) + ((MAX_TOK * ks + 15) & ~(size_t)15) + ((16 * ks + 15) & ~(size_t)15) +
         (size_t)(DW - 1) * 64 * sizeof(f32x4);
}

// Activation blocks per thread: m * cols/32 blocks over DT threads.
int x_rounds(int m, int cols) { return (m * (cols / 32) + DT - 1) / DT; }

// Register budget of a wave's K run, rounded up to an instantiated size:
// 7 and 3 are the 7168- and 3072-wide K of the expert, 1 the tiny shapes.
int steps_bucket(int cols) {
  const int ns = (cols / 128 + DW - 1) / DW;
  return ns <= 1 ? 1 : ns <= 3 ? 3 : ns <= 7 ? 7 : MAX_STEPS;
}

struct DecodeArgs {
  const uint16_t* x; int m, H, I;
  const uint8_t *w1, *w1s, *w3, *w3s, *w2, *w2s;
  const uint8_t *pk1, *pk2;   // tile-major L1 / L2 codes, or null
  uint16_t *h, *y;
};

template <int XR, int NS>
void launch_l1(const DecodeArgs& a, hipStream_t s) {
  k_decode_l1<XR, NS><<<a.I / 8, DT, decode_lds(a.H), s>>>(a.x, a.m, a.H, a.I, a.w1, a.w1s, a.w3, a.w3s, a.pk1,
                                                           a.h);
}

template <int XR, int NS>
void launch_l2(const DecodeArgs& a, hipStream_t s) {
  k_decode_l2<XR, NS><<<a.H / 16, DT, decode_lds(a.I), s>>>(a.h, a.m, a.H, a.I, a.w2, a.w2s, a.pk2, a.y);
}

template <int XR>
void launch_l1_ns(const DecodeArgs& a, hipStream_t s) {
  switch (steps_bucket(a.H)) {
    case 1: launch_l1<XR, 1>(a, s); break;
    case 3: launch_l1<XR, 3>(a, s); break;
    case 7: launch_l1<XR, 7>(a, s); break;
    default: launch_l1<XR, MAX_STEPS>(a, s); break;
  }
}

template <int XR>
void launch_l2_ns(const DecodeArgs& a, hipStream_t s) {
  switch (steps_bucket(a.I)) {
    case 1: launch_l2<XR, 1>(a, s); break;
    case 3: launch_l2<XR, 3>(a, s); break;
    case 7: launch_l2<XR, 7>(a, s); break;
    default: launch_l2<XR, MAX_STEPS>(a, s); break;
  }
}

// Weight tiles per workgroup of the 9..512-token L2 kernel (32 w2 rows); the
// L1 kernel holds two as well, the gate and up rows of 16 intermediate columns.
constexpr int SK_TILES = 2;

// Up to 2 chunks (32 tokens) the L1 takes two gate/up pairs per workgroup and
// re-quantises h itself, which saves the h quantiser's launch; past that the
// halved workgroup count (96 for the expert's 3072 columns, on 256 CUs) costs
// more than the launch, and the L1 takes one pair per workgroup and writes h
// in bf16 for the quantiser. Measured on the shared expert (7168 x 3072): 18.9
// against 20.5 us at 16 tokens, 20.3 against 21.1 at 32; 24.0 against 23.6 at
// 64, 32.2 against 28.6 at 128.
constexpr int SK_L1_FUSED_CHUNKS = 2;

bool skinny_l1_fused(int m) { return (m + 15) / 16 <= SK_L1_FUSED_CHUNKS; }

template <int NC, int NS>
void launch_skinny_l1(const DecodeArgs& a, const uint8_t* xq, const uint8_t* xs, uint8_t* hq, uint8_t* hs,
                      hipStream_t s) {
  if constexpr (NC <= SK_L1_FUSED_CHUNKS) {
    k_skinny_l1<2, NC, NS, true><<<a.I / 32, DT, 0, s>>>(xq, xs, a.m, a.H, a.I, a.w1, a.w1s, a.w3, a.w3s, a.pk1,
                                                          a.h, hq, hs);
  } else {
    k_skinny_l1<1, NC, NS, false><<<a.I / 16, DT, 0, s>>>(xq, xs, a.m, a.H, a.I, a.w1, a.w1s, a.w3, a.w3s, a.pk1,
                                                           a.h, hq, hs);
  }
}

template <int NC, int NS>
void launch_skinny_l2(const DecodeArgs& a, const uint8_t* hq, const uint8_t* hs, hipStream_t s) {
  k_skinny_l2<SK_TILES, NC, NS><<<a.H / (16 * SK_TILES), DT, 0, s>>>(hq, hs, a.m, a.H, a.I, a.w2, a.w2s, a.pk2,
                                                                    a.y);
}

template <int NC>
void launch_skinny_l1_ns(const DecodeArgs& a, const uint8_t* xq, const uint8_t* xs, uint8_t* hq, uint8_t* hs,
                         hipStream_t s) {
  switch (steps_bucket(a.H)) {
    case 1: launch_skinny_l1<NC, 1>(a, xq, xs, hq, hs, s); break;
    case 3: launch_skinny_l1<NC, 3>(a, xq, xs, hq, hs, s); break;
    case 7: launch_skinny_l1<NC, 7>(a, xq, xs, hq, hs, s); break;
    default: launch_skinny_l1<NC, MAX_STEPS>(a, xq, xs, hq, hs, s); break;
  }
}

template <int NC>
void launch_skinny_l2_ns(const DecodeArgs& a, const uint8_t* hq, const uint8_t* hs, hipStream_t s) {
  switch (steps_bucket(a.I)) {
    case 1: launch_skinny_l2<NC, 1>(a, hq, hs, s); break;
    case 3: launch_skinny_l2<NC, 3>(a, hq, hs, s); break;
    case 7: launch_skinny_l2<NC, 7>(a, hq, hs, s); break;
    default: launch_skinny_l2<NC, MAX_STEPS>(a, hq, hs, s); break;
  }
}

// Weight tiles per workgroup of the routed kernels: two. The token operand of
// a step is loaded once for both, and the NVFP4 L2 converts it to bf16 once
// for both (it does so in every workgroup of the expert). Measured on the
// 8-token tail of the skewed batch (28 experts of 7168 x 3072, hipGraph
// replay), one / two / four tiles: NVFP4 277 / 242 / 252 us (four take 163
// VGPRs, one workgroup per CU); at 72 tokens 575 / 458 us with two tiles in
// both kernels. Hidden and intermediate sizes are multiples of 128, so 8 and
// 16 RT_TILES divide them.
constexpr int RT_TILES = 2;

template <int NS>
void launch_routed_l1_ns(const RoutedArgs& a, hipStream_t s) {
  constexpr int MT = RT_TILES;
  const dim3 grid(a.I / (8 * MT), a.E);
  if (a.H / 128 == DW * NS)
    k_routed_l1<NS, MT, true><<<grid, DT, 0, s>>>(a.xq, a.xs, a.row_token, a.expert_off, a.H, a.I, a.w1, a.w1s,
                                                  a.w3, a.w3s, a.pk1, a.pk1_estride, a.h);
  else
    k_routed_l1<NS, MT, false><<<grid, DT, 0, s>>>(a.xq, a.xs, a.row_token, a.expert_off, a.H, a.I, a.w1, a.w1s,
                                                   a.w3, a.w3s, a.pk1, a.pk1_estride, a.h);
}

template <int OP, int NS>
void launch_routed_l2_ns(const RoutedArgs& a, hipStream_t s) {
  constexpr int MT = RT_TILES;
  const dim3 grid(a.H / (16 * MT), a.E);
  // the NVFP4 operand keeps the zero steps: without them the compiler hoists
  // every conversion of the run (162 VGPRs, one workgroup per CU; the 8-token
  // tail 246 -> 253 us); the FP4 one gains (MXFP4 tail 218.5 -> 214.6 us)
  constexpr bool FP4 = OP == RT_FP4;
  if (FP4 && a.I / 128 == DW * NS)
    k_routed_l2<OP, NS, MT, FP4><<<grid, DT, 0, s>>>(a.hq, a.hs, a.expert_off, a.row_slot, a.row_weight, a.scale,
                                                      a.scale_ptr, a.H, a.I, a.w2, a.w2s, a.pk2, a.pk2_estride, a.o);
  else
    k_routed_l2<OP, NS, MT, false><<<grid, DT, 0, s>>>(a.hq, a.hs, a.expert_off, a.row_slot, a.row_weight, a.scale,
                                                       a.scale_ptr, a.H, a.I, a.w2, a.w2s, a.pk2, a.pk2_estride,
                                                       a.o);
}

template <int OP>
void launch_routed_l2_op(const RoutedArgs& a, hipStream_t s) {
  switch (steps_bucket(a.I)) {
    case 1: launch_routed_l2_ns<OP, 1>(a, s); break;
    case 3: launch_routed_l2_ns<OP, 3>(a, s); break;
    case 7: launch_routed_l2_ns<OP, 7>(a, s); break;
    default: launch_routed_l2_ns<OP, MAX_STEPS>(a, s); break;
  }
}

}  // namespace

// Every workgroup reads all m token rows, so the token traffic grows with m;
// past 128 tokens the kernels take them in groups of 128 (the accumulators'
// register budget) with the weights still read once. Measured on the shared
// expert (7168 x 3072, hipGraph replay over rotating weight copies): 28.7 /
// 40.3 / 49.7 / 62.4 / 74.0 us at 128 / 256 / 300 / 512 / 640 tokens, against
// 51 / 64 / 69 / 77 / 71 us for the tiled GEMMs.
constexpr int SK_MAX_TOKENS = 512;

bool skinny_fits(int64_t m, int64_t hidden, int64_t inter) {
  if (m < 1 || m > SK_MAX_TOKENS) return false;
  if (hidden > DW * MAX_STEPS * 128 || inter > DW * MAX_STEPS * 128) return false;
  if (inter % 32 != 0 || hidden % (16 * SK_TILES) != 0) return false;
  return 16 * (hidden / 32) <= 8 * DT && 16 * (inter / 32) <= 8 * DT;
}

hipError_t launch_skinny_mlp(const uint16_t* x, int m, int H, int I, const uint8_t* w1, const uint8_t* w1s,
                             const uint8_t* w3, const uint8_t* w3s, const uint8_t* w2, const uint8_t* w2s,
                             const uint8_t* pk1, const uint8_t* pk2, uint8_t* xq, uint8_t* xs, uint16_t* h,
                             uint8_t* hq, uint8_t* hs, uint16_t* y, hipStream_t s) {
  const DecodeArgs a{x, m, H, I, w1, w1s, w3, w3s, w2, w2s, pk1, pk2, h, y};
  hipError_t e = launch_quant_mxfp4_chunked(x, m, H, xq, xs, s);
  if (e != hipSuccess) return e;
  const int nc = (m + 15) / 16;
  if (nc <= 1) launch_skinny_l1_ns<1>(a, xq, xs, hq, hs, s);
  else if (nc <= 2) launch_skinny_l1_ns<2>(a, xq, xs, hq, hs, s);
  else if (nc <= 4) launch_skinny_l1_ns<4>(a, xq, xs, hq, hs, s);
  else launch_skinny_l1_ns<8>(a, xq, xs, hq, hs, s);
  if (!skinny_l1_fused(m)) {
    e = launch_quant_mxfp4_chunked(h, m, I, hq, hs, s);
    if (e != hipSuccess) return e;
  }
  if (nc <= 1) launch_skinny_l2_ns<1>(a, hq, hs, s);
  else if (nc <= 2) launch_skinny_l2_ns<2>(a, hq, hs, s);
  else if (nc <= 4) launch_skinny_l2_ns<4>(a, hq, hs, s);
  else launch_skinny_l2_ns<8>(a, hq, hs, s);
  return hipGetLastError();
}

bool decode_fits(int64_t m, int64_t hidden, int64_t inter) {
  if (m < 1 || m > MAX_TOK) return false;
  // every K step of a wave is held in registers
  if (hidden > DW * MAX_STEPS * 128 || inter > DW * MAX_STEPS * 128) return false;
  if (inter % 8 != 0 || hidden % 16 != 0) return false;
  // at most 4 activation blocks and two scale dwords per thread
  if (x_rounds((int)m, (int)hidden) > 4 || x_rounds((int)m, (int)inter) > 4) return false;
  if (16 * (hidden / 32) > 8 * DT || 16 * (inter / 32) > 8 * DT) return false;
  return decode_lds((int)hidden) <= 64 * 1024 && decode_lds((int)inter) <= 64 * 1024;
}

hipError_t launch_decode_mlp(const uint16_t* x, int m, int H, int I, const uint8_t* w1, const uint8_t* w1s,
                             const uint8_t* w3, const uint8_t* w3s, const uint8_t* w2, const uint8_t* w2s,
                             const uint8_t* pk1, const uint8_t* pk2, uint16_t* h, uint16_t* y, hipStream_t s) {
  const DecodeArgs a{x, m, H, I, w1, w1s, w3, w3s, w2, w2s, pk1, pk2, h, y};
  const int r1 = x_rounds(m, H), r2 = x_rounds(m, I);
  if (r1 <= 1) launch_l1_ns<1>(a, s);
  else if (r1 <= 2) launch_l1_ns<2>(a, s);
  else launch_l1_ns<4>(a, s);
  if (r2 <= 1) launch_l2_ns<1>(a, s);
  else if (r2 <= 2) launch_l2_ns<2>(a, s);
  else launch_l2_ns<4>(a, s);
  return hipGetLastError();
}

// Mean rows per expert up to which the routed weight-streaming kernels run
// instead of the tiled GEMMs. Each workgroup reads all rows of its expert, so
// their load instructions and MFMAs grow with the rows, while the GEMMs' time
// at this size hardly depends on them. Measured over 48 experts of 7168 x 3072
// (hipGraph replay, uniform top-8), streaming against GEMMs: with MXFP4
// re-quantisation 239 / 275 / 294 / 337 / 352 / 368 against 277 / 300 / 308 /
// 362 / 364 / 366 us at 8 / 12 / 16 / 24 / 32 / 48 tokens; with NVFP4, whose
// GEMM L2 converts both operands to bf16 per tile, 284 / 433 / 604 / 739
// against 511 / 694 / 699 / 704 us at 8 / 64 / 128 / 192 tokens.
constexpr int64_t RT_MAX_MEAN_ROWS_MXFP4 = 6;
constexpr int64_t RT_MAX_MEAN_ROWS_NVFP4 = 24;

bool routed_stream_fits(int64_t T, int64_t hidden, int64_t inter, int k, int E, bool nvfp4) {
  const int64_t mean_rows = nvfp4 ? RT_MAX_MEAN_ROWS_NVFP4 : RT_MAX_MEAN_ROWS_MXFP4;
  if (T < 1 || T * (int64_t)k > mean_rows * E) return false;
  if (hidden > DW * MAX_STEPS * 128 || inter > DW * MAX_STEPS * 128) return false;
  if (inter % 128 != 0 || hidden % 128 != 0) return false;
  return 16 * (hidden / 32) <= 8 * DT && 16 * (inter / 32) <= 8 * DT;
}

hipError_t launch_routed_l1(const RoutedArgs& a, hipStream_t s) {
  switch (steps_bucket(a.H)) {
    case 1: launch_routed_l1_ns<1>(a, s); break;
    case 3: launch_routed_l1_ns<3>(a, s); break;
    case 7: launch_routed_l1_ns<7>(a, s); break;
    default: launch_routed_l1_ns<MAX_STEPS>(a, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_routed_l2(const RoutedArgs& a, hipStream_t s) {
  if (a.nvfp4) launch_routed_l2_op<RT_NV>(a, s);
  else launch_routed_l2_op<RT_FP4>(a, s);
  return hipGetLastError();
}

}  // namespace mx
