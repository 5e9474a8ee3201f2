// Block-scaled FP4 x FP4 GEMM on gfx950 matrix cores (V_MFMA_SCALE_F32_32X32X64_F8F6F4),
// with the epilogues of the expert MLP.
//
// What it computes: D[n][m] = sum_k W[n][k] * X[m][k] where W (weight rows) and
// X (token rows) are MXFP4: E2M1 codes packed two per byte, low nibble first,
// and one E8M0 scale per row per 32 logical columns (page "2026-05-08 DeepSeek
// V4 Pro NVFP4 Quantization", sections "Script update" and "FP4 (E2M1) expert
// weight format confirmed"). The L1 epilogue applies SiLU(gate) * up and
// re-quantises to FP4, the L2 epilogue writes bf16 (page "Current Bug: vLLM
// produces empty/garbage output", section "Revised Plan", Phase 1: L1 GEMM,
// SiLU, re-quant, L2 GEMM; Phase 3 keeps the SiLU output and the final scatter
// in BF16).
//
// Design (gfx950, one 512-thread workgroup per CU, two waves per SIMD):
//  * Workgroup tile 256 weight rows x 256 token rows. Each of the 8 waves owns
//    128 x 64 = 4 x 2 MFMA blocks of 32 x 32 (128 fp32 accumulators per lane).
//    At FP4 rate the tile needs 32 B/clk/CU of operand bytes from L2.
//  * The packed layout is already the MFMA operand layout: a lane holds 32
//    consecutive K values of one row (16 bytes) and that block's E8M0 byte.
//    A 256-wide K stage is four MFMA steps; in step s lane half h takes the
//    32-column chunk 4h + s, so the lane's four scale bytes for the stage are one
//    aligned dword and s is the byte select (op_sel) of the instruction.
//    Both operands use the same K order, so the sum is unchanged.
//  * Global -> LDS with GLOBAL_LOAD_LDS_DWORDX4 (16 B per lane, no VGPR staging),
//    issued by every wave between its MFMAs of a stage's last K step,
//    2 LDS slots of 68 KB: each copy brings whole 128-byte lines (8 rows x 128 B
//    per wave instruction), which doubles the bytes per outstanding L1 miss
//    compared with half-line copies. LDS rows are 128 B; chunk c of row r sits at
//    slot c ^ ((r >> 1) & 7) so the 16 rows a quarter-wave reads hit distinct banks.
//  * Operand fragments are double-buffered in registers: the LDS reads of the
//    next step are interleaved with the MFMAs of the current one.
//  * blockIdx -> tile mapping is XCD aware: consecutive tiles (the m-tiles of one
//    expert's weight n-tile) land on the same XCD and share its L2.
#include <atomic>

#include "gemm_common.h"

namespace mx {

namespace {

constexpr int ROW_BYTES = BK / 2;                     // 128 code bytes per row per stage
constexpr int SC_BYTES = BK / 32;                     // 8 scale bytes per row per stage
constexpr int W_BYTES = BN * ROW_BYTES;               // 32768
constexpr int X_BYTES = BM * ROW_BYTES;               // 32768
constexpr int WS_BYTES = BN * SC_BYTES;               // 2048
constexpr int XS_BYTES = BM * SC_BYTES;               // 2048
constexpr int OFF_X = W_BYTES;
constexpr int OFF_WS = W_BYTES + X_BYTES;
constexpr int OFF_XS = OFF_WS + WS_BYTES;
constexpr int STAGE_BYTES = OFF_XS + XS_BYTES;        // 69632
constexpr int SMEM_BYTES = NSTAGE * STAGE_BYTES;
constexpr int NWAVES = GEMM_THREADS / 64;             // 8: 2 along weight rows x 4 along tokens
constexpr int W_DMA = W_BYTES / 1024 / NWAVES;        // 16-byte copies per wave per stage (W)
constexpr int X_DMA = X_BYTES / 1024 / NWAVES;
constexpr int VM_PER_STAGE = W_DMA + X_DMA + 2;       // + two dword copies of the scale tiles
static_assert(VM_PER_STAGE == 10, "the vmcnt immediate below assumes 10 copies per stage");
static_assert(NSTAGE == 2, "the pipeline below is written for 2 LDS slots");
static_assert(WS_BYTES + XS_BYTES == GEMM_THREADS * 8, "two scale dwords per thread per stage");
static_assert(SMEM_BYTES >= TILE_LDS_TOTAL, "the bf16 epilogue stages its tile in the K-loop LDS");

// Zero bytes for the upper half of a K stage when K % 256 == 128: zero codes with
// zero scale bytes (2^-127) contribute exactly 0 to every sum.
__device__ __attribute__((aligned(256))) uint8_t g_zero_page[256];

// Global -> LDS copies. Lane i of the wave writes LDS bytes [m0 + i*size, +size).
// They are issued as inline asm so that the compiler neither waits for them
// before every LDS read nor at every barrier: the K loop waits for exactly the
// stage it needs (s_waitcnt vmcnt) before its barrier. Waits the compiler
// emits for its own loads can only become longer because of them, never shorter.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_off)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* src, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds_off)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

struct Frags {
  uint4 A[4];   // weight rows wn*128 + f*32 + r32: 32 K values (16 bytes) each
  uint4 B[2];   // token rows wm*64 + g*32 + r32
};

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *(const uint4*)p; }

__device__ __forceinline__ i32x8 opnd(const uint4& v) {
  return i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

// No stage copies between the MFMAs of a step.
struct NoCopy {
  __device__ __forceinline__ void operator()(int) const {}
};

// The eight MFMAs of K step S (chunk 4*hh + S, scale byte S) from `cur`,
// interleaved with the six LDS reads that fill `nxt` for the next step (when
// READ), so that the reads issue while the matrix core is busy. `copy(i)` runs
// before MFMA i: the last step of a stage spreads the next slot's global -> LDS
// copies over its MFMAs this way.
template <int S, bool READ, class Copy>
__device__ __forceinline__ void k_step(const Frags& cur, Frags& nxt, const uint8_t* sbn, int coffn,
                                       int wrow_off, int xrow_off, const uint32_t (&sa)[4],
                                       const uint32_t (&sb)[2], f32x16 (&acc)[4][2], const Copy& copy) {
#pragma unroll
  for (int f = 0; f < 4; ++f) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int i = f * 2 + g;
      copy(i);
      acc[f][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(opnd(cur.A[f]), opnd(cur.B[g]), acc[f][g], 4,
                                                                 4, S, (int)sa[f], S, (int)sb[g]);
      // After MFMA i (0..5) read fragment i of the next step, in the order the
      // next step's MFMAs consume them (A0 B0 B1 A1 A2 A3): every read then has
      // at least six MFMAs of this wave before its first use.
      if (READ && i < 6) {
        if (i == 0) nxt.A[0] = lds16(sbn + wrow_off + coffn);
        else if (i == 1) nxt.B[0] = lds16(sbn + xrow_off + coffn);
        else if (i == 2) nxt.B[1] = lds16(sbn + xrow_off + 32 * ROW_BYTES + coffn);
        else nxt.A[i - 2] = lds16(sbn + wrow_off + (i - 2) * 32 * ROW_BYTES + coffn);
      }
    }
  }
  if (READ) {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
}

// One 32 x 32 block of the L1 epilogue, as this lane holds it: gate `ga` and up
// `ua` are D[n][m] of token row ml within the tile and j = j0 + 8*(v/4) + 4*hh + v%4.
// h = bf16(silu(g) * u) is re-quantised per 32 j (MXFP4: one E8M0 byte; NVFP4:
// two E4M3 bytes per 16 j and the fp32 global scale) and stored with the codes.
// Returns (MXFP4) the max |h| of the block row as bf16 bits, 0 for padding rows.
template <int EPI>
__device__ __forceinline__ uint32_t l1_block(const GemmArgs& a, const Tile& t, const f32x16& ga, const f32x16& ua,
                                             int j0, int ml, int hh) {
  const int I = a.n_rows;
  const bool valid = (ml < t.rows) && (j0 < I);
  const int row = t.row0 + ml;
  // h as bf16 pairs: hp[2q] = (v = 4q, 4q+1), hp[2q+1] = (4q+2, 4q+3)
  uint32_t hp[8];
#pragma unroll
  for (int v = 0; v < 16; v += 2) {
    hp[v >> 1] = bf16x2_rne(silu_mul(ga[v], ua[v]), silu_mul(ga[v + 1], ua[v + 1]));
  }
  uint32_t bytes_lo, bytes_hi;   // this lane's 8 code bytes (positions 4q + 2hh + {0,1})
  uint32_t block_amax = 0;
  if constexpr (EPI == EPI_SWIGLU_MXFP4) {
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = max(am, amax2(hp[i]));
    am = max(am, (uint32_t)__shfl_xor((int)am, 32));
    const uint32_t sbyte = mx_scale_from_amax_bits(am);
    block_amax = valid ? am : 0u;
    uint32_t w01[2];
    quant_pairs_e8m0<8>(hp, sbyte, w01);
    bytes_lo = w01[0];
    bytes_hi = w01[1];
    if (valid && hh == 0) {
      // row-major [rows][I/32], or tile-major for the L2's copies: m-tile
      // t.mt, L2 stage j0/256, tile row ml, byte (j0/32) % 8
      const int64_t at = a.h_scales_packed
                             ? ((int64_t)t.mt * ((I + BK - 1) / BK) + (j0 >> 8)) * SC_TILE_STAGE_BYTES +
                                   ml * SC_BYTES + ((j0 >> 5) & 7)
                             : (int64_t)row * (I >> 5) + (j0 >> 5);
      a.h_scales[at] = (uint8_t)sbyte;
    }
  } else {
    // NVFP4: 16-blocks j0..j0+15 (v = 0..7) and j0+16..j0+31 (v = 8..15).
    const float gsc = a.nv_gptr != nullptr ? *a.nv_gptr : a.nv_global;
    const float t6 = 6.0f * gsc;
    uint32_t w01[2];
    uint32_t sbytes[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      uint32_t am = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) am = max(am, amax2(hp[blk * 4 + i]));
      am = max(am, (uint32_t)__shfl_xor((int)am, 32));
      // a block holding an infinity or a NaN gets the E4M3 NaN byte 0x7F
      const uint32_t sbyte = am >= 0x7F80u ? 0x7Fu : e4m3_rne_satfinite(bf16_to_f32(am) / t6);
      sbytes[blk] = sbyte;
      const float d = e4m3_to_f32(sbyte) * gsc;
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t pr = hp[blk * 4 + i];
        float v0 = bf16_to_f32(pr & 0xFFFFu), v1 = bf16_to_f32(pr >> 16);
        if (sbyte == 0) {
          v0 *= 0.0f;
          v1 *= 0.0f;
        } else {
          v0 = fminf(fmaxf(v0 / d, -6.0f), 6.0f);
          v1 = fminf(fmaxf(v1 / d, -6.0f), 6.0f);
        }
        if (i == 0) w = quant_pair_f32_unit<0>(w, v0, v1);
        else if (i == 1) w = quant_pair_f32_unit<1>(w, v0, v1);
        else if (i == 2) w = quant_pair_f32_unit<2>(w, v0, v1);
        else w = quant_pair_f32_unit<3>(w, v0, v1);
      }
      w01[blk] = w;
    }
    bytes_lo = w01[0];
    bytes_hi = w01[1];
    if (valid && hh == 0) {
      const uint16_t two = (uint16_t)(sbytes[0] | (sbytes[1] << 8));
      *(uint16_t*)(a.h_scales + (int64_t)row * (I >> 4) + (j0 >> 4)) = two;
    }
  }
  // Lane hh=0 holds byte positions {0,1,4,5,8,9,12,13} of the 16-byte block row,
  // hh=1 holds {2,3,6,7,10,11,14,15}; bytes_lo = q0p0,q0p1,q1p0,q1p1, bytes_hi = q2.., q3...
  // Exchange so that hh=0 writes bytes 0..7 and hh=1 writes 8..15.
  const uint32_t send = hh ? bytes_lo : bytes_hi;
  const uint32_t recv = (uint32_t)__shfl_xor((int)send, 32);
  uint32_t o0, o1;
  if (hh == 0) {
    o0 = (bytes_lo & 0xFFFFu) | ((recv & 0xFFFFu) << 16);
    o1 = (bytes_lo >> 16) | (recv & 0xFFFF0000u);
  } else {
    o0 = (recv & 0xFFFFu) | ((bytes_hi & 0xFFFFu) << 16);
    o1 = (recv >> 16) | (bytes_hi & 0xFFFF0000u);
  }
  if (valid) {
    *(uint2*)(a.h_codes + (int64_t)row * (I >> 1) + (j0 >> 1) + hh * 8) = make_uint2(o0, o1);
  }
  return block_amax;
}

// NVFP4 warm-up: fold this wave's max |h| into *amax (one atomic per wave).
__device__ __forceinline__ void wave_amax_atomic(uint32_t* amax, uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  if ((threadIdx.x & 63) == 0) atomicMax(amax, v);
}

// One 256 x 256 output tile: K loop and epilogue. All LDS reads and copies of
// the tile have completed when it returns.
template <int EPI>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, const Tile& t, uint8_t* smem) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // wave -> (wn, wm): consecutive waves share a token block, so the token blocks
  // of a partly filled tile are spread over the SIMDs (waves 0-3 run on four
  // different SIMDs, and wave w + 4 on the SIMD of wave w)
  const int wn = wave & 1, wm = wave >> 1;
  // a wave whose 64 token rows are all past the tile's rows skips its MFMAs and
  // fragment reads (it still copies and meets every barrier)
  const bool act = wm * 64 < t.rows;
  const int K = a.k;
  const int kb = K >> 1;                    // code bytes per row
  const int ks = K >> 5;                    // scale bytes per row
  const int nst_all = (K + BK - 1) / BK;
  // this tile's K stages [ks0, ks1): all of them, or one split's share
  const int nst = t.ks1 - t.ks0;
  const int kc0 = t.ks0 * ROW_BYTES;        // code byte offset of the first stage
  const bool half_tail = (K % BK) != 0 && t.ks1 == nst_all;   // the last stage holds 128 columns only
  constexpr bool l1 = (EPI == EPI_SWIGLU_MXFP4 || EPI == EPI_SWIGLU_NVFP4 || EPI == EPI_PART_L1);

  const uint8_t* wa = a.wa + (int64_t)t.e * a.w_estride;
  const uint8_t* wa_s = a.wa_s + (int64_t)t.e * a.ws_estride;
  const uint8_t* wb = l1 ? a.wb + (int64_t)t.e * a.w_estride : nullptr;
  const uint8_t* wb_s = l1 ? a.wb_s + (int64_t)t.e * a.ws_estride : nullptr;

  // ---- per-thread source rows of the stage copies ----
  // W tile row R -> (matrix, row). L1: R = wn*128 + f*32 + r holds gate rows
  // (f = 0, 1) and up rows (f = 2, 3) of the same j = j0 + wn*64 + (f&1)*32 + r.
  auto w_row = [&](int R, const uint8_t*& base, const uint8_t*& sbase) -> int {
    int row;
    if (l1) {
      const int f = (R >> 5) & 3;
      row = t.nt * L1_J_PER_TILE + (R >> 7) * 64 + (f & 1) * 32 + (R & 31);
      base = (f < 2) ? wa : wb;
      sbase = (f < 2) ? wa_s : wb_s;
    } else {
      row = t.nt * BN + R;
      base = wa;
      sbase = wa_s;
    }
    return min(row, a.n_rows - 1);
  };
  auto x_token = [&](int R) -> int {
    const int r = t.row0 + min(R, t.rows - 1);
    return a.row_token ? a.row_token[r] : r;
  };

  // Copy (wave, i) writes LDS bytes [(wave*W_DMA + i) * 1024, +1024): rows q*8 + lane/8,
  // 16-byte slot lane%8 holding chunk (lane%8) ^ ((row >> 1) & 7).
  const uint8_t* wsrc[W_DMA];
  bool whi[W_DMA];   // chunk in the upper half of the stage (columns 128..255)
#pragma unroll
  for (int i = 0; i < W_DMA; ++i) {
    const int R = (wave * W_DMA + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((R >> 1) & 7);
    const uint8_t *base, *sbase;
    const int row = w_row(R, base, sbase);
    wsrc[i] = base + (int64_t)row * kb + kc0 + c * 16;
    whi[i] = c >= 4;
  }
  const uint8_t* xsrc[X_DMA];
  bool xhi[X_DMA];
#pragma unroll
  for (int i = 0; i < X_DMA; ++i) {
    const int R = (wave * X_DMA + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((R >> 1) & 7);
    xsrc[i] = a.x + (int64_t)x_token(R) * kb + kc0 + c * 16;
    xhi[i] = c >= 4;
  }
  // Scale tiles (8 bytes per row per stage): thread tid copies dword tid & 1 of
  // weight row tid / 2 and of token row tid / 2, from the row-major scales
  // (stage stride 8 bytes) or from a tile-major copy, where a stage of the
  // tile is 2 KB in one piece (stage stride 2 KB).
  const uint8_t *wssrc, *xssrc;
  int wsc_stride = SC_BYTES, xsc_stride = SC_BYTES;
  {
    const int tid = wave * 64 + lane;
    if (a.w_spk != nullptr) {
      wssrc = a.w_spk + (int64_t)t.e * a.wspk_estride + ((int64_t)t.nt * nst_all + t.ks0) * SC_TILE_STAGE_BYTES +
              tid * 4;
      wsc_stride = SC_TILE_STAGE_BYTES;
    } else {
      const uint8_t *base, *sbase;
      const int row = w_row(tid >> 1, base, sbase);
      wssrc = sbase + (int64_t)row * ks + t.ks0 * SC_BYTES + (tid & 1) * 4;
    }
    if (a.x_s_packed) {
      // rows past the tile's end read the last valid row, as the code copies do
      xssrc = a.x_s + ((int64_t)t.mt * nst_all + t.ks0) * SC_TILE_STAGE_BYTES + min(tid >> 1, t.rows - 1) * SC_BYTES +
              (tid & 1) * 4;
      xsc_stride = SC_TILE_STAGE_BYTES;
    } else {
      xssrc = a.x_s + (int64_t)x_token(tid >> 1) * ks + t.ks0 * SC_BYTES + (tid & 1) * 4;
    }
  }

  const uint32_t lds0 = lds_addr(smem);
  // the zero page's address, taken once: referenced inside the K loop, the
  // compiler reloads it there with a scalar load whose wait (lgkmcnt(0)) also
  // drains the LDS reads in flight
  const uint8_t* zpage = g_zero_page;
  asm volatile("" : "+s"(zpage));
  const bool shi = (lane & 1) != 0;   // scale dword of columns 128..255
  // Copy c (0..9) of stage st: W_DMA weight copies, X_DMA token copies, then
  // the two scale dwords.
  auto copy_one = [&](int st, int c) {
    const uint32_t sb = lds0 + (st % NSTAGE) * STAGE_BYTES;
    const int ko = st * ROW_BYTES;
    const bool tail = half_tail && st == nst - 1;
    if (c < W_DMA) {
      lds_dma16((tail && whi[c]) ? (const void*)zpage : (const void*)(wsrc[c] + ko),
                sb + (wave * W_DMA + c) * 1024);
    } else if (c < W_DMA + X_DMA) {
      const int i = c - W_DMA;
      lds_dma16((tail && xhi[i]) ? (const void*)zpage : (const void*)(xsrc[i] + ko),
                sb + OFF_X + (wave * X_DMA + i) * 1024);
    } else if (c == W_DMA + X_DMA) {
      lds_dma4((tail && shi) ? (const void*)zpage : (const void*)(wssrc + st * wsc_stride),
               sb + OFF_WS + wave * 256);
    } else {
      lds_dma4((tail && shi) ? (const void*)zpage : (const void*)(xssrc + st * xsc_stride),
               sb + OFF_XS + wave * 256);
    }
  };
  auto issue = [&](int st) {
#pragma unroll
    for (int c = 0; c < VM_PER_STAGE; ++c) copy_one(st, c);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[f][g][v] = 0.0f;

  // per-lane LDS read offsets
  const int r32 = lane & 31, hh = lane >> 5;
  const int swz = (r32 >> 1) & 7;
  const int wrow_off = (wn * 128 + r32) * ROW_BYTES;
  const int xrow_off = OFF_X + (wm * 64 + r32) * ROW_BYTES;
  const int wsc_off = OFF_WS + (wn * 128 + r32) * SC_BYTES + hh * 4;
  const int xsc_off = OFF_XS + (wm * 64 + r32) * SC_BYTES + hh * 4;
  int coff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) coff[q] = ((hh * 4 + q) ^ swz) * 16;

  // this lane's scale dwords of stage s
  auto read_scales = [&](int s, uint32_t (&sa)[4], uint32_t (&sx)[2]) {
    const uint8_t* rs = smem + (s % NSTAGE) * STAGE_BYTES;
#pragma unroll
    for (int f = 0; f < 4; ++f) sa[f] = *(const uint32_t*)(rs + wsc_off + f * 32 * SC_BYTES);
#pragma unroll
    for (int g = 0; g < 2; ++g) sx[g] = *(const uint32_t*)(rs + xsc_off + g * 32 * SC_BYTES);
  };

  // Output rows and gate weights of the bf16 epilogue, loaded now so that their
  // latency hides behind the K loop (they complete before stage 0's copies,
  // which the prologue waits for).
  TileRows<2> rows;
  if constexpr (EPI == EPI_BF16) rows = load_tile_rows<2>(a, t, wm, lane);

  // Prologue: stages 0 and 1 in flight; wait for stage 0 and read its first step.
  issue(0);
  if (nst > 1) {
    issue(1);
    asm volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  }

  if (act) {
    Frags F0, F1;
    uint32_t sa[4], sx[2];
    read_scales(0, sa, sx);
    // the order of the K loop's reads (A0 B0 B1 A1 A2 A3), so the loop entry
    // needs no longer wait than its back edge
    F0.A[0] = lds16(smem + wrow_off + coff[0]);
#pragma unroll
    for (int g = 0; g < 2; ++g) F0.B[g] = lds16(smem + xrow_off + g * 32 * ROW_BYTES + coff[0]);
#pragma unroll
    for (int f = 1; f < 4; ++f) F0.A[f] = lds16(smem + wrow_off + f * 32 * ROW_BYTES + coff[0]);

    // One K stage. Every read of slot st is issued by the end of step 2: retire
    // them, wait for stage st+1 (the only copies in flight) and run the last
    // step, whose MFMAs overlap `copy` (the refill of slot st with stage st+2)
    // and the reads of stage st+1's first step. In the last stage those reads
    // fetch bytes that are never used.
    auto stage = [&](int st, const auto& copy) {
      const uint8_t* sb = smem + (st % NSTAGE) * STAGE_BYTES;
      k_step<0, true>(F0, F1, sb, coff[1], wrow_off, xrow_off, sa, sx, acc, NoCopy{});
      k_step<1, true>(F1, F0, sb, coff[2], wrow_off, xrow_off, sa, sx, acc, NoCopy{});
      k_step<2, true>(F0, F1, sb, coff[3], wrow_off, xrow_off, sa, sx, acc, NoCopy{});
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const uint8_t* sbn = smem + ((st + 1) % NSTAGE) * STAGE_BYTES;
      uint32_t san[4], sxn[2];
      read_scales(st + 1, san, sxn);
      k_step<3, true>(F1, F0, sbn, coff[0], wrow_off, xrow_off, sa, sx, acc, copy);
#pragma unroll
      for (int q = 0; q < 4; ++q) sa[q] = san[q];
      sx[0] = sxn[0];
      sx[1] = sxn[1];
    };
    // Two loops rather than a branch per stage: with a branch the compiler hoists
    // the last step's MFMAs (identical on both sides) above the barrier, and the
    // copies and reads after it no longer overlap any matrix work.
    int st = 0;
    for (; st + 2 < nst; ++st) {
      const int nx = st + 2;
      stage(st, [&](int i) {   // copies 2i and 2i+1 of stage st+2 before MFMA i
        if (2 * i < VM_PER_STAGE) copy_one(nx, 2 * i);
        if (2 * i + 1 < VM_PER_STAGE) copy_one(nx, 2 * i + 1);
      });
    }
    for (; st < nst; ++st) stage(st, NoCopy{});
  } else {
    // the same copies and barriers as `stage`, without MFMAs (accumulators stay
    // zero): one barrier per stage, so that every wave meets the same barriers
    for (int st = 0; st < nst; ++st) {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (st + 2 < nst) issue(st + 2);
    }
  }

  // ---------------------------------------------------------------- epilogues
  // acc[f][g][v] is D[n][m] with n = (tile n base) + wn*128 + f*32 + 8*(v/4) + 4*hh + v%4
  // and m = wm*64 + g*32 + r32 within the token tile.
  if constexpr (EPI == EPI_F32) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int ml = wm * 64 + g * 32 + r32;
      if (ml >= t.rows) continue;
      const int m = t.row0 + ml;
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = t.nt * BN + wn * 128 + f * 32 + 8 * q + 4 * hh;
          if (n < a.n_rows) {
            float4 o = make_float4(acc[f][g][4 * q], acc[f][g][4 * q + 1], acc[f][g][4 * q + 2],
                                   acc[f][g][4 * q + 3]);
            *(float4*)(a.c_f32 + (int64_t)m * a.n_rows + n) = o;
          }
        }
    }
  } else if constexpr (EPI == EPI_BF16) {
    store_tile_bf16_lds<2>(a, t, acc, rows, wn, wm, lane, 1.0f, smem, GEMM_THREADS);
  } else if constexpr (EPI == EPI_PART_L1) {
    // split-K partial: the accumulators as this lane holds them, 64 contiguous
    // bytes per lane and block (waves of all-padding token rows write nothing)
    if (act) {
      const int mtiles = (a.m_rows + BM - 1) / BM;
      const int tiles = a.grid_tiles / a.k_splits;
      float* pb = a.c_f32 + (((int64_t)t.sp * tiles + t.nt * mtiles + t.mt) * 8 + wave) * (8 * 64 * 16);
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 2; ++g) *(f32x16*)(pb + ((f * 2 + g) * 64 + lane) * 16) = acc[f][g];
    }
  } else {
    // L1: gate in acc[f][g], up in acc[f + 2][g] for f = 0, 1.
    uint32_t amax = 0;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int j0 = t.nt * L1_J_PER_TILE + wn * 64 + f * 32;   // 32-aligned block of j
#pragma unroll
      for (int g = 0; g < 2; ++g)
        amax = max(amax, l1_block<EPI>(a, t, acc[f][g], acc[f + 2][g], j0, wm * 64 + g * 32 + r32, hh));
    }
    if (a.h_amax != nullptr) wave_amax_atomic(a.h_amax, amax);
  }
}

// Persistent kernel: one workgroup per CU. Workgroup b runs on XCD b % 8 (the
// dispatcher deals workgroups to the XCDs in turn); the tiles are cut into 8
// contiguous ranges, one per XCD, and the workgroups of an XCD walk their range
// in lock-step rounds. The 32 tiles of a round share weight and token rows and
// stream the same K slabs at the same time, so those slabs are read once into
// the XCD's L2 and reused from there.
template <int EPI>
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_gemm(const GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM_BYTES];
  __shared__ TileTables tt;
  load_tile_tables(a, tt);
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3, per_xcd_wgs = gridDim.x >> 3;
  const int total = tile_count(a, tt);
  const int per = (total + 7) >> 3;
  const int end = min((xcd + 1) * per, total);
  for (int L = xcd * per + local; L < end; L += per_xcd_wgs) {
    gemm_tile<EPI>(a, decode_tile(a, tt, L), smem);
    // the next tile's first copies overwrite LDS that this tile's waves read
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

// Split-K sum of L1. One 64-thread block per (tile, wave, gate block (f, g)
// with f < 2) of the GEMM's layout: each lane adds the k_splits partials of its
// 16 gate and 16 up accumulators in split order (fixed, so the result does not
// depend on timing), then runs the epilogue the unsplit GEMM runs on its registers.
__device__ __forceinline__ Tile part_tile(const GemmArgs& a, int tix) {
  const int mtiles = (a.m_rows + BM - 1) / BM;
  Tile t;
  t.e = 0;
  t.nt = tix / mtiles;
  t.mt = tix - t.nt * mtiles;
  t.row0 = t.mt * BM;
  t.rows = min(BM, a.m_rows - t.row0);
  t.sp = 0;
  t.ks0 = t.ks1 = 0;
  return t;
}

// Sum of blocks blk0 and blk1 over the splits. The loads of four splits are
// issued before their additions, which stay in split order.
__device__ __forceinline__ void part_sum2(const GemmArgs& a, int tix, int wave, int blk0, int blk1, int lane,
                                          f32x16& s0, f32x16& s1) {
  const int tiles = a.grid_tiles / a.k_splits;
  const int64_t split_stride = (int64_t)tiles * PART_TILE_FLOATS;
  const float* p = a.c_f32 + ((int64_t)tix * 8 + wave) * (8 * 64 * 16) + lane * 16;
  const float* p0 = p + blk0 * 64 * 16;
  const float* p1 = p + blk1 * 64 * 16;
  s0 = f32x16{};
  s1 = f32x16{};
  int sp = 0;
  for (; sp + 4 <= a.k_splits; sp += 4) {
    f32x16 u0[4], u1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u0[i] = *(const f32x16*)(p0 + (sp + i) * split_stride);
      u1[i] = *(const f32x16*)(p1 + (sp + i) * split_stride);
    }
    asm volatile("" ::: "memory");   // all eight loads in flight before the first addition
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s0 += u0[i];
      s1 += u1[i];
    }
  }
  for (; sp < a.k_splits; ++sp) {
    s0 += *(const f32x16*)(p0 + sp * split_stride);
    s1 += *(const f32x16*)(p1 + sp * split_stride);
  }
}

// L1: blocks (f, g) with f < 2; gate in block (f, g), up in (f + 2, g).
__global__ __launch_bounds__(64) void k_part_l1(const GemmArgs a) {
  const int lane = threadIdx.x;
  const int fg = blockIdx.x & 3, wave = (blockIdx.x >> 2) & 7, tix = blockIdx.x >> 5;
  const int f = fg >> 1, g = fg & 1, wn = wave & 1, wm = wave >> 1;
  const Tile t = part_tile(a, tix);
  if (wm * 64 + g * 32 >= t.rows) return;   // token rows all padding: no partials were written
  f32x16 ga, ua;
  part_sum2(a, tix, wave, f * 2 + g, (f + 2) * 2 + g, lane, ga, ua);
  const uint32_t amax = l1_block<EPI_SWIGLU_MXFP4>(a, t, ga, ua, t.nt * L1_J_PER_TILE + wn * 64 + f * 32,
                                                   wm * 64 + g * 32 + (lane & 31), lane >> 5);
  if (a.h_amax != nullptr) wave_amax_atomic(a.h_amax, amax);
}

}  // namespace

hipError_t launch_part_l1(const GemmArgs& a, hipStream_t s) {
  const int tiles = a.grid_tiles / a.k_splits;
  if (tiles <= 0) return hipSuccess;
  k_part_l1<<<tiles * 8 * 4, 64, 0, s>>>(a);
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_gemm(Epilogue epi, const GemmArgs& a, int max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  // one workgroup per CU, at most as many as there can be tiles, a multiple of 8 (XCDs)
  const int cus = cu_count();
  int grid = max_tiles < cus ? max_tiles : cus;
  const int g8 = (grid + 7) & ~7;
  switch (epi) {
    case EPI_F32: k_gemm<EPI_F32><<<g8, GEMM_THREADS, 0, s>>>(a); break;
    case EPI_SWIGLU_MXFP4: k_gemm<EPI_SWIGLU_MXFP4><<<g8, GEMM_THREADS, 0, s>>>(a); break;
    case EPI_SWIGLU_NVFP4: k_gemm<EPI_SWIGLU_NVFP4><<<g8, GEMM_THREADS, 0, s>>>(a); break;
    case EPI_BF16: k_gemm<EPI_BF16><<<g8, GEMM_THREADS, 0, s>>>(a); break;
    case EPI_PART_L1: k_gemm<EPI_PART_L1><<<g8, GEMM_THREADS, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mx
