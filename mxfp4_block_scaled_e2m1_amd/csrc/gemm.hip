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
// Design (gfx950):
//  * One workgroup = 4 waves = a 256 (weight rows) x 128 (token rows) tile; each
//    wave owns 128 x 64 = 4 x 2 MFMA blocks of 32 x 32 (128 fp32 accumulators).
//  * The packed layout is already the MFMA operand layout: a lane holds 32
//    consecutive K values of one row (16 bytes) and that block's E8M0 byte. Over a
//    256-wide K stage, lane half h takes 32-column chunks 4h..4h+3 in its four
//    MFMA steps, so each lane's scales for a stage are one aligned dword and the
//    step index is the byte select (op_sel) of the instruction. Both operands
//    use the same K order, so the sum is unchanged.
//  * Global -> LDS with GLOBAL_LOAD_LDS_DWORDX4 (16 B per lane, no VGPR staging),
//    3 LDS stages in flight (51 KB each). Rows are 128 B in LDS; the 16-byte
//    chunk c of row r sits at slot c ^ ((r >> 1) & 7) so that the 16 rows read
//    by a quarter-wave spread over all banks.
//  * blockIdx -> tile mapping is XCD aware: consecutive tiles (the m-tiles of one
//    expert's weight n-tile) land on the same XCD and share its L2.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

namespace {

constexpr int ROW_BYTES = BK / 2;                     // 128 code bytes per row per stage
constexpr int W_BYTES = BN * ROW_BYTES;               // 32768
constexpr int X_BYTES = BM * ROW_BYTES;               // 16384
constexpr int WS_BYTES = BN * (BK / 32);              // 2048
constexpr int XS_BYTES = BM * (BK / 32);              // 1024
constexpr int OFF_X = W_BYTES;
constexpr int OFF_WS = W_BYTES + X_BYTES;
constexpr int OFF_XS = OFF_WS + WS_BYTES;
constexpr int STAGE_BYTES = OFF_XS + XS_BYTES;        // 52224
constexpr int VM_PER_STAGE = 8 + 4 + 2 + 1;           // global_load_lds per thread per stage

__device__ __attribute__((aligned(256))) uint8_t g_zero_page[256];

struct Tile {
  int e;         // expert
  int nt;        // tile index along weight rows
  int row0;      // first row (sorted order) of the token tile
  int rows;      // valid rows in the token tile
};

// Returns false when this workgroup has no tile.
__device__ __forceinline__ bool map_tile(const GemmArgs& a, Tile& t) {
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  int total;
  if (a.expert_off == nullptr) total = a.grid_tiles;
  else total = a.tile_base[a.n_experts] * a.n_tiles;
  const int per = (total + 7) >> 3;
  if (local >= per) return false;
  const int L = xcd * per + local;
  if (L >= total) return false;
  if (a.expert_off == nullptr) {
    const int mtiles = (a.m_rows + BM - 1) / BM;
    t.e = 0;
    t.nt = L / mtiles;
    const int mt = L - t.nt * mtiles;
    t.row0 = mt * BM;
    t.rows = min(BM, a.m_rows - t.row0);
    return true;
  }
  // expert e with tile_base[e] * n_tiles <= L < tile_base[e + 1] * n_tiles
  int lo = 0, hi = a.n_experts - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.tile_base[mid] * a.n_tiles <= L) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int tb = a.tile_base[e];
  const int nte = a.tile_base[e + 1] - tb;
  const int r = L - tb * a.n_tiles;
  t.e = e;
  t.nt = r / nte;
  const int mt = r - t.nt * nte;
  const int off = a.expert_off[e];
  t.row0 = off + mt * BM;
  t.rows = min(BM, a.expert_off[e + 1] - t.row0);
  return true;
}

// Global -> LDS copies. Lane i of the wave writes LDS bytes [m0 + i*size, +size).
// They are issued as inline asm so that the compiler neither waits for them
// before every LDS read nor at every barrier: the K loop waits for exactly the
// stage it needs (s_waitcnt vmcnt) before its barrier. Code the compiler emits
// itself can only wait longer because of them, never shorter.
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

// One 64-wide K step of a wave's 4 x 2 block of 32 x 32 MFMAs from LDS stage `sb`.
// S selects both the 32-column chunk (4*hh + S) and the scale byte (op_sel).
template <int S>
__device__ __forceinline__ void mfma_step(const uint8_t* sb, int wrow_off, int xrow_off, int hh, int swz,
                                          const uint32_t (&sa)[4], const uint32_t (&sbx)[2],
                                          f32x16 (&acc)[4][2]) {
  const int coff = ((hh * 4 + S) ^ swz) * 16;
  i32x8 A[4], B[2];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const uint4 v = *(const uint4*)(sb + wrow_off + f * 32 * ROW_BYTES + coff);
    A[f] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const uint4 v = *(const uint4*)(sb + xrow_off + g * 32 * ROW_BYTES + coff);
    B[g] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
      acc[f][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[f], B[g], acc[f][g], 4, 4, S,
                                                                 (int)sa[f], S, (int)sbx[g]);
}

template <int EPI>
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_gemm(const GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * STAGE_BYTES];

  Tile t;
  if (!map_tile(a, t)) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave >> 1, wm = wave & 1;
  const int K = a.k;
  const int kb = K >> 1;                    // code bytes per row
  const int ks = K >> 5;                    // scale bytes per row
  const int nst = (K + BK - 1) / BK;
  const bool half_tail = (K % BK) != 0;     // last stage holds 128 columns only
  const bool l1 = (EPI == EPI_SWIGLU_MXFP4 || EPI == EPI_SWIGLU_NVFP4);

  const uint8_t* wa = a.wa + (int64_t)t.e * a.w_estride;
  const uint8_t* wa_s = a.wa_s + (int64_t)t.e * a.ws_estride;
  const uint8_t* wb = l1 ? a.wb + (int64_t)t.e * a.w_estride : nullptr;
  const uint8_t* wb_s = l1 ? a.wb_s + (int64_t)t.e * a.ws_estride : nullptr;

  // ---- per-thread source rows for the stage loads ----
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

  const uint8_t* wsrc[8];
  int wchunk[8];
  for (int i = 0; i < 8; ++i) {
    const int q = wave * 8 + i;
    const int R = q * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((R >> 1) & 7);
    const uint8_t *base, *sbase;
    const int row = w_row(R, base, sbase);
    wsrc[i] = base + (int64_t)row * kb + c * 16;
    wchunk[i] = c;
  }
  const uint8_t* xsrc[4];
  int xchunk[4];
  for (int i = 0; i < 4; ++i) {
    const int q = wave * 4 + i;
    const int R = q * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((R >> 1) & 7);
    xsrc[i] = a.x + (int64_t)x_token(R) * kb + c * 16;
    xchunk[i] = c;
  }
  const uint8_t* wssrc[2];
  int wshalf[2];
  for (int i = 0; i < 2; ++i) {
    const int d = (wave * 2 + i) * 64 + lane;
    const uint8_t *base, *sbase;
    const int row = w_row(d >> 1, base, sbase);
    wssrc[i] = sbase + (int64_t)row * ks + (d & 1) * 4;
    wshalf[i] = d & 1;
  }
  const int dxs = wave * 64 + lane;
  const uint8_t* xssrc = a.x_s + (int64_t)x_token(dxs >> 1) * ks + (dxs & 1) * 4;
  const int xshalf = dxs & 1;

  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int st) {
    const uint32_t sb = lds0 + (st % NSTAGE) * STAGE_BYTES;
    const bool tail = half_tail && st == nst - 1;
    const int ko = st * ROW_BYTES;
    const int kso = st * (BK / 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const void* src = (tail && wchunk[i] >= 4) ? (const void*)g_zero_page : (const void*)(wsrc[i] + ko);
      lds_dma16(src, sb + (wave * 8 + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const void* src = (tail && xchunk[i] >= 4) ? (const void*)g_zero_page : (const void*)(xsrc[i] + ko);
      lds_dma16(src, sb + OFF_X + (wave * 4 + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const void* src = (tail && wshalf[i]) ? (const void*)g_zero_page : (const void*)(wssrc[i] + kso);
      lds_dma4(src, sb + OFF_WS + (wave * 2 + i) * 256);
    }
    {
      const void* src = (tail && xshalf) ? (const void*)g_zero_page : (const void*)(xssrc + kso);
      lds_dma4(src, sb + OFF_XS + wave * 256);
    }
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
  const int wsc_off = OFF_WS + (wn * 128 + r32) * 8 + hh * 4;
  const int xsc_off = OFF_XS + (wm * 64 + r32) * 8 + hh * 4;

  issue(0);
  if (nst > 1) issue(1);

  for (int st = 0; st < nst; ++st) {
    // Stage st has landed once at most one younger stage (15 copies) is in flight;
    // the barrier then publishes every wave's copies and retires the reads of the
    // slot that the next issue overwrites (their MFMAs consumed them already).
    if (st + 1 < nst) asm volatile("s_waitcnt vmcnt(15)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    static_assert(VM_PER_STAGE == 15, "vmcnt immediate above assumes 15 loads per stage");
    if (st + 2 < nst) issue(st + 2);

    const uint8_t* sb = smem + (st % NSTAGE) * STAGE_BYTES;
    uint32_t sa[4], sbx[2];
#pragma unroll
    for (int f = 0; f < 4; ++f) sa[f] = *(const uint32_t*)(sb + wsc_off + f * 32 * 8);
#pragma unroll
    for (int g = 0; g < 2; ++g) sbx[g] = *(const uint32_t*)(sb + xsc_off + g * 32 * 8);

    mfma_step<0>(sb, wrow_off, xrow_off, hh, swz, sa, sbx, acc);
    mfma_step<1>(sb, wrow_off, xrow_off, hh, swz, sa, sbx, acc);
    mfma_step<2>(sb, wrow_off, xrow_off, hh, swz, sa, sbx, acc);
    mfma_step<3>(sb, wrow_off, xrow_off, hh, swz, sa, sbx, acc);
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
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int ml = wm * 64 + g * 32 + r32;
      if (ml >= t.rows) continue;
      const int row = t.row0 + ml;
      int64_t out_row = row;
      float wgt = 1.0f;
      if (a.row_slot != nullptr) {
        const int slot = a.row_slot[row];
        out_row = slot;
        wgt = a.slot_weight[slot];
      }
      uint16_t* dst = a.out_bf16 + out_row * a.n_rows;
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = t.nt * BN + wn * 128 + f * 32 + 8 * q + 4 * hh;
          if (n < a.n_rows) {
            uint32_t p0 = f32_to_bf16_rne(acc[f][g][4 * q] * wgt) |
                          (f32_to_bf16_rne(acc[f][g][4 * q + 1] * wgt) << 16);
            uint32_t p1 = f32_to_bf16_rne(acc[f][g][4 * q + 2] * wgt) |
                          (f32_to_bf16_rne(acc[f][g][4 * q + 3] * wgt) << 16);
            *(uint2*)(dst + n) = make_uint2(p0, p1);
          }
        }
    }
  } else {
    // L1: gate in acc[f][g], up in acc[f + 2][g] for f = 0, 1.
    const int I = a.n_rows;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int j0 = t.nt * L1_J_PER_TILE + wn * 64 + f * 32;   // 32-aligned block of j
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int ml = wm * 64 + g * 32 + r32;
        const bool valid = (ml < t.rows) && (j0 < I);
        const int row = t.row0 + ml;
        // h as bf16 bit patterns, packed in pairs: hp[q*2 + 0] = (v=4q, 4q+1), hp[q*2+1] = (4q+2, 4q+3)
        uint32_t hp[8];
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const uint32_t lo = f32_to_bf16_rne(silu_mul(acc[f][g][v], acc[f + 2][g][v]));
          const uint32_t hi = f32_to_bf16_rne(silu_mul(acc[f][g][v + 1], acc[f + 2][g][v + 1]));
          hp[v >> 1] = lo | (hi << 16);
        }
        uint32_t bytes_lo, bytes_hi;   // this lane's 8 code bytes (positions 4q + 2hh + {0,1})
        if constexpr (EPI == EPI_SWIGLU_MXFP4) {
          uint32_t am = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) am = max(am, amax2(hp[i]));
          am = max(am, (uint32_t)__shfl_xor((int)am, 32));
          const uint32_t sbyte = mx_scale_from_amax_bits(am);
          uint32_t w0 = 0, w1 = 0;
          // byte order within (w0, w1): q=0 pair0, q=0 pair1, q=1 pair0, q=1 pair1 | q=2 ..., q=3 ...
          w0 = quant_pair_e8m0<0>(w0, hp[0], sbyte);
          w0 = quant_pair_e8m0<1>(w0, hp[1], sbyte);
          w0 = quant_pair_e8m0<2>(w0, hp[2], sbyte);
          w0 = quant_pair_e8m0<3>(w0, hp[3], sbyte);
          w1 = quant_pair_e8m0<0>(w1, hp[4], sbyte);
          w1 = quant_pair_e8m0<1>(w1, hp[5], sbyte);
          w1 = quant_pair_e8m0<2>(w1, hp[6], sbyte);
          w1 = quant_pair_e8m0<3>(w1, hp[7], sbyte);
          bytes_lo = w0;
          bytes_hi = w1;
          if (valid && hh == 0) a.h_scales[(int64_t)row * (I >> 5) + (j0 >> 5)] = (uint8_t)sbyte;
        } else {
          // NVFP4: 16-blocks j0..j0+15 (v = 0..7) and j0+16..j0+31 (v = 8..15).
          const float gsc = a.nv_global;
          const float t6 = 6.0f * gsc;
          uint32_t w01[2];
          uint32_t sbytes[2];
#pragma unroll
          for (int blk = 0; blk < 2; ++blk) {
            uint32_t am = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) am = max(am, amax2(hp[blk * 4 + i]));
            am = max(am, (uint32_t)__shfl_xor((int)am, 32));
            const float r = bf16_to_f32(am) / t6;
            const uint32_t sbyte = e4m3_rne_satfinite(r);
            sbytes[blk] = sbyte;
            const float d = e4m3_to_f32(sbyte) * gsc;
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t pr = hp[blk * 4 + i];
              float v0 = bf16_to_f32(pr & 0xFFFFu), v1 = bf16_to_f32(pr >> 16);
              if (sbyte == 0) { v0 *= 0.0f; v1 *= 0.0f; }
              else {
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
            uint16_t two = (uint16_t)(sbytes[0] | (sbytes[1] << 8));
            *(uint16_t*)(a.h_scales + (int64_t)row * (I >> 4) + (j0 >> 4)) = two;
          }
        }
        // Lane hh=0 holds byte positions {0,1,4,5,8,9,12,13} of the 16-byte block row,
        // hh=1 holds {2,3,6,7,10,11,14,15}; bytes_lo = q0p0,q0p1,q1p0,q1p1, bytes_hi = q2.., q3...
        // Exchange so hh=0 writes bytes 0..7 and hh=1 writes 8..15.
        const uint32_t send = hh ? bytes_lo : bytes_hi;
        const uint32_t recv = (uint32_t)__shfl_xor((int)send, 32);
        uint32_t o0, o1;
        if (hh == 0) {
          // positions 0,1 = my q0; 2,3 = peer q0; 4,5 = my q1; 6,7 = peer q1
          o0 = (bytes_lo & 0xFFFFu) | ((recv & 0xFFFFu) << 16);
          o1 = (bytes_lo >> 16) | (recv & 0xFFFF0000u);
        } else {
          // positions 8,9 = peer q2; 10,11 = my q2; 12,13 = peer q3; 14,15 = my q3
          o0 = (recv & 0xFFFFu) | ((bytes_hi & 0xFFFFu) << 16);
          o1 = (recv >> 16) | (bytes_hi & 0xFFFF0000u);
        }
        if (valid) {
          *(uint2*)(a.h_codes + (int64_t)row * (I >> 1) + (j0 >> 1) + hh * 8) = make_uint2(o0, o1);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(Epilogue epi, const GemmArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  const int g8 = (grid + 7) & ~7;
  switch (epi) {
    case EPI_F32: k_gemm<EPI_F32><<<g8, GEMM_THREADS, 0, s>>>(a); break;
    case EPI_SWIGLU_MXFP4: k_gemm<EPI_SWIGLU_MXFP4><<<g8, GEMM_THREADS, 0, s>>>(a); break;
    case EPI_SWIGLU_NVFP4: k_gemm<EPI_SWIGLU_NVFP4><<<g8, GEMM_THREADS, 0, s>>>(a); break;
    case EPI_BF16: k_gemm<EPI_BF16><<<g8, GEMM_THREADS, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mx
