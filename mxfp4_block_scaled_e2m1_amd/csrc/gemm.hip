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
//    A 128-wide half stage is two MFMA steps; in step s lane half h takes the
//    32-column chunk 2h + s, so the lane's two scale bytes are bytes 2h, 2h+1 of
//    the row's scale dword for the half stage: shifted right by 16h they are
//    bytes 0 and 1, and s is the byte select (op_sel) of the instruction.
//    Both operands use the same K order, so the sum is unchanged.
//  * Global -> LDS with GLOBAL_LOAD_LDS_DWORDX4 (16 B per lane, no VGPR staging)
//    over half stages of 128 K (64 code bytes per row), four LDS slots of 34 KB:
//    half stages h+1 and h+2 are in flight while h is read, and the copies of
//    h+3 go to the slot that h-1 left, spread over the MFMAs of both steps of h
//    (a few per step, never a burst that would hold every wave at the memory
//    issue port while the matrix core idles; measured: spreading the same copies
//    over a stage takes L1 from 0.81 to 0.74 ms). LDS rows are 64 B; chunk c of
//    row r sits at slot c ^ ((r >> 2) & 3) so the 16 rows a quarter-wave reads
//    hit distinct banks.
//  * Operand fragments are double-buffered in registers: the LDS reads of the
//    next step are interleaved with the MFMAs of the current one.
//  * blockIdx -> tile mapping is XCD aware: consecutive tiles (the m-tiles of one
//    expert's weight n-tile) land on the same XCD and share its L2.
#include <atomic>
#include <type_traits>

#include "gemm_common.h"

namespace mx {

namespace {

// The K loop runs over half stages of HK = 128 logical columns: 64 code bytes
// and 4 scale bytes per row. NSLOT = 4 LDS slots hold half stages h, h+1, h+2
// (arriving) and the one being read.
constexpr int HK = BK / 2;                            // 128 logical columns per half stage
constexpr int HROW = HK / 2;                          // 64 code bytes per row per half stage
constexpr int HSC = HK / 32;                          // 4 scale bytes per row per half stage
constexpr int NSLOT = 4;
constexpr int W_BYTES = BN * HROW;                    // 16384
constexpr int X_BYTES = BM * HROW;                    // 16384
constexpr int WS_BYTES = BN * HSC;                    // 1024
constexpr int XS_BYTES = BM * HSC;                    // 1024
constexpr int OFF_X = W_BYTES;
constexpr int OFF_WS = W_BYTES + X_BYTES;
constexpr int OFF_XS = OFF_WS + WS_BYTES;
constexpr int SLOT_BYTES = OFF_XS + XS_BYTES;         // 34816
constexpr int SMEM_BYTES = NSLOT * SLOT_BYTES;        // 139264
constexpr int NWAVES = GEMM_THREADS / 64;             // 8: 2 along weight rows x 4 along tokens
constexpr int W_DMA = W_BYTES / 1024 / NWAVES;        // 16-byte copies per wave per half stage (W): 2
constexpr int X_DMA = X_BYTES / 1024 / NWAVES;        // 2
constexpr int VM_PER_HALF = W_DMA + X_DMA + 1;        // + one dword copy of a scale tile (W: waves 0-3, X: 4-7)
static_assert(VM_PER_HALF == 5, "the vmcnt immediates below assume 5 copies per half stage");
static_assert(WS_BYTES + XS_BYTES == GEMM_THREADS * 4, "one scale dword per thread per half stage");
static_assert(SMEM_BYTES >= TILE_LDS_TOTAL, "the bf16 epilogue stages its tile in the K-loop LDS");
static_assert(CODE_BLOCK_BYTES == W_BYTES, "a tile-major code block is the image of a W slot");

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

// The eight MFMAs of K step S of a half stage (chunk 2*hh + S, scale byte S of
// the lane's shifted scale dword) from `cur`, interleaved with the six LDS reads
// that fill `nxt` for the next step (when READ), so that the reads issue while
// the matrix core is busy. `copy(i)` runs before MFMA i: the global -> LDS
// copies of a later half stage are spread over the MFMAs this way.
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
        else if (i == 2) nxt.B[1] = lds16(sbn + xrow_off + 32 * HROW + coffn);
        else nxt.A[i - 2] = lds16(sbn + wrow_off + (i - 2) * 32 * HROW + coffn);
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
  // this tile's half stages: those of the 256-column stages [ks0, ks1) (all of
  // them, or one split's share); K % 128 == 0, so every half stage is full
  const int nh = min(2 * t.ks1, K / HK) - 2 * t.ks0;
  const int kc0 = t.ks0 * 2 * HROW;         // code byte offset of the first half stage
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

  // Copy (wave, i) writes LDS bytes [(wave*W_DMA + i) * 1024, +1024) of the W
  // (or X) tile: 16 rows of 64 bytes, lane -> row (wave*W_DMA + i)*16 + lane/4,
  // 16-byte slot lane%4 holding chunk (lane%4) ^ ((row >> 2) & 3). The 16 rows a
  // quarter-wave reads then hit 16 distinct 16-byte bank groups.
  // With the tile-major codes (pack.hip) the slot image of half stage h of this
  // tile is one 16 KB block: copy (wave, i) reads its 1 KB of it in one piece.
  const uint8_t* wsrc[W_DMA];
  int w_hstride;   // source bytes between consecutive half stages
  if (a.w_cpk != nullptr) {
    const uint8_t* tb = a.w_cpk + (int64_t)t.e * a.wcpk_estride +
                        ((int64_t)t.nt * (K / HK) + 2 * t.ks0) * CODE_BLOCK_BYTES;
#pragma unroll
    for (int i = 0; i < W_DMA; ++i) wsrc[i] = tb + (wave * W_DMA + i) * 1024 + lane * 16;
    w_hstride = CODE_BLOCK_BYTES;
  } else {
#pragma unroll
    for (int i = 0; i < W_DMA; ++i) {
      const int R = (wave * W_DMA + i) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ ((R >> 2) & 3);
      const uint8_t *base, *sbase;
      const int row = w_row(R, base, sbase);
      wsrc[i] = base + (int64_t)row * kb + kc0 + c * 16;
    }
    w_hstride = HROW;
  }
  const uint8_t* xsrc[X_DMA];
  int x_hstride;
  if (a.x_tiled) {
    // token codes already tile-major (the L1 epilogue wrote h so): one 16 KB
    // block per m-tile and half stage, read in 1 KB pieces as the weights
    const uint8_t* tb = a.x + ((int64_t)t.mt * (K / HK) + 2 * t.ks0) * CODE_BLOCK_BYTES;
#pragma unroll
    for (int i = 0; i < X_DMA; ++i) xsrc[i] = tb + (wave * X_DMA + i) * 1024 + lane * 16;
    x_hstride = CODE_BLOCK_BYTES;
  } else {
#pragma unroll
    for (int i = 0; i < X_DMA; ++i) {
      const int R = (wave * X_DMA + i) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ ((R >> 2) & 3);
      xsrc[i] = a.x + (int64_t)x_token(R) * kb + kc0 + c * 16;
    }
    x_hstride = HROW;
  }
  // Scale tiles (4 bytes per row per half stage): waves 0-3 copy the weight
  // rows' dwords (row 64*wave + lane), waves 4-7 the token rows' (row
  // 64*(wave-4) + lane), from the row-major scales (half stage h at byte 4h of
  // the row) or from a tile-major copy, where a 256-column stage of the tile is
  // 2 KB in one piece with 8 bytes per row (half stage h: piece h/2, dword h%2).
  const bool scale_w = wave < 4;
  const uint8_t* ssrc;
  int piece_stride;   // bytes between the pieces of consecutive 256-column stages
  {
    const int R = (wave & 3) * 64 + lane;
    if (scale_w) {
      if (a.w_spk != nullptr) {
        ssrc = a.w_spk + (int64_t)t.e * a.wspk_estride + ((int64_t)t.nt * nst_all + t.ks0) * SC_TILE_STAGE_BYTES +
               R * SC_STAGE_BYTES;
        piece_stride = SC_TILE_STAGE_BYTES;
      } else {
        const uint8_t *base, *sbase;
        const int row = w_row(R, base, sbase);
        ssrc = sbase + (int64_t)row * ks + t.ks0 * SC_STAGE_BYTES;
        piece_stride = SC_STAGE_BYTES;
      }
    } else if (a.x_s_packed) {
      // rows past the tile's end read the last valid row, as the code copies do
      ssrc = a.x_s + ((int64_t)t.mt * nst_all + t.ks0) * SC_TILE_STAGE_BYTES + min(R, t.rows - 1) * SC_STAGE_BYTES;
      piece_stride = SC_TILE_STAGE_BYTES;
    } else {
      ssrc = a.x_s + (int64_t)x_token(R) * ks + t.ks0 * SC_STAGE_BYTES;
      piece_stride = SC_STAGE_BYTES;
    }
  }
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t sc_lds = (scale_w ? OFF_WS : OFF_XS) + (wave & 3) * 256;
  // Copy c (0..4) of half stage h into slot h % NSLOT: W_DMA weight copies,
  // X_DMA token copies, then the scale dword.
  auto copy_one = [&](int h, int c) {
    const uint32_t sb = lds0 + (h % NSLOT) * SLOT_BYTES;
    if (c < W_DMA) {
      lds_dma16(wsrc[c] + (int64_t)h * w_hstride, sb + (wave * W_DMA + c) * 1024);
    } else if (c < W_DMA + X_DMA) {
      const int i = c - W_DMA;
      lds_dma16(xsrc[i] + (int64_t)h * x_hstride, sb + OFF_X + (wave * X_DMA + i) * 1024);
    } else {
      lds_dma4(ssrc + (h >> 1) * piece_stride + (h & 1) * HSC, sb + sc_lds);
    }
  };
  auto issue = [&](int h) {
#pragma unroll
    for (int c = 0; c < VM_PER_HALF; ++c) copy_one(h, c);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[f][g][v] = 0.0f;

  // per-lane LDS read offsets: row r32 (+32 per block) of the lane's weight and
  // token blocks; in step s lane half hh reads chunk 2*hh + s
  const int r32 = lane & 31, hh = lane >> 5;
  const int swz = (r32 >> 2) & 3;
  const int wrow_off = (wn * 128 + r32) * HROW;
  const int xrow_off = OFF_X + (wm * 64 + r32) * HROW;
  const int wsc_off = OFF_WS + (wn * 128 + r32) * HSC;
  const int xsc_off = OFF_XS + (wm * 64 + r32) * HSC;
  int coff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) coff[s] = ((hh * 2 + s) ^ swz) * 16;

  // this lane's scale dwords of half stage h, shifted so that the bytes of its
  // chunks 2*hh, 2*hh + 1 are bytes 0 and 1 (the MFMA's byte select is the step)
  auto read_scales = [&](int h, uint32_t (&sa)[4], uint32_t (&sx)[2]) {
    const uint8_t* rs = smem + (h % NSLOT) * SLOT_BYTES;
#pragma unroll
    for (int f = 0; f < 4; ++f) sa[f] = *(const uint32_t*)(rs + wsc_off + f * 32 * HSC) >> (16 * hh);
#pragma unroll
    for (int g = 0; g < 2; ++g) sx[g] = *(const uint32_t*)(rs + xsc_off + g * 32 * HSC) >> (16 * hh);
  };

  // Output rows and gate weights of the bf16 epilogue, loaded now so that their
  // latency hides behind the K loop (they complete before half stage 0's
  // copies, which the prologue waits for).
  TileRows<2> rows;
  if constexpr (EPI == EPI_BF16) rows = load_tile_rows<2>(a, t, wm, lane);

  // Prologue: half stages 0, 1, 2 in flight; wait for half stage 0.
  issue(0);
  if (nh > 2) {
    issue(1);
    issue(2);
    asm volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory");
  } else if (nh > 1) {
    issue(1);
    asm volatile("s_waitcnt vmcnt(5)\n\ts_barrier" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  }

  // Half stage h, in every wave: step 0's MFMAs (reading step 1's fragments),
  // then a wait for half stage h+1 (own copies: vmcnt; everyone's: the
  // barrier), then step 1's MFMAs (reading half stage h+1's first fragments).
  // Copies of half stage h+3 go to slot (h+3) % 4 = (h-1) % 4, whose last reads
  // (step 0 of h-1) precede the barrier of h-1: three of them before MFMAs 0, 3
  // and 6 of step 0, two before MFMAs 1 and 5 of step 1. At the barrier of h the
  // copies allowed in flight are those of h+2 and the three of h+3: vmcnt(8);
  // near the end, vmcnt(5) (no copies of h+3) and vmcnt(0).
  // WAIT is that count: 8 (with copies), 5 or 0 (without).
  if (act) {
    Frags F0, F1;
    uint32_t sa[4], sx[2];
    read_scales(0, sa, sx);
    // the order of the K loop's reads (A0 B0 B1 A1 A2 A3), so the loop entry
    // needs no longer wait than its back edge
    F0.A[0] = lds16(smem + wrow_off + coff[0]);
#pragma unroll
    for (int g = 0; g < 2; ++g) F0.B[g] = lds16(smem + xrow_off + g * 32 * HROW + coff[0]);
#pragma unroll
    for (int f = 1; f < 4; ++f) F0.A[f] = lds16(smem + wrow_off + f * 32 * HROW + coff[0]);

    auto half = [&](int h, auto wait_tag) {
      constexpr int WAIT = decltype(wait_tag)::value;
      const uint8_t* sb = smem + (h % NSLOT) * SLOT_BYTES;
      k_step<0, true>(F0, F1, sb, coff[1], wrow_off, xrow_off, sa, sx, acc, [&](int i) {
        if constexpr (WAIT == 8) {
          if (i == 0) copy_one(h + 3, 0);
          else if (i == 3) copy_one(h + 3, 1);
          else if (i == 6) copy_one(h + 3, 2);
        }
      });
      // keep all eight MFMAs of step 0 above the wait: moved below it (the
      // wait's asm does not order register-only instructions), they leave the
      // matrix core idle while the wave waits for its last fragment read
      // (measured: L1 0.786 -> 0.767 ms, L2 0.432 -> 0.425 ms)
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (WAIT == 8) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else if constexpr (WAIT == 5) asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const uint8_t* sbn = smem + ((h + 1) % NSLOT) * SLOT_BYTES;
      uint32_t san[4], sxn[2];
      read_scales(h + 1, san, sxn);
      k_step<1, true>(F1, F0, sbn, coff[0], wrow_off, xrow_off, sa, sx, acc, [&](int i) {
        if constexpr (WAIT == 8) {
          if (i == 1) copy_one(h + 3, 3);
          else if (i == 5) copy_one(h + 3, 4);
        }
      });
#pragma unroll
      for (int q = 0; q < 4; ++q) sa[q] = san[q];
      sx[0] = sxn[0];
      sx[1] = sxn[1];
    };
    // Separate loops rather than a branch per half stage: with a branch the
    // compiler hoists MFMAs that are identical on both sides above the barrier,
    // and the copies and reads after it no longer overlap any matrix work. In the
    // last half stage the reads of the "next" slot fetch bytes never used.
    int h = 0;
    for (; h + 3 < nh; ++h) half(h, std::integral_constant<int, 8>{});
    if (h + 2 < nh) half(h++, std::integral_constant<int, 5>{});
    for (; h < nh; ++h) half(h, std::integral_constant<int, 0>{});
  } else {
    // the same copies and barriers as `half`, without MFMAs (accumulators stay
    // zero): every wave meets the same barriers
    int h = 0;
    for (; h + 3 < nh; ++h) {
      copy_one(h + 3, 0);
      copy_one(h + 3, 1);
      copy_one(h + 3, 2);
      asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      copy_one(h + 3, 3);
      copy_one(h + 3, 4);
    }
    if (h + 2 < nh) {
      asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      ++h;
    }
    for (; h < nh; ++h) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
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
