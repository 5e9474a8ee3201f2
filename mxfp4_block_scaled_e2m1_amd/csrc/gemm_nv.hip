// GEMMs with NVFP4 operands, on bf16 or fp16 matrix cores: the L2 down GEMM of
// the NVFP4 re-quantisation variant (bf16) and the GEMMs of NVFP4 weights (fp16).
//
// The intermediate h arrives as NVFP4: E2M1 codes, one E4M3 scale per 16
// columns and an fp32 global scale g (page "Current Bug: vLLM produces
// empty/garbage output", section "Revised Plan", Phase 1 names the warm-up
// based global scale of the runner; the pages do not spell the format out, so
// the block of 16 with an E4M3 scale is the plain reading of the name). The
// weights stay MXFP4 (page "2026-05-08 DeepSeek V4 Pro NVFP4 Quantization",
// section "FP4 (E2M1) expert weight format confirmed").
//
// The scaled FP4 MFMA of gfx950 takes one E8M0 (power of two) scale per 32 K
// values, which cannot carry an E4M3 scale per 16. Both operands are therefore
// dequantised exactly into a 16-bit type:
//  * MXFP4 w: code * 2^(e-127) has at most 2 significant bits; exact in bf16
//    for scale bytes up to 252 (above that, 6 * 2^126 exceeds the bf16 range),
//    and far outside the fp16 range, so MXFP4 weights take bf16.
//  * NVFP4 (h, or NVFP4 w): code * s with s an E4M3 value: at most 2 + 4
//    significant bits in [2^-10, 2688] (or 0), exact in bf16 and in fp16.
// With NVFP4 weights both operands are fp16 (a cheaper conversion, below). The
// product sum runs in fp32 (V_MFMA_F32_32X32X16_BF16 / _F16) and the epilogue
// multiplies by g (and, for routed experts, by the gate weight), so
// y = g * sum_k (code_h * s_h)(code_w * scale_w) up to fp32 summation order.
//
// Design: persistent 512-thread workgroups on 256 x 256 tiles, the same tile
// order and XCD mapping as the FP4 kernel. Per 64-wide K stage each thread
// loads 16 code bytes of one weight row and 16 of one token row (plus their
// scale bytes) into registers two stages ahead, and in the current stage
// converts the next stage's bytes (before or after its MFMAs, by wave) and
// writes the 16-bit tile into the other of two 64 KB LDS slots. Every operand
// element is converted once per workgroup.
#include "gemm_common.h"
#include "nv_linear.h"

namespace mx {

namespace {

constexpr int NV_BK = 64;                   // logical K per stage
constexpr int NV_ROW = NV_BK * 2;           // 128 bytes of bf16 per row per stage
constexpr int NV_OPND = BN * NV_ROW;        // 32 KB per operand tile
constexpr int NV_SLOT = 2 * NV_OPND;        // weight tile + token tile
static_assert(BN == 256 && BM == 256, "the copy assignment below assumes 256-row tiles");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// LDS byte offset of 16-byte chunk c (0..7) of row r of an operand tile: chunk
// c sits at slot c ^ s(r), s(r) = 2 * ((r / 2) % 4) + (r / 8) % 2. Measured on
// gfx950: a 16-byte read is served 16 lanes at a time over 256 bytes of banks,
// a 16-byte write 8 consecutive lanes at a time over 128 bytes (the slot,
// address bits 4..6). The fragment reads (lane l: row l % 32, chunk 2k + l / 32)
// hit 16 distinct 16-byte bank groups per cycle, for either grouping of the
// read lanes; the stores below give each 8 lanes 8 distinct slots. With the
// former layout ((r / 2) % 8, no reordering of the stores) the writes were 2-way
// conflicted: 29 % of the LDS cycles.
__device__ __forceinline__ int nv_swz(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int nv_off(int r, int c) { return r * NV_ROW + ((c ^ nv_swz(r)) << 4); }

// One thread's raw bytes of a stage: 32 logical columns of a weight row and of
// a token row.
struct NvRaw {
  uint4 wc;         // 16 weight code bytes
  uint32_t we;      // their E8M0 scale byte (MXFP4 weights) or two E4M3 bytes (NVFP4 weights)
  uint4 hc;         // 16 NVFP4 code bytes
  uint32_t hs;      // their two E4M3 scale bytes (16 columns each)
};

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return bf16x2_rne(lo, hi);
}

// MXFP4 -> bf16 for one dword of codes (8 columns): code * 2^(e-127), exact.
__device__ __forceinline__ uint4 w_to_bf16(uint32_t d, uint32_t e) {
  if (e == 0xFFu) return make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);   // NaN scale
  const float sc = e8m0_to_f32(e);
  return make_uint4(dequant_pair<0>(d, sc), dequant_pair<1>(d, sc), dequant_pair<2>(d, sc),
                    dequant_pair<3>(d, sc));
}

// NVFP4 codes -> bf16 for one dword (8 columns) with block scale s: code * s,
// exact in fp32 and in bf16 (at most 6 significant bits).
__device__ __forceinline__ uint4 h_to_bf16(uint32_t d, float s) {
  uint32_t r[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f32x2 v;
    if (b == 0) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
    else if (b == 1) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
    else if (b == 2) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
    else v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
    r[b] = bf16_pair(v[0] * s, v[1] * s);
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// NVFP4 codes -> fp16 for one dword (8 columns) with block scale s (an E4M3
// value, exact in fp16): unit-scale conversion, then one packed fp16 multiply
// per pair. code * s has at most 6 significant bits and lies in [2^-10, 2688]
// (or is 0), so it is exact and normal in fp16. The scaled conversion
// instruction applies only the power of two of its scale operand (measured on
// gfx950 over all codes and E4M3 scales), so s cannot go into it.
__device__ __forceinline__ uint4 nv_to_f16(uint32_t d, _Float16 s) {
  const f16x2 sc = {s, s};
  f16x2 v[4];
  v[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * sc;
  v[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * sc;
  v[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * sc;
  v[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * sc;
  return make_uint4(__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                    __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3]));
}

__device__ __forceinline__ f16x8 as_f16x8(const uint4& v) { return __builtin_bit_cast(f16x8, v); }

// One MFMA of a K step: fp16 operands when both are NVFP4 (NVW), bf16 when the
// weights are MXFP4 (their E8M0 scales reach far outside the fp16 range).
template <bool NVW>
__device__ __forceinline__ f32x16 nv_mfma(const uint4& a, const uint4& b, const f32x16& c) {
  if constexpr (NVW) return __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(a), as_f16x8(b), c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// One 256 x 256 tile of o = g * h . w^T (h NVFP4; w MXFP4, or NVFP4 when NVW,
// whose E4M3 scales [rows, k/16] are in wa_s and whose global scale is folded
// into g by the caller).
// SWIGLU (NVFP4 weights): the fused gate/up L1. The weight tile holds gate rows
// (wa, wa_s) and up rows (wb, wb_s) of 128 intermediate columns j, in the row
// order of the FP4 L1 tile, so a wave's gate block acc[f][g] and up block
// acc[f + 2][g] cover the same j; the epilogue forms g = bf16(gate * sg),
// u = bf16(up * su), h = bf16(silu(g) * u) and re-quantises h to NVFP4 with the
// fp32 global h_nv_global (codes and E4M3 scales row-major, as k_quant_nvfp4
// writes them): the two bf16 GEMMs, the SiLU * up and the quantiser in one pass.
template <bool NVW, bool SWIGLU>
__device__ __forceinline__ void nv_tile(const GemmArgs& a, const Tile& t, uint8_t* smem) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;   // token blocks of a partly filled tile spread over the SIMDs
  const bool act = wm * 64 < t.rows;         // else this wave's token rows are all padding: no MFMAs
  const int K = a.k;
  const int kb = K >> 1, kse = K >> 5, ksn = K >> 4;   // code bytes, E8M0 and E4M3 bytes per row
  const int nst = K / NV_BK;

  // copy assignment: row R = tid / 2 of both tiles, columns (tid & 1) * 32 .. +31
  const int R = tid >> 1, half = tid & 1;
  const uint8_t* wmat = a.wa;
  const uint8_t* wsmat = a.wa_s;
  int wrow;
  if constexpr (SWIGLU) {
    const int f = (R >> 5) & 3;   // tile rows of blocks f = 0, 1: gate; f = 2, 3: up (same j)
    wrow = t.nt * L1_J_PER_TILE + (R >> 7) * 64 + (f & 1) * 32 + (R & 31);
    if (f >= 2) {
      wmat = a.wb;
      wsmat = a.wb_s;
    }
  } else {
    wrow = t.nt * BN + R;
  }
  wrow = min(wrow, a.n_rows - 1);
  const uint8_t* wsrc = wmat + (int64_t)t.e * a.w_estride + (int64_t)wrow * kb + half * 16;
  const uint8_t* wesrc = NVW ? wsmat + (int64_t)t.e * a.ws_estride + (int64_t)wrow * ksn + half * 2
                             : wsmat + (int64_t)t.e * a.ws_estride + (int64_t)wrow * kse + half;
  const int hrow = t.row0 + min(R, t.rows - 1);
  const uint8_t* hsrc = a.x + (int64_t)hrow * kb + half * 16;
  const uint8_t* hssrc = a.x_s + (int64_t)hrow * ksn + half * 2;

  auto load = [&](int st, NvRaw& r) {
    r.wc = *(const uint4*)(wsrc + st * (NV_BK / 2));
    if constexpr (NVW) r.we = *(const uint16_t*)(wesrc + st * (NV_BK / 16));
    else r.we = wesrc[st * (NV_BK / 32)];
    r.hc = *(const uint4*)(hsrc + st * (NV_BK / 2));
    r.hs = *(const uint16_t*)(hssrc + st * (NV_BK / 16));
  };
  auto store = [&](int slot, const NvRaw& r) {
    uint8_t* wt = smem + slot * NV_SLOT;
    uint8_t* ht = wt + NV_OPND;
    const uint32_t wd[4] = {r.wc.x, r.wc.y, r.wc.z, r.wc.w};
    const uint32_t hd[4] = {r.hc.x, r.hc.y, r.hc.z, r.hc.w};
    const float s0 = e4m3_to_f32(r.hs & 0xFFu), s1 = e4m3_to_f32(r.hs >> 8);
    _Float16 w0 = 0, w1 = 0, t0 = 0, t1 = 0;
    if constexpr (NVW) {
      w0 = (_Float16)e4m3_to_f32(r.we & 0xFFu);
      w1 = (_Float16)e4m3_to_f32(r.we >> 8);
      t0 = (_Float16)s0;
      t1 = (_Float16)s1;
    }
    // store i writes chunk half*4 + (i ^ swap): odd rows swap the chunks of each
    // pair (a pair shares its E4M3 scale), so the 8 lanes of rows 4q .. 4q+3
    // that one write cycle serves hit 8 distinct slots
    const bool swap = R & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = half * 4 + (i ^ (swap ? 1 : 0));
      const uint32_t wdi = swap ? wd[i ^ 1] : wd[i];
      const uint32_t hdi = swap ? hd[i ^ 1] : hd[i];
      if constexpr (NVW) {
        *(uint4*)(wt + nv_off(R, c)) = nv_to_f16(wdi, i < 2 ? w0 : w1);
        *(uint4*)(ht + nv_off(R, c)) = nv_to_f16(hdi, i < 2 ? t0 : t1);
      } else {
        *(uint4*)(wt + nv_off(R, c)) = w_to_bf16(wdi, r.we);
        *(uint4*)(ht + nv_off(R, c)) = h_to_bf16(hdi, i < 2 ? s0 : s1);
      }
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[f][g][v] = 0.0f;

  const int r32 = lane & 31, hh = lane >> 5;
  TileRows<2> rows;   // for the bf16 epilogue, loaded early
  if constexpr (!SWIGLU) rows = load_tile_rows<2>(a, t, wm, lane);
  // raw bytes of two stages in flight: stage st+2 is loaded while stage st is
  // multiplied and stage st+1 converted, so the loads have two stages of MFMAs
  // to arrive in. `cur` held stage st (already in LDS), `nxt` holds stage st+1.
  // The load is unconditional (the last two stages re-read stage nst-1): with a
  // branch around it, the compiler's wait before the conversion was vmcnt(0),
  // a wait for the loads of stage st+2 just issued.
  // One stage's 32 MFMAs per wave (4 K steps of 16). The fragments of step
  // k16+1 are read between the MFMAs of step k16: token fragment g after MFMA
  // 2g, weight fragment f after MFMA 2f+1, the last one that reads the register
  // it replaces (so the weight fragments need one register set, the token
  // fragments two). Every read then has at least five MFMAs of this wave before
  // its first use; only the first step of a stage waits for its reads.
  auto mfmas = [&](int st) {
    const uint8_t* wt = smem + (st & 1) * NV_SLOT;
    const uint8_t* ht = wt + NV_OPND;
    // rows wn*128 + f*32 + r32 and wm*64 + g*32 + r32 all have the swizzle of
    // r32 (it depends on row bits 1..3 only): a fragment's address is a lane
    // base, an immediate row offset and the swizzled chunk of the step
    const int swz = nv_swz(r32);
    const uint8_t* wb = wt + (wn * 128 + r32) * NV_ROW;
    const uint8_t* hb = ht + (wm * 64 + r32) * NV_ROW;
    uint4 A[4], B[2][2];
#pragma unroll
    for (int f = 0; f < 4; ++f) A[f] = *(const uint4*)(wb + f * 32 * NV_ROW + ((hh ^ swz) << 4));
#pragma unroll
    for (int g = 0; g < 2; ++g) B[0][g] = *(const uint4*)(hb + g * 32 * NV_ROW + ((hh ^ swz) << 4));
#pragma unroll
    for (int k16 = 0; k16 < NV_BK / 16; ++k16) {
      const int p = k16 & 1, q = p ^ 1;
      // chunk of step k16+1: lane half hh holds K values 8*hh .. 8*hh+7 of a step
      const int co = (((k16 + 1) * 2 + hh) ^ swz) << 4;
      const bool more = k16 + 1 < NV_BK / 16;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int f = i >> 1, g = i & 1;
        acc[f][g] = nv_mfma<NVW>(A[f], B[p][g], acc[f][g]);
        if (more) {
          if (i == 0) B[q][0] = *(const uint4*)(hb + co);
          else if (i == 2) B[q][1] = *(const uint4*)(hb + 32 * NV_ROW + co);
          if (g == 1) A[f] = *(const uint4*)(wb + f * 32 * NV_ROW + co);
        }
      }
      if (more) {
        // MFMA 0, B0, MFMA 1, A0, MFMA 2, B1, MFMA 3, A1, MFMA 4, MFMA 5, A2, MFMA 6, MFMA 7, A3
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };
  // Waves w and w + 4 share a SIMD. In every stage waves 0-3 run their MFMAs
  // before converting the next stage and waves 4-7 after it, so that on each
  // SIMD one wave's conversion (VALU work) overlaps the other wave's MFMAs,
  // instead of all eight waves converting while the matrix cores idle. The
  // conversion writes the other slot (its last reads were before the previous
  // barrier) and the MFMAs read this stage's slot, so the order is free.
  const bool conv_first = wave >= 4;
  auto stage = [&](int st, NvRaw& cur, NvRaw& nxt) {
    load(min(st + 2, nst - 1), cur);   // unconditional: see below
    const bool conv = st + 1 < nst;
    if (conv_first && conv) store((st + 1) & 1, nxt);
    if (act) mfmas(st);
    if (!conv_first && conv) store((st + 1) & 1, nxt);
    __syncthreads();
  };
  NvRaw ra, rb;
  load(0, ra);
  if (nst > 1) load(1, rb);
  store(0, ra);
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    stage(st, ra, rb);
    if (st + 1 < nst) stage(st + 1, rb, ra);
  }
  if constexpr (SWIGLU) {
    const float sg = a.e_global != nullptr ? a.nv_global * a.e_global[t.e] : a.nv_global;
    const float su = a.e_global2 != nullptr ? a.nv_global2 * a.e_global2[t.e] : a.nv_global2;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int j0 = t.nt * L1_J_PER_TILE + wn * 64 + f * 32;   // 32-aligned block of j
#pragma unroll
      for (int g = 0; g < 2; ++g)
        l1_block<EPI_SWIGLU_NVFP4, true>(a, t, acc[f][g], acc[f + 2][g], j0, wm * 64 + g * 32 + r32, hh, sg, su);
    }
  } else {
    const float g = a.nv_gptr != nullptr ? *a.nv_gptr : a.nv_global;
    const float scale = a.e_global != nullptr ? g * a.e_global[t.e] : g;
    store_tile_bf16_lds<2>(a, t, acc, rows, wn, wm, lane, scale, smem, GEMM_THREADS);
  }
}

// Persistent kernel with the tile order and XCD mapping of the FP4 GEMM.
template <bool NVW, bool SWIGLU>
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_gemm_nv(const GemmArgs a) {
  // the two K-stage slots, or the bf16 output tile of the epilogue
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * NV_SLOT > TILE_LDS_TOTAL ? 2 * NV_SLOT : TILE_LDS_TOTAL];
  __shared__ TileTables tt;
  load_tile_tables(a, tt);
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3, per_xcd_wgs = gridDim.x >> 3;
  const int total = tile_count(a, tt);
  const int per = (total + 7) >> 3;
  const int end = min((xcd + 1) * per, total);
  for (int L = xcd * per + local; L < end; L += per_xcd_wgs) {
    nv_tile<NVW, SWIGLU>(a, decode_tile(a, tt, L), smem);
    __syncthreads();   // the next tile's first stores overwrite slot 0
  }
}

}  // namespace

hipError_t launch_gemm_nv_l2(const GemmArgs& a, int max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const int cus = cu_count();
  const int grid = ((max_tiles < cus ? max_tiles : cus) + 7) & ~7;
  k_gemm_nv<false, false><<<grid, GEMM_THREADS, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_nv_w(const GemmArgs& a, int max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const int cus = cu_count();
  const int grid = ((max_tiles < cus ? max_tiles : cus) + 7) & ~7;
  k_gemm_nv<true, false><<<grid, GEMM_THREADS, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_nv_w_swiglu(const GemmArgs& a, int max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const int cus = cu_count();
  const int grid = ((max_tiles < cus ? max_tiles : cus) + 7) & ~7;
  k_gemm_nv<true, true><<<grid, GEMM_THREADS, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mx
