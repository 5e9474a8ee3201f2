// Tile bookkeeping shared by the GEMM kernels (FP4 scaled MFMA and the bf16
// variant): the tile order of a launch and the bf16 output epilogue.
#pragma once

#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

struct Tile {
  int e;         // expert
  int nt;        // tile index along weight rows
  int row0;      // first row (sorted order) of the token tile
  int rows;      // valid rows in the token tile
  int mt;        // m-tile index within the launch (tile-major scale layouts)
  int sp;        // K split of a split-K launch (0 otherwise)
  int ks0, ks1;  // the split's K stages [ks0, ks1) of 256 columns
};

// Routed launches keep the expert offsets and m-tile bases (E+1 each) in LDS:
// the tile decode at the start of every tile then reads LDS instead of a chain
// of dependent global loads (a binary search and the offsets). Dense launches
// need neither.
struct TileTables {
  int tile_base[ROUTE_MAX_EXPERTS + 1];
  int expert_off[ROUTE_MAX_EXPERTS + 1];
};

// Fill the tables (all threads of the workgroup; ends with a barrier).
static __device__ __forceinline__ void load_tile_tables(const GemmArgs& a, TileTables& tt) {
  if (a.expert_off != nullptr) {
    for (int i = threadIdx.x; i <= a.n_experts; i += blockDim.x) {
      tt.tile_base[i] = a.tile_base[i];
      tt.expert_off[i] = a.expert_off[i];
    }
  }
  __syncthreads();
}

// Number of tiles of this launch (device-side for the routed experts).
static __device__ __forceinline__ int tile_count(const GemmArgs& a, const TileTables& tt) {
  if (a.expert_off == nullptr) return a.grid_tiles;
  return tt.tile_base[a.n_experts] * a.n_tiles;
}

// Tile L of the launch. Tiles are ordered (expert, n-tile, m-tile) with the
// m-tile fastest, so consecutive tiles share their weight rows.
static __device__ __forceinline__ Tile decode_tile(const GemmArgs& a, const TileTables& tt, int L) {
  Tile t;
  const int nst = (a.k + BK - 1) / BK;
  t.sp = 0;
  t.ks0 = 0;
  t.ks1 = nst;
  if (a.expert_off == nullptr) {
    const int mtiles = (a.m_rows + BM - 1) / BM;
    if (a.k_splits > 1) {
      // split-K: tile L + sp * (tiles of one split) covers stages
      // [sp * nst / S, (sp + 1) * nst / S)
      const int per_split = a.grid_tiles / a.k_splits;
      t.sp = L / per_split;
      L -= t.sp * per_split;
      t.ks0 = t.sp * nst / a.k_splits;
      t.ks1 = (t.sp + 1) * nst / a.k_splits;
    }
    t.e = 0;
    t.nt = L / mtiles;
    const int mt = L - t.nt * mtiles;
    t.row0 = mt * BM;
    t.rows = min(BM, a.m_rows - t.row0);
    t.mt = mt;
    return t;
  }
  // expert e with tile_base[e] * n_tiles <= L < tile_base[e + 1] * n_tiles
  int lo = 0, hi = a.n_experts - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tt.tile_base[mid] * a.n_tiles <= L) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int tb = tt.tile_base[e];
  const int nte = tt.tile_base[e + 1] - tb;
  const int r = L - tb * a.n_tiles;
  t.e = e;
  t.nt = r / nte;
  const int mt = r - t.nt * nte;
  const int off = tt.expert_off[e];
  t.row0 = off + mt * BM;
  t.rows = min(BM, tt.expert_off[e + 1] - t.row0);
  t.mt = tb + mt;
  return t;
}

// bf16 output of a 256 x 256 tile whose waves each hold 128 weight rows x
// NG*32 token rows as 4 x NG 32x32 MFMA blocks: acc[f][g][v] is D[n][m] with
// n = nt*BN + wn*128 + f*32 + 8*(v/4) + 4*(lane/32) + v%4 and
// m = wm*NG*32 + g*32 + lane%32 within the token tile. Dense: y[m][n] =
// bf16(scale * D). Routed: o[row_slot[m]][n] = bf16(scale * D * row_weight[m]).
//
// The tile goes through LDS: the waves put their bf16 values into a row-major
// [256 token rows][256 columns] tile in `smem` (row stride TILE_LDS_STRIDE: the
// 16 bytes of padding spread the 32 rows a wave writes at once over the banks),
// then every thread copies 16-byte chunks, so each output row leaves as one
// contiguous 512-byte run. The per-row output slots and gate weights are loaded
// by the caller at the start of the tile (TileRows), so no load latency is
// exposed here. `smem` must hold TILE_LDS_TOTAL bytes; this function begins
// with a barrier (the K loop's last LDS reads) and the caller must place a
// barrier before the next use of `smem`.
constexpr int TILE_LDS_STRIDE = 256 * 2 + 16;
constexpr int TILE_LDS_BYTES = 256 * TILE_LDS_STRIDE;
constexpr int TILE_LDS_TOTAL = TILE_LDS_BYTES + 256 * 4;   // + the output row of each token row

// Per-thread rows of a tile's bf16 epilogue: the gate weights of this lane's NG
// token rows, and (threads < 256) the output row of token row threadIdx.x.
template <int NG>
struct TileRows {
  float w[NG];
  int out_row;
};

template <int NG>
static __device__ __forceinline__ TileRows<NG> load_tile_rows(const GemmArgs& a, const Tile& t, int wm, int lane) {
  TileRows<NG> r;
  const int r32 = lane & 31;
#pragma unroll
  for (int g = 0; g < NG; ++g) r.w[g] = 1.0f;
  r.out_row = t.row0 + min((int)threadIdx.x, t.rows - 1);
  if (a.row_slot != nullptr) {
#pragma unroll
    for (int g = 0; g < NG; ++g) r.w[g] = a.row_weight[t.row0 + min(wm * NG * 32 + g * 32 + r32, t.rows - 1)];
    if (threadIdx.x < 256) r.out_row = a.row_slot[r.out_row];
  }
  return r;
}

template <int NG>
static __device__ __forceinline__ void store_tile_bf16_lds(const GemmArgs& a, const Tile& t,
                                                           const f32x16 (&acc)[4][NG], const TileRows<NG>& rows,
                                                           int wn, int wm, int lane, float scale, uint8_t* smem,
                                                           int nthreads) {
  const int r32 = lane & 31, hh = lane >> 5;
  int* out_rows = (int*)(smem + TILE_LDS_BYTES);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (threadIdx.x < 256) out_rows[threadIdx.x] = rows.out_row;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int ml = wm * NG * 32 + g * 32 + r32;
    const float wgt = scale * rows.w[g];
    uint8_t* trow = smem + ml * TILE_LDS_STRIDE;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wn * 128 + f * 32 + 8 * q + 4 * hh;
        const uint32_t p0 = bf16x2_rne(acc[f][g][4 * q] * wgt, acc[f][g][4 * q + 1] * wgt);
        const uint32_t p1 = bf16x2_rne(acc[f][g][4 * q + 2] * wgt, acc[f][g][4 * q + 3] * wgt);
        *(uint2*)(trow + nl * 2) = make_uint2(p0, p1);
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // 256 rows x 32 chunks of 16 bytes
  const int c = threadIdx.x & 31;
  const int n = t.nt * BN + c * 8;
  if (n < a.n_rows) {
#pragma unroll 4
    for (int r = threadIdx.x >> 5; r < t.rows; r += nthreads / 32)
      *(uint4*)(a.out_bf16 + (int64_t)out_rows[r] * a.n_rows + n) = *(const uint4*)(smem + r * TILE_LDS_STRIDE + c * 16);
  }
}

// One 32 x 32 block of the L1 epilogue, as this lane holds it: gate `ga` and up
// `ua` are D[n][m] of token row ml within the tile and j = j0 + 8*(v/4) + 4*hh + v%4.
// h = bf16(silu(g) * u) is re-quantised per 32 j (MXFP4: one E8M0 byte; NVFP4:
// two E4M3 bytes per 16 j and the fp32 global scale) and stored with the codes.
// With ROUND_GU (the GEMMs whose gate and up outputs are defined as bf16, e.g.
// NVFP4 weights) g = bf16(ga * sg) and u = bf16(ua * su) first, as two bf16
// linears followed by the elementwise SiLU * up would give them.
// Returns (MXFP4) the max |h| of the block row as bf16 bits, 0 for padding rows.
template <int EPI, bool ROUND_GU = false>
static __device__ __forceinline__ uint32_t l1_block(const GemmArgs& a, const Tile& t, const f32x16& ga,
                                                    const f32x16& ua, int j0, int ml, int hh, float sg = 1.0f,
                                                    float su = 1.0f) {
  const int I = a.n_rows;
  const bool valid = (ml < t.rows) && (j0 < I);
  const int row = t.row0 + ml;
  // h as bf16 pairs: hp[2q] = (v = 4q, 4q+1), hp[2q+1] = (4q+2, 4q+3)
  uint32_t hp[8];
#pragma unroll
  for (int v = 0; v < 16; v += 2) {
    if constexpr (ROUND_GU) {
      const uint32_t gp = bf16x2_rne(ga[v] * sg, ga[v + 1] * sg), up = bf16x2_rne(ua[v] * su, ua[v + 1] * su);
      hp[v >> 1] = bf16x2_rne(silu_mul(bf16_to_f32(gp & 0xFFFFu), bf16_to_f32(up & 0xFFFFu)),
                              silu_mul(bf16_to_f32(gp >> 16), bf16_to_f32(up >> 16)));
    } else {
      hp[v >> 1] = bf16x2_rne(silu_mul(ga[v], ua[v]), silu_mul(ga[v + 1], ua[v + 1]));
    }
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
                                   ml * SC_STAGE_BYTES + ((j0 >> 5) & 7)
                             : (int64_t)row * (I >> 5) + (j0 >> 5);
      a.h_scales[at] = (uint8_t)sbyte;
    }
  } else {
    // NVFP4: 16-blocks j0..j0+15 (v = 0..7) and j0+16..j0+31 (v = 8..15).
    const float gsc = a.nv_gptr != nullptr ? *a.nv_gptr : a.h_nv_global;
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
    // row-major [rows][I/2], or tile-major for the L2's copies (h_codes_tiled):
    // block (m-tile t.mt, half stage j0/128 of the L2's K) of 16 KB, tile row ml
    // at ml*64, this 16-byte chunk (32 j) at ((j0/32) % 4) ^ ((ml >> 2) & 3)
    const int64_t at = a.h_codes_tiled
                           ? ((int64_t)t.mt * (I >> 7) + (j0 >> 7)) * CODE_BLOCK_BYTES + ml * 64 +
                                 ((((j0 >> 5) & 3) ^ ((ml >> 2) & 3)) << 4)
                           : (int64_t)row * (I >> 1) + (j0 >> 1);
    *(uint2*)(a.h_codes + at + hh * 8) = make_uint2(o0, o1);
  }
  return block_amax;
}

// NVFP4 warm-up: fold this wave's max |h| into *amax (one atomic per wave).
static __device__ __forceinline__ void wave_amax_atomic(uint32_t* amax, uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  if ((threadIdx.x & 63) == 0) atomicMax(amax, v);
}

}  // namespace mx
