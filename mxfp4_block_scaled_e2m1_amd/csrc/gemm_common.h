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

}  // namespace mx
