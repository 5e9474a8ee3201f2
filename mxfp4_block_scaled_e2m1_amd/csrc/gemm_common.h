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
};

// Number of tiles of this launch (device-side for the routed experts).
static __device__ __forceinline__ int tile_count(const GemmArgs& a) {
  if (a.expert_off == nullptr) return a.grid_tiles;
  return a.tile_base[a.n_experts] * a.n_tiles;
}

// Tile L of the launch. Tiles are ordered (expert, n-tile, m-tile) with the
// m-tile fastest, so consecutive tiles share their weight rows.
static __device__ __forceinline__ Tile decode_tile(const GemmArgs& a, int L) {
  Tile t;
  if (a.expert_off == nullptr) {
    const int mtiles = (a.m_rows + BM - 1) / BM;
    t.e = 0;
    t.nt = L / mtiles;
    const int mt = L - t.nt * mtiles;
    t.row0 = mt * BM;
    t.rows = min(BM, a.m_rows - t.row0);
    return t;
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
  return t;
}

// bf16 output of a 256 x 256 tile held as 8 waves x (4 x 2) 32x32 MFMA blocks:
// acc[f][g][v] is D[n][m] with n = nt*BN + wn*128 + f*32 + 8*(v/4) + 4*(lane/32) + v%4
// and m = wm*64 + g*32 + lane%32 within the token tile. Dense: y[m][n] =
// bf16(scale * D). Routed: o[slot(m)][n] = bf16(scale * D * gate_weight[slot]).
static __device__ __forceinline__ void store_tile_bf16(const GemmArgs& a, const Tile& t, const f32x16 (&acc)[4][2],
                                                       int wn, int wm, int lane, float scale) {
  const int r32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int ml = wm * 64 + g * 32 + r32;
    if (ml >= t.rows) continue;
    const int row = t.row0 + ml;
    int64_t out_row = row;
    float wgt = scale;
    if (a.row_slot != nullptr) {
      const int slot = a.row_slot[row];
      out_row = slot;
      wgt = scale * a.slot_weight[slot];
    }
    uint16_t* dst = a.out_bf16 + out_row * a.n_rows;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = t.nt * BN + wn * 128 + f * 32 + 8 * q + 4 * hh;
        if (n < a.n_rows) {
          uint32_t p0 = f32_to_bf16_rne(acc[f][g][4 * q] * wgt) | (f32_to_bf16_rne(acc[f][g][4 * q + 1] * wgt) << 16);
          uint32_t p1 =
              f32_to_bf16_rne(acc[f][g][4 * q + 2] * wgt) | (f32_to_bf16_rne(acc[f][g][4 * q + 3] * wgt) << 16);
          *(uint2*)(dst + n) = make_uint2(p0, p1);
        }
      }
  }
}

}  // namespace mx
