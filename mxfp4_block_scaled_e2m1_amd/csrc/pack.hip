// Tile-major copies of E8M0 scale matrices and FP4 weight codes for the FP4 GEMM.
//
// The GEMM copies, per 256-wide K stage, 8 scale bytes of each of the 256
// weight rows and 256 token rows of its tile into LDS. In the row-major layout
// of the format (one E8M0 byte per row per 32 columns, page "2026-05-08
// DeepSeek V4 Pro NVFP4 Quantization", section "Script update") those are 512
// separate 8-byte pieces per stage, each a memory request of its own. The
// tile-major layout stores the 2 KB a stage needs for one tile contiguously:
//
//   packed[tile][stage][r][8]: bytes 8*stage .. 8*stage+7 of row(tile, r)
//
// with zero bytes past the end of a row (K % 256 == 128). The weight codes have
// a tile-major copy too (k_pack_weight_codes): per tile and 128-wide half stage,
// the 16 KB the GEMM's LDS slot holds, in that slot's byte order, so that each
// 16-byte copy lane reads consecutive bytes and a wave's copy is 1 KB in one
// piece (whole cache lines). The weight layouts are
// built once after the weights are loaded (the pages' runner prepares its
// weights once at start-up: page "Current Bug: vLLM produces empty/garbage
// output", section "Revised Plan", Phase 1); the activation layout is built
// per call from the quantiser's output.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

namespace {

// Bytes 8*st .. 8*st+7 of a scale row of ks bytes (ks % 4 == 0), zero past ks.
__device__ __forceinline__ uint2 stage_bytes(const uint8_t* __restrict__ row, int ks, int st) {
  const int b = st * SC_STAGE_BYTES;
  const uint32_t lo = b < ks ? *(const uint32_t*)(row + b) : 0u;
  const uint32_t hi = b + 4 < ks ? *(const uint32_t*)(row + b + 4) : 0u;
  return make_uint2(lo, hi);
}

// Weight scales: block (tile, stage), expert blockIdx.y; thread r = tile row.
// L1 tiles interleave gate rows (a_s) and up rows (b_s): tile row r holds
// matrix (r / 32) % 4 < 2 ? gate : up, row nt*128 + (r / 128)*64 + ((r / 32) % 2)*32 + r % 32,
// the row order of the GEMM's L1 weight tile. Rows past n_rows repeat the last row.
__global__ __launch_bounds__(256) void k_pack_weight_scales(const uint8_t* __restrict__ a_s,
                                                            const uint8_t* __restrict__ b_s, int l1, int n_rows,
                                                            int ks, int ntiles, int nst, int64_t src_estride,
                                                            uint8_t* __restrict__ out) {
  const int nt = blockIdx.x / nst, st = blockIdx.x - nt * nst, e = blockIdx.y, r = threadIdx.x;
  const uint8_t* src;
  int row;
  if (l1) {
    const int f = (r >> 5) & 3;
    row = nt * L1_J_PER_TILE + (r >> 7) * 64 + (f & 1) * 32 + (r & 31);
    src = f < 2 ? a_s : b_s;
  } else {
    row = nt * BN + r;
    src = a_s;
  }
  row = min(row, n_rows - 1);
  const uint2 v = stage_bytes(src + (int64_t)e * src_estride + (int64_t)row * ks, ks, st);
  *(uint2*)(out + (((int64_t)e * ntiles + nt) * nst + st) * SC_TILE_STAGE_BYTES + r * SC_STAGE_BYTES) = v;
}

// Activation scales of the token tiles of a launch: block (m-tile, group of
// ACT_STAGES stages), thread r = tile row. Routed: m-tile mt of expert e
// (tile_base[e] <= mt < tile_base[e+1]) covers sorted rows expert_off[e] +
// 256*(mt - tile_base[e]) + r, whose token is row_token[row]. Dense: rows
// 256*mt + r. Rows past the tile's end are not written (the GEMM reads the last
// valid row for them). The tile bases go through LDS so that the search for
// the expert costs one round trip to memory instead of one per step.
constexpr int ACT_STAGES = 4;
static_assert(ACT_STAGES == 4, "the 16-byte load path below fills four stages");
__global__ __launch_bounds__(256) void k_pack_act_scales(const uint8_t* __restrict__ x_s, int ks, int nst,
                                                         const int32_t* __restrict__ row_token,
                                                         const int32_t* __restrict__ expert_off,
                                                         const int32_t* __restrict__ tile_base, int n_experts,
                                                         int m_rows, uint8_t* __restrict__ out) {
  __shared__ int tb[ROUTE_MAX_EXPERTS + 1];
  const int mt = blockIdx.x, st0 = blockIdx.y * ACT_STAGES, r = threadIdx.x;
  int row0, rows;
  if (expert_off != nullptr) {
    for (int i = r; i <= n_experts; i += 256) tb[i] = tile_base[i];
    __syncthreads();
    if (mt >= tb[n_experts]) return;
    int lo = 0, hi = n_experts - 1;   // expert e with tb[e] <= mt < tb[e + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tb[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    row0 = expert_off[lo] + (mt - tb[lo]) * BM;
    rows = expert_off[lo + 1] - row0;
  } else {
    row0 = mt * BM;
    rows = m_rows - row0;
  }
  if (r >= rows) return;
  const int64_t src_row = row_token != nullptr ? row_token[row0 + r] : row0 + r;
  const uint8_t* src = x_s + src_row * ks;
  uint2 v[ACT_STAGES];
  if (ks % (ACT_STAGES * SC_STAGE_BYTES) == 0) {
    // whole 32-byte groups (K % 1024 == 0, the model's shapes): two 16-byte loads
    const uint4 a = *(const uint4*)(src + st0 * SC_STAGE_BYTES);
    const uint4 b = *(const uint4*)(src + st0 * SC_STAGE_BYTES + 16);
    v[0] = make_uint2(a.x, a.y); v[1] = make_uint2(a.z, a.w);
    v[2] = make_uint2(b.x, b.y); v[3] = make_uint2(b.z, b.w);
  } else {
#pragma unroll
    for (int i = 0; i < ACT_STAGES; ++i) v[i] = stage_bytes(src, ks, min(st0 + i, nst - 1));
  }
#pragma unroll
  for (int i = 0; i < ACT_STAGES; ++i)
    if (st0 + i < nst)
      *(uint2*)(out + ((int64_t)mt * nst + st0 + i) * SC_TILE_STAGE_BYTES + r * SC_STAGE_BYTES) = v[i];
}

}  // namespace

hipError_t launch_pack_weight_scales(const uint8_t* a_s, const uint8_t* b_s, int n_experts, int n_rows, int k,
                                     uint8_t* out, hipStream_t s) {
  const int l1 = b_s != nullptr;
  const int ntiles = l1 ? (n_rows + L1_J_PER_TILE - 1) / L1_J_PER_TILE : (n_rows + BN - 1) / BN;
  const int nst = (k + BK - 1) / BK, ks = k / 32;
  if (n_experts <= 0 || ntiles <= 0) return hipSuccess;
  dim3 grid(ntiles * nst, n_experts);
  k_pack_weight_scales<<<grid, 256, 0, s>>>(a_s, b_s, l1, n_rows, ks, ntiles, nst, (int64_t)n_rows * ks, out);
  return hipGetLastError();
}

// Weight codes: block (tile, half stage h), expert blockIdx.y; thread R = tile
// row, the GEMM's row order (L1: gate and up rows interleaved as for the
// scales; rows past n_rows repeat the last row). The block is the LDS image of
// the half stage: row R at R * 64, its 16-byte chunk c (32 K values) at slot
// c ^ ((R >> 2) & 3), the swizzle the GEMM reads with.
__global__ __launch_bounds__(256) void k_pack_weight_codes(const uint8_t* __restrict__ a,
                                                           const uint8_t* __restrict__ b, int l1, int n_rows,
                                                           int kb, int ntiles, int nh, int64_t src_estride,
                                                           uint8_t* __restrict__ out) {
  const int nt = blockIdx.x / nh, h = blockIdx.x - nt * nh, e = blockIdx.y, R = threadIdx.x;
  const uint8_t* src;
  int row;
  if (l1) {
    const int f = (R >> 5) & 3;
    row = nt * L1_J_PER_TILE + (R >> 7) * 64 + (f & 1) * 32 + (R & 31);
    src = f < 2 ? a : b;
  } else {
    row = nt * BN + R;
    src = a;
  }
  row = min(row, n_rows - 1);
  const uint4* p = (const uint4*)(src + (int64_t)e * src_estride + (int64_t)row * kb + h * 64);
  uint4 v[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = p[c];
  uint8_t* dst = out + (((int64_t)e * ntiles + nt) * nh + h) * CODE_BLOCK_BYTES + R * 64;
#pragma unroll
  for (int c = 0; c < 4; ++c) *(uint4*)(dst + ((c ^ ((R >> 2) & 3)) * 16)) = v[c];
}

hipError_t launch_pack_weight_codes(const uint8_t* a, const uint8_t* b, int n_experts, int n_rows, int k,
                                    uint8_t* out, hipStream_t s) {
  const int l1 = b != nullptr;
  const int ntiles = l1 ? (n_rows + L1_J_PER_TILE - 1) / L1_J_PER_TILE : (n_rows + BN - 1) / BN;
  const int nh = k / 128, kb = k / 2;
  if (n_experts <= 0 || ntiles <= 0 || nh <= 0) return hipSuccess;
  dim3 grid(ntiles * nh, n_experts);
  k_pack_weight_codes<<<grid, 256, 0, s>>>(a, b, l1, n_rows, kb, ntiles, nh, (int64_t)n_rows * kb, out);
  return hipGetLastError();
}

hipError_t launch_pack_act_scales(const uint8_t* x_s, int k, const int32_t* row_token, const int32_t* expert_off,
                                  const int32_t* tile_base, int n_experts, int m_rows, int max_mtiles,
                                  uint8_t* out, hipStream_t s) {
  if (max_mtiles <= 0) return hipSuccess;
  const int nst = (k + BK - 1) / BK, ks = k / 32;
  const dim3 grid(max_mtiles, (nst + ACT_STAGES - 1) / ACT_STAGES);
  k_pack_act_scales<<<grid, 256, 0, s>>>(x_s, ks, nst, row_token, expert_off, tile_base, n_experts, m_rows, out);
  return hipGetLastError();
}

}  // namespace mx
