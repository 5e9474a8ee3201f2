// Token -> expert permutation for the routed experts, and the weighted un-permute.
//
// The routed MoE adds routing, top-k and a scatter to the shared-expert pipeline
// (page "Current Bug: vLLM produces empty/garbage output", section "Revised
// Plan", Phase 1, which describes the shared expert as the MoE pipeline minus
// those steps; 48 local experts per rank in "Config values"; the final scatter
// stays in BF16 per Phase 3). Router logits and top-k selection are inputs.
//
// Route: pairs p = t*k + j (token t, slot j) are ordered by expert, and by p
// within an expert (stable, so the layout is the same on every run). Two kernels:
//   1. per-chunk expert histogram (LDS counters),
//   2. scatter with the scan folded in (see k_route_scatter).
// Ids outside [0, E) belong to experts on other ranks and are skipped.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_route_count(const int32_t* __restrict__ ids, int64_t P, int E,
                                                     int32_t* __restrict__ block_counts) {
  __shared__ int cnt[ROUTE_MAX_EXPERTS];
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * ROUTE_CHUNK;
  for (int i = threadIdx.x; i < ROUTE_CHUNK; i += 256) {
    const int64_t p = base + i;
    if (p < P) {
      const int e = ids[p];
      if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) block_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// One block of ROUTE_CHUNK threads (16 waves) per chunk of pairs, one pair per
// thread. Each block recomputes, from the chunk histograms, the expert totals
// (-> expert offsets and m-tile bases, written by block 0) and its own base
// within every expert. Inside the block a pair's rank among the earlier pairs
// of its expert is the sum of the counts of the earlier waves plus its rank in
// its own wave: lanes that share an expert find each other with a ballot and
// count the set bits below them. Order within an expert is pair order.
__global__ __launch_bounds__(ROUTE_CHUNK) void k_route_scatter(
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int64_t P, int k, int E,
    const int32_t* __restrict__ block_counts, int nblocks, int32_t* __restrict__ expert_off,
    int32_t* __restrict__ tile_base, int32_t* __restrict__ row_token, int32_t* __restrict__ row_slot,
    float* __restrict__ row_weight) {
  extern __shared__ int sm[];
  constexpr int NW = ROUTE_CHUNK / 64;
  int* tot = sm;              // [E] pairs per expert (all chunks)
  int* pre = sm + E;          // [E] pairs per expert in earlier chunks
  int* off = sm + 2 * E;      // [E] exclusive prefix of tot
  int* wc = sm + 3 * E;       // [NW][E] pairs per expert in each wave of this chunk
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.x;
  for (int i = tid; i < (3 + NW) * E; i += ROUTE_CHUNK) sm[i] = 0;
  __syncthreads();
  for (int i = tid; i < nblocks * E; i += ROUTE_CHUNK) {
    const int c = block_counts[i];
    const int e = i % E;
    atomicAdd(&tot[e], c);
    if (i / E < b) atomicAdd(&pre[e], c);
  }
  const int64_t p = (int64_t)b * ROUTE_CHUNK + tid;
  const int e = (p < P) ? ids[p] : -1;
  const bool valid = (p < P) && ((unsigned)e < (unsigned)E);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank = 0;
  uint64_t todo = __ballot(valid);
  while (todo) {
    const int leader = __ffsll((long long)todo) - 1;
    const int ee = __shfl(e, leader);
    const uint64_t m = __ballot(valid && e == ee);
    if (valid && e == ee) rank = __popcll(m & below);
    if (lane == leader) wc[w * E + ee] = __popcll(m);
    todo &= ~m;
  }
  __syncthreads();
  if (tid == 0) {
    int o = 0, tb = 0;
    for (int x = 0; x < E; ++x) {
      off[x] = o;
      if (b == 0) {
        expert_off[x] = o;
        tile_base[x] = tb;
      }
      o += tot[x];
      tb += (tot[x] + BM - 1) / BM;
    }
    if (b == 0) {
      expert_off[E] = o;
      tile_base[E] = tb;
    }
  }
  __syncthreads();
  if (valid) {
    int pos = off[e] + pre[e] + rank;
    for (int x = 0; x < w; ++x) pos += wc[x * E + e];
    row_token[pos] = (int)(p / k);
    row_slot[pos] = (int)p;
    row_weight[pos] = wts[p];
  }
}

constexpr int COMBINE_BATCH = 8;   // slots whose rows are loaded together

// Sorted row r of the routed pairs gets token row_token[r] of a row-major
// [T, width] byte matrix (width a multiple of 8): one thread per 8 bytes.
// Rows past the last routed pair (ids on other ranks) are left as they are.
__global__ __launch_bounds__(256) void k_gather_rows(const uint8_t* __restrict__ src, int width,
                                                     const int32_t* __restrict__ row_token,
                                                     const int32_t* __restrict__ n_valid, int64_t P,
                                                     uint8_t* __restrict__ dst) {
  const int per = width >> 3;
  const int64_t rows = min((int64_t)*n_valid, P);
  const int64_t n = rows * per;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    const int64_t r = i / per;
    const int c = (int)(i - r * per);
    *(uint2*)(dst + r * width + c * 8) = *(const uint2*)(src + (int64_t)row_token[r] * width + c * 8);
  }
}

// y[t][n] = bf16( sum_j o[t*k + j][n] ) over slots j with a local expert, in j order.
// o rows already carry the gate weight. One thread per 8 columns (16 bytes).
// o is read once and y written once, both as streaming accesses that bypass the
// caches (measured over 48 experts x 4096 tokens, top-8: 0.109 -> 0.089 ms).
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ o,
                                                 const int32_t* __restrict__ ids, int64_t T, int k,
                                                 int E, int H, uint16_t* __restrict__ y) {
  const int per_row = H >> 3;
  const int64_t n = T * per_row;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    const int64_t t = i / per_row;
    const int c = (int)(i - t * per_row) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // Eight slots at a time, all loads issued before any sum: the row of every
    // slot exists (skipped slots' rows are simply not added), so no load waits
    // for an id check.
    for (int j0 = 0; j0 < k; j0 += COMBINE_BATCH) {
      uint4 v[COMBINE_BATCH];
      bool ok[COMBINE_BATCH];
#pragma unroll
      for (int q = 0; q < COMBINE_BATCH; ++q) {
        const int j = min(j0 + q, k - 1);
        ok[q] = j0 + q < k && (unsigned)ids[t * k + j] < (unsigned)E;
        v[q] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)(o + (t * k + j) * (int64_t)H + c)));
      }
#pragma unroll
      for (int q = 0; q < COMBINE_BATCH; ++q) {
        if (!ok[q]) continue;
        const uint32_t w[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += bf16_to_f32(w[i] & 0xFFFFu);
          acc[2 * i + 1] += bf16_to_f32(w[i] >> 16);
        }
      }
    }
    uint32_t r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = bf16x2_rne(acc[2 * q], acc[2 * q + 1]);
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, make_uint4(r[0], r[1], r[2], r[3])), (u32x4_t*)(y + t * (int64_t)H + c));
  }
}

}  // namespace

hipError_t launch_route(const int32_t* topk_ids, const float* topk_w, int64_t tokens, int k, int n_experts,
                        const RouteBuffers& rb, hipStream_t s) {
  const int64_t P = tokens * k;
  const int nblocks = (int)((P + ROUTE_CHUNK - 1) / ROUTE_CHUNK);
  if (nblocks == 0) return hipSuccess;
  k_route_count<<<nblocks, 256, 0, s>>>(topk_ids, P, n_experts, rb.block_counts);
  const size_t lds = (size_t)(3 + ROUTE_CHUNK / 64) * n_experts * sizeof(int);
  k_route_scatter<<<nblocks, ROUTE_CHUNK, lds, s>>>(topk_ids, topk_w, P, k, n_experts, rb.block_counts, nblocks,
                                                    rb.expert_off, rb.tile_base, rb.row_token, rb.row_slot,
                                                    rb.row_weight);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const uint8_t* src, int width, const int32_t* row_token, const int32_t* n_valid,
                              int64_t P, uint8_t* dst, hipStream_t s) {
  const int64_t n = P * (width / 8);
  if (n == 0) return hipSuccess;
  int64_t g = (n + 255) / 256;
  if (g > 8192) g = 8192;
  k_gather_rows<<<(int)g, 256, 0, s>>>(src, width, row_token, n_valid, P, dst);
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* o, const int32_t* topk_ids, int64_t tokens, int k,
                          int n_experts, int hidden, uint16_t* y, hipStream_t s) {
  const int64_t n = tokens * (hidden / 8);
  if (n == 0) return hipSuccess;
  int64_t g = (n + 255) / 256;
  if (g > 16384) g = 16384;
  k_combine<<<(int)g, 256, 0, s>>>(o, topk_ids, tokens, k, n_experts, hidden, y);
  return hipGetLastError();
}

}  // namespace mx
