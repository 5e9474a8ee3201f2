// Token -> expert permutation for the routed experts, and the weighted un-permute.
//
// The routed MoE adds routing, top-k and a scatter to the shared-expert pipeline
// (page "Current Bug: vLLM produces empty/garbage output", section "Revised
// Plan", Phase 1, which describes the shared expert as the MoE pipeline minus
// those steps; 48 local experts per rank in "Config values"; the final scatter
// stays in BF16 per Phase 3). Router logits and top-k selection are inputs.
//
// Route: pairs p = t*k + j (token t, slot j) are ordered by expert, and by p
// within an expert (stable, so the layout is the same on every run). Three kernels:
//   1. per-chunk expert histogram (LDS counters),
//   2. one block turns the histograms into each chunk's base within every expert
//      and the expert offsets and m-tile bases,
//   3. scatter: every pair's place is its chunk's base plus its rank in the chunk.
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

// One block of ROUTE_SCAN_THREADS threads over the [nblocks, E] chunk
// histograms. Thread (g, e) owns expert e in the g-th of G = threads / E
// contiguous runs of chunks: it sums its run, the run sums are scanned over g,
// and it rewrites its run in place as exclusive prefixes, so that
// block_counts[c * E + e] becomes the number of expert-e pairs in chunks before
// c. Wave 0 then scans the expert totals into expert_off (pair offsets) and
// tile_base (offsets in m-tiles of BM rows), each with a final entry E.
constexpr int ROUTE_SCAN_THREADS = 1024;
static_assert(ROUTE_SCAN_THREADS >= 2 * ROUTE_MAX_EXPERTS, "two chunk runs per expert at least");

__global__ __launch_bounds__(ROUTE_SCAN_THREADS) void k_route_scan(int32_t* __restrict__ block_counts,
                                                                    int64_t nblocks, int E,
                                                                    int32_t* __restrict__ expert_off,
                                                                    int32_t* __restrict__ tile_base) {
  __shared__ int part[ROUTE_SCAN_THREADS];   // [G][E] run sums, then their exclusive prefix over g
  __shared__ int tot[ROUTE_MAX_EXPERTS];
  const int tid = threadIdx.x;
  const int G = ROUTE_SCAN_THREADS / E;
  const int g = tid / E, e = tid - g * E;
  const bool on = g < G;
  const int64_t lo = nblocks * g / G, hi = nblocks * (g + 1) / G;
  // runs can be long (16384 chunks of 48 experts: ~780 per thread), so the
  // loads go eight at a time, independent of the sums
  constexpr int U = 8;
  if (on) {
    int sum = 0;
    int64_t c = lo;
    for (; c + U <= hi; c += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = block_counts[(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < U; ++u) sum += v[u];
    }
    for (; c < hi; ++c) sum += block_counts[c * E + e];
    part[tid] = sum;
  }
  __syncthreads();
  if (tid < E) {
    int acc = 0;
    for (int x = 0; x < G; ++x) {
      const int v = part[x * E + tid];
      part[x * E + tid] = acc;
      acc += v;
    }
    tot[tid] = acc;
  }
  __syncthreads();
  if (on) {
    int acc = part[tid];
    int64_t c = lo;
    for (; c + U <= hi; c += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = block_counts[(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        block_counts[(c + u) * E + e] = acc;
        acc += v[u];
      }
    }
    for (; c < hi; ++c) {
      const int v = block_counts[c * E + e];
      block_counts[c * E + e] = acc;
      acc += v;
    }
  }
  if (tid < 64) {
    // lane l scans experts [l * per, (l + 1) * per) after the lanes below it
    const int per = (E + 63) / 64;
    const int x0 = min(tid * per, E), x1 = min(x0 + per, E);
    int ps = 0, ts = 0;
    for (int x = x0; x < x1; ++x) {
      ps += tot[x];
      ts += (tot[x] + BM - 1) / BM;
    }
    int pi = ps, ti = ts;   // inclusive scans over the lanes
    for (int d = 1; d < 64; d <<= 1) {
      const int pu = __shfl_up(pi, d), tu = __shfl_up(ti, d);
      if (tid >= d) {
        pi += pu;
        ti += tu;
      }
    }
    int o = pi - ps, tb = ti - ts;
    for (int x = x0; x < x1; ++x) {
      expert_off[x] = o;
      tile_base[x] = tb;
      o += tot[x];
      tb += (tot[x] + BM - 1) / BM;
    }
    if (tid == 63) {
      expert_off[E] = pi;
      tile_base[E] = ti;
    }
  }
}

// One block of ROUTE_CHUNK threads (16 waves) per chunk of pairs, one pair per
// thread. A pair's place is its expert's offset, plus the expert's pairs in
// earlier chunks (the scanned histograms), plus its rank in this chunk: the
// counts of the earlier waves plus its rank in its own wave, where lanes that
// share an expert find each other with a ballot and count the set bits below
// them. Order within an expert is pair order.
__global__ __launch_bounds__(ROUTE_CHUNK) void k_route_scatter(
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int64_t P, int k, int E,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ expert_off,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_slot, float* __restrict__ row_weight) {
  extern __shared__ int wc[];   // [NW][E] pairs per expert in each wave of this chunk
  constexpr int NW = ROUTE_CHUNK / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t b = blockIdx.x;
  for (int i = tid; i < NW * E; i += ROUTE_CHUNK) wc[i] = 0;
  __syncthreads();
  const int64_t p = b * ROUTE_CHUNK + tid;
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
  if (valid) {
    int pos = expert_off[e] + chunk_base[b * E + e] + rank;
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
  k_route_scan<<<1, ROUTE_SCAN_THREADS, 0, s>>>(rb.block_counts, nblocks, n_experts, rb.expert_off, rb.tile_base);
  const size_t lds = (size_t)(ROUTE_CHUNK / 64) * n_experts * sizeof(int);
  k_route_scatter<<<nblocks, ROUTE_CHUNK, lds, s>>>(topk_ids, topk_w, P, k, n_experts, rb.block_counts,
                                                    rb.expert_off, rb.row_token, rb.row_slot, rb.row_weight);
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
