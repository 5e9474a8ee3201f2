// C-ABI entry points of libmxfp4: host-side validation, workspace layout and
// kernel sequencing. Every check runs before anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/mxfp4.h"
#include "mx_internal.h"
#include "nv_linear.h"
#include "fp8_linear.h"

using namespace mx;

namespace {

thread_local char g_err[512] = "";

mx_status fail(mx_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

mx_status ok() {
  g_err[0] = 0;
  return MX_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ---------------------------------------------------------------- profiler
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Profiler g_prof;

template <class F>
hipError_t phase(const char* name, hipStream_t s, F&& launch) {
  if (!g_prof.on) return launch();
  std::lock_guard<std::mutex> lk(g_prof.mu);
  hipEvent_t a = g_prof.get(), b = g_prof.get();
  if (a) hipEventRecord(a, s);
  hipError_t e = launch();
  if (b) hipEventRecord(b, s);
  if (a && b) g_prof.recs.push_back({name, a, b});
  return e;
}

mx_status hip_fail(hipError_t e, const char* what) {
  return fail(MX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------- workspace
struct Carve {
  uint8_t* base;
  size_t off = 0;
  explicit Carve(void* b) : base((uint8_t*)b) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  }
};

// Dense (one expert) workspace, by path (MXFP4 re-quantisation picks the
// weight-streaming paths for small M):
//   few tokens (M <= 8): h, the bf16 SiLU output;
//   9 <= M <= 96:        xq, xs, hq, hs, then h;
//   GEMM path:           xq, xs, hq, hs, xs_pk, then the L1 split-K partials
//                        when L1 is split.
// On the GEMM path xs_pk is the tile-major copy of xs that L1 reads, and with
// MXFP4 re-quantisation hs is tile-major over the m-tiles (L2 reads it so);
// with NVFP4 hs is row-major E4M3 per 16.
enum DensePath { DENSE_DECODE, DENSE_SKINNY, DENSE_GEMM };

// Split-K of the L1 GEMM on the dense path (MXFP4 re-quantisation, one
// m-tile): with so few tiles most CUs would idle while each tile streams all of
// K one stage at a time, so the K stages are split over about 256 workgroups
// (the CUs of an MI355X), at least 4 stages and at most 8 splits each. Returns
// 1 for no split. Measured on the shared expert (7168 x 3072): 80 -> 57 us per
// call at 128 tokens. Splitting L2 too, or splitting two m-tiles, was slower:
// the fp32 partials (about 20 MB) cost more than the split saves.
int l1_splits(int64_t M, int64_t H, int64_t I, mx_format rq) {
  if (rq != MX_FMT_MXFP4 || M > BM) return 1;
  int64_t s = 256 / ((I + L1_J_PER_TILE - 1) / L1_J_PER_TILE);
  s = std::min<int64_t>(s, ((H + BK - 1) / BK) / 4);
  s = std::min<int64_t>(s, 8);
  return s >= 2 ? (int)s : 1;
}

struct DenseWs {
  DensePath path;
  int l1_split;
  uint8_t *xq, *xs, *hq, *hs, *xs_pk;
  uint16_t* h;
  float* part;
  size_t bytes;
};
DenseWs dense_ws(void* base, int64_t M, int64_t H, int64_t I, mx_format rq) {
  Carve c(base);
  DenseWs w;
  w.xq = w.xs = w.hq = w.hs = w.xs_pk = nullptr;
  w.h = nullptr;
  w.part = nullptr;
  w.l1_split = 1;
  if (rq == MX_FMT_MXFP4 && decode_fits(M, H, I)) {
    w.path = DENSE_DECODE;
    w.h = (uint16_t*)c.take((size_t)(M * I * 2));
  } else {
    w.path = (rq == MX_FMT_MXFP4 && skinny_fits(M, H, I)) ? DENSE_SKINNY : DENSE_GEMM;
    const int64_t mtiles = (M + BM - 1) / BM;
    // the weight-streaming path's token operands: chunked, whole 16-row chunks
    const int64_t mq = w.path == DENSE_SKINNY ? (M + 15) / 16 * 16 : M;
    w.xq = (uint8_t*)c.take((size_t)(mq * H / 2));
    w.xs = (uint8_t*)c.take(w.path == DENSE_SKINNY ? (size_t)chunked_scale_bytes(M) : (size_t)(M * H / 32));
    // h codes: tile-major for the L2 GEMM's copies on the MXFP4 GEMM path
    w.hq = (uint8_t*)c.take((rq == MX_FMT_MXFP4 && w.path == DENSE_GEMM) ? (size_t)packed_code_bytes(mtiles, I)
                                                                         : (size_t)(mq * I / 2));
    if (rq == MX_FMT_NVFP4) w.hs = (uint8_t*)c.take((size_t)(M * I / 16));
    else if (w.path == DENSE_GEMM) w.hs = (uint8_t*)c.take((size_t)packed_scale_bytes(mtiles, I));
    else w.hs = (uint8_t*)c.take((size_t)chunked_scale_bytes(M));
    if (w.path == DENSE_SKINNY) {
      w.h = (uint16_t*)c.take((size_t)(M * I * 2));
    } else {
      w.xs_pk = (uint8_t*)c.take((size_t)packed_scale_bytes(mtiles, H));
      w.l1_split = l1_splits(M, H, I, rq);
      if (w.l1_split > 1) {
        const int64_t tiles = (int64_t)w.l1_split * mtiles * ((I + L1_J_PER_TILE - 1) / L1_J_PER_TILE);
        w.part = (float*)c.take((size_t)(tiles * PART_TILE_FLOATS * 4));
      }
    }
  }
  w.bytes = c.off;
  return w;
}

// Routed workspace: xq, xs, the route buffers, hq, hs, o, xs_pk. As on the
// dense GEMM path, xs_pk is the tile-major copy of the gathered xs and, with
// MXFP4 re-quantisation, hq and hs are tile-major over the m-tiles.
//
// With few rows per expert (routed_stream_fits) the weight-streaming kernels
// run instead of the GEMMs: xq, xs, the route buffers, h (bf16), hq, hs
// (row-major, E8M0 per 32 or E4M3 per 16), then o; no xs_pk.
struct GroupWs {
  bool stream;
  uint8_t *xq, *xs, *hq, *hs, *xs_pk;
  uint16_t *o, *h;
  RouteBuffers rb;
  size_t bytes;
};
// Upper bound of the m-tiles of a routed launch: every expert adds at most one
// partly filled tile.
int64_t max_route_mtiles(int64_t P, int E) { return (P + (int64_t)E * (BM - 1)) / BM; }
GroupWs group_ws(void* base, int64_t T, int64_t H, int64_t I, int k, int E, mx_format rq) {
  Carve c(base);
  GroupWs w;
  const int64_t P = T * k;
  const int64_t nblocks = (P + ROUTE_CHUNK - 1) / ROUTE_CHUNK;
  const int64_t mtiles = max_route_mtiles(P, E);
  w.stream = routed_stream_fits(T, H, I, k, E, rq == MX_FMT_NVFP4);
  w.h = nullptr;
  w.xs_pk = nullptr;
  w.xq = (uint8_t*)c.take((size_t)(T * H / 2));
  w.xs = (uint8_t*)c.take((size_t)(T * H / 32));
  w.rb.block_counts = (int32_t*)c.take((size_t)(nblocks * E * 4));
  w.rb.expert_off = (int32_t*)c.take((size_t)(E + 1) * 4);
  w.rb.tile_base = (int32_t*)c.take((size_t)(E + 1) * 4);
  w.rb.row_token = (int32_t*)c.take((size_t)P * 4);
  w.rb.row_slot = (int32_t*)c.take((size_t)P * 4);
  w.rb.row_weight = (float*)c.take((size_t)P * 4);
  if (w.stream) {
    w.h = (uint16_t*)c.take((size_t)(P * I * 2));
    w.hq = (uint8_t*)c.take((size_t)(P * I / 2));
    w.hs = (uint8_t*)c.take(rq == MX_FMT_NVFP4 ? (size_t)(P * I / 16) : (size_t)(P * I / 32));
    w.o = (uint16_t*)c.take((size_t)(P * H * 2));
    w.bytes = c.off;
    return w;
  }
  // h codes: tile-major over the m-tiles for the L2 GEMM's copies (MXFP4)
  w.hq = (uint8_t*)c.take(rq == MX_FMT_NVFP4 ? (size_t)(P * I / 2) : (size_t)packed_code_bytes(mtiles, I));
  w.hs = (uint8_t*)c.take(rq == MX_FMT_NVFP4 ? (size_t)(P * I / 16) : (size_t)packed_scale_bytes(mtiles, I));
  w.o = (uint16_t*)c.take((size_t)(P * H * 2));
  w.xs_pk = (uint8_t*)c.take((size_t)packed_scale_bytes(mtiles, H));
  w.bytes = c.off;
  return w;
}

// The tile-major weight scales written by mx_pack_weight_scales: for each
// expert, L1 (gate/up pairs, tiles of 128 j) and then, after all experts' L1
// parts, L2 (tiles of 256 rows).
struct PackedWeights {
  int64_t l1_estride, l2_estride, l1_bytes, bytes;
};
PackedWeights packed_weights(int64_t H, int64_t I, int64_t E) {
  PackedWeights p;
  p.l1_estride = packed_scale_bytes((I + L1_J_PER_TILE - 1) / L1_J_PER_TILE, H);
  p.l2_estride = packed_scale_bytes((H + BN - 1) / BN, I);
  p.l1_bytes = E * p.l1_estride;
  p.bytes = p.l1_bytes + E * p.l2_estride;
  return p;
}

// The tile-major weight codes written by mx_pack_weight_codes, laid out as the
// scales: each expert's L1 blocks, then (after all experts) the L2 blocks.
PackedWeights packed_codes_layout(int64_t H, int64_t I, int64_t E) {
  PackedWeights p;
  p.l1_estride = packed_code_bytes((I + L1_J_PER_TILE - 1) / L1_J_PER_TILE, H);
  p.l2_estride = packed_code_bytes((H + BN - 1) / BN, I);
  p.l1_bytes = E * p.l1_estride;
  p.bytes = p.l1_bytes + E * p.l2_estride;
  return p;
}

// ---------------------------------------------------------------- checks
mx_status check_mlp_dims(int64_t M, int64_t H, int64_t I) {
  if (M < 0) return fail(MX_ERR_SHAPE, "token count %lld is negative", (long long)M);
  if (H < 128 || H % 128 != 0) return fail(MX_ERR_SHAPE, "hidden %lld must be a positive multiple of 128", (long long)H);
  if (I < 128 || I % 128 != 0) return fail(MX_ERR_SHAPE, "inter %lld must be a positive multiple of 128", (long long)I);
  if (H > (1 << 20) || I > (1 << 20)) return fail(MX_ERR_SHAPE, "hidden/inter above 2^20");
  if (M > ((int64_t)1 << 30)) return fail(MX_ERR_SHAPE, "token count %lld above 2^30", (long long)M);
  return MX_OK;
}

mx_status check_global(float g) {
  if (!std::isfinite(g) || !(g >= 0x1p-117f))
    return fail(MX_ERR_VALUE, "NVFP4 global scale %g must be finite and >= 2^-117", (double)g);
  return MX_OK;
}

// A global scale in device memory: present and 4-byte aligned. Its value is
// read by the kernels in stream order, so the host cannot check it.
mx_status check_global_ptr(const float* g) {
  if (g == nullptr) return fail(MX_ERR_NULL, "the NVFP4 global scale pointer is NULL");
  if (!aligned(g, 4)) return fail(MX_ERR_ALIGN, "the NVFP4 global scale pointer is not 4-byte aligned");
  return MX_OK;
}

mx_status check_requant(mx_format rq, const float* g) {
  if (rq == MX_FMT_MXFP4) return MX_OK;
  if (rq == MX_FMT_NVFP4) return check_global_ptr(g);
  return fail(MX_ERR_FORMAT, "requant format %d is not MXFP4 or NVFP4", (int)rq);
}

#define MX_REQUIRE_PTR(p) \
  do { if ((p) == nullptr) return fail(MX_ERR_NULL, "%s is NULL", #p); } while (0)
#define MX_REQUIRE_ALIGN(p, a) \
  do { if (!aligned((p), (a))) return fail(MX_ERR_ALIGN, "%s is not %d-byte aligned", #p, (int)(a)); } while (0)
#define MX_TRY(expr) \
  do { mx_status st_ = (expr); if (st_ != MX_OK) return st_; } while (0)
#define MX_HIP(expr, what) \
  do { hipError_t e_ = (expr); if (e_ != hipSuccess) return hip_fail(e_, what); } while (0)

GemmArgs base_args() {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  return a;
}

}  // namespace

extern "C" {

const char* mx_status_string(mx_status s) {
  switch (s) {
    case MX_OK: return "ok";
    case MX_ERR_NULL: return "null pointer";
    case MX_ERR_SHAPE: return "bad shape";
    case MX_ERR_ALIGN: return "misaligned pointer";
    case MX_ERR_FORMAT: return "unsupported format";
    case MX_ERR_WORKSPACE: return "workspace too small";
    case MX_ERR_HIP: return "HIP error";
    case MX_ERR_VALUE: return "bad value";
  }
  return "unknown status";
}

const char* mx_last_error(void) { return g_err; }

mx_status mx_profile_start(void) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (auto& r : g_prof.recs) {
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.recs.clear();
  g_prof.on = true;
  return ok();
}

mx_status mx_profile_stop(mx_phase_stat* stats, int32_t max_stats, int32_t* n_stats) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = false;
  std::vector<mx_phase_stat> agg;
  mx_status st = MX_OK;
  for (auto& r : g_prof.recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) st = hip_fail(e, "profiler event");
    size_t i = 0;
    for (; i < agg.size(); ++i)
      if (strcmp(agg[i].name, r.name) == 0) break;
    if (i == agg.size()) {
      mx_phase_stat z;
      memset(&z, 0, sizeof(z));
      snprintf(z.name, sizeof(z.name), "%s", r.name);
      agg.push_back(z);
    }
    agg[i].total_ms += ms;
    agg[i].launches += 1;
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.recs.clear();
  const int n = (int)agg.size() < max_stats ? (int)agg.size() : max_stats;
  if (stats)
    for (int i = 0; i < n; ++i) stats[i] = agg[i];
  if (n_stats) *n_stats = (int32_t)agg.size();
  if (st == MX_OK) ok();
  return st;
}

mx_status mx_dequant(mx_format fmt, const void* codes, const void* scales, const float* global_scale,
                     int64_t rows, int64_t cols, uint16_t* out, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (rows < 0 || cols < 0) return fail(MX_ERR_SHAPE, "rows %lld / cols %lld negative", (long long)rows, (long long)cols);
  if (rows * cols > ((int64_t)1 << 40)) return fail(MX_ERR_SHAPE, "matrix too large");
  if (fmt == MX_FMT_MXFP4) {
    if (cols % 32 != 0) return fail(MX_ERR_SHAPE, "cols %lld %% 32 != 0", (long long)cols);
  } else if (fmt == MX_FMT_FP8_B128 || fmt == MX_FMT_NVFP4) {
    if (cols % 16 != 0) return fail(MX_ERR_SHAPE, "cols %lld %% 16 != 0", (long long)cols);
  } else {
    return fail(MX_ERR_FORMAT, "unknown format %d", (int)fmt);
  }
  if (rows == 0 || cols == 0) return ok();
  MX_REQUIRE_PTR(codes);
  MX_REQUIRE_PTR(scales);
  MX_REQUIRE_PTR(out);
  MX_REQUIRE_ALIGN(out, 16);
  hipError_t e;
  if (fmt == MX_FMT_MXFP4) {
    MX_REQUIRE_ALIGN(codes, 16);
    e = phase("dequant_mxfp4", s, [&] {
      return launch_dequant_mxfp4((const uint8_t*)codes, (const uint8_t*)scales, rows, cols, out, s);
    });
  } else if (fmt == MX_FMT_FP8_B128) {
    MX_REQUIRE_ALIGN(codes, 16);
    e = phase("dequant_fp8_block", s, [&] {
      return launch_dequant_fp8_block((const uint8_t*)codes, (const uint8_t*)scales, rows, cols, out, s);
    });
  } else {
    MX_TRY(check_global_ptr(global_scale));
    MX_REQUIRE_ALIGN(codes, 8);
    e = phase("dequant_nvfp4", s, [&] {
      return launch_dequant_nvfp4((const uint8_t*)codes, (const uint8_t*)scales, 0.0f, global_scale, rows, cols,
                                  out, s);
    });
  }
  if (e != hipSuccess) return hip_fail(e, "dequant launch");
  return ok();
}

mx_status mx_quantize_act(mx_format fmt, const uint16_t* x, int64_t rows, int64_t cols,
                          const float* global_scale, uint8_t* codes, uint8_t* scales, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (rows < 0 || cols < 0) return fail(MX_ERR_SHAPE, "rows %lld / cols %lld negative", (long long)rows, (long long)cols);
  if (rows * cols > ((int64_t)1 << 40)) return fail(MX_ERR_SHAPE, "matrix too large");
  if (fmt == MX_FMT_MXFP4) {
    if (cols % 32 != 0) return fail(MX_ERR_SHAPE, "cols %lld %% 32 != 0", (long long)cols);
  } else if (fmt == MX_FMT_NVFP4) {
    if (cols % 16 != 0) return fail(MX_ERR_SHAPE, "cols %lld %% 16 != 0", (long long)cols);
    MX_TRY(check_global_ptr(global_scale));
  } else if (fmt == MX_FMT_MXFP8) {
    if (cols % 32 != 0) return fail(MX_ERR_SHAPE, "cols %lld %% 32 != 0", (long long)cols);
  } else {
    return fail(MX_ERR_FORMAT, "quantize_act supports MXFP4, NVFP4 and MXFP8, not format %d", (int)fmt);
  }
  if (rows == 0 || cols == 0) return ok();
  MX_REQUIRE_PTR(x);
  MX_REQUIRE_PTR(codes);
  MX_REQUIRE_PTR(scales);
  MX_REQUIRE_ALIGN(x, 16);
  hipError_t e;
  if (fmt == MX_FMT_MXFP4) {
    MX_REQUIRE_ALIGN(codes, 16);
    e = phase("quant_mxfp4", s, [&] { return launch_quant_mxfp4(x, rows, cols, codes, scales, s); });
  } else if (fmt == MX_FMT_MXFP8) {
    MX_REQUIRE_ALIGN(codes, 16);
    e = phase("quant_mxfp8", s, [&] { return launch_quant_mxfp8(x, rows, cols, codes, scales, s); });
  } else {
    MX_REQUIRE_ALIGN(codes, 8);
    e = phase("quant_nvfp4", s, [&] { return launch_quant_nvfp4(x, rows, cols, 0.0f, global_scale, codes, scales, s); });
  }
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return ok();
}

size_t mx_expert_mlp_workspace_size(int64_t M, int64_t hidden, int64_t inter, mx_format requant) {
  if (M < 0 || hidden < 0 || inter < 0) return 0;
  return dense_ws(nullptr, M, hidden, inter, requant).bytes;
}

size_t mx_grouped_expert_mlp_workspace_size(int64_t T, int64_t hidden, int64_t inter, int32_t k, int32_t E,
                                            mx_format requant) {
  if (T < 0 || hidden < 0 || inter < 0 || k < 1 || E < 1) return 0;
  return group_ws(nullptr, T, hidden, inter, k, E, requant).bytes;
}

static mx_status check_weights(const uint8_t* w1, const uint8_t* w1_s, const uint8_t* w3, const uint8_t* w3_s,
                               const uint8_t* w2, const uint8_t* w2_s) {
  MX_REQUIRE_PTR(w1);
  MX_REQUIRE_PTR(w1_s);
  MX_REQUIRE_PTR(w3);
  MX_REQUIRE_PTR(w3_s);
  MX_REQUIRE_PTR(w2);
  MX_REQUIRE_PTR(w2_s);
  MX_REQUIRE_ALIGN(w1, 16);
  MX_REQUIRE_ALIGN(w3, 16);
  MX_REQUIRE_ALIGN(w2, 16);
  MX_REQUIRE_ALIGN(w1_s, 4);
  MX_REQUIRE_ALIGN(w3_s, 4);
  MX_REQUIRE_ALIGN(w2_s, 4);
  return MX_OK;
}

size_t mx_packed_weight_scales_size(int64_t hidden, int64_t inter, int32_t E) {
  if (hidden < 0 || inter < 0 || E < 1) return 0;
  return (size_t)packed_weights(hidden, inter, E).bytes;
}

mx_status mx_pack_weight_scales(const uint8_t* w1_s, const uint8_t* w3_s, const uint8_t* w2_s, int64_t hidden,
                                int64_t inter, int32_t E, uint8_t* packed, size_t packed_bytes, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  MX_TRY(check_mlp_dims(0, hidden, inter));
  if (E < 1 || E > ROUTE_MAX_EXPERTS) return fail(MX_ERR_SHAPE, "E %d outside [1, %d]", E, ROUTE_MAX_EXPERTS);
  MX_REQUIRE_PTR(w1_s);
  MX_REQUIRE_PTR(w3_s);
  MX_REQUIRE_PTR(w2_s);
  MX_REQUIRE_PTR(packed);
  MX_REQUIRE_ALIGN(w1_s, 4);
  MX_REQUIRE_ALIGN(w3_s, 4);
  MX_REQUIRE_ALIGN(w2_s, 4);
  MX_REQUIRE_ALIGN(packed, 256);
  const PackedWeights pw = packed_weights(hidden, inter, E);
  if (packed_bytes < (size_t)pw.bytes)
    return fail(MX_ERR_WORKSPACE, "packed buffer %zu bytes < required %lld", packed_bytes, (long long)pw.bytes);
  MX_HIP(phase("pack_w_scales", s, [&] {
           hipError_t e = launch_pack_weight_scales(w1_s, w3_s, E, (int)inter, (int)hidden, packed, s);
           if (e != hipSuccess) return e;
           return launch_pack_weight_scales(w2_s, nullptr, E, (int)hidden, (int)inter, packed + pw.l1_bytes, s);
         }), "pack_w_scales");
  return ok();
}

mx_status mx_pack_weight_codes(const uint8_t* w1, const uint8_t* w3, const uint8_t* w2, int64_t hidden,
                               int64_t inter, int32_t E, uint8_t* packed, size_t packed_bytes, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  MX_TRY(check_mlp_dims(0, hidden, inter));
  if (E < 1 || E > ROUTE_MAX_EXPERTS) return fail(MX_ERR_SHAPE, "E %d outside [1, %d]", E, ROUTE_MAX_EXPERTS);
  MX_REQUIRE_PTR(w1);
  MX_REQUIRE_PTR(w3);
  MX_REQUIRE_PTR(w2);
  MX_REQUIRE_PTR(packed);
  MX_REQUIRE_ALIGN(w1, 16);
  MX_REQUIRE_ALIGN(w3, 16);
  MX_REQUIRE_ALIGN(w2, 16);
  MX_REQUIRE_ALIGN(packed, 256);
  const PackedWeights pc = packed_codes_layout(hidden, inter, E);
  if (packed_bytes < (size_t)pc.bytes)
    return fail(MX_ERR_WORKSPACE, "packed buffer %zu bytes < required %lld", packed_bytes, (long long)pc.bytes);
  MX_HIP(phase("pack_w_codes", s, [&] {
           hipError_t e = launch_pack_weight_codes(w1, w3, E, (int)inter, (int)hidden, packed, s);
           if (e != hipSuccess) return e;
           return launch_pack_weight_codes(w2, nullptr, E, (int)hidden, (int)inter, packed + pc.l1_bytes, s);
         }), "pack_w_codes");
  return ok();
}

size_t mx_packed_weight_codes_size(int64_t hidden, int64_t inter, int32_t E) {
  if (hidden < 128 || inter < 128 || hidden % 128 != 0 || inter % 128 != 0 || E < 1 || E > ROUTE_MAX_EXPERTS) return 0;
  return (size_t)packed_codes_layout(hidden, inter, E).bytes;
}

mx_status mx_expert_mlp(const uint16_t* x, int64_t M, int64_t hidden, int64_t inter, const uint8_t* w1,
                        const uint8_t* w1_s, const uint8_t* w3, const uint8_t* w3_s, const uint8_t* w2,
                        const uint8_t* w2_s, const uint8_t* packed_scales, const uint8_t* packed_codes,
                        mx_format requant, const float* requant_global, uint16_t* y, void* workspace,
                        size_t ws_bytes, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  MX_TRY(check_mlp_dims(M, hidden, inter));
  MX_TRY(check_requant(requant, requant_global));
  if (M == 0) return ok();
  MX_REQUIRE_PTR(x);
  MX_REQUIRE_PTR(y);
  MX_REQUIRE_ALIGN(x, 16);
  MX_REQUIRE_ALIGN(y, 16);
  MX_TRY(check_weights(w1, w1_s, w3, w3_s, w2, w2_s));
  MX_REQUIRE_ALIGN(packed_scales, 256);
  MX_REQUIRE_ALIGN(packed_codes, 256);
  const size_t need = mx_expert_mlp_workspace_size(M, hidden, inter, requant);
  MX_REQUIRE_PTR(workspace);
  MX_REQUIRE_ALIGN(workspace, 256);
  if (ws_bytes < need)
    return fail(MX_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  DenseWs w = dense_ws(workspace, M, hidden, inter, requant);
  const int H = (int)hidden, I = (int)inter, m = (int)M;
  const PackedWeights pc = packed_codes_layout(hidden, inter, 1);
  const uint8_t* pk1 = packed_codes;
  const uint8_t* pk2 = packed_codes ? packed_codes + pc.l1_bytes : nullptr;

  if (w.path == DENSE_DECODE) {
    // few tokens: two weight-streaming kernels, activations quantised in LDS
    MX_HIP(phase("decode_mlp", s, [&] {
             return launch_decode_mlp(x, m, H, I, w1, w1_s, w3, w3_s, w2, w2_s, pk1, pk2, w.h, y, s);
           }), "decode_mlp");
    return ok();
  }
  if (w.path == DENSE_SKINNY) {
    // up to 96 tokens: quantise x, stream the weights with the token rows as
    // operands, quantise h, stream w2
    MX_HIP(phase("skinny_mlp", s, [&] {
             return launch_skinny_mlp(x, m, H, I, w1, w1_s, w3, w3_s, w2, w2_s, pk1, pk2, w.xq, w.xs, w.h, w.hq,
                                      w.hs, y, s);
           }), "skinny_mlp");
    return ok();
  }

  const int mtiles = (m + BM - 1) / BM;
  const PackedWeights pw = packed_weights(hidden, inter, 1);
  MX_HIP(phase("quant_x", s, [&] {
           hipError_t e = launch_quant_mxfp4(x, M, hidden, w.xq, w.xs, s);
           if (e != hipSuccess) return e;
           return launch_pack_act_scales(w.xs, H, nullptr, nullptr, nullptr, 1, m, mtiles, w.xs_pk, s);
         }), "quant_x");

  GemmArgs l1 = base_args();
  l1.wa = w1; l1.wa_s = w1_s; l1.wb = w3; l1.wb_s = w3_s;
  l1.w_spk = packed_scales; l1.wspk_estride = pw.l1_estride;
  l1.w_cpk = packed_codes; l1.wcpk_estride = pc.l1_estride;
  l1.n_rows = I; l1.k = H;
  l1.x = w.xq; l1.x_s = w.xs_pk; l1.x_s_packed = 1;
  l1.m_rows = m; l1.n_experts = 1;
  l1.n_tiles = (I + L1_J_PER_TILE - 1) / L1_J_PER_TILE;
  l1.grid_tiles = mtiles * l1.n_tiles;
  l1.h_codes = w.hq; l1.h_scales = w.hs; l1.nv_gptr = requant_global;
  l1.h_scales_packed = requant == MX_FMT_MXFP4;
  l1.h_codes_tiled = requant == MX_FMT_MXFP4;
  const Epilogue l1_epi = requant == MX_FMT_NVFP4 ? EPI_SWIGLU_NVFP4 : EPI_SWIGLU_MXFP4;
  if (w.l1_split > 1) {
    // split-K: fp32 partials, then their sum through the same epilogue
    l1.k_splits = w.l1_split;
    l1.grid_tiles *= w.l1_split;
    l1.c_f32 = w.part;
    MX_HIP(phase("l1_gemm", s, [&] {
             hipError_t e = launch_gemm(EPI_PART_L1, l1, l1.grid_tiles, s);
             if (e != hipSuccess) return e;
             return launch_part_l1(l1, s);
           }), "l1_gemm");
  } else {
    MX_HIP(phase("l1_gemm", s, [&] { return launch_gemm(l1_epi, l1, l1.grid_tiles, s); }), "l1_gemm");
  }

  GemmArgs l2 = base_args();
  l2.wa = w2; l2.wa_s = w2_s;
  l2.w_spk = packed_scales ? packed_scales + pw.l1_bytes : nullptr; l2.wspk_estride = pw.l2_estride;
  l2.w_cpk = pk2; l2.wcpk_estride = pc.l2_estride;
  l2.n_rows = H; l2.k = I;
  l2.x = w.hq; l2.x_s = w.hs; l2.x_s_packed = requant == MX_FMT_MXFP4; l2.x_tiled = requant == MX_FMT_MXFP4;
  l2.m_rows = m; l2.n_experts = 1;
  l2.n_tiles = (H + BN - 1) / BN;
  l2.grid_tiles = mtiles * l2.n_tiles;
  l2.out_bf16 = y;
  if (requant == MX_FMT_NVFP4) {
    l2.nv_gptr = requant_global;
    MX_HIP(phase("l2_gemm_bf16", s, [&] { return launch_gemm_nv_l2(l2, l2.grid_tiles, s); }), "l2_gemm_bf16");
  } else {
    MX_HIP(phase("l2_gemm", s, [&] { return launch_gemm(EPI_BF16, l2, l2.grid_tiles, s); }), "l2_gemm");
  }
  return ok();
}

mx_status mx_grouped_expert_mlp(const uint16_t* x, int64_t T, int64_t hidden, int64_t inter,
                                const int32_t* topk_ids, const float* topk_w, int32_t k, int32_t E,
                                const uint8_t* w1, const uint8_t* w1_s, const uint8_t* w3, const uint8_t* w3_s,
                                const uint8_t* w2, const uint8_t* w2_s, const uint8_t* packed_scales,
                                const uint8_t* packed_codes, mx_format requant, const float* requant_global,
                                uint16_t* y, void* workspace, size_t ws_bytes, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  MX_TRY(check_mlp_dims(T, hidden, inter));
  MX_TRY(check_requant(requant, requant_global));
  if (E < 1 || E > ROUTE_MAX_EXPERTS) return fail(MX_ERR_SHAPE, "E %d outside [1, %d]", E, ROUTE_MAX_EXPERTS);
  if (k < 1 || k > E) return fail(MX_ERR_SHAPE, "k %d outside [1, E=%d]", k, E);
  if (T * (int64_t)k > ((int64_t)1 << 30)) return fail(MX_ERR_SHAPE, "T*k above 2^30");
  if (T == 0) return ok();
  MX_REQUIRE_PTR(x);
  MX_REQUIRE_PTR(y);
  MX_REQUIRE_PTR(topk_ids);
  MX_REQUIRE_PTR(topk_w);
  MX_REQUIRE_ALIGN(x, 16);
  MX_REQUIRE_ALIGN(y, 16);
  MX_REQUIRE_ALIGN(topk_ids, 4);
  MX_REQUIRE_ALIGN(topk_w, 4);
  MX_TRY(check_weights(w1, w1_s, w3, w3_s, w2, w2_s));
  MX_REQUIRE_ALIGN(packed_scales, 256);
  MX_REQUIRE_ALIGN(packed_codes, 256);
  const size_t need = mx_grouped_expert_mlp_workspace_size(T, hidden, inter, k, E, requant);
  MX_REQUIRE_PTR(workspace);
  MX_REQUIRE_ALIGN(workspace, 256);
  if (ws_bytes < need)
    return fail(MX_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  GroupWs w = group_ws(workspace, T, hidden, inter, k, E, requant);
  const int H = (int)hidden, I = (int)inter;
  const int64_t P = T * k;
  const int max_mtiles = (int)max_route_mtiles(P, E);
  const PackedWeights pw = packed_weights(hidden, inter, E);
  const PackedWeights pc = packed_codes_layout(hidden, inter, E);

  MX_HIP(phase("quant_x", s, [&] { return launch_quant_mxfp4(x, T, hidden, w.xq, w.xs, s); }), "quant_x");
  if (w.stream) {
    MX_HIP(phase("route", s, [&] { return launch_route(topk_ids, topk_w, T, k, E, w.rb, s); }), "route");
    RoutedArgs ra;
    ra.H = H; ra.I = I; ra.E = E;
    ra.xq = w.xq; ra.xs = w.xs;
    ra.row_token = w.rb.row_token; ra.row_slot = w.rb.row_slot; ra.expert_off = w.rb.expert_off;
    ra.row_weight = w.rb.row_weight;
    ra.w1 = w1; ra.w1s = w1_s; ra.w3 = w3; ra.w3s = w3_s; ra.w2 = w2; ra.w2s = w2_s;
    ra.pk1 = packed_codes; ra.pk1_estride = pc.l1_estride;
    ra.pk2 = packed_codes ? packed_codes + pc.l1_bytes : nullptr; ra.pk2_estride = pc.l2_estride;
    ra.h = w.h; ra.hq = w.hq; ra.hs = w.hs; ra.nvfp4 = requant == MX_FMT_NVFP4;
    ra.scale = 1.0f;
    ra.scale_ptr = requant == MX_FMT_NVFP4 ? requant_global : nullptr;
    ra.o = w.o;
    MX_HIP(phase("l1_stream", s, [&] { return launch_routed_l1(ra, s); }), "l1_stream");
    MX_HIP(phase("requant_h", s, [&] {
             if (requant == MX_FMT_MXFP4) return launch_quant_mxfp4(w.h, P, inter, w.hq, w.hs, s);
             return launch_quant_nvfp4(w.h, P, inter, 0.0f, requant_global, w.hq, w.hs, s);
           }), "requant_h");
    MX_HIP(phase("l2_stream", s, [&] { return launch_routed_l2(ra, s); }), "l2_stream");
    MX_HIP(phase("combine", s, [&] { return launch_combine(w.o, topk_ids, T, k, E, H, y, s); }), "combine");
    return ok();
  }
  MX_HIP(phase("route", s, [&] {
           hipError_t e = launch_route(topk_ids, topk_w, T, k, E, w.rb, s);
           if (e != hipSuccess) return e;
           return launch_pack_act_scales(w.xs, H, w.rb.row_token, w.rb.expert_off, w.rb.tile_base, E, 0,
                                         max_mtiles, w.xs_pk, s);
         }), "route");

  GemmArgs l1 = base_args();
  l1.wa = w1; l1.wa_s = w1_s; l1.wb = w3; l1.wb_s = w3_s;
  l1.w_estride = (int64_t)I * H / 2; l1.ws_estride = (int64_t)I * H / 32;
  l1.w_spk = packed_scales; l1.wspk_estride = pw.l1_estride;
  l1.w_cpk = packed_codes; l1.wcpk_estride = pc.l1_estride;
  l1.n_rows = I; l1.k = H;
  l1.x = w.xq; l1.x_s = w.xs_pk; l1.x_s_packed = 1; l1.row_token = w.rb.row_token;
  l1.expert_off = w.rb.expert_off; l1.tile_base = w.rb.tile_base; l1.n_experts = E;
  l1.n_tiles = (I + L1_J_PER_TILE - 1) / L1_J_PER_TILE;
  l1.h_codes = w.hq; l1.h_scales = w.hs; l1.nv_gptr = requant_global;
  l1.h_scales_packed = requant == MX_FMT_MXFP4;
  l1.h_codes_tiled = requant == MX_FMT_MXFP4;
  const Epilogue l1_epi = requant == MX_FMT_NVFP4 ? EPI_SWIGLU_NVFP4 : EPI_SWIGLU_MXFP4;
  MX_HIP(phase("l1_gemm", s, [&] { return launch_gemm(l1_epi, l1, max_mtiles * l1.n_tiles, s); }), "l1_gemm");

  GemmArgs l2 = base_args();
  l2.wa = w2; l2.wa_s = w2_s;
  l2.w_estride = (int64_t)H * I / 2; l2.ws_estride = (int64_t)H * I / 32;
  l2.w_spk = packed_scales ? packed_scales + pw.l1_bytes : nullptr; l2.wspk_estride = pw.l2_estride;
  l2.w_cpk = packed_codes ? packed_codes + pc.l1_bytes : nullptr; l2.wcpk_estride = pc.l2_estride;
  l2.n_rows = H; l2.k = I;
  l2.x = w.hq; l2.x_s = w.hs; l2.x_s_packed = requant == MX_FMT_MXFP4; l2.x_tiled = requant == MX_FMT_MXFP4;
  l2.expert_off = w.rb.expert_off; l2.tile_base = w.rb.tile_base; l2.n_experts = E;
  l2.n_tiles = (H + BN - 1) / BN;
  l2.out_bf16 = w.o; l2.row_slot = w.rb.row_slot; l2.row_weight = w.rb.row_weight;
  if (requant == MX_FMT_NVFP4) {
    l2.nv_gptr = requant_global;
    MX_HIP(phase("l2_gemm_bf16", s, [&] { return launch_gemm_nv_l2(l2, max_mtiles * l2.n_tiles, s); }),
           "l2_gemm_bf16");
  } else {
    MX_HIP(phase("l2_gemm", s, [&] { return launch_gemm(EPI_BF16, l2, max_mtiles * l2.n_tiles, s); }), "l2_gemm");
  }

  MX_HIP(phase("combine", s, [&] { return launch_combine(w.o, topk_ids, T, k, E, H, y, s); }), "combine");
  return ok();
}

}  // extern "C"

namespace {

// NVFP4 warm-up workspace: the L1 inputs and outputs of the MXFP4 path (no L2
// rows), then the |h| max word. k == 0: one expert, T token rows.
struct WarmWs {
  uint8_t *xq, *xs, *hq, *hs, *xs_pk;
  RouteBuffers rb;
  uint32_t* amax;
  size_t bytes;
};
WarmWs warm_ws(void* base, int64_t T, int64_t H, int64_t I, int k, int E) {
  Carve c(base);
  WarmWs w;
  memset(&w, 0, sizeof(w));
  const bool routed = k > 0;
  const int64_t P = routed ? T * k : T;
  const int64_t mtiles = routed ? max_route_mtiles(P, E) : (T + BM - 1) / BM;
  w.xq = (uint8_t*)c.take((size_t)(T * H / 2));
  w.xs = (uint8_t*)c.take((size_t)(T * H / 32));
  if (routed) {
    const int64_t nblocks = (P + ROUTE_CHUNK - 1) / ROUTE_CHUNK;
    w.rb.block_counts = (int32_t*)c.take((size_t)(nblocks * E * 4));
    w.rb.expert_off = (int32_t*)c.take((size_t)(E + 1) * 4);
    w.rb.tile_base = (int32_t*)c.take((size_t)(E + 1) * 4);
    w.rb.row_token = (int32_t*)c.take((size_t)P * 4);
    w.rb.row_slot = (int32_t*)c.take((size_t)P * 4);
    w.rb.row_weight = (float*)c.take((size_t)P * 4);
  }
  w.hq = (uint8_t*)c.take((size_t)(P * I / 2));
  w.hs = (uint8_t*)c.take((size_t)packed_scale_bytes(mtiles, I));
  w.xs_pk = (uint8_t*)c.take((size_t)packed_scale_bytes(mtiles, H));
  w.amax = (uint32_t*)c.take(4);
  w.bytes = c.off;
  return w;
}

}  // namespace

extern "C" {

size_t mx_nvfp4_global_warmup_workspace_size(int64_t T, int64_t hidden, int64_t inter, int32_t k, int32_t E) {
  if (T < 0 || hidden < 0 || inter < 0 || k < 0 || (k > 0 && E < 1)) return 0;
  return warm_ws(nullptr, T, hidden, inter, k, E).bytes;
}

mx_status mx_nvfp4_global_warmup(const uint16_t* x, int64_t T, int64_t hidden, int64_t inter,
                                 const int32_t* topk_ids, const float* topk_w, int32_t k, int32_t E,
                                 const uint8_t* w1, const uint8_t* w1_s, const uint8_t* w3, const uint8_t* w3_s,
                                 const uint8_t* packed_scales, float* global_out, void* workspace, size_t ws_bytes,
                                 void* stream) {
  hipStream_t s = (hipStream_t)stream;
  MX_TRY(check_mlp_dims(T, hidden, inter));
  const bool routed = topk_ids != nullptr;
  if (routed) {
    if (E < 1 || E > ROUTE_MAX_EXPERTS) return fail(MX_ERR_SHAPE, "E %d outside [1, %d]", E, ROUTE_MAX_EXPERTS);
    if (k < 1 || k > E) return fail(MX_ERR_SHAPE, "k %d outside [1, E=%d]", k, E);
    if (T * (int64_t)k > ((int64_t)1 << 30)) return fail(MX_ERR_SHAPE, "T*k above 2^30");
    MX_REQUIRE_PTR(topk_w);
    MX_REQUIRE_ALIGN(topk_ids, 4);
    MX_REQUIRE_ALIGN(topk_w, 4);
  } else if (k != 0) {
    return fail(MX_ERR_SHAPE, "k %d: without topk_ids (one expert) k must be 0", k);
  }
  MX_REQUIRE_PTR(global_out);
  MX_REQUIRE_ALIGN(global_out, 4);
  MX_REQUIRE_PTR(w1);
  MX_REQUIRE_PTR(w1_s);
  MX_REQUIRE_PTR(w3);
  MX_REQUIRE_PTR(w3_s);
  MX_REQUIRE_ALIGN(w1, 16);
  MX_REQUIRE_ALIGN(w3, 16);
  MX_REQUIRE_ALIGN(w1_s, 4);
  MX_REQUIRE_ALIGN(w3_s, 4);
  MX_REQUIRE_ALIGN(packed_scales, 256);
  if (T > 0) {
    MX_REQUIRE_PTR(x);
    MX_REQUIRE_ALIGN(x, 16);
  }
  const size_t need = mx_nvfp4_global_warmup_workspace_size(T, hidden, inter, routed ? k : 0, routed ? E : 1);
  MX_REQUIRE_PTR(workspace);
  MX_REQUIRE_ALIGN(workspace, 256);
  if (ws_bytes < need)
    return fail(MX_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  const int ne = routed ? E : 1;
  WarmWs w = warm_ws(workspace, T, hidden, inter, routed ? k : 0, ne);
  const int H = (int)hidden, I = (int)inter;
  MX_HIP(launch_amax_clear(w.amax, s), "amax_clear");
  if (T > 0) {
    const int64_t P = routed ? T * k : T;
    const int mtiles = routed ? (int)max_route_mtiles(P, ne) : (int)((T + BM - 1) / BM);
    MX_HIP(launch_quant_mxfp4(x, T, hidden, w.xq, w.xs, s), "quant_x");
    if (routed) {
      MX_HIP(launch_route(topk_ids, topk_w, T, k, E, w.rb, s), "route");
      MX_HIP(launch_pack_act_scales(w.xs, H, w.rb.row_token, w.rb.expert_off, w.rb.tile_base, E, 0, mtiles, w.xs_pk,
                                    s), "pack_act_scales");
    } else {
      MX_HIP(launch_pack_act_scales(w.xs, H, nullptr, nullptr, nullptr, 1, (int)T, mtiles, w.xs_pk, s),
             "pack_act_scales");
    }
    const PackedWeights pw = packed_weights(hidden, inter, ne);
    GemmArgs l1 = base_args();
    l1.wa = w1; l1.wa_s = w1_s; l1.wb = w3; l1.wb_s = w3_s;
    l1.w_estride = (int64_t)I * H / 2; l1.ws_estride = (int64_t)I * H / 32;
    l1.w_spk = packed_scales; l1.wspk_estride = pw.l1_estride;
    l1.n_rows = I; l1.k = H;
    l1.x = w.xq; l1.x_s = w.xs_pk; l1.x_s_packed = 1;
    l1.n_tiles = (I + L1_J_PER_TILE - 1) / L1_J_PER_TILE;
    l1.h_codes = w.hq; l1.h_scales = w.hs; l1.h_scales_packed = 1;
    l1.h_amax = w.amax;
    if (routed) {
      l1.row_token = w.rb.row_token;
      l1.expert_off = w.rb.expert_off; l1.tile_base = w.rb.tile_base; l1.n_experts = E;
    } else {
      l1.m_rows = (int)T; l1.n_experts = 1;
      l1.grid_tiles = mtiles * l1.n_tiles;
    }
    MX_HIP(launch_gemm(EPI_SWIGLU_MXFP4, l1, mtiles * l1.n_tiles, s), "l1_gemm");
  }
  MX_HIP(launch_nvfp4_global(w.amax, global_out, s), "nvfp4_global");
  return ok();
}

size_t mx_fp8_block_linear_workspace_size(int64_t M, int64_t K) {
  if (M < 0 || K < 0) return 0;
  Carve c(nullptr);
  c.take((size_t)(M * K));
  c.take((size_t)(M * (K / 32)));
  return c.off;
}

mx_status mx_fp8_block_linear(const uint16_t* x, int64_t M, int64_t K, const uint8_t* w, const uint8_t* w_s,
                              int64_t N, uint16_t* y, void* workspace, size_t ws_bytes, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (M < 0 || K < 0 || N < 0) return fail(MX_ERR_SHAPE, "negative size");
  if (K < 128 || K % 128 != 0) return fail(MX_ERR_SHAPE, "K %lld must be a positive multiple of 128", (long long)K);
  if (!fp8_linear_fits(K)) return fail(MX_ERR_SHAPE, "K %lld above 8192", (long long)K);
  if (N < 128 || N % 128 != 0) return fail(MX_ERR_SHAPE, "N %lld must be a positive multiple of 128", (long long)N);
  if (N > (1 << 20) || M > ((int64_t)1 << 30) || M * K > ((int64_t)1 << 40) || M * N > ((int64_t)1 << 40))
    return fail(MX_ERR_SHAPE, "matrix too large");
  if (M == 0) return ok();
  MX_REQUIRE_PTR(x);
  MX_REQUIRE_PTR(w);
  MX_REQUIRE_PTR(w_s);
  MX_REQUIRE_PTR(y);
  MX_REQUIRE_ALIGN(x, 16);
  MX_REQUIRE_ALIGN(w, 16);
  MX_REQUIRE_ALIGN(y, 16);
  MX_REQUIRE_PTR(workspace);
  MX_REQUIRE_ALIGN(workspace, 256);
  const size_t need = mx_fp8_block_linear_workspace_size(M, K);
  if (ws_bytes < need) return fail(MX_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  Carve c(workspace);
  uint8_t* xq = (uint8_t*)c.take((size_t)(M * K));
  uint8_t* xs = (uint8_t*)c.take((size_t)(M * (K / 32)));
  MX_HIP(phase("quant_x8", s, [&] { return launch_quant_mxfp8(x, M, K, xq, xs, s); }), "quant_x8");
  MX_HIP(phase("fp8_gemm", s, [&] { return launch_fp8_gemm(xq, xs, w, w_s, (int)M, (int)N, (int)K, y, s); }),
         "fp8_gemm");
  return ok();
}

size_t mx_nvfp4_linear_workspace_size(int64_t M, int64_t K) {
  if (M < 0 || K < 0) return 0;
  Carve c(nullptr);
  c.take((size_t)(M * K / 2));
  c.take((size_t)(M * (K / 16)));
  return c.off;
}

mx_status mx_nvfp4_linear(const uint16_t* x, int64_t M, int64_t K, const uint8_t* w, const uint8_t* w_s,
                          float w_global, int64_t N, float x_global, uint16_t* y, void* workspace, size_t ws_bytes,
                          void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (M < 0 || K < 0 || N < 0) return fail(MX_ERR_SHAPE, "negative size");
  if (K < 128 || K % 128 != 0) return fail(MX_ERR_SHAPE, "K %lld must be a positive multiple of 128", (long long)K);
  if (N < 128 || N % 128 != 0) return fail(MX_ERR_SHAPE, "N %lld must be a positive multiple of 128", (long long)N);
  if (K > (1 << 20) || N > (1 << 20) || M > ((int64_t)1 << 30) || M * K > ((int64_t)1 << 40))
    return fail(MX_ERR_SHAPE, "matrix too large");
  MX_TRY(check_global(x_global));
  if (!std::isfinite(w_global) || !(w_global > 0.f))
    return fail(MX_ERR_VALUE, "weight global scale %g must be finite and positive", (double)w_global);
  const float g = x_global * w_global;
  if (!std::isfinite(g)) return fail(MX_ERR_VALUE, "product of the global scales overflows");
  if (M == 0) return ok();
  MX_REQUIRE_PTR(x);
  MX_REQUIRE_PTR(w);
  MX_REQUIRE_PTR(w_s);
  MX_REQUIRE_PTR(y);
  MX_REQUIRE_ALIGN(x, 16);
  MX_REQUIRE_ALIGN(w, 16);
  MX_REQUIRE_ALIGN(w_s, 2);
  MX_REQUIRE_ALIGN(y, 16);
  MX_REQUIRE_PTR(workspace);
  MX_REQUIRE_ALIGN(workspace, 256);
  const size_t need = mx_nvfp4_linear_workspace_size(M, K);
  if (ws_bytes < need) return fail(MX_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  Carve c(workspace);
  uint8_t* xq = (uint8_t*)c.take((size_t)(M * K / 2));
  uint8_t* xs = (uint8_t*)c.take((size_t)(M * (K / 16)));
  MX_HIP(phase("quant_nvfp4", s, [&] { return launch_quant_nvfp4(x, M, K, x_global, nullptr, xq, xs, s); }), "quant_x");
  GemmArgs a = base_args();
  a.wa = w; a.wa_s = w_s;
  a.n_rows = (int)N; a.k = (int)K;
  a.x = xq; a.x_s = xs;
  a.m_rows = (int)M; a.n_experts = 1;
  a.n_tiles = (int)((N + BN - 1) / BN);
  a.grid_tiles = (int)((M + BM - 1) / BM) * a.n_tiles;
  a.out_bf16 = y;
  a.nv_global = g;
  MX_HIP(phase("nv_gemm", s, [&] { return launch_gemm_nv_w(a, a.grid_tiles, s); }), "nv_gemm");
  return ok();
}

size_t mx_nvfp4_expert_mlp_workspace_size(int64_t M, int64_t hidden, int64_t inter) {
  if (M < 0 || hidden < 0 || inter < 0) return 0;
  Carve c(nullptr);
  c.take((size_t)(M * hidden / 2));
  c.take((size_t)(M * (hidden / 16)));
  c.take((size_t)(M * inter / 2));
  c.take((size_t)(M * (inter / 16)));
  return c.off;
}

mx_status mx_nvfp4_expert_mlp(const uint16_t* x, int64_t M, int64_t hidden, int64_t inter, const uint8_t* w1,
                              const uint8_t* w1_s, float w1_global, const uint8_t* w3, const uint8_t* w3_s,
                              float w3_global, const uint8_t* w2, const uint8_t* w2_s, float w2_global,
                              float x_global, float h_global, uint16_t* y, void* workspace, size_t ws_bytes,
                              void* stream) {
  hipStream_t s = (hipStream_t)stream;
  MX_TRY(check_mlp_dims(M, hidden, inter));
  if (M * hidden > ((int64_t)1 << 40) || M * inter > ((int64_t)1 << 40)) return fail(MX_ERR_SHAPE, "matrix too large");
  MX_TRY(check_global(x_global));
  MX_TRY(check_global(h_global));
  const float wg[3] = {w1_global, w3_global, w2_global};
  for (int i = 0; i < 3; ++i)
    if (!std::isfinite(wg[i]) || !(wg[i] > 0.f) || !std::isfinite(wg[i] * (i < 2 ? x_global : h_global)))
      return fail(MX_ERR_VALUE, "weight global scale %d (%g) must be finite and positive, and its product "
                                "with the activation global finite", i, (double)wg[i]);
  if (M == 0) return ok();
  MX_REQUIRE_PTR(x);
  MX_REQUIRE_PTR(y);
  MX_REQUIRE_ALIGN(x, 16);
  MX_REQUIRE_ALIGN(y, 16);
  const uint8_t* wp[6] = {w1, w1_s, w3, w3_s, w2, w2_s};
  for (int i = 0; i < 6; ++i) {
    if (wp[i] == nullptr) return fail(MX_ERR_NULL, "NVFP4 weight or scale pointer %d is NULL", i);
    if (!aligned(wp[i], i % 2 ? 2 : 16)) return fail(MX_ERR_ALIGN, "NVFP4 weight or scale pointer %d misaligned", i);
  }
  MX_REQUIRE_PTR(workspace);
  MX_REQUIRE_ALIGN(workspace, 256);
  const size_t need = mx_nvfp4_expert_mlp_workspace_size(M, hidden, inter);
  if (ws_bytes < need) return fail(MX_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  Carve c(workspace);
  uint8_t* xq = (uint8_t*)c.take((size_t)(M * hidden / 2));
  uint8_t* xs = (uint8_t*)c.take((size_t)(M * (hidden / 16)));
  uint8_t* hq = (uint8_t*)c.take((size_t)(M * inter / 2));
  uint8_t* hs = (uint8_t*)c.take((size_t)(M * (inter / 16)));
  auto gemm = [&](const uint8_t* aq, const uint8_t* as, const uint8_t* w, const uint8_t* ws, int64_t N, int64_t K,
                  float gscale, uint16_t* out) {
    GemmArgs a = base_args();
    a.wa = w; a.wa_s = ws;
    a.n_rows = (int)N; a.k = (int)K;
    a.x = aq; a.x_s = as;
    a.m_rows = (int)M; a.n_experts = 1;
    a.n_tiles = (int)((N + BN - 1) / BN);
    a.grid_tiles = (int)((M + BM - 1) / BM) * a.n_tiles;
    a.out_bf16 = out;
    a.nv_global = gscale;
    return launch_gemm_nv_w(a, a.grid_tiles, s);
  };
  MX_HIP(phase("quant_nvfp4", s, [&] { return launch_quant_nvfp4(x, M, hidden, x_global, nullptr, xq, xs, s); }), "quant_x");
  // gate and up in one GEMM whose epilogue forms h and re-quantises it
  GemmArgs l1 = base_args();
  l1.wa = w1; l1.wa_s = w1_s; l1.wb = w3; l1.wb_s = w3_s;
  l1.n_rows = (int)inter; l1.k = (int)hidden;
  l1.x = xq; l1.x_s = xs;
  l1.m_rows = (int)M; l1.n_experts = 1;
  l1.n_tiles = (int)((inter + L1_J_PER_TILE - 1) / L1_J_PER_TILE);
  l1.grid_tiles = (int)((M + BM - 1) / BM) * l1.n_tiles;
  l1.nv_global = x_global * w1_global; l1.nv_global2 = x_global * w3_global;
  l1.h_codes = hq; l1.h_scales = hs; l1.h_nv_global = h_global;
  MX_HIP(phase("nv_gemm_swiglu", s, [&] { return launch_gemm_nv_w_swiglu(l1, l1.grid_tiles, s); }), "nv_gemm_l1");
  MX_HIP(phase("nv_gemm", s, [&] { return gemm(hq, hs, w2, w2_s, hidden, inter, h_global * w2_global, y); }),
         "nv_gemm_l2");
  return ok();
}

namespace {
// Routed NVFP4-weight workspace: xq, xs (per token), the route buffers, the
// gathered xq/xs (sorted rows), hq, hs (the fused gate/up GEMM's NVFP4 h), o
// (per pair row).
struct NvGroupWs {
  uint8_t *xq, *xs, *gq, *gs, *hq, *hs;
  uint16_t* o;
  RouteBuffers rb;
  size_t bytes;
};
NvGroupWs nv_group_ws(void* base, int64_t T, int64_t H, int64_t I, int k, int E) {
  Carve c(base);
  NvGroupWs w;
  const int64_t P = T * k;
  const int64_t nblocks = (P + ROUTE_CHUNK - 1) / ROUTE_CHUNK;
  w.xq = (uint8_t*)c.take((size_t)(T * H / 2));
  w.xs = (uint8_t*)c.take((size_t)(T * H / 16));
  w.rb.block_counts = (int32_t*)c.take((size_t)(nblocks * E * 4));
  w.rb.expert_off = (int32_t*)c.take((size_t)(E + 1) * 4);
  w.rb.tile_base = (int32_t*)c.take((size_t)(E + 1) * 4);
  w.rb.row_token = (int32_t*)c.take((size_t)P * 4);
  w.rb.row_slot = (int32_t*)c.take((size_t)P * 4);
  w.rb.row_weight = (float*)c.take((size_t)P * 4);
  w.gq = (uint8_t*)c.take((size_t)(P * H / 2));
  w.gs = (uint8_t*)c.take((size_t)(P * H / 16));
  w.hq = (uint8_t*)c.take((size_t)(P * I / 2));
  w.hs = (uint8_t*)c.take((size_t)(P * I / 16));
  w.o = (uint16_t*)c.take((size_t)(P * H * 2));
  w.bytes = c.off;
  return w;
}
}  // namespace

size_t mx_grouped_nvfp4_expert_mlp_workspace_size(int64_t T, int64_t hidden, int64_t inter, int32_t k, int32_t E) {
  if (T < 0 || hidden < 0 || inter < 0 || k < 1 || E < 1) return 0;
  return nv_group_ws(nullptr, T, hidden, inter, k, E).bytes;
}

mx_status mx_grouped_nvfp4_expert_mlp(const uint16_t* x, int64_t T, int64_t hidden, int64_t inter,
                                      const int32_t* topk_ids, const float* topk_w, int32_t k, int32_t E,
                                      const uint8_t* w1, const uint8_t* w1_s, const float* w1_global,
                                      const uint8_t* w3, const uint8_t* w3_s, const float* w3_global,
                                      const uint8_t* w2, const uint8_t* w2_s, const float* w2_global,
                                      float x_global, float h_global, uint16_t* y, void* workspace,
                                      size_t ws_bytes, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  MX_TRY(check_mlp_dims(T, hidden, inter));
  MX_TRY(check_global(x_global));
  MX_TRY(check_global(h_global));
  if (E < 1 || E > ROUTE_MAX_EXPERTS) return fail(MX_ERR_SHAPE, "E %d outside [1, %d]", E, ROUTE_MAX_EXPERTS);
  if (k < 1 || k > E) return fail(MX_ERR_SHAPE, "k %d outside [1, E=%d]", k, E);
  if (T * (int64_t)k > ((int64_t)1 << 30)) return fail(MX_ERR_SHAPE, "T*k above 2^30");
  if (T == 0) return ok();
  MX_REQUIRE_PTR(x);
  MX_REQUIRE_PTR(y);
  MX_REQUIRE_PTR(topk_ids);
  MX_REQUIRE_PTR(topk_w);
  MX_REQUIRE_ALIGN(x, 16);
  MX_REQUIRE_ALIGN(y, 16);
  MX_REQUIRE_ALIGN(topk_ids, 4);
  MX_REQUIRE_ALIGN(topk_w, 4);
  const uint8_t* wp[6] = {w1, w1_s, w3, w3_s, w2, w2_s};
  for (int i = 0; i < 6; ++i) {
    if (wp[i] == nullptr) return fail(MX_ERR_NULL, "NVFP4 weight or scale pointer %d is NULL", i);
    if (!aligned(wp[i], i % 2 ? 2 : 16)) return fail(MX_ERR_ALIGN, "NVFP4 weight or scale pointer %d misaligned", i);
  }
  MX_REQUIRE_PTR(w1_global);
  MX_REQUIRE_PTR(w3_global);
  MX_REQUIRE_PTR(w2_global);
  MX_REQUIRE_ALIGN(w1_global, 4);
  MX_REQUIRE_ALIGN(w3_global, 4);
  MX_REQUIRE_ALIGN(w2_global, 4);
  MX_REQUIRE_PTR(workspace);
  MX_REQUIRE_ALIGN(workspace, 256);
  const size_t need = mx_grouped_nvfp4_expert_mlp_workspace_size(T, hidden, inter, k, E);
  if (ws_bytes < need) return fail(MX_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  NvGroupWs w = nv_group_ws(workspace, T, hidden, inter, k, E);
  const int64_t P = T * k;
  const int max_mtiles = (int)max_route_mtiles(P, E);
  MX_HIP(phase("quant_nvfp4", s, [&] { return launch_quant_nvfp4(x, T, hidden, x_global, nullptr, w.xq, w.xs, s); }),
         "quant_x");
  MX_HIP(phase("route", s, [&] {
           hipError_t e = launch_route(topk_ids, topk_w, T, k, E, w.rb, s);
           if (e != hipSuccess) return e;
           e = launch_gather_rows(w.xq, (int)(hidden / 2), w.rb.row_token, w.rb.expert_off + E, P, w.gq, s);
           if (e != hipSuccess) return e;
           return launch_gather_rows(w.xs, (int)(hidden / 16), w.rb.row_token, w.rb.expert_off + E, P, w.gs, s);
         }), "route");
  auto gemm = [&](const uint8_t* aq, const uint8_t* as, const uint8_t* wc, const uint8_t* wsc, const float* eg,
                  int64_t N, int64_t K, float gscale, uint16_t* out, bool pairs) {
    GemmArgs a = base_args();
    a.wa = wc; a.wa_s = wsc;
    a.w_estride = N * K / 2; a.ws_estride = N * K / 16;
    a.n_rows = (int)N; a.k = (int)K;
    a.x = aq; a.x_s = as;
    a.expert_off = w.rb.expert_off; a.tile_base = w.rb.tile_base; a.n_experts = E;
    a.n_tiles = (int)((N + BN - 1) / BN);
    a.out_bf16 = out;
    if (pairs) {
      a.row_slot = w.rb.row_slot;
      a.row_weight = w.rb.row_weight;
    }
    a.nv_global = gscale;
    a.e_global = eg;
    return launch_gemm_nv_w(a, max_mtiles * a.n_tiles, s);
  };
  // gate and up in one GEMM whose epilogue forms h and re-quantises it
  GemmArgs l1 = base_args();
  l1.wa = w1; l1.wa_s = w1_s; l1.wb = w3; l1.wb_s = w3_s;
  l1.w_estride = inter * hidden / 2; l1.ws_estride = inter * hidden / 16;
  l1.n_rows = (int)inter; l1.k = (int)hidden;
  l1.x = w.gq; l1.x_s = w.gs;
  l1.expert_off = w.rb.expert_off; l1.tile_base = w.rb.tile_base; l1.n_experts = E;
  l1.n_tiles = (int)((inter + L1_J_PER_TILE - 1) / L1_J_PER_TILE);
  l1.nv_global = x_global; l1.e_global = w1_global;
  l1.nv_global2 = x_global; l1.e_global2 = w3_global;
  l1.h_codes = w.hq; l1.h_scales = w.hs; l1.h_nv_global = h_global;
  MX_HIP(phase("nv_gemm_swiglu", s, [&] { return launch_gemm_nv_w_swiglu(l1, max_mtiles * l1.n_tiles, s); }),
         "nv_gemm_l1");
  MX_HIP(phase("nv_gemm", s, [&] {
           return gemm(w.hq, w.hs, w2, w2_s, w2_global, hidden, inter, h_global, w.o, true);
         }), "nv_gemm_l2");
  MX_HIP(phase("combine", s, [&] { return launch_combine(w.o, topk_ids, T, k, E, (int)hidden, y, s); }), "combine");
  return ok();
}

size_t mx_fp8_expert_mlp_workspace_size(int64_t M, int64_t hidden, int64_t inter) {
  if (M < 0 || hidden < 0 || inter < 0) return 0;
  Carve c(nullptr);
  c.take((size_t)(M * hidden));
  c.take((size_t)(M * (hidden / 32)));
  c.take((size_t)(M * inter * 2));   // h
  c.take((size_t)(M * inter));
  c.take((size_t)(M * (inter / 32)));
  return c.off;
}

mx_status mx_fp8_expert_mlp(const uint16_t* x, int64_t M, int64_t hidden, int64_t inter, const uint8_t* w1,
                            const uint8_t* w1_s, const uint8_t* w3, const uint8_t* w3_s, const uint8_t* w2,
                            const uint8_t* w2_s, uint16_t* y, void* workspace, size_t ws_bytes, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  MX_TRY(check_mlp_dims(M, hidden, inter));
  if (!fp8_linear_fits(hidden) || !fp8_linear_fits(inter))
    return fail(MX_ERR_SHAPE, "hidden %lld / inter %lld above 8192", (long long)hidden, (long long)inter);
  if (M * hidden > ((int64_t)1 << 40) || M * inter > ((int64_t)1 << 40)) return fail(MX_ERR_SHAPE, "matrix too large");
  if (M == 0) return ok();
  MX_REQUIRE_PTR(x);
  MX_REQUIRE_PTR(y);
  MX_REQUIRE_ALIGN(x, 16);
  MX_REQUIRE_ALIGN(y, 16);
  const uint8_t* wp[6] = {w1, w1_s, w3, w3_s, w2, w2_s};
  for (int i = 0; i < 6; ++i)
    if (wp[i] == nullptr) return fail(MX_ERR_NULL, "FP8 weight or scale pointer %d is NULL", i);
  MX_REQUIRE_ALIGN(w1, 16);
  MX_REQUIRE_ALIGN(w3, 16);
  MX_REQUIRE_ALIGN(w2, 16);
  MX_REQUIRE_PTR(workspace);
  MX_REQUIRE_ALIGN(workspace, 256);
  const size_t need = mx_fp8_expert_mlp_workspace_size(M, hidden, inter);
  if (ws_bytes < need) return fail(MX_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  Carve c(workspace);
  uint8_t* xq = (uint8_t*)c.take((size_t)(M * hidden));
  uint8_t* xs = (uint8_t*)c.take((size_t)(M * (hidden / 32)));
  uint16_t* h = (uint16_t*)c.take((size_t)(M * inter * 2));
  uint8_t* hq = (uint8_t*)c.take((size_t)(M * inter));
  uint8_t* hs = (uint8_t*)c.take((size_t)(M * (inter / 32)));
  const int m = (int)M, H = (int)hidden, I = (int)inter;
  MX_HIP(phase("quant_x8", s, [&] { return launch_quant_mxfp8(x, M, hidden, xq, xs, s); }), "quant_x8");
  // gate and up in one GEMM whose epilogue applies SiLU * up to their bf16 outputs
  MX_HIP(phase("fp8_swiglu", s, [&] { return launch_fp8_swiglu(xq, xs, w1, w1_s, w3, w3_s, m, I, H, h, s); }),
         "fp8_swiglu");
  MX_HIP(phase("quant_x8", s, [&] { return launch_quant_mxfp8(h, M, inter, hq, hs, s); }), "quant_h8");
  MX_HIP(phase("fp8_gemm", s, [&] { return launch_fp8_gemm(hq, hs, w2, w2_s, m, H, I, y, s); }), "fp8_gemm_l2");
  return ok();
}

mx_status mx_debug_gemm_f32(const uint8_t* a, const uint8_t* a_s, const uint8_t* b, const uint8_t* b_s,
                            int64_t M, int64_t N, int64_t K, float* c, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (M < 0 || N < 0 || K < 0) return fail(MX_ERR_SHAPE, "negative size");
  if (K < 128 || K % 128 != 0) return fail(MX_ERR_SHAPE, "K %lld must be a positive multiple of 128", (long long)K);
  if (N % 4 != 0) return fail(MX_ERR_SHAPE, "N %lld %% 4 != 0", (long long)N);
  if (M > ((int64_t)1 << 30) || N > ((int64_t)1 << 30) || K > (1 << 20)) return fail(MX_ERR_SHAPE, "too large");
  if (M == 0 || N == 0) return ok();
  MX_REQUIRE_PTR(a);
  MX_REQUIRE_PTR(a_s);
  MX_REQUIRE_PTR(b);
  MX_REQUIRE_PTR(b_s);
  MX_REQUIRE_PTR(c);
  MX_REQUIRE_ALIGN(a, 16);
  MX_REQUIRE_ALIGN(b, 16);
  MX_REQUIRE_ALIGN(c, 16);
  MX_REQUIRE_ALIGN(a_s, 4);
  MX_REQUIRE_ALIGN(b_s, 4);
  GemmArgs g = base_args();
  g.wa = b; g.wa_s = b_s;
  g.n_rows = (int)N; g.k = (int)K;
  g.x = a; g.x_s = a_s;
  g.m_rows = (int)M; g.n_experts = 1;
  g.n_tiles = (int)((N + BN - 1) / BN);
  g.grid_tiles = (int)((M + BM - 1) / BM) * g.n_tiles;
  g.c_f32 = c;
  MX_HIP(phase("debug_gemm", s, [&] { return launch_gemm(EPI_F32, g, g.grid_tiles, s); }), "debug_gemm");
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------- no-allocation entry point
// mx_expert_mlp_noalloc runs mx_expert_mlp on a file-scope device array instead
// of a caller workspace, for callers that cannot allocate device memory. Each
// device holds its own copy of the array (64 MiB, for as long as the process
// runs); its address on a device is looked up once, with that device current,
// and kept. Host code never passes `scratch` itself to a kernel: in host code
// the name is a stand-in, not a device address.
namespace {

constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES];

// The current device's copy of `scratch`, looked up on its first use.
mx_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return fail(MX_ERR_HIP, "device %d above the supported %d", dev,
                                                         NOALLOC_MAX_DEVICES);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(MX_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MX_OK;
}

}  // namespace

extern "C" {

size_t mx_expert_mlp_noalloc_max_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

mx_status mx_expert_mlp_noalloc(const uint16_t* x, int64_t M, int64_t hidden, int64_t inter, const uint8_t* w1,
                                const uint8_t* w1_s, const uint8_t* w3, const uint8_t* w3_s, const uint8_t* w2,
                                const uint8_t* w2_s, const uint8_t* packed_scales, const uint8_t* packed_codes,
                                mx_format requant, const float* requant_global, uint16_t* y, void* stream) {
  MX_TRY(check_mlp_dims(M, hidden, inter));
  MX_TRY(check_requant(requant, requant_global));
  if (M == 0) return ok();
  const size_t need = mx_expert_mlp_workspace_size(M, hidden, inter, requant);
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(MX_ERR_WORKSPACE,
                "M %lld, hidden %lld, inter %lld need %zu bytes of scratch, above the %zu bytes of the "
                "no-allocation entry point (use mx_expert_mlp with a workspace)",
                (long long)M, (long long)hidden, (long long)inter, need, NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  MX_TRY(scratch_ptr(&ws));
  return mx_expert_mlp(x, M, hidden, inter, w1, w1_s, w3, w3_s, w2, w2_s, packed_scales, packed_codes, requant,
                       requant_global, y, ws, NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- runner
// Routed-expert runner: workspace allocated once, the whole call captured once
// into a hipGraph and replayed. The pages' serving plan is a runner with
// pre-allocated buffers whose calls are CUDA-graph safe (page "Current Bug:
// vLLM produces empty/garbage output", section "Revised Plan", Phase 1);
// mx_grouped_expert_mlp allocates nothing and never synchronises the host, so
// the runner only owns its workspace and a graph of one call over fixed device
// buffers, whose contents the caller refreshes in place between replays.
struct mx_moe_runner {
  void* workspace = nullptr;
  hipStream_t capture = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

namespace {

void runner_release(mx_moe_runner* r) {
  if (r->exec) hipGraphExecDestroy(r->exec);
  if (r->graph) hipGraphDestroy(r->graph);
  if (r->capture) hipStreamDestroy(r->capture);
  if (r->workspace) hipFree(r->workspace);
  delete r;
}

}  // namespace

extern "C" {

mx_status mx_moe_runner_create(const uint16_t* x, int64_t T, int64_t hidden, int64_t inter,
                               const int32_t* topk_ids, const float* topk_w, int32_t k, int32_t E,
                               const uint8_t* w1, const uint8_t* w1_s, const uint8_t* w3, const uint8_t* w3_s,
                               const uint8_t* w2, const uint8_t* w2_s, const uint8_t* packed_scales,
                               const uint8_t* packed_codes, mx_format requant, const float* requant_global,
                               uint16_t* y, mx_moe_runner** out) {
  MX_REQUIRE_PTR(out);
  *out = nullptr;
  if (T < 1) return fail(MX_ERR_SHAPE, "runner token count %lld must be positive", (long long)T);
  if (g_prof.on) return fail(MX_ERR_VALUE, "profiling is on: stop it before capturing a runner");
  MX_TRY(check_mlp_dims(T, hidden, inter));
  if (E < 1 || E > ROUTE_MAX_EXPERTS || k < 1 || k > E) return fail(MX_ERR_SHAPE, "k %d / E %d out of range", k, E);
  const size_t bytes = mx_grouped_expert_mlp_workspace_size(T, hidden, inter, k, E, requant);
  mx_moe_runner* r = new (std::nothrow) mx_moe_runner;
  if (r == nullptr) return fail(MX_ERR_HIP, "runner: out of host memory");
  hipError_t e = hipMalloc(&r->workspace, bytes);
  if (e != hipSuccess) {
    runner_release(r);
    return hip_fail(e, "runner workspace");
  }
  // The eager call below runs on a private stream that is not ordered after the
  // caller's streams: wait for all work already enqueued on the device (the
  // caller may just have written x, topk_ids, topk_w or the global scale).
  e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    runner_release(r);
    return hip_fail(e, "runner set-up synchronisation");
  }
  // a private stream of default priority for the capture
  e = hipStreamCreateWithFlags(&r->capture, hipStreamNonBlocking);
  if (e != hipSuccess) {
    runner_release(r);
    return hip_fail(e, "runner stream");
  }
  // one eager call first: it validates every argument (nothing is captured if
  // it fails) and leaves y valid
  mx_status st = mx_grouped_expert_mlp(x, T, hidden, inter, topk_ids, topk_w, k, E, w1, w1_s, w3, w3_s, w2, w2_s,
                                       packed_scales, packed_codes, requant, requant_global, y, r->workspace, bytes,
                                       r->capture);
  if (st != MX_OK) {
    runner_release(r);
    return st;
  }
  e = hipStreamSynchronize(r->capture);
  if (e == hipSuccess) e = hipStreamBeginCapture(r->capture, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    runner_release(r);
    return hip_fail(e, "runner capture");
  }
  st = mx_grouped_expert_mlp(x, T, hidden, inter, topk_ids, topk_w, k, E, w1, w1_s, w3, w3_s, w2, w2_s,
                             packed_scales, packed_codes, requant, requant_global, y, r->workspace, bytes, r->capture);
  e = hipStreamEndCapture(r->capture, &r->graph);
  if (st != MX_OK) {
    runner_release(r);
    return st;
  }
  if (e == hipSuccess) e = hipGraphInstantiate(&r->exec, r->graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    runner_release(r);
    return hip_fail(e, "runner graph");
  }
  *out = r;
  return ok();
}

mx_status mx_moe_runner_replay(mx_moe_runner* r, void* stream) {
  MX_REQUIRE_PTR(r);
  MX_HIP(hipGraphLaunch(r->exec, (hipStream_t)stream), "runner replay");
  return ok();
}

mx_status mx_moe_runner_destroy(mx_moe_runner* r) {
  if (r == nullptr) return ok();
  MX_HIP(hipStreamSynchronize(r->capture), "runner destroy");
  runner_release(r);
  return ok();
}

// ---------------------------------------------------------------- measurement probes
mx_status mx_probe_mfma_fp4(const uint32_t* operands, int64_t iters, int32_t workgroups, float* out,
                            void* stream) {
  if (workgroups < 1 || workgroups > 65536) return fail(MX_ERR_VALUE, "workgroups %d not in [1, 65536]", workgroups);
  if (iters < 1 || iters > ((int64_t)1 << 20)) return fail(MX_ERR_VALUE, "iters %lld not in [1, 2^20]", (long long)iters);
  MX_REQUIRE_PTR(operands);
  MX_REQUIRE_PTR(out);
  MX_REQUIRE_ALIGN(operands, 16);
  MX_REQUIRE_ALIGN(out, 4);
  hipStream_t s = (hipStream_t)stream;
  MX_HIP(phase("probe_mfma", s, [&] { return launch_probe_mfma(operands, iters, workgroups, out, s); }),
         "probe_mfma");
  return ok();
}

mx_status mx_probe_read(int32_t mode, int32_t loads_per_wave, int32_t workgroups, const void* src, int64_t bytes,
                        uint32_t* out, void* stream) {
  if (mode != 0 && mode != 1) return fail(MX_ERR_VALUE, "mode %d is not 0 (registers) or 1 (LDS)", mode);
  if (loads_per_wave != 8 && loads_per_wave != 32)
    return fail(MX_ERR_VALUE, "loads_per_wave %d is not 8 or 32", loads_per_wave);
  if (workgroups < 1 || workgroups > 65536) return fail(MX_ERR_VALUE, "workgroups %d not in [1, 65536]", workgroups);
  const int64_t chunk = (int64_t)loads_per_wave * 1024;
  if (bytes <= 0 || bytes % chunk != 0)
    return fail(MX_ERR_SHAPE, "bytes %lld is not a positive multiple of %lld", (long long)bytes, (long long)chunk);
  MX_REQUIRE_PTR(src);
  MX_REQUIRE_PTR(out);
  MX_REQUIRE_ALIGN(src, 16);
  MX_REQUIRE_ALIGN(out, 4);
  hipStream_t s = (hipStream_t)stream;
  MX_HIP(phase("probe_read", s, [&] { return launch_probe_read(mode, loads_per_wave, workgroups, src, bytes, out, s); }),
         "probe_read");
  return ok();
}

mx_status mx_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return fail(MX_ERR_SHAPE, "bytes %lld is not a multiple of 16", (long long)bytes);
  if (bytes == 0) return ok();
  MX_REQUIRE_PTR(src);
  MX_REQUIRE_PTR(dst);
  MX_REQUIRE_ALIGN(src, 16);
  MX_REQUIRE_ALIGN(dst, 16);
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + (uintptr_t)bytes && b < a + (uintptr_t)bytes) return fail(MX_ERR_VALUE, "src and dst overlap");
  hipStream_t s = (hipStream_t)stream;
  MX_HIP(phase("probe_copy", s, [&] { return launch_probe_copy(src, dst, bytes, s); }), "probe_copy");
  return ok();
}

}  // extern "C"

