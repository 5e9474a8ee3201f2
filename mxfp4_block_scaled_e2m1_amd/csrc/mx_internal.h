// Internal interfaces between the C-ABI layer (mx_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mx {

// ---- GEMM tile geometry (block-scaled FP4 MFMA kernels) --------------------
// One workgroup computes BN weight rows x BM token rows; the K loop moves
// BK logical columns (BK/2 bytes per row) per LDS stage.
constexpr int BN = 256;
constexpr int BM = 256;
constexpr int BK = 256;
constexpr int NSTAGE = 2;
constexpr int GEMM_THREADS = 512;
constexpr int L1_J_PER_TILE = BN / 2;    // L1 tiles hold gate and up rows for 128 j

// Tile-major scale layout (pack.hip): per tile and K stage, the 8 scale bytes
// of each of the tile's 256 rows, contiguous.
constexpr int SC_STAGE_BYTES = BK / 32;                           // 8
constexpr int SC_TILE_STAGE_BYTES = 256 * SC_STAGE_BYTES;         // 2048
// Bytes of the tile-major layout of `tiles` tiles over K.
constexpr int64_t packed_scale_bytes(int64_t tiles, int64_t k) { return tiles * ((k + BK - 1) / BK) * SC_TILE_STAGE_BYTES; }
// Tile-major weight codes: one block per 256-row weight tile and 128-wide half
// stage of K, the tile's 256 rows x 64 code bytes (16 KB).
constexpr int CODE_BLOCK_BYTES = 256 * 64;
constexpr int64_t packed_code_bytes(int64_t tiles, int64_t k) { return tiles * (k / 128) * CODE_BLOCK_BYTES; }

// Epilogue kinds of the scaled-MFMA GEMM.
enum Epilogue : int {
  EPI_F32 = 0,          // C[m][n] fp32 (test hook)
  EPI_SWIGLU_MXFP4 = 1, // L1: h = bf16(silu(g) * u) -> MXFP4 codes + E8M0 per 32 j
  EPI_SWIGLU_NVFP4 = 2, // L1: h -> NVFP4 codes + E4M3 per 16 j (fp32 global)
  EPI_BF16 = 3,         // L2: y[m][n] = bf16(acc) (dense) or o[slot][n] = bf16(w * acc) (grouped)
  EPI_PART_L1 = 4,      // split-K partial of L1 (gate/up rows): fp32 accumulators as the lanes hold them
};

// Split-K partial layout: per split, tile (nt * m-tiles + mt), wave, 32 x 32
// block (f * 2 + g) and lane, the lane's 16 fp32 accumulators (64 bytes).
constexpr int64_t PART_TILE_FLOATS = 8 * 8 * 64 * 16;   // 256 KB per tile and split

struct GemmArgs {
  // MFMA A operand: weight rows (MXFP4). For L1 `wa` is w1 (gate) and `wb`
  // is w3 (up); otherwise `wb` is null. Expert e starts at w + e * w_estride.
  const uint8_t* wa;
  const uint8_t* wa_s;
  const uint8_t* wb;
  const uint8_t* wb_s;
  int64_t w_estride;    // bytes between experts' code matrices
  int64_t ws_estride;   // bytes between experts' scale matrices
  // Optional tile-major copy of the weight scales (pack.hip): when set, the
  // GEMM reads it instead of wa_s/wb_s. Expert e starts at w_spk + e * wspk_estride.
  const uint8_t* w_spk;
  int64_t wspk_estride;
  // Optional tile-major copy of the weight codes (pack.hip): when set, the FP4
  // GEMM copies each half stage of its weight tile as one contiguous block laid
  // out as its LDS slot. Expert e starts at w_cpk + e * wcpk_estride.
  const uint8_t* w_cpk;
  int64_t wcpk_estride;
  int n_rows;           // logical weight rows per matrix (inter for L1, hidden for L2)
  int k;                // logical K (multiple of 128)

  // MFMA B operand: token rows (MXFP4) [rows, k/2] + [rows, k/32].
  const uint8_t* x;
  const uint8_t* x_s;         // [rows, k/32], or tile-major over the m-tiles when x_s_packed
  const int32_t* row_token;   // grouped L1: sorted row -> token; null = identity
  int x_s_packed;
  int x_tiled;                // x holds tile-major codes: per m-tile and half stage, the
                              // LDS image of the slot (the L2's h from an L1 with h_codes_tiled)

  // Row groups: grouped mode has expert_off/tile_base on the device;
  // dense mode (expert_off == null) is a single group of m_rows rows.
  const int32_t* expert_off;  // [E+1] first sorted row of each expert
  const int32_t* tile_base;   // [E+1] first m-tile of each expert
  int n_experts;
  int m_rows;                 // dense mode rows
  int n_tiles;                // tiles along the weight rows
  int grid_tiles;             // dense: exact count of tiles (times k_splits)
  int k_splits;               // dense: K splits (0 or 1: none); EPI_PART_L1: c_f32 holds the partials

  // Outputs.
  float* c_f32;               // EPI_F32: [m_rows, n_rows]; EPI_PART_L1: split-K partials
  uint8_t* h_codes;           // L1: [rows, n_rows/2]
  uint8_t* h_scales;          // L1: [rows, n_rows/32] (MXFP4) or [rows, n_rows/16] (NVFP4)
  int h_scales_packed;        // L1 MXFP4: h_scales tile-major over the m-tiles (the L2's x_s)
  int h_codes_tiled;          // L1 MXFP4: h_codes tile-major over the m-tiles (the L2's x, x_tiled)
  float nv_global;            // bf16-MFMA GEMMs: epilogue scale (fused gate/up: the gate's)
  float nv_global2;           // bf16-MFMA fused gate/up: the up GEMM's epilogue scale
  float h_nv_global;          // L1 NVFP4 re-quant global scale when nv_gptr is null
  const float* nv_gptr;       // when set, the kernel reads nv_global from this device float
  const float* e_global;      // bf16-MFMA GEMMs, optional: per-expert factor on nv_global [E]
  const float* e_global2;     // bf16-MFMA fused gate/up: per-expert factor on nv_global2 [E]
  uint32_t* h_amax;           // L1 MXFP4, optional: running max of |h| (bf16 bits) over the valid rows
  uint16_t* out_bf16;         // EPI_BF16: dense y [m_rows, n_rows]; grouped o [slots, n_rows]
  const int32_t* row_slot;    // grouped L2: sorted row -> slot (t*k + j)
  const float* row_weight;    // grouped L2: gate weight of each sorted row
};

// max_tiles: an upper bound on the tiles of the launch (the routed case only knows
// its exact count on the device); the kernel is persistent with one workgroup per CU.
hipError_t launch_gemm(Epilogue epi, const GemmArgs& a, int max_tiles, hipStream_t s);

// L2 of the NVFP4 re-quantisation variant: x/x_s are NVFP4 h codes and E4M3
// scales per 16 columns, nv_global the fp32 global scale; bf16 matrix cores on
// exactly dequantised operands, output as EPI_BF16 times nv_global.
hipError_t launch_gemm_nv_l2(const GemmArgs& a, int max_tiles, hipStream_t s);

// Split-K sum of a dense L1 launch `a` (its k_splits partials in a.c_f32),
// followed by the SiLU * up and MXFP4 re-quantisation epilogue (a.h_codes,
// a.h_scales, tile-major when a.h_scales_packed).
hipError_t launch_part_l1(const GemmArgs& a, hipStream_t s);

// Compute units of the current device (cached per device).
int cu_count();

// Tile-major scale copies (pack.hip). Weights: b_s null for a plain matrix of
// n_rows rows (tiles of 256 rows), else the L1 pair (a_s gate, b_s up, tiles
// of 128 rows of each); out holds n_experts * tiles * stages * 2048 bytes.
hipError_t launch_pack_weight_scales(const uint8_t* a_s, const uint8_t* b_s, int n_experts, int n_rows, int k,
                                     uint8_t* out, hipStream_t s);
// Activations: the m-tiles of a routed (expert_off set, tokens via row_token)
// or dense (m_rows rows) launch; out holds max_mtiles * stages * 2048 bytes.
// Tile-major weight codes (pack_weight_codes): L1 when b != null (gate rows in a,
// up rows in b, the GEMM's interleaved L1 tile rows), else L2; k % 128 == 0.
hipError_t launch_pack_weight_codes(const uint8_t* a, const uint8_t* b, int n_experts, int n_rows, int k,
                                    uint8_t* out, hipStream_t s);
hipError_t launch_pack_act_scales(const uint8_t* x_s, int k, const int32_t* row_token, const int32_t* expert_off,
                                  const int32_t* tile_base, int n_experts, int m_rows, int max_mtiles,
                                  uint8_t* out, hipStream_t s);

// ---- Elementwise kernels ---------------------------------------------------
hipError_t launch_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                int64_t cols, uint16_t* out, hipStream_t s);
hipError_t launch_dequant_fp8_block(const uint8_t* q, const uint8_t* scales, int64_t rows,
                                    int64_t cols, uint16_t* out, hipStream_t s);
// NVFP4 kernels take their fp32 global either as a value or, when gptr is not
// null, from device memory (*gptr, read in stream order).
hipError_t launch_dequant_nvfp4(const uint8_t* codes, const uint8_t* scales, float global, const float* gptr,
                                int64_t rows, int64_t cols, uint16_t* out, hipStream_t s);
hipError_t launch_quant_mxfp4(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes,
                              uint8_t* scales, hipStream_t s);
// The same codes and scales in the chunked layout of the weight-streaming
// kernels (rows in chunks of 16, padded with zero codes; cols % 128 == 0, rows
// <= 512). Codes: per chunk c and 128-wide K step s one 1 KB block, lane
// l = 16 q + r at bytes 16 l .. +15 holding columns 128 s + 32 q .. +31 of row
// 16 c + r. Scales: the K steps are split over the kernels' STREAM_WAVES waves
// in balanced runs (the first ksteps % STREAM_WAVES waves take one more), and
// per chunk c, wave w and lane l the 8 bytes at ((c * STREAM_WAVES + w) * 64 +
// l) * 8 are the scales of lane l's 32 columns in the steps of w's run (bytes
// past the run are not written).
constexpr int STREAM_WAVES = 8;
inline int64_t chunked_scale_bytes(int64_t rows) { return (rows + 15) / 16 * STREAM_WAVES * 64 * 8; }
hipError_t launch_quant_mxfp4_chunked(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes,
                                      uint8_t* scales, hipStream_t s);
hipError_t launch_quant_nvfp4(const uint16_t* x, int64_t rows, int64_t cols, float global, const float* gptr,
                              uint8_t* codes, uint8_t* scales, hipStream_t s);
// NVFP4 warm-up: clear the |h| max word; turn it into g = f32(max / (6 * 448)).
hipError_t launch_amax_clear(uint32_t* amax, hipStream_t s);
hipError_t launch_nvfp4_global(const uint32_t* amax, float* g, hipStream_t s);

// ---- Routing ----------------------------------------------------------------
constexpr int ROUTE_CHUNK = 1024;    // pairs per counting/scatter block
constexpr int ROUTE_MAX_EXPERTS = 512;   // LDS of the scatter: 16 * E ints

struct RouteBuffers {
  int32_t* block_counts;   // [nblocks, E] chunk histograms, scanned in place into chunk bases
  int32_t* expert_off;     // [E+1]
  int32_t* tile_base;      // [E+1]
  int32_t* row_token;      // [P]
  int32_t* row_slot;       // [P]
  float* row_weight;       // [P] gate weight of each sorted row
};

hipError_t launch_route(const int32_t* topk_ids, const float* topk_w, int64_t tokens, int k, int n_experts,
                        const RouteBuffers& rb, hipStream_t s);

// dst[r] = src[row_token[r]] for the *n_valid sorted rows (n_valid: the route's
// expert_off[E], on the device); rows are `width` bytes, width % 8 == 0.
hipError_t launch_gather_rows(const uint8_t* src, int width, const int32_t* row_token, const int32_t* n_valid,
                              int64_t P, uint8_t* dst, hipStream_t s);

hipError_t launch_combine(const uint16_t* o, const int32_t* topk_ids, int64_t tokens, int k,
                          int n_experts, int hidden, uint16_t* y, hipStream_t s);

// ---- Few-token paths: weight streaming, see decode.hip ----------------------
// pk1 / pk2: the expert's tile-major L1 / L2 weight codes (mx_pack_weight_codes)
// or null: the kernels then read the row-major codes. Up to 8 tokens the
// activations are quantised in LDS; h: bf16 scratch [m, inter].
bool decode_fits(int64_t m, int64_t hidden, int64_t inter);
// 9 <= M <= 512: x and h quantised by the MXFP4 quantiser into the workspace in
// the chunked layout (xq, hq: ceil(m/16)*16 rows), the weights streamed once by
// two kernels that read the token rows as MFMA operands, 16 at a time.
bool skinny_fits(int64_t m, int64_t hidden, int64_t inter);
hipError_t launch_skinny_mlp(const uint16_t* x, int m, int H, int I, const uint8_t* w1, const uint8_t* w1s,
                             const uint8_t* w3, const uint8_t* w3s, const uint8_t* w2, const uint8_t* w2s,
                             const uint8_t* pk1, const uint8_t* pk2, uint8_t* xq, uint8_t* xs, uint16_t* h,
                             uint8_t* hq, uint8_t* hs, uint16_t* y, hipStream_t s);
hipError_t launch_decode_mlp(const uint16_t* x, int m, int H, int I, const uint8_t* w1, const uint8_t* w1s,
                             const uint8_t* w3, const uint8_t* w3s, const uint8_t* w2, const uint8_t* w2s,
                             const uint8_t* pk1, const uint8_t* pk2, uint16_t* h, uint16_t* y, hipStream_t s);

// Routed experts with few rows each (mean T*k/E at most 2 with MXFP4, 12 with
// NVFP4 re-quantisation): the weights of each
// expert with rows streamed once by two kernels (see decode.hip). L1 writes
// h (bf16, [P, inter], sorted row order); the caller re-quantises it into
// hq/hs row-major, MXFP4 or (nvfp4) NVFP4, in which case L2 converts code *
// s to bf16 and multiplies by `scale` = g. L2 writes o[row_slot[p]] rows, as
// the GEMM's routed epilogue.
struct RoutedArgs {
  int H, I, E;
  const uint8_t *xq, *xs;
  const int32_t *row_token, *row_slot, *expert_off;
  const float* row_weight;
  const uint8_t *w1, *w1s, *w3, *w3s, *w2, *w2s;
  const uint8_t *pk1, *pk2;          // tile-major L1 / L2 codes of expert 0 (mx_pack_weight_codes), or null
  int64_t pk1_estride, pk2_estride;  // their bytes per expert
  uint16_t* h;
  const uint8_t *hq, *hs;
  bool nvfp4;           // hq/hs are NVFP4 (E4M3 per 16), else MXFP4
  float scale;
  const float* scale_ptr;   // when set, L2 reads `scale` from this device float
  uint16_t* o;
};
bool routed_stream_fits(int64_t T, int64_t hidden, int64_t inter, int k, int E, bool nvfp4);
hipError_t launch_routed_l1(const RoutedArgs& a, hipStream_t s);
hipError_t launch_routed_l2(const RoutedArgs& a, hipStream_t s);

// ---- FP8 block-scaled linear (fp8_linear.hip) -----------------------------
hipError_t launch_quant_mxfp8(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                              hipStream_t s);
// y [M, N] = bf16(dequant(xq, xs) . dequant(w, ws)^T); K % 128 == 0, N % 128 == 0.
hipError_t launch_fp8_gemm(const uint8_t* xq, const uint8_t* xs, const uint8_t* w, const uint8_t* ws, int M, int N,
                           int K, uint16_t* y, hipStream_t s);
bool fp8_linear_fits(int64_t K);
// h = bf16(silu(g) * u) elementwise over n values (n % 8 == 0, 16-byte aligned).
hipError_t launch_silu_mul_bf16(const uint16_t* g, const uint16_t* u, int64_t n, uint16_t* h, hipStream_t s);

// Measurement probes (probe.hip). mode 0: reads into registers, 1: into LDS;
// loads_per_wave 8 or 32; bytes a multiple of loads_per_wave KiB; out holds
// workgroups * 4 words. operands: 512 x 16 words; out: workgroups * 512 floats.
hipError_t launch_probe_mfma(const uint32_t* operands, int64_t iters, int workgroups, float* out, hipStream_t s);
hipError_t launch_probe_read(int mode, int loads_per_wave, int workgroups, const void* src, int64_t bytes,
                             uint32_t* out, hipStream_t s);
hipError_t launch_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);

}  // namespace mx
