/*
 * libmxfp4 -- block-scaled FP4 (MXFP4: E2M1 x E8M0) expert MLP for AMD MI355X (gfx950).
 *
 * C ABI. Every tensor argument is a DEVICE pointer owned by the caller; the
 * library never allocates device memory, never synchronises the host and never
 * keeps a pointer after a call returns -- except the runner (mx_moe_runner_*),
 * which allocates its workspace and synchronises once when it is created and
 * destroyed, and keeps the buffers it was created over. Work is enqueued on the caller's HIP
 * stream (`stream` is a hipStream_t; NULL means the default stream). Tensors are
 * row-major and contiguous. bf16 tensors are passed as uint16_t bit patterns;
 * FP4 codes and E8M0/E4M3 scales are raw bytes (a checkpoint's int8 storage is
 * read as unsigned bytes).
 *
 * Formats, from the pages this library is built from:
 *  - MXFP4 ("2026-05-08 DeepSeek V4 Pro NVFP4 Quantization", sections "Script
 *    update" item 2 and "FP4 (E2M1) expert weight format confirmed"): a logical
 *    [R, C] matrix is stored as codes [R, C/2] (two E2M1 codes per byte, element
 *    2j in the low nibble, code 8 = -0.0) and scales [R, C/32] (one E8M0 byte
 *    2^(b-127) per row per 32 columns; 0xFF is NaN). Expert weights are w1/w3
 *    [inter, hidden] and w2 [hidden, inter]; for the pages' model hidden = 7168,
 *    inter = 3072 (codes [3072, 3584] + scales [3072, 224] -> [3072, 7168]).
 *  - FP8 block ("Script update" item 1): float8_e4m3fn [R, C] with one E8M0
 *    scale per 128 x 128 block, scales [ceil(R/128), ceil(C/128)] row-major;
 *    value = e4m3 * 2^(b-127).
 *  - NVFP4 (named, not defined, on "Current Bug: vLLM produces empty/garbage
 *    output", "Revised Plan" Phases 1-2): E2M1 codes as above, one E4M3 scale
 *    per 16 columns [R, C/16] and a positive fp32 global scale g; value =
 *    e2m1 * e4m3 * g. Used for the re-quantised intermediate (g in DEVICE
 *    memory: mx_dequant, mx_quantize_act, the MLP entry points and the runner
 *    take `const float*` and read g in stream order, so the value written by
 *    mx_nvfp4_global_warmup feeds them without a host read-back), and for
 *    weights and activations by the mx_*nvfp4_* entry points (host values).
 *  - MXFP8 (activations of the FP8 linear): float8_e4m3fn [R, C] with one E8M0
 *    scale per 32 columns [R, C/32], shared exponent floor(log2 amax) - 8.
 *
 * The expert MLP ("Current Bug ...", "Revised Plan", Phase 1: L1 GEMM -> SiLU ->
 * re-quant -> L2 GEMM; the shared expert is the MoE pipeline with one expert and
 * no routing; Phase 3 keeps the SiLU output and the final scatter in BF16):
 *      xq = MXFP4(x)                                  per token, per 32 columns
 *      g  = xq . w1^T,  u = xq . w3^T                 FP4 x FP4, fp32 accumulation
 *      h  = bf16(silu(g) * u)                         silu(g) = g / (1 + e^-g)
 *      hq = MXFP4(h)  (or NVFP4(h, g_global))
 *      y  = bf16(hq . w2^T)
 * MXFP4(.) is the OCP MX rule: shared exponent floor(log2 amax) - 2 (clamped to
 * the E8M0 range), E2M1 round to nearest even, saturating at 6, sign kept.
 * The routed form sums k experts per token: y[t] = bf16(sum_j w[t,j] * y_j(t)).
 *
 * Errors: every entry point validates its arguments on the host before it
 * enqueues anything. On a failed check it enqueues nothing and returns a
 * non-zero mx_status; mx_last_error() then describes the failure (the text is
 * per calling thread and stays valid until that thread's next call). A HIP
 * launch error returns MX_ERR_HIP. Data that can only be checked on the device
 * is not checked: E8M0 0xFF and E4M3 NaN codes propagate NaN, expert ids
 * outside [0, E) are skipped (they belong to other ranks), non-finite
 * activations give unspecified codes.
 *
 * Thread safety: calls on different streams may run concurrently; the library
 * holds no mutable state besides the per-thread error text and the optional
 * profiler (mx_profile_*), which must not be toggled while other threads call.
 */
#ifndef MXFP4_H_
#define MXFP4_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define MX_API __attribute__((visibility("default")))
#else
#define MX_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mx_status {
  MX_OK = 0,
  MX_ERR_NULL = 1,       /* a required pointer is NULL */
  MX_ERR_SHAPE = 2,      /* a size is negative, not a required multiple, or too large */
  MX_ERR_ALIGN = 3,      /* a pointer is not aligned as documented */
  MX_ERR_FORMAT = 4,     /* format not valid for this entry point */
  MX_ERR_WORKSPACE = 5,  /* workspace smaller than the matching *_workspace_size() */
  MX_ERR_HIP = 6,        /* a HIP runtime call or kernel launch failed */
  MX_ERR_VALUE = 7,      /* a scalar argument is out of range (e.g. a non-finite global scale) */
  /* not statuses: they make every int32 value a valid mx_status
   * (mx_status_string of an unknown value is defined) */
  MX_STATUS_RESERVED_MIN_ = -2147483647 - 1,
  MX_STATUS_RESERVED_MAX_ = 2147483647
} mx_status;

typedef enum mx_format {
  MX_FMT_MXFP4 = 0,      /* E2M1 codes + E8M0 per 1x32 */
  MX_FMT_FP8_B128 = 1,   /* float8_e4m3fn + E8M0 per 128x128 block (dequant only) */
  MX_FMT_NVFP4 = 2,      /* E2M1 codes + E4M3 per 1x16 + fp32 global scale */
  MX_FMT_MXFP8 = 3,      /* float8_e4m3fn codes + E8M0 per 1x32 (activation quantisation only) */
  /* not formats: they make every int32 value a valid mx_format, so a caller's
   * unknown value reaches the library's check (MX_ERR_FORMAT) with defined
   * behaviour in C++ as in C */
  MX_FMT_RESERVED_MIN_ = -2147483647 - 1,
  MX_FMT_RESERVED_MAX_ = 2147483647
} mx_format;

/*
 * mx_dequant -- dequantise a block-scaled matrix to bf16. The operation is the
 * pages' offline dequant script: the FP8 weights times their 128 x 128 block
 * scale, and the packed E2M1 experts through the E2M1 table times 2^(e-127)
 * with the width doubled ("2026-05-08 DeepSeek V4 Pro NVFP4 Quantization",
 * section "Script update", items 1-2; shapes in "FP4 (E2M1) expert weight
 * format confirmed").
 *   MX_FMT_MXFP4:    codes [rows, cols/2], scales [rows, cols/32]; cols % 32 == 0.
 *   MX_FMT_FP8_B128: codes [rows, cols] (e4m3fn), scales [ceil(rows/128), ceil(cols/128)];
 *                    cols % 16 == 0.
 *   MX_FMT_NVFP4:    codes [rows, cols/2], scales [rows, cols/16] (e4m3fn), global_scale:
 *                    DEVICE pointer to g (required: MX_ERR_NULL if NULL); cols % 16 == 0.
 * global_scale is ignored (may be NULL) except for NVFP4. out_bf16 is [rows, cols].
 * Exact: every MXFP4 and FP8 product is representable in bf16 unless it
 * overflows (then +-inf); NVFP4 products are rounded to bf16 once (RNE).
 * Alignment: codes and out_bf16 16 bytes (NVFP4 codes 8 bytes), global_scale 4.
 */
MX_API mx_status mx_dequant(mx_format fmt, const void* codes, const void* scales, const float* global_scale,
                     int64_t rows, int64_t cols, uint16_t* out_bf16, void* stream);

/*
 * mx_quantize_act -- quantise bf16 activations x [rows, cols] per row: the
 * quantisation step before each FP4 GEMM of the pages' pipeline (page
 * "Current Bug: vLLM produces empty/garbage output", section "Revised Plan",
 * Phase 1: L1 GEMM, SiLU, re-quant, L2 GEMM), in the MXFP4 format of
 * "2026-05-08 DeepSeek V4 Pro NVFP4 Quantization", "Script update" item 2.
 *   MX_FMT_MXFP4: codes [rows, cols/2], scales [rows, cols/32] (E8M0); cols % 32 == 0.
 *   MX_FMT_NVFP4: codes [rows, cols/2], scales [rows, cols/16] (E4M3), global_scale: DEVICE
 *                 pointer to g (required), g > 0 finite and >= 2^-117 (not checked: the
 *                 value lives on the device). Steps in fp32: s = E4M3_RNE_sat(amax / (6 g)),
 *                 code = E2M1_RNE_sat(x / (s g)); s == 0 gives signed zero codes.
 *   MX_FMT_MXFP8: codes [rows, cols] (e4m3fn), scales [rows, cols/32] (E8M0); cols % 32 == 0.
 *                 Scale byte clamp(floor(log2 amax) - 8 + 127, 0, 254); elements
 *                 rounded to nearest even E4M3, saturating at +-448, sign kept.
 * Alignment: x and codes 16 bytes (NVFP4 codes 8 bytes), global_scale 4.
 */
MX_API mx_status mx_quantize_act(mx_format fmt, const uint16_t* x_bf16, int64_t rows, int64_t cols,
                          const float* global_scale, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * mx_expert_mlp -- one expert (the shared expert), M tokens, no routing: the
 * pages' shared-expert pipeline L1 GEMM -> SiLU -> re-quant -> L2 GEMM, the MoE
 * pipeline with one group and no routing (page "Current Bug: vLLM produces
 * empty/garbage output", section "Revised Plan", Phase 1; BF16 SiLU output per
 * Phase 3; weight shapes from "2026-05-08 DeepSeek V4 Pro NVFP4 Quantization",
 * "FP4 (E2M1) expert weight format confirmed").
 *   x  [M, hidden] bf16            w1, w3 codes [inter, hidden/2], scales [inter, hidden/32]
 *   y  [M, hidden] bf16            w2 codes [hidden, inter/2], scales [hidden, inter/32]
 * hidden % 128 == 0 and inter % 128 == 0.
 * requant selects the format of the intermediate h between the two GEMMs:
 *   MX_FMT_MXFP4: E8M0 per 32 (requant_global ignored); both GEMMs run on FP4
 *     matrix cores. Up to 512 tokens the weights are streamed once by two
 *     kernels that take the tokens as the MFMA's second operand (M <= 8:
 *     activations quantised in LDS; 9..512: quantised beforehand, in 16-token
 *     chunks); larger M runs the tiled GEMMs.
 *   MX_FMT_NVFP4: E4M3 per 16 with the fp32 global scale g at the DEVICE
 *     pointer requant_global (required; g finite and >= 2^-117, not checked,
 *     read in stream order, e.g. straight from mx_nvfp4_global_warmup); the L2
 *     GEMM runs on bf16 matrix cores on exactly dequantised operands,
 *     y = bf16(g * sum (code*s)(w)).
 *     Exact for w2 scale bytes <= 252 (6 * 2^126 exceeds bf16 above that).
 *   anything else: MX_ERR_FORMAT.
 * A stacked gate_up tensor [2*inter, hidden/2] is passed as w1 = w13 and
 * w3 = w13 + inter*hidden/2 (scales likewise).
 * packed_scales: NULL, or the output of mx_pack_weight_scales() for these
 * weights (E = 1, same hidden and inter), 256-byte aligned. The GEMM path then
 * reads the weight scales from it; the results are identical either way.
 * packed_codes: NULL, or the output of mx_pack_weight_codes() for these weights
 * (E = 1, same hidden and inter), 256-byte aligned: every path then reads the
 * weight codes from it (the GEMMs copy whole 1 KB pieces, the weight-streaming
 * kernels read 512 or 1024 contiguous bytes per 128-wide K step instead of 16
 * separate 64-byte row pieces); the results are identical either way. w1, w3
 * and w2 are still required.
 * workspace: device memory of at least mx_expert_mlp_workspace_size() bytes,
 * 256-byte aligned; its contents are scratch. y must not alias x or workspace.
 * Alignment: x, y, codes 16 bytes; scales and requant_global 4 bytes.
 */
MX_API mx_status mx_expert_mlp(const uint16_t* x, int64_t M, int64_t hidden, int64_t inter,
                        const uint8_t* w1, const uint8_t* w1_s, const uint8_t* w3,
                        const uint8_t* w3_s, const uint8_t* w2, const uint8_t* w2_s,
                        const uint8_t* packed_scales, const uint8_t* packed_codes, mx_format requant,
                        const float* requant_global, uint16_t* y, void* workspace, size_t ws_bytes,
                        void* stream);

/* Workspace bytes of mx_expert_mlp for these sizes (the caller-owned scratch of
 * the pages' pre-allocated runner: "Current Bug ...", "Revised Plan", Phase 1);
 * 0 for negative sizes. */
MX_API size_t mx_expert_mlp_workspace_size(int64_t M, int64_t hidden, int64_t inter, mx_format requant);

/*
 * mx_expert_mlp_noalloc -- mx_expert_mlp for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation and results, with the workspace
 * taken from a fixed device array inside the library instead of a caller
 * buffer. The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).
 *   Arguments, formats, alignment and errors as for mx_expert_mlp, without
 *   workspace and ws_bytes.
 *   Limit: the sizes must need at most mx_expert_mlp_noalloc_max_bytes()
 *   (64 MiB) of workspace, i.e. mx_expert_mlp_workspace_size(M, hidden, inter,
 *   requant) <= 64 MiB (M = 4096 at hidden 7168, inter 3072 needs 23 MiB);
 *   larger sizes return MX_ERR_WORKSPACE and enqueue nothing.
 *   Each GPU holds its own 64 MiB array for the life of the process (its
 *   address is looked up on the first call on that device). Every call on one
 *   GPU uses that GPU's array: calls that overlap in time on one GPU (different
 *   streams, different threads without ordering) race and give wrong results.
 */
MX_API mx_status mx_expert_mlp_noalloc(const uint16_t* x, int64_t M, int64_t hidden, int64_t inter,
                                       const uint8_t* w1, const uint8_t* w1_s, const uint8_t* w3,
                                       const uint8_t* w3_s, const uint8_t* w2, const uint8_t* w2_s,
                                       const uint8_t* packed_scales, const uint8_t* packed_codes,
                                       mx_format requant, const float* requant_global, uint16_t* y,
                                       void* stream);
/* Bytes of the fixed device array behind mx_expert_mlp_noalloc (64 MiB). */
MX_API size_t mx_expert_mlp_noalloc_max_bytes(void);

/*
 * mx_grouped_expert_mlp -- E local routed experts as a ragged grouped GEMM: the
 * pages' MoE pipeline (routing, top-k, scatter around the same L1 GEMM -> SiLU
 * -> re-quant -> L2 GEMM; page "Current Bug: vLLM produces empty/garbage
 * output", section "Revised Plan", Phase 1, with the final scatter in BF16 per
 * Phase 3), for the 48 experts of one expert-parallel rank ("Config values").
 *   x        [T, hidden] bf16 tokens
 *   topk_ids [T, k] int32 expert of each (token, slot); ids outside [0, E) are skipped
 *   topk_w   [T, k] fp32 gate weight of each (token, slot)
 *   w1, w3   codes [E, inter, hidden/2], scales [E, inter, hidden/32]
 *   w2       codes [E, hidden, inter/2], scales [E, hidden, inter/32]
 *   y        [T, hidden] bf16: y[t] = bf16(sum_j topk_w[t,j] * expert_{ids[t,j]}(x[t]))
 * Steps: x is quantised once per token; pairs are sorted by expert (stable in
 * t*k + j order) with a ballot-based scan; the L1 GEMM gathers token rows and
 * fuses SiLU*up and the re-quantisation; the L2 GEMM multiplies by the gate
 * weight and writes one bf16 row per pair; a final pass sums each token's k
 * rows in slot order in fp32 (deterministic: no atomics).
 * 1 <= k <= E <= 512; hidden % 128 == 0; inter % 128 == 0. requant,
 * requant_global, packed_scales and packed_codes (here for all E experts) as
 * for mx_expert_mlp.
 * Alignment as for mx_expert_mlp; topk_ids and topk_w 4 bytes.
 */
MX_API mx_status mx_grouped_expert_mlp(const uint16_t* x, int64_t T, int64_t hidden, int64_t inter,
                                const int32_t* topk_ids, const float* topk_w, int32_t k, int32_t E,
                                const uint8_t* w1, const uint8_t* w1_s, const uint8_t* w3,
                                const uint8_t* w3_s, const uint8_t* w2, const uint8_t* w2_s,
                                const uint8_t* packed_scales, const uint8_t* packed_codes, mx_format requant,
                                const float* requant_global, uint16_t* y, void* workspace, size_t ws_bytes,
                                void* stream);

/* Workspace bytes of mx_grouped_expert_mlp for these sizes (caller-owned
 * scratch of the pages' pre-allocated runner: "Current Bug: vLLM produces
 * empty/garbage output", "Revised Plan", Phase 1); 0 for invalid sizes. */
MX_API size_t mx_grouped_expert_mlp_workspace_size(int64_t T, int64_t hidden, int64_t inter, int32_t k,
                                            int32_t E, mx_format requant);

/*
 * mx_pack_weight_scales -- re-lay the E8M0 weight scales of E experts once,
 * after the weights are loaded, in the order the FP4 GEMM copies them: for
 * each 256-row weight tile and 256-wide K stage, the 8 scale bytes of the
 * tile's rows are contiguous (2 KB), so that a stage's scales arrive in a
 * few whole cache lines instead of 256 separate 8-byte pieces. The runner on
 * the pages prepares its weights once before serving (page "Current Bug: vLLM
 * produces empty/garbage output", section "Revised Plan", Phase 1).
 *   w1_s, w3_s [E, inter, hidden/32]; w2_s [E, hidden, inter/32] (E8M0 bytes).
 *   packed: device buffer of mx_packed_weight_scales_size(hidden, inter, E)
 *   bytes, 256-byte aligned, owned by the caller and passed to mx_expert_mlp
 *   (E = 1) or mx_grouped_expert_mlp as packed_scales. Its layout is internal.
 * Shapes as for mx_grouped_expert_mlp; MX_ERR_WORKSPACE if packed_bytes is
 * too small. Alignment: scales 4 bytes.
 */
MX_API mx_status mx_pack_weight_scales(const uint8_t* w1_s, const uint8_t* w3_s, const uint8_t* w2_s,
                                       int64_t hidden, int64_t inter, int32_t E, uint8_t* packed,
                                       size_t packed_bytes, void* stream);

MX_API size_t mx_packed_weight_scales_size(int64_t hidden, int64_t inter, int32_t E);

/*
 * mx_pack_weight_codes -- re-lay the FP4 weight codes of E experts once, after
 * the weights are loaded, in the order the FP4 GEMM copies them into LDS: for
 * each 256-row weight tile (L1: the tile's gate and up rows; L2: w2 rows) and
 * each 128-wide half stage of K, one 16 KB block that is the byte image of the
 * GEMM's LDS slot. A copy then reads whole cache lines, 1 KB in one piece,
 * instead of 16 rows x 64 bytes scattered over 16 rows of the matrix. As for
 * the scales, the pages' runner prepares its weights once before serving (page
 * "Current Bug: vLLM produces empty/garbage output", section "Revised Plan",
 * Phase 1).
 *   w1, w3 [E, inter, hidden/2]; w2 [E, hidden, inter/2] (E2M1 codes), 16-byte
 *   aligned. packed: device buffer of mx_packed_weight_codes_size(hidden,
 *   inter, E) bytes (as large as the three code tensors, rounded up to whole
 *   tiles), 256-byte aligned, owned by the caller and passed to mx_expert_mlp
 *   (E = 1), mx_expert_mlp_noalloc, mx_grouped_expert_mlp or
 *   mx_moe_runner_create as packed_codes. Its layout is internal.
 * Shapes as for mx_grouped_expert_mlp; MX_ERR_WORKSPACE if packed_bytes is too
 * small.
 */
MX_API mx_status mx_pack_weight_codes(const uint8_t* w1, const uint8_t* w3, const uint8_t* w2, int64_t hidden,
                                      int64_t inter, int32_t E, uint8_t* packed, size_t packed_bytes,
                                      void* stream);

/* Bytes of mx_pack_weight_codes' output (the re-laid E2M1 codes of
 * "2026-05-08 DeepSeek V4 Pro NVFP4 Quantization", "FP4 (E2M1) expert weight
 * format confirmed"); 0 for invalid sizes. */
MX_API size_t mx_packed_weight_codes_size(int64_t hidden, int64_t inter, int32_t E);

/*
 * mx_nvfp4_global_warmup -- the fp32 global scale g of the NVFP4 re-quantisation
 * of h, from a warm-up batch, computed on the device: g = f32(max |h| / (6 * 448))
 * over every (token, expert) pair of the batch, or 1 when h is all zero. h is
 * bf16(silu(x . w1^T) * (x . w3^T)) as the MLP computes it (x quantised to
 * MXFP4, the FP4 L1 GEMM, the same SiLU and rounding), so the largest |h| maps
 * onto the largest E2M1 value (6) times the largest E4M3 scale (448). The pages'
 * runner plans a global scale taken from a warm-up pass, computed once before
 * serving (page "Current Bug: vLLM produces empty/garbage output", section
 * "Revised Plan", Phase 1); the mapping is the plain reading of that plan.
 *   topk_ids == NULL: one expert (the shared expert), T token rows; k must be 0
 *     and topk_w, E are ignored (packed_scales then holds one expert).
 *   otherwise: routed exactly as mx_grouped_expert_mlp (topk_ids, topk_w, k, E).
 *   w1, w3 (and scales) as for mx_expert_mlp / mx_grouped_expert_mlp; w2 is not read.
 *   global_out: one fp32 in device memory, written by the call in stream order;
 *     pass the same pointer as requant_global (no host read-back needed).
 * workspace: mx_nvfp4_global_warmup_workspace_size(T, hidden, inter, k, E) bytes
 * (k = 0 for one expert), 256-byte aligned; contents are scratch.
 * Alignment as for the MLP entry points; global_out 4 bytes.
 */
MX_API mx_status mx_nvfp4_global_warmup(const uint16_t* x, int64_t T, int64_t hidden, int64_t inter,
                                        const int32_t* topk_ids, const float* topk_w, int32_t k, int32_t E,
                                        const uint8_t* w1, const uint8_t* w1_s, const uint8_t* w3,
                                        const uint8_t* w3_s, const uint8_t* packed_scales, float* global_out,
                                        void* workspace, size_t ws_bytes, void* stream);

MX_API size_t mx_nvfp4_global_warmup_workspace_size(int64_t T, int64_t hidden, int64_t inter, int32_t k,
                                                    int32_t E);

/*
 * mx_fp8_block_linear -- y = bf16(MXFP8(x) . W^T): the FP8 block-scaled linear
 * of the original checkpoint's shared expert (page "2026-05-11 - DeepSeek V4
 * NVFP4 vLLM Serving: Full End-to-End", "Architecture Map" and "What We
 * Fixed" item 1; page "2026-05-08 DeepSeek V4 Pro NVFP4 Quantization",
 * "Status").
 *   x   [M, K] bf16, quantised per row and 32 columns to MXFP8 as
 *       mx_quantize_act(MX_FMT_MXFP8) does (into the workspace)
 *   w   [N, K] float8_e4m3fn codes, row-major
 *   w_s [N/128, K/128] E8M0, one byte per 128 x 128 tile (multiplies)
 *   y   [M, N] bf16, fp32 accumulation rounded once
 * K % 128 == 0, K <= 8192, N % 128 == 0; M >= 0 (M == 0 does nothing).
 * workspace: at least mx_fp8_block_linear_workspace_size(M, K) bytes, 256-byte
 * aligned; scratch. y must not alias x, w or the workspace.
 * Alignment: x, w and y 16 bytes. E4M3 NaN codes or E8M0 byte 255 give NaN.
 */
MX_API mx_status mx_fp8_block_linear(const uint16_t* x, int64_t M, int64_t K, const uint8_t* w,
                                     const uint8_t* w_s, int64_t N, uint16_t* y, void* workspace,
                                     size_t ws_bytes, void* stream);
MX_API size_t mx_fp8_block_linear_workspace_size(int64_t M, int64_t K);

/*
 * mx_nvfp4_linear -- y = bf16(NVFP4(x) . W^T) with NVFP4 weights: the GEMM of
 * the routed experts as the pages run them on B200 (w13/w2 in NVFP4: page
 * "2026-05-11 - DeepSeek V4 NVFP4 vLLM Serving: Full End-to-End", "Architecture
 * Map"; per-matrix weight_scale_2 and the activations' input scale: page
 * "Current Bug: vLLM produces empty/garbage output", "Revised Plan", Phase 2).
 *   x   [M, K] bf16, quantised to NVFP4 with the fp32 global x_global exactly
 *       as mx_quantize_act(MX_FMT_NVFP4) does (into the workspace)
 *   w   [N, K/2] E2M1 codes (low nibble first), w_s [N, K/16] E4M3 scales,
 *       w_global the fp32 weight global scale: value = code * s * w_global
 *   y   [M, N] bf16 = bf16((x_global * w_global) * sum (code s)(code s)),
 *       on bf16 matrix cores (code * s is exact in bf16)
 * K % 128 == 0, N % 128 == 0. x_global finite and >= 2^-117, w_global finite
 * and > 0 (else MX_ERR_VALUE). workspace: mx_nvfp4_linear_workspace_size(M, K)
 * bytes, 256-byte aligned. Alignment: x, w, y 16 bytes; w_s 2 bytes.
 */
MX_API mx_status mx_nvfp4_linear(const uint16_t* x, int64_t M, int64_t K, const uint8_t* w,
                                 const uint8_t* w_s, float w_global, int64_t N, float x_global, uint16_t* y,
                                 void* workspace, size_t ws_bytes, void* stream);
MX_API size_t mx_nvfp4_linear_workspace_size(int64_t M, int64_t K);

/*
 * mx_nvfp4_expert_mlp -- one expert with NVFP4 weights, as the pages run the
 * experts on B200 (gate and up with their own weight_scale_2: page "Current
 * Bug: vLLM produces empty/garbage output", "Revised Plan", Phase 2):
 *   g = NVLIN(x, w1, w1_global), u = NVLIN(x, w3, w3_global) (x quantised to
 *   NVFP4 with x_global), h = bf16(silu(g) * u), y = NVLIN(h, w2, w2_global)
 *   with h quantised to NVFP4 with h_global; NVLIN is the mx_nvfp4_linear
 *   computation, so g and u are bf16 before the SiLU.
 *   w1, w3 [inter, hidden/2] codes + [inter, hidden/16] E4M3; w2 [hidden, inter/2] + [hidden, inter/16].
 * hidden, inter multiples of 128. x_global, h_global finite and >= 2^-117;
 * weight globals finite and > 0 (else MX_ERR_VALUE). workspace:
 * mx_nvfp4_expert_mlp_workspace_size(M, hidden, inter) bytes, 256-byte aligned.
 * Alignment: x, y, codes 16 bytes; E4M3 scales 2 bytes.
 */
MX_API mx_status mx_nvfp4_expert_mlp(const uint16_t* x, int64_t M, int64_t hidden, int64_t inter,
                                     const uint8_t* w1, const uint8_t* w1_s, float w1_global,
                                     const uint8_t* w3, const uint8_t* w3_s, float w3_global,
                                     const uint8_t* w2, const uint8_t* w2_s, float w2_global,
                                     float x_global, float h_global, uint16_t* y, void* workspace,
                                     size_t ws_bytes, void* stream);
MX_API size_t mx_nvfp4_expert_mlp_workspace_size(int64_t M, int64_t hidden, int64_t inter);

/*
 * mx_grouped_nvfp4_expert_mlp -- E routed experts with NVFP4 weights, as the
 * pages run the MoE on B200 (w13/w2 in NVFP4 with per-expert weight_scale_2).
 * Routing, gate weights, ids outside [0, E) and the combine as for
 * mx_grouped_expert_mlp; each pair runs the steps of mx_nvfp4_expert_mlp with
 * its expert's globals:
 *   w1, w3 codes [E, inter, hidden/2], E4M3 scales [E, inter, hidden/16]
 *   w2 codes [E, hidden, inter/2], E4M3 scales [E, hidden, inter/16]
 *   w1_global, w3_global, w2_global: DEVICE arrays of E fp32 (finite, > 0;
 *     not checked on the host)
 *   x_global, h_global: fp32 activation and intermediate globals (host values)
 * 1 <= k <= E <= 512; hidden % 128 == 0; inter % 128 == 0. workspace:
 * mx_grouped_nvfp4_expert_mlp_workspace_size(T, hidden, inter, k, E) bytes,
 * 256-byte aligned. Alignment: x, y, codes 16 bytes; E4M3 scales 2 bytes;
 * ids, gate weights and globals 4 bytes.
 */
MX_API mx_status mx_grouped_nvfp4_expert_mlp(const uint16_t* x, int64_t T, int64_t hidden, int64_t inter,
                                             const int32_t* topk_ids, const float* topk_w, int32_t k,
                                             int32_t E, const uint8_t* w1, const uint8_t* w1_s,
                                             const float* w1_global, const uint8_t* w3, const uint8_t* w3_s,
                                             const float* w3_global, const uint8_t* w2, const uint8_t* w2_s,
                                             const float* w2_global, float x_global, float h_global,
                                             uint16_t* y, void* workspace, size_t ws_bytes, void* stream);
MX_API size_t mx_grouped_nvfp4_expert_mlp_workspace_size(int64_t T, int64_t hidden, int64_t inter, int32_t k,
                                                         int32_t E);

/*
 * mx_fp8_expert_mlp -- the shared expert in the original checkpoint's FP8
 * format (page "2026-05-08 DeepSeek V4 Pro NVFP4 Quantization", "Status"):
 *   g = FP8LIN(x, w1), u = FP8LIN(x, w3), h = bf16(silu(g) * u), y = FP8LIN(h, w2)
 * with FP8LIN the mx_fp8_block_linear computation (MXFP8 activations, bf16
 * output), so g and u are bf16 before the SiLU. g and u come from one GEMM
 * over w1 and w3 whose epilogue forms h, so they are never stored; the
 * workspace holds the MXFP8 x, h and the MXFP8 h.
 *   x  [M, hidden] bf16; y [M, hidden] bf16
 *   w1, w3 [inter, hidden] e4m3fn, scales [inter/128, hidden/128] E8M0
 *   w2 [hidden, inter] e4m3fn, scales [hidden/128, inter/128] E8M0
 * hidden, inter multiples of 128 and <= 8192. workspace: at least
 * mx_fp8_expert_mlp_workspace_size(M, hidden, inter) bytes, 256-byte aligned.
 * Alignment: x, y and weight codes 16 bytes.
 */
MX_API mx_status mx_fp8_expert_mlp(const uint16_t* x, int64_t M, int64_t hidden, int64_t inter,
                                   const uint8_t* w1, const uint8_t* w1_s, const uint8_t* w3,
                                   const uint8_t* w3_s, const uint8_t* w2, const uint8_t* w2_s, uint16_t* y,
                                   void* workspace, size_t ws_bytes, void* stream);
MX_API size_t mx_fp8_expert_mlp_workspace_size(int64_t M, int64_t hidden, int64_t inter);

/*
 * mx_debug_gemm_f32 -- test hook, not part of the hot path: the L1/L2 contraction of
 * the pages' pipeline ("Current Bug ...", "Revised Plan", Phase 1) with an fp32
 * output instead of the fused epilogues: C[M, N] = A . B^T in fp32
 * for MXFP4 A (codes [M, K/2], scales [M, K/32]) and B (codes [N, K/2], scales
 * [N, K/32]) through the same scaled-MFMA kernel as the MLP. K % 128 == 0,
 * N % 4 == 0. Alignment: codes and c 16 bytes, scales 4 bytes.
 */
MX_API mx_status mx_debug_gemm_f32(const uint8_t* a, const uint8_t* a_s, const uint8_t* b,
                            const uint8_t* b_s, int64_t M, int64_t N, int64_t K, float* c,
                            void* stream);

/*
 * mx_moe_runner -- the routed experts as a serving runner: its workspace is
 * allocated once (hipMalloc at creation) and one mx_grouped_expert_mlp call
 * over fixed device buffers is captured once into a hipGraph, which
 * mx_moe_runner_replay launches on any stream. The pages' serving plan is a
 * runner with pre-allocated buffers whose calls are CUDA-graph safe (page
 * "Current Bug: vLLM produces empty/garbage output", section "Revised Plan",
 * Phase 1).
 *   create: the arguments of mx_grouped_expert_mlp (T >= 1) without workspace
 *     and stream. It waits for the device to finish the work already enqueued
 *     (so inputs just written on any stream are seen), runs the call once
 *     eagerly on a private stream (validating every argument; on failure nothing
 *     is captured and *out stays NULL), synchronises, then captures it. Every
 *     pointer is fixed in the graph; the NVFP4 global is read from
 *     *requant_global at each replay. Fails with MX_ERR_VALUE while
 *     mx_profile_start() is on.
 *   replay: the captured call on `stream`, reading the current contents of x,
 *     topk_ids, topk_w and *requant_global (the caller refreshes them in place)
 *     and writing y.
 *     Replays on one runner must not overlap (they share the workspace).
 *   destroy: waits for the runner's stream, frees the graph and the workspace.
 *     The caller must have finished its replays (synchronise their streams).
 * The bound buffers must outlive the runner.
 */
typedef struct mx_moe_runner mx_moe_runner;
MX_API mx_status mx_moe_runner_create(const uint16_t* x, int64_t T, int64_t hidden, int64_t inter,
                                      const int32_t* topk_ids, const float* topk_w, int32_t k, int32_t E,
                                      const uint8_t* w1, const uint8_t* w1_s, const uint8_t* w3,
                                      const uint8_t* w3_s, const uint8_t* w2, const uint8_t* w2_s,
                                      const uint8_t* packed_scales, const uint8_t* packed_codes,
                                      mx_format requant, const float* requant_global, uint16_t* y,
                                      mx_moe_runner** out);
MX_API mx_status mx_moe_runner_replay(mx_moe_runner* r, void* stream);
MX_API mx_status mx_moe_runner_destroy(mx_moe_runner* r);

/* Status text (static) and the calling thread's last error detail: the clear
 * failure messages the pages' debugging history calls for (wrong scale
 * handling, shape mistakes: "2026-05-11 - DeepSeek V4 NVFP4 vLLM Serving: Full
 * End-to-End", "What We Fixed" and "Outstanding Issues"). */
MX_API const char* mx_status_string(mx_status s);
MX_API const char* mx_last_error(void);

/*
 * Profiler (measurement support, not a step of the pages' pipeline): while
 * enabled, every kernel the library enqueues is bracketed by two
 * hipEvents recorded on the same stream. mx_profile_stop() waits for them and
 * returns, per kernel name, the summed duration and the launch count.
 */
typedef struct mx_phase_stat {
  char name[32];
  double total_ms;
  int64_t launches;
} mx_phase_stat;

MX_API mx_status mx_profile_start(void);
MX_API mx_status mx_profile_stop(mx_phase_stat* stats, int32_t max_stats, int32_t* n_stats);

/*
 * Measurement probes (not steps of the pages' pipeline): kernels whose measured
 * rates stand beside MI355X's published peaks (10.1 PFLOP/s dense FP4 matrix
 * math, 8 TB/s HBM3E) as the ceilings this machine reaches. Each result can be
 * checked, so a rate never comes from work the compiler dropped.
 *   mx_probe_mfma_fp4: `workgroups` x 8 waves, each running `iters` iterations
 *     of four independent V_MFMA_SCALE_F32_32X32X64_F8F6F4 on FP4 operands held
 *     in registers (scale bytes 127). FLOPs = workgroups * 8 * iters * 4 * 131072.
 *     operands: DEVICE, 512 x 16 uint32, the same for every workgroup, 16-byte
 *     aligned: thread t's FP4 A operand is words [16t, 16t+4) and its B operand
 *     words [16t+8, 16t+12) (32 E2M1 codes each; the other words are not read).
 *     out: DEVICE, workgroups * 512 floats, out[w * 512 + t] = the sum of
 *     thread t's 64 accumulator values. 1 <= workgroups <= 65536,
 *     1 <= iters <= 2^20.
 *   mx_probe_read: reads `bytes` of src once. mode 0 into registers
 *     (GLOBAL_LOAD_DWORDX4), mode 1 into LDS (GLOBAL_LOAD_LDS_DWORDX4, the copies
 *     of the tiled GEMMs); each wave issues loads_per_wave (8 or 32) 16-byte
 *     loads per lane at once, 256-thread workgroups. bytes > 0 and a multiple
 *     of loads_per_wave * 1024; src 16-byte aligned; out: DEVICE, workgroups *
 *     4 uint32 whose XOR equals the XOR of all 32-bit words of src.
 *   mx_probe_copy: dst[0, bytes) = src[0, bytes); bytes % 16 == 0, both 16-byte
 *     aligned, not overlapping.
 * Errors as for every entry point (MX_ERR_NULL / SHAPE / ALIGN / VALUE / HIP).
 */
MX_API mx_status mx_probe_mfma_fp4(const uint32_t* operands, int64_t iters, int32_t workgroups, float* out,
                                   void* stream);
MX_API mx_status mx_probe_read(int32_t mode, int32_t loads_per_wave, int32_t workgroups, const void* src,
                               int64_t bytes, uint32_t* out, void* stream);
MX_API mx_status mx_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H_ */
