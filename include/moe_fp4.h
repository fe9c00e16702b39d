/*
 * moe_fp4 — block-scaled FP4 mixture-of-experts layer for AMD MI355X (gfx950).
 *
 * The layer (b12x PR #22, "rp-native tiny-decode kernel for w4a8_mx (M=1)",
 * What section, FC1 and FC2 bullets): for every token t and every route j of
 * its top-k, with expert e = ids[t][j],
 *     gate_n = sum_h x[t][h] * W13[e][n][h],        n in [0, I)
 *     up_n   = sum_h x[t][h] * W13[e][I + n][h]
 *     a_n    = gate_n / (1 + exp(-gate_n)) * up_n     (SiLU(gate) * up)
 *     y_h    = sum_n a_n * W2[e][h][n]
 *     out[t][h] = bf16( sum_j w[t][j] * y_h )         (fp32 sum, one rounding)
 * Weights are E2M1 nibbles with block scales:
 *   MXFP4: one UE8M0 scale byte (2^(b-127)) per 32 consecutive K elements;
 *   NVFP4: one E4M3 scale byte per 16 consecutive K elements, times an fp32
 *          global multiplier per expert per matrix (g13[e] for W13, g2[e]
 *          for W2).
 * A route whose id is negative or >= E reads no weights and contributes
 * nothing (b12x PR #311, commit message on the FC2-only endpoint, and its
 * review of tiny_decode.py); a token with no valid route yields +0.
 *
 * Logical weight layout (the input of moe_fp4_prepare), row-major, G = 32
 * (MXFP4) or 16 (NVFP4), for the gated activations (relu2: W13 has I rows):
 *   w13_codes  u8[E][2I][H/2]  rows [0, I) gate, [I, 2I) up; element 2b of a
 *                              row in the low nibble of byte b, 2b+1 in the high
 *   w13_scales u8[E][2I][H/G]
 *   w2_codes   u8[E][H][I/2]
 *   w2_scales  u8[E][H][I/G]
 *   g13, g2    f32[E]          NVFP4 only (NULL for MXFP4)
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned device memory; the library allocates
 *     nothing, keeps no global state (except moe_fp4_forward_noalloc's
 *     workspace, below) and never synchronises.  Work is queued on `stream`
 *     (a hipStream_t; NULL is the default stream).
 *   - Inputs are never written.  Arguments are checked before any launch; a
 *     rejected call launches nothing.  A failed launch returns MOE_FP4_EHIP.
 *   - Data conditions are not errors: invalid ids contribute zero; NaN or Inf
 *     in scales, globals or activations of valid routes propagate.
 */
#ifndef MOE_FP4_H
#define MOE_FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_FP4_OK = 0,
  MOE_FP4_EINVAL = 1,      /* null/misaligned pointer, bad size or count */
  MOE_FP4_EUNSUPPORTED = 2,/* valid request outside what the library handles */
  MOE_FP4_EWORKSPACE = 3,  /* workspace or prepared buffer too small */
  MOE_FP4_EHIP = 4         /* a HIP launch or runtime call failed */
} moe_fp4_status;

typedef enum {
  MOE_FP4_MXFP4 = 1, /* E2M1 + UE8M0 scale per 32 */
  MOE_FP4_NVFP4 = 2  /* E2M1 + E4M3 scale per 16, times an fp32 global */
} moe_fp4_format;

/* Activation format of the grouped path.
 *   BF16:  x and SiLU(gate) * up enter the GEMMs at bf16 precision or better
 *          (the layer as defined above).
 *   MXFP8: the W4A8-MX variant (b12x PR #22, Measured table and its note on
 *          the dynamic path, which quantises activations to MXFP8; MXFP4
 *          weights only).  x is quantised per token in blocks of 32 along H,
 *          and SiLU(gate) * up (from fp32 FC1 outputs, rounded to fp32) per
 *          route in blocks of 32 along I, each to MXFP8 as the OCP MX format
 *          defines it: one UE8M0 scale 2^(floor(log2(max |v|)) - 8) per
 *          block (clamped to 2^[-127, 127]; a zero block gets byte 0, a
 *          block with a NaN or an infinity byte 255), elements v / scale
 *          rounded to nearest-even E4M3 with magnitudes capped at 448 (a
 *          NaN/Inf block's codes are all 0x7F).  FC1 and FC2 then run on the
 *          scaled matrix instruction with fp32 accumulation.  The decode
 *          path (small M) keeps bf16 activations in both modes, as the
 *          pages' M = 1 kernel does. */
typedef enum {
  MOE_FP4_ACT_BF16 = 0,
  MOE_FP4_ACT_MXFP8 = 1
} moe_fp4_act_format;

/* Gated activation a = f(gate, up) between FC1 and FC2.  The pages name
 * SiLU (b12x PR #22, What: FC2 applies SiLU inline), gelu_tanh and
 * swigluoai_uninterleave with alpha, beta and limit (flashinfer #4285,
 * reviews of moe_activation.py and of the direct micro kernel's activation
 * coverage) without formulas; these are the standard definitions:
 *   SILU:      gate * sigmoid(gate) * up
 *   GELU_TANH: 0.5 * gate * (1 + tanh(sqrt(2/pi) * (gate + 0.044715 * gate^3))) * up
 *   SWIGLUOAI: g = min(gate, limit), u = max(min(up, limit), -limit),
 *              g * sigmoid(alpha * g) * (u + beta)
 *              (act_alpha, act_beta finite, act_limit > 0 or +inf; gate and
 *              up are the separate halves of W13; a NaN passes the clamps)
 *   RELU2:     not gated (b12x PR #311, commit message on the FP4 quantiser,
 *              which treats relu2 apart from the gated activations): W13 has
 *              I rows (w13_codes u8[E][I][H/2], w13_scales u8[E][I][H/G]),
 *              h = x . W13[n] and a_n = max(h, 0)^2; I must be a multiple
 *              of 64 (else MOE_FP4_EUNSUPPORTED)
 * Every path applies the same function. */
typedef enum {
  MOE_FP4_FN_SILU = 0,
  MOE_FP4_FN_GELU_TANH = 1,
  MOE_FP4_FN_SWIGLUOAI = 2,
  MOE_FP4_FN_RELU2 = 3
} moe_fp4_act_fn;

/* Resident form of the block scales (scale_format in moe_fp4_desc).
 *   PLAIN: the scale bytes as given.
 *   CSF:   in addition, each weight row's scale bytes compressed as a row
 *          base byte plus an offset per block, one bit (MXFP4, offset 0 or
 *          1) or four bits (NVFP4, 0..15), the byte being base + offset
 *          (b12x PR #459, "Reduce NVFP4-CSF scale reconstruction overhead",
 *          commit messages: one-bit MXFP4 and four-bit NVFP4 offsets from a
 *          row base byte).  The base is the row's smallest byte; a row whose
 *          bytes span more than the offsets reach, or whose smallest byte is
 *          255, is an exception read from the plain bytes.  Lossless: every
 *          result equals the PLAIN one bit for bit.  The decode path reads
 *          the compressed scales (one 4-byte word of base byte and offsets
 *          per row and 24 (MXFP4) or 3 (NVFP4) chunks of 32 weights, against
 *          1 or 2 plain bytes per chunk) and the plain bytes of exception
 *          rows only; the grouped path and moe_fp4_unprepare read the plain
 *          bytes.  The prepared buffer grows by the compressed blocks
 *          (moe_fp4_prepared_bytes). */
typedef enum {
  MOE_FP4_SCALES_PLAIN = 0,
  MOE_FP4_SCALES_CSF = 1
} moe_fp4_scale_format;

/* Shape of one MoE layer.  H and I must be multiples of 32 for both formats
 * (the kernels work in 32-element units); max_tokens is the largest M that
 * later forward calls will pass, used only to size the workspace.
 * act_format is a moe_fp4_act_format (0 keeps bf16 activations); MXFP8 with
 * NVFP4 weights returns MOE_FP4_EUNSUPPORTED.  act_fn and its parameters
 * choose the gated activation (0 and zeros: SiLU).  scale_format is a
 * moe_fp4_scale_format (0: plain). */
typedef struct {
  int32_t format;      /* moe_fp4_format */
  int32_t num_experts; /* E, resident experts; ids outside [0, E) are invalid */
  int32_t hidden;      /* H: K of FC1, N of FC2 */
  int32_t inter;       /* I: intermediate size */
  int32_t top_k;       /* k: routes per token */
  int32_t max_tokens;  /* capacity for workspace sizing */
  int32_t act_format;  /* moe_fp4_act_format */
  int32_t act_fn;      /* moe_fp4_act_fn (0: SiLU) */
  float act_alpha;     /* SWIGLUOAI only, else ignored */
  float act_beta;
  float act_limit;
  int32_t scale_format; /* moe_fp4_scale_format */
} moe_fp4_desc;

/* Human-readable name of a status code (static string).  A diagnostic hook
 * of this library's own; no page defines one. */
const char* moe_fp4_status_string(moe_fp4_status s);

/* Bytes of the prepared (resident) weight buffer for `desc`.  It holds the
 * same codes, scale bytes and fp32 globals as the logical tensors, reordered,
 * plus zero padding to whole tiles (b12x PR #459, "Reduce NVFP4-CSF scale
 * reconstruction overhead", commit messages: preparation keeps checkpoint
 * bytes and prepared memory sizes). */
moe_fp4_status moe_fp4_prepared_bytes(const moe_fp4_desc* desc, size_t* bytes);

/* Weight preparation, once per layer at load time (b12x PR #459, "Reduce
 * NVFP4-CSF scale reconstruction overhead", commit messages: keep the exact
 * FP4 nibbles and scale bytes, no requantisation, reorder resident offsets
 * for contiguous decoding).  A pure byte permutation of the logical tensors
 * above into `prepared` (device, 256-byte aligned, `prepared_bytes` >=
 * moe_fp4_prepared_bytes).  Logical inputs must be 16-byte aligned device
 * buffers; g13/g2 are required for NVFP4 and must be NULL for MXFP4. */
moe_fp4_status moe_fp4_prepare(const moe_fp4_desc* desc, const uint8_t* w13_codes,
                               const uint8_t* w13_scales, const uint8_t* w2_codes,
                               const uint8_t* w2_scales, const float* g13, const float* g2,
                               void* prepared, size_t prepared_bytes, void* stream);

/* Inverse of moe_fp4_prepare: writes the logical tensors back from a
 * prepared buffer (used to check that preparation is a bijection). */
moe_fp4_status moe_fp4_unprepare(const moe_fp4_desc* desc, const void* prepared,
                                 uint8_t* w13_codes, uint8_t* w13_scales, uint8_t* w2_codes,
                                 uint8_t* w2_scales, float* g13, float* g2, void* stream);

/* Workspace bytes for forward calls on `desc` (device scratch, 256-byte
 * aligned, caller-owned).  The size depends only on the descriptor, so one
 * workspace serves every M <= max_tokens; `M` is checked against max_tokens
 * (b12x PR #311, review comment on the intermediate_cache13 sizing: a
 * workspace must hold the largest requirement over every token count the
 * caller plans, or a smaller launch under-allocates).
 * The grouped path needs about 4I + 4H bytes per route (max_tokens * k
 * routes) with bf16 activations, and about I + 4H per route plus H per
 * token with MXFP8 activations.  Its contents on entry do not matter and
 * are overwritten. */
moe_fp4_status moe_fp4_workspace_bytes(const moe_fp4_desc* desc, int32_t M, size_t* bytes);

/* The layer.  x: bf16 [M][H]; topk_ids: int32 [M][k]; topk_w: fp32 [M][k]
 * (used as given, no renormalisation); out: bf16 [M][H], overwritten.  All
 * device pointers, 16-byte aligned except topk_ids (element size) and topk_w
 * (4-byte).  M may be 0 (nothing is launched).  Calls that share a workspace
 * must be ordered on one stream.
 *
 * Two execution paths, chosen by M (both compute the layer above):
 *   decode  FC1 and FC2 as streamed FP4 GEMVs in one launch each, FC1
 *           over chunks of up to C = min(16, 64 / k) tokens, each routed
 *           expert's weights read once per chunk (b12x PR #22, What);
 *           results are bit-reproducible.  Taken for M <= C; with bf16
 *           activations for M <= 2C, and for M <= 6C when the chunks'
 *           route slots ceil(M / C) * C * k are fewer than E (few routes
 *           per expert); and for every M when E > 8192.
 *   grouped (any other M): routes grouped by expert in route order, FC1 and
 *           FC2 as grouped GEMMs on the matrix cores over bf16 operands (FP4
 *           dequantised exactly) with fp32 accumulation, per-route fp32 rows
 *           summed per token in route order and cast once (flashinfer #4285,
 *           description: the prefill kernel's per-expert tiles; b12x PR #311,
 *           commit message on the prefill fused-sum epilogue).  The
 *           activation enters FC2 as a pair of bf16 values (hi + lo, 16
 *           significant bits), as in the decode path.  With act_format =
 *           MXFP8 both GEMMs instead take MXFP8 activations on the scaled
 *           FP8 x FP4 matrix instruction (the W4A8-MX variant above).
 *           Results are bit-reproducible.
 * The activation function (act_fn) is the same on both paths.
 * Returns MOE_FP4_EUNSUPPORTED when max_tokens * k > 2^22, or when the path
 * the call needs cannot run it: the grouped path with E > 8192, the decode
 * path with k > 64 or M > 65535. */
moe_fp4_status moe_fp4_forward(const moe_fp4_desc* desc, const void* prepared,
                               const uint16_t* x, int32_t M, const int32_t* topk_ids,
                               const float* topk_w, uint16_t* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Same, with int64 route ids (any int64 value outside [0, E) is invalid).
 * Both id widths are served (b12x PR #459, "Reduce NVFP4-CSF scale
 * reconstruction overhead", commit messages: programs kept for both routing
 * integer types). */
moe_fp4_status moe_fp4_forward_i64(const moe_fp4_desc* desc, const void* prepared,
                                   const uint16_t* x, int32_t M, const int64_t* topk_ids,
                                   const float* topk_w, uint16_t* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): moe_fp4_forward
 * (int32 ids) without a workspace argument.  The workspace is a block of
 * 64 MiB of device memory that the library itself holds, one per GPU it
 * runs on, from the first call on that GPU until the process ends; the call
 * allocates nothing.  `desc` must need at most that much workspace
 * (moe_fp4_workspace_bytes <= 64 MiB), else MOE_FP4_EWORKSPACE; other
 * arguments, checks and results are those of moe_fp4_forward.  The stream
 * must belong to the current device.  All calls on one GPU share that
 * GPU's block: calls that overlap on one GPU (other streams, other host
 * threads without ordering) race on it and give wrong results; calls
 * ordered on one stream are safe.  Its contents on entry do not matter. */
moe_fp4_status moe_fp4_forward_noalloc(const moe_fp4_desc* desc, const void* prepared,
                                       const uint16_t* x, int32_t M, const int32_t* topk_ids,
                                       const float* topk_w, uint16_t* out, void* stream);

/* Test hook of this library's own: dequantise one expert matrix from the
 * prepared buffer with the same decode instructions the forward kernels use,
 * into fp32 row-major `out` ([2I][H] for which = 0 (W13), [H][I] for
 * which = 1 (W2); device, 4-byte aligned, caller-owned).  Each value is
 * (E2M1 code * block scale) rounded to fp32, times the global (NVFP4), so
 * the tests can compare every prepared byte with the oracle's dequantisation
 * bit for bit (b12x PR #459, PR body: every arm is checked against an exact
 * byte oracle). */
moe_fp4_status moe_fp4_dequant_export(const moe_fp4_desc* desc, const void* prepared,
                                      int32_t expert, int32_t which, float* out,
                                      void* stream);

/* Execution path selector for moe_fp4_forward_ex. */
typedef enum {
  MOE_FP4_PATH_AUTO = 0,    /* by M, as moe_fp4_forward */
  MOE_FP4_PATH_DECODE = 1,  /* decode path (in chunks); MOE_FP4_EUNSUPPORTED when k > 64 or M > 65535 */
  MOE_FP4_PATH_GROUPED = 2  /* grouped path at any M */
} moe_fp4_path;

/* Launch shape of the decode kernels and the path; 0 in a field keeps the
 * built-in choice.
 *   fc1_chunks_per_wave: 32-element K chunks per FC1 wave (4, 8 or 16)
 *   fc1_rows: FC1 rows per workgroup, half gate and half up (16 or 32)
 *   fc2_rows: FC2 rows of H per workgroup (8, 16 or 32; at least 64 divided
 *             by FC2's chunk lanes, which is 4, 8 or 16 for I up to 128, 256
 *             or beyond)
 *   path: a moe_fp4_path */
typedef struct {
  int32_t fc1_chunks_per_wave;
  int32_t fc1_rows;
  int32_t fc2_rows;
  int32_t path;
} moe_fp4_tuning;

/* Measurement and test hook: moe_fp4_forward (int32 ids) with an explicit
 * launch shape and path (`tuning` may be NULL) and only part of the call
 * queued, so a caller can put events between the two halves: phases = 1
 * queues the first half (decode: FC1; grouped: routing and FC1), which fills
 * the workspace's activation; 2 queues the second half (FC2 and the combine
 * into `out`; it must follow a phase-1 call with the same arguments on the
 * same stream); 3 queues both.  On the grouped path, 4 queues only its
 * routing (the grouping of the routes by expert) and 8 only its combine
 * (which reads what a phase-2 call left), so the two GEMM launches can be
 * timed on their own; the decode path rejects 4 and 8. */
moe_fp4_status moe_fp4_forward_ex(const moe_fp4_desc* desc, const void* prepared,
                                  const uint16_t* x, int32_t M, const int32_t* topk_ids,
                                  const float* topk_w, uint16_t* out, void* workspace,
                                  size_t workspace_bytes, const moe_fp4_tuning* tuning,
                                  int32_t phases, void* stream);

/* The path and launch shape that moe_fp4_forward_ex takes for M tokens with
 * `tuning` (NULL: moe_fp4_forward's choice), written to `plan` with every
 * field resolved: path is MOE_FP4_PATH_DECODE or MOE_FP4_PATH_GROUPED, and
 * the decode shape fields are 0 on the grouped path.  Returns what
 * moe_fp4_forward_ex would return for an invalid or unsupported request;
 * launches nothing. */
moe_fp4_status moe_fp4_plan(const moe_fp4_desc* desc, int32_t M, const moe_fp4_tuning* tuning,
                            moe_fp4_tuning* plan);

/* The MXFP8 quantisation of the MXFP8 activation format (see
 * moe_fp4_act_format), as the grouped path applies it to x: bf16 `x`
 * [rows][cols] (device, 16-byte aligned, cols a multiple of 32) to E4M3
 * `codes` [rows][cols] (device, 8-byte aligned) and UE8M0 `scales`
 * [rows][cols / 32] (device), one scale per 32 consecutive values of a row.
 * rows may be 0 (nothing is launched). */
moe_fp4_status moe_fp4_mxfp8_quantize(const uint16_t* x, int64_t rows, int32_t cols, uint8_t* codes,
                                      uint8_t* scales, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP4_H */
