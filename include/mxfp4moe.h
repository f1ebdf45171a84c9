/*
 * mxfp4moe.h -- C ABI of the MI355X (gfx950) MXFP4 weight-quantized mixture-of-experts MLP.
 *
 * Sources, cited by page title and section:
 *   [EN] "Transformers 4.40 performance upgrades for OpenAI GPT-OSS: zero-build kernels, MXFP4
 *        quantization, parallelism, and faster loading" (agentlenshq.com, English page),
 *        section "MXFP4 4-Bit Quantization" (subsections "What MXFP4 Is", "Native Support in
 *        transformers", "Memory Savings"); section "Zero-Build Kernels from the Hub" (the MoE MLP
 *        kernel is the MegaBlocks MoE layer there).
 *   [GGUF] "Hugging Face Transformers GGUF 지원" (agentlenshq.com, Korean page), section
 *        "ggml Metal 커널 통합": the quantized matmul reads packed weights without expanding
 *        them first, and MoE expert selection is a top-k.
 * The pages fix: E2M1 elements (1 sign, 2 exponent, 1 mantissa bit) and one shared scale per
 * 32-element block. The library fixes what they leave open, the same way everywhere:
 *   - scale: E8M0 byte b, value 2^(b-127); b = clamp(floor(log2 amax) - 2, -127, 127) + 127,
 *     amax = 0 gives b = 0; a block with NaN/Inf gets b = 255 (decodes to NaN) and codes 0;
 *   - elements: nearest E2M1 value to x / 2^(b-127), ties to the even code, magnitudes above 6
 *     saturate to 6; sign bit = sign bit of x;
 *   - layout ("packed MXFP4 tensor" [rows][K]): row-major, K contiguous; packed bytes
 *     uint8[rows][K/2] with element 2j in the low nibble of byte j; scales uint8[rows][K/32];
 *   - MoE expert: gate_up rows [0, F) = gate, [F, 2F) = up; h = silu(gate) * up, rounded to bf16;
 *     expert output = h W_down^T; token output = sum over its k experts of weight * output;
 *   - router: logits = x W_r^T + b; top-k by (logit desc, expert index asc); softmax over the k.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked host. bf16 tensors are passed as uint16_t bit
 *     patterns. The caller owns every buffer; the library never allocates or frees memory and
 *     never synchronizes (the diagnostics mx_get_device_error, mx_workspace_status and
 *     mx_profile_read are the exceptions). Work is enqueued on `stream` (a hipStream_t; NULL =
 *     the default stream) and outputs are valid once it completes.
 *   - Inputs and outputs must not alias.
 *   - Argument errors are found on the host before anything is launched and return a status
 *     (never a C++ exception); mx_last_error() then describes it. A failed launch returns
 *     MX_ERR_HIP. Faults inside kernels surface at the caller's next synchronization.
 *   - The library runs on gfx950 only: other devices get MX_ERR_UNSUPPORTED.
 *   - Zero-sized work (rows = 0, T = 0, M = 0) returns MX_OK and launches nothing.
 */
#ifndef MXFP4MOE_H
#define MXFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MX_OK = 0,
  MX_ERR_NULL = 1,        /* a required pointer is NULL */
  MX_ERR_SHAPE = 2,       /* a size is negative, not a multiple of 32 where required, or too big */
  MX_ERR_ALIGN = 3,       /* a pointer lacks the alignment the entry point states */
  MX_ERR_DTYPE = 4,       /* unknown dtype enum */
  MX_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the matching *_workspace() query */
  MX_ERR_UNSUPPORTED = 6, /* not a gfx950 device, or an unknown flag / descriptor version */
  MX_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed */
} mx_status;

typedef enum { MX_F32 = 0, MX_BF16 = 1 } mx_dtype;

/* Activation variant: the GEMM A-operands (x along H, and the bf16 SwiGLU output h along F) are
 * themselves MXFP4-quantized with the rule above and multiplied on the scaled FP4 matrix cores. */
#define MX_ACT_MXFP4 0x1u
/* The expert weights of mxfp4_moe_mlp are in the tiled layout written by mxfp4_tile_weights. */
#define MX_WEIGHTS_TILED 0x2u
/* mxfp4_moe_mlp runs the whole MLP (routing included) as one persistent launch whose steps wait
 * for each other on the GPU; for decode-sized batches (see mxfp4_moe_mlp). */
#define MX_SINGLE_LAUNCH 0x4u

/* Upper limits checked on the host. */
#define MX_MAX_EXPERTS 256
#define MX_MAX_TOPK 8
#define MX_MAX_K 8192            /* reduction length K of mxfp4_linear */
#define MX_MAX_MOE_DIM 3072      /* H and F of the MoE MLP */

/* ------------------------------------------------------------------------------------------------
 * mxfp4_quantize -- pack `rows` rows of K values into MXFP4 ([EN] "What MXFP4 Is").
 *   src     [rows][K] fp32 (src_dtype MX_F32) or bf16 bits (MX_BF16), row-major.
 *   packed  [rows][K/2] bytes out; scales [rows][K/32] bytes out (layout above).
 *   K % 32 == 0 (else MX_ERR_SHAPE); src 16-byte aligned (fp32) or 8-byte aligned (bf16),
 *   packed 16-byte aligned (else MX_ERR_ALIGN). Bit-exact: the result depends only on the values.
 * ---------------------------------------------------------------------------------------------- */
mx_status mxfp4_quantize(const void* src, mx_dtype src_dtype, int64_t rows, int64_t K,
                         uint8_t* packed, uint8_t* scales, void* stream);

/* ------------------------------------------------------------------------------------------------
 * mxfp4_dequantize -- exact values code * 2^(b-127) ([EN] "Memory Savings": the de-quantized
 * model is the bf16 one).
 *   packed [rows][K/2], scales [rows][K/32]; dst [rows][K] fp32 or bf16 bits (dst_dtype).
 *   Every value is exact in both types except overflow past the type's max (-> +-Inf, as IEEE
 *   rounding gives) and scale byte 255 (-> NaN). K % 32 == 0; packed 16-byte aligned; dst
 *   16-byte aligned.
 * ---------------------------------------------------------------------------------------------- */
mx_status mxfp4_dequantize(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t K,
                           void* dst, mx_dtype dst_dtype, void* stream);

/* ------------------------------------------------------------------------------------------------
 * mxfp4_tile_weights -- rearrange G packed matrices [R][K] into the layout in which the grouped
 * GEMMs of mxfp4_moe_mlp (flag MX_WEIGHTS_TILED) read every weight stage as whole cache lines.
 * The pages put the MXFP4 conversion at model load, through the quantizer and its integration
 * hooks ([EN] "MXFP4 4-Bit Quantization" > "Native Support in transformers"), and have the
 * quantized matmul read the packed weights as they are stored ([GGUF] "ggml Metal 커널 통합");
 * this is that load-time step for these kernels: weights are static, so it runs once, and it is
 * a pure permutation of bytes (every weight stays packed, nothing is decoded):
 *   packed [G][R][K/2], scales [G][R][K/32] in (the layout above);
 *   packed_t [G][R/16][K/32][16][16] out: the 16 code bytes of block b of rows 16q..16q+15 as
 *     one 256-byte run, row r at byte 16*(r % 16);
 *   scales_t [G][K/32][R] out: the scale byte of (row r, block b) at b*R + r.
 *   R % 16 == 0, K % 32 == 0 (MX_ERR_SHAPE); packed and packed_t 16-byte aligned (MX_ERR_ALIGN);
 *   outputs must not overlap the inputs. Buffers are owned by the caller.
 * For the MoE weights: gate_up G = E, R = 2F, K = H; down G = E, R = H, K = F.
 * ---------------------------------------------------------------------------------------------- */
mx_status mxfp4_tile_weights(const uint8_t* packed, const uint8_t* scales, int64_t G, int64_t R,
                             int64_t K, uint8_t* packed_t, uint8_t* scales_t, void* stream);
/* mxfp4_tile_weights_ex -- the same with flags: MX_TILE_DEINTERLEAVE moves rows 2i to i and rows
 * 2i + 1 to R/2 + i while tiling (interleaved gate/up rows -> gate rows, then up rows; R % 32 ==
 * 0). Unknown flags: MX_ERR_UNSUPPORTED. */
#define MX_TILE_DEINTERLEAVE 0x1u
mx_status mxfp4_tile_weights_ex(const uint8_t* packed, const uint8_t* scales, int64_t G,
                                int64_t R, int64_t K, uint32_t flags, uint8_t* packed_t,
                                uint8_t* scales_t, void* stream);

/* ------------------------------------------------------------------------------------------------
 * moe_route_topk -- router logits, top-k expert selection and softmax over the k selected
 * ([GGUF] "ggml Metal 커널 통합": top-k expert selection for MoE; the router itself is a reading).
 *   x [T][H] bf16, wr [E][H] bf16, br [E] fp32 or NULL (no bias).
 *   logits [T][E] fp32 out, or NULL (not stored: every workgroup then covers all experts of its
 *   16 tokens and selects from on-chip memory, which leaves small batches on fewer CUs);
 *   topk_idx [T][k] int32 out, in rank order (logit descending, lower expert index first on
 *   equal logits); topk_w [T][k] fp32 out.
 *   Limits: 1 <= k <= min(E, MX_MAX_TOPK), 1 <= E <= MX_MAX_EXPERTS, H % 32 == 0 (MX_ERR_SHAPE);
 *   x and wr 16-byte aligned (MX_ERR_ALIGN). Logits are fp32 sums of bf16 products; the top-k
 *   is exact given those logits.
 * ---------------------------------------------------------------------------------------------- */
mx_status moe_route_topk(const uint16_t* x, const uint16_t* wr, const float* br, int32_t T,
                         int32_t H, int32_t E, int32_t k, float* logits, int32_t* topk_idx,
                         float* topk_w, void* stream);

/* ------------------------------------------------------------------------------------------------
 * moe_permute -- group the T*k (token, slot) pairs by expert: histogram over experts, exclusive
 * prefix sum, stable scatter in (token, slot) order (the row grouping an MoE MLP kernel such as
 * [EN] "Zero-Build Kernels from the Hub"'s MegaBlocks MoE layer runs its grouped GEMMs on).
 *   topk_idx [T][k] int32 in.
 *   offsets [E+1] int32 out: expert e owns permuted rows [offsets[e], offsets[e+1]).
 *   perm [T*k] int32 out: perm[row] = t*k + j of the pair at permuted row `row`.
 *   inv [T*k] int32 out: inv[t*k + j] = its permuted row.
 *   ws: device workspace of moe_permute_workspace(T, k, E) bytes, 256-byte aligned, owned by the
 *   caller (contents need not be initialized). Large batches are then permuted by many
 *   workgroups (a histogram of every 1024-pair slice, then each slice placed from all slice
 *   histograms; from T*k >= 8192). ws may be NULL (ws_bytes ignored): one workgroup then does the whole
 *   permutation, with the same results element for element. A non-NULL ws smaller than the
 *   query is MX_ERR_WORKSPACE. The query is 0 for small batches.
 *   Indices outside [0, E) are left out of perm, their inv entry is -1, and the device error
 *   word gets MX_DEVERR_ROUTING (mx_get_device_error).
 *   Deterministic (no ordering by atomics). Limits as for moe_route_topk; T*k < 2^31.
 * ---------------------------------------------------------------------------------------------- */
size_t moe_permute_workspace(int32_t T, int32_t k, int32_t E);
mx_status moe_permute(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E, int32_t* offsets,
                      int32_t* perm, int32_t* inv, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------------
 * mxfp4_moe_mlp -- the whole MoE MLP: route -> permute -> gate_up grouped GEMM with fused SwiGLU
 * -> down grouped GEMM -> combine over the k experts, each scaled by its routing weight. The grouped
 * GEMMs read the packed weights and decode them in registers, never materializing bf16 weights
 * ([GGUF] "ggml Metal 커널 통합"; [EN] "MXFP4 4-Bit Quantization": MXFP4 weights served by
 * dedicated kernels instead of a bf16 fallback).
 * ---------------------------------------------------------------------------------------------- */
typedef struct mx_moe_desc {
  size_t struct_size;          /* sizeof(mx_moe_desc) or MX_MOE_DESC_SIZE_V1; else MX_ERR_UNSUPPORTED */
  int32_t T, H, F, E, k;       /* tokens, hidden, expert FFN width, experts, experts per token */
  uint32_t flags;              /* MX_ACT_MXFP4, MX_WEIGHTS_TILED, MX_SINGLE_LAUNCH, or 0 */
  mx_dtype out_dtype;          /* dtype of `out` */
  const uint16_t* x;           /* [T][H] bf16 */
  const uint16_t* wr;          /* [E][H] bf16 router weight; unused if topk_idx_in is given */
  const float* br;             /* [E] fp32 router bias, NULL = none */
  const int32_t* topk_idx_in;  /* [T][k] caller routing, NULL = route internally */
  const float* topk_w_in;      /* [T][k] caller routing weights (required with topk_idx_in) */
  const uint8_t* gu_packed;    /* [E][2F][H/2] (MX_WEIGHTS_TILED: mxfp4_tile_weights layout) */
  const uint8_t* gu_scales;    /* [E][2F][H/32] (tiled: [E][H/32][2F]) */
  const uint8_t* dn_packed;    /* [E][H][F/2] (tiled: mxfp4_tile_weights layout) */
  const uint8_t* dn_scales;    /* [E][H][F/32] (tiled: [E][F/32][H]) */
  void* out;                   /* [T][H] out_dtype */
  int32_t* topk_idx_out;       /* [T][k], NULL = not stored (internal routing only) */
  float* topk_w_out;           /* [T][k], NULL = not stored */
  float* logits_out;           /* [T][E], NULL = not stored */
  /* ---- expert activation (descriptors that end at logits_out -- struct_size ==
   * MX_MOE_DESC_SIZE_V1 -- read all of these as zero): the released gpt-oss models' clamped,
   * scaled SwiGLU with biases, which the pages leave open (the library's reading):
   *   a = x W_gu^T + gu_bias[e]; g, u = gate and up pre-activations of output column f;
   *   if swiglu_limit > 0: g = min(g, limit), u = clamp(u, -limit, limit) (gate clamped above);
   *   h = bf16(g * sigmoid(alpha * g) * (u + swiglu_up_shift)), alpha = swiglu_alpha or 1 if 0;
   *   expert output = h W_dn^T + dn_bias[e], then weighted by the routing weight and summed.
   * All zero: h = silu(g) * u, no biases -- the SwiGLU above. */
  uint32_t act_flags;          /* MX_GU_INTERLEAVED or 0 */
  float swiglu_alpha;          /* sigmoid scale (0 = 1) */
  float swiglu_limit;          /* clamp limit (<= 0: no clamp) */
  float swiglu_up_shift;       /* added to the (clamped) up value */
  const float* gu_bias;        /* [E][2F] fp32 in the caller's gate_up row order, NULL = none */
  const float* dn_bias;        /* [E][H] fp32, 16-byte aligned, NULL = none */
} mx_moe_desc;
/* The descriptor size before the expert activation fields (still accepted). */
#define MX_MOE_DESC_SIZE_V1 (offsetof(mx_moe_desc, act_flags))
/* act_flags: the caller's gate_up rows alternate gate and up (row 2i gate i, row 2i + 1 up i), as
 * in the released checkpoints. The kernels take gate rows first: such weights must be tiled with
 * mxfp4_tile_weights_ex(..., MX_TILE_DEINTERLEAVE, ...) and passed with MX_WEIGHTS_TILED
 * (row-major interleaved weights are MX_ERR_UNSUPPORTED); gu_bias stays in the caller's order. */
#define MX_GU_INTERLEAVED 0x1u

/* Bytes of workspace mxfp4_moe_mlp needs for this descriptor (0 if the shapes are invalid). */
size_t mxfp4_moe_mlp_workspace(const mx_moe_desc* desc);

/*   desc (host pointer) as above; ws: device workspace of at least mxfp4_moe_mlp_workspace(desc)
 *   bytes, 256-byte aligned, owned by the caller, contents need not be initialized.
 *   Limits: H, F multiples of 32 and <= MX_MAX_MOE_DIM; E, k as for moe_route_topk; all weight, x and
 *   out pointers 16-byte aligned. Routing indices outside [0, E) (caller routing) are skipped and
 *   flagged in the workspace status word (read it with mx_workspace_status); their tokens'
 *   outputs then lack those experts (the device error word gets MX_DEVERR_ROUTING too).
 *   Concurrent calls must use distinct workspaces.
 *   Internal routing is moe_route_topk's up to the fp32 summation order of the logits (small
 *   batches split H over more workgroups, partial sums added in a fixed order, so results do not
 *   depend on timing); the top-k is exact given the logits it reports.
 *   MX_SINGLE_LAUNCH ([GGUF] "생성 루프 최적화": generation is bound by the host-GPU round trips
 *   around each step): the same computation in one kernel launch -- routing, permutation,
 *   gate_up, down and combine wait for each other through counters the library keeps on each
 *   device -- with the same results up to the fp32 summation order of the logits. For
 *   decode-sized batches: T*k <= 2048, bf16 activations (with MX_ACT_MXFP4:
 *   MX_ERR_UNSUPPORTED). Calls with this flag must not overlap on one device (different streams
 *   or threads: serialize them); a wait that gives up (never in a correct run) sets
 *   MX_DEVERR_SYNC and leaves the outputs invalid. On MI355X the per-step launches (the flag
 *   left out) measured faster at the decode shapes tried; the flag serves callers that need the
 *   call to be a single kernel launch. */
mx_status mxfp4_moe_mlp(const mx_moe_desc* desc, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------------
 * mxfp4_moe_mlp_noalloc -- mxfp4_moe_mlp for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels, with the workspace taken from an array the library holds on each device
 * (MX_NOALLOC_SCRATCH_BYTES per device, kept until the process ends). The call allocates
 * nothing; the caller still owns desc's inputs and outputs.
 *   Problems whose workspace (mxfp4_moe_mlp_workspace(desc)) exceeds MX_NOALLOC_SCRATCH_BYTES
 *   return MX_ERR_WORKSPACE before anything is launched (32 MiB covers batches of up to about
 *   1900 token-expert pairs at H = F = 2880 with bf16 activations: 484 tokens at top-4).
 *   Every call on a device shares that device's array, which keeps the last call's contents
 *   (no call needs it cleared): calls that overlap on one device -- on different streams, or from
 *   different threads -- race and must be serialized by the caller. Other errors as for
 *   mxfp4_moe_mlp; mx_workspace_status does not apply (read mx_get_device_error instead).
 * ---------------------------------------------------------------------------------------------- */
#define MX_NOALLOC_SCRATCH_BYTES (32u << 20)
mx_status mxfp4_moe_mlp_noalloc(const mx_moe_desc* desc, void* stream);

/* ------------------------------------------------------------------------------------------------
 * mxfp4_linear -- dense weight-only linear y = x W^T with W packed MXFP4 [N][K] (the single
 * matrix product the MoE MLP's grouped GEMMs are made of; [EN] "MXFP4 4-Bit Quantization").
 *   x [M][K] bf16; packed [N][K/2], scales [N][K/32]; y [M][N] fp32 or bf16 (y_dtype).
 *   flags: 0 or MX_ACT_MXFP4 (x is MXFP4-quantized along K first; needs the workspace).
 *   ws: mxfp4_linear_workspace(M, K, N, flags) bytes, 256-byte aligned, owned by the caller,
 *   contents need not be initialized (ws may be NULL when that size is 0); it holds the
 *   quantized x (MX_ACT_MXFP4) and, for decode-sized M (<= 64), the fp32 partial sums of the
 *   workgroups that split K (summed in a fixed order: results do not depend on timing).
 *   K % 32 == 0, K <= MX_MAX_K; x, packed, y 16-byte aligned.
 * ---------------------------------------------------------------------------------------------- */
size_t mxfp4_linear_workspace(int32_t M, int32_t K, int32_t N, uint32_t flags);
mx_status mxfp4_linear(const uint16_t* x, int32_t M, int32_t K, const uint8_t* packed,
                       const uint8_t* scales, int32_t N, void* y, mx_dtype y_dtype, uint32_t flags,
                       void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Diagnostics.
 * ---------------------------------------------------------------------------------------------- */
/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* mx_last_error(void);
/* Errors the kernels found in the data (not in the arguments), as bits of the device error word
 * the library keeps for each device (the current one is read): */
#define MX_DEVERR_ROUTING 0x1  /* a routing index outside [0, E) was skipped (moe_permute,
                                  mxfp4_moe_mlp with caller routing) */
#define MX_DEVERR_SYNC 0x2     /* a wait inside an MX_SINGLE_LAUNCH call gave up: its outputs
                                  are invalid */
/* Synchronizes `stream`, copies the current device's error word to *code_host (host pointer; 0 =
 * none) and clears it. Calls on other streams of the device share the word. For tests and
 * debugging: it synchronizes. */
mx_status mx_get_device_error(void* stream, int32_t* code_host);
/* Synchronizes `stream`, then copies the status word of an mxfp4_moe_mlp workspace to *status
 * (host pointer): 0 = fine, 1 = routing index outside [0, E) seen by that call. */
mx_status mx_workspace_status(const void* ws, void* stream, int32_t* status);
/* Library version string. */
const char* mx_version(void);

/* ------------------------------------------------------------------------------------------------
 * Kernel timing, for benchmarks. While enabled, every kernel the entry points above launch is
 * bracketed by two HIP events recorded on the caller's stream (small per-launch overhead).
 * mx_profile_enable(0|1) clears what was recorded and switches recording off or on.
 * mx_profile_read synchronizes the recorded events, writes up to `max` entries (one per kernel
 * kind that ran: name, launch count, summed milliseconds) to `out` (host array), clears the
 * record and returns the number of kinds.
 * ---------------------------------------------------------------------------------------------- */
typedef struct {
  const char* name;
  int32_t launches;
  double total_ms;
} mx_kernel_time;
mx_status mx_profile_enable(int enable);
int32_t mx_profile_read(mx_kernel_time* out, int32_t max);

#ifdef __cplusplus
}
#endif
#endif /* MXFP4MOE_H */
