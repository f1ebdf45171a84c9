/*
 * mx_oracle.h -- CPU oracle for the MXFP4 weight-quantized mixture-of-experts MLP.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library. The product path (the HIP library under
 * mxfp4_weight_quantized_amd/) shares no code, header, table or constant with it.
 *
 * Plain, slow, obviously correct: loops in the order the definitions give, fp64 arithmetic,
 * rounding only at the precision points listed per function. OpenMP splits independent rows or
 * tokens across threads; nothing is blocked, fused or reordered inside a row.
 *
 * Sources (cited by page title and section):
 *   [EN] "Transformers 4.40 performance upgrades for OpenAI GPT-OSS: zero-build kernels, MXFP4
 *        quantization, parallelism, and faster loading" (agentlenshq.com, English page),
 *        section "MXFP4 4-Bit Quantization", subsections "What MXFP4 Is" and "Memory Savings".
 *   [ZH] the Chinese version of the same page, section "MXFP4 是什么".
 *   [FR] "GPT-OSS ... améliorations OpenAI" (otomatix.tech), section "Quantification MXFP4 :
 *        un format atypique".
 * The pages fix the element format (E2M1: 1 sign, 2 exponent, 1 mantissa bit) and that every
 * 32 consecutive elements share one scale. Every other rule here (the E8M0 scale choice, rounding,
 * packing, routing, SwiGLU) is a reading of an open point; each is stated where it is used.
 */
#ifndef MX_ORACLE_H
#define MX_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Value of a 4-bit E2M1 code (0..15) built from its bit fields. */
double mxo_e2m1_value(unsigned code);
/* Value of an E8M0 scale byte: 2^(b-127); 255 is NaN. */
double mxo_e8m0_value(unsigned b);
/* fp64 -> bf16 bit pattern, round to nearest even, one rounding step, subnormals kept. */
uint16_t mxo_bf16_from_double(double d);
double mxo_double_from_bf16(uint16_t b);

/* Quantize rows of K values (K % 32 == 0) in 32-element blocks along K.
 * packed: rows*K/2 bytes, element 2j in the low nibble of byte j; scales: rows*K/32 bytes. */
void mxo_quantize_f32(const float* src, int64_t rows, int64_t K, uint8_t* packed, uint8_t* scales);
void mxo_quantize_bf16(const uint16_t* src, int64_t rows, int64_t K, uint8_t* packed, uint8_t* scales);
/* Value weight element (code, scale byte b) takes in the matrix products: mx_act == 0, the bf16
 * operand of a bf16 product (code * 2^(b-127) rounded to nearest even bf16: exact except past
 * bf16's range, which gives +-Inf); mx_act != 0, the exact value. Byte 255 gives NaN. */
double mxo_weight_operand(unsigned code, unsigned b, int mx_act);
/* Exact dequantization to fp64. */
void mxo_dequantize(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t K, double* dst);

/* Router: logits[t][e] = fp32(sum_h x[t][h]*wr[e][h] + br[e]) with the sum in fp64 (br nullable). */
void mxo_router_logits(const uint16_t* x, const uint16_t* wr, const float* br, int T, int H, int E,
                       float* logits);
/* Top-k by (logit descending, expert index ascending); softmax over the k selected, fp64 -> fp32. */
void mxo_topk_softmax(const float* logits, int T, int E, int k, int32_t* idx, float* w);
/* Stable counting sort of the T*k (token, slot) pairs by expert.
 * Returns 0, or -1 if an index lies outside [0, E). */
int mxo_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets, int32_t* perm, int32_t* inv);

/* Dense weight-only linear y[m][n] = sum_k x[m][k] * W^[n][k] in fp64, W^ the weight operand
 * above (bf16 for mx_act == 0, exact for mx_act != 0).
 * mx_act != 0: the rows of x are first quantized and dequantized along K (activation variant). */
void mxo_linear(const uint16_t* x, int M, int K, const uint8_t* packed, const uint8_t* scales, int N,
                int mx_act, double* y);

/* MoE MLP for a list of tokens (tokens == NULL: all T tokens, in order), given the routing.
 * out: [n_tokens][H] fp64.  h_out (nullable): [n_tokens][k][F] bf16 bits of the SwiGLU output.
 * Returns 0, or -1 on an expert index outside [0, E). */
int mxo_moe_mlp(int T, int H, int F, int E, int k, int mx_act, const uint16_t* x,
                const int32_t* topk_idx, const float* topk_w,
                const uint8_t* gu_packed, const uint8_t* gu_scales,
                const uint8_t* dn_packed, const uint8_t* dn_scales,
                const int32_t* tokens, int n_tokens, double* out, uint16_t* h_out);
/* The same, plus (activation variant only) the h quantization decisions that an fp32
 * implementation could legitimately take the other way. acc_c scales the assumed fp32 error of
 * g and u: acc_c * 2^-24 * sqrt(H * sum of squared terms). h_alt_out (nullable, [n][k][F]): the
 * other bf16 of each such element, else h itself. slack_out (nullable, [n][H]): bound on the
 * output change those decisions can cause (0 everywhere when mx_act == 0). */
int mxo_moe_mlp_ex(int T, int H, int F, int E, int k, int mx_act, const uint16_t* x,
                   const int32_t* topk_idx, const float* topk_w,
                   const uint8_t* gu_packed, const uint8_t* gu_scales,
                   const uint8_t* dn_packed, const uint8_t* dn_scales,
                   const int32_t* tokens, int n_tokens, double* out, uint16_t* h_out,
                   double acc_c, uint16_t* h_alt_out, double* slack_out);

/* The expert activation of the released gpt-oss models, which the pages do not spell out (reading
 * of an open point, parameterised so that the zero / NULL parameters give the SwiGLU above):
 *   a = x W_gu^T + gu_bias[e]   (gu_bias [E][2F] in the weight rows' order, NULL = none)
 *   g = a[gate_row(f)], u = a[up_row(f)]: rows f and F + f, or (interleaved) 2f and 2f + 1
 *   limit > 0: g = min(g, limit), u = clamp(u, -limit, limit)   (the gate is clamped above only)
 *   h = bf16( g * sigmoid(alpha * g) * (u + up_shift) )          (alpha 0 means 1)
 *   y = h W_dn^T + dn_bias[e]   (dn_bias [E][H], NULL = none), then weighted and summed.
 * The fragile-decision aid of the activation variant uses the same h. */
typedef struct {
  int interleaved;
  double alpha, limit, up_shift;
  const float* gu_bias;
  const float* dn_bias;
} mxo_act_params;
int mxo_moe_mlp_act(int T, int H, int F, int E, int k, int mx_act, const uint16_t* x,
                    const int32_t* topk_idx, const float* topk_w,
                    const uint8_t* gu_packed, const uint8_t* gu_scales,
                    const uint8_t* dn_packed, const uint8_t* dn_scales,
                    const int32_t* tokens, int n_tokens, double* out, uint16_t* h_out,
                    double acc_c, uint16_t* h_alt_out, double* slack_out,
                    const mxo_act_params* act);

/* Number of OpenMP threads the oracle uses. */
int mxo_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
