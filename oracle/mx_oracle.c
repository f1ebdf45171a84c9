/*
 * mx_oracle.c -- CPU oracle for the MXFP4 weight-quantized mixture-of-experts MLP.
 *
 * TEST INFRASTRUCTURE: loaded only by tests/, the smoke check and the benchmark's CPU-baseline
 * leg. It shares no code with the HIP library. Build: gcc -O2 -fno-fast-math -fopenmp -shared.
 *
 * Page citations are by title and section; see mx_oracle.h for the list of pages.
 * Every floating-point step runs in fp64; values are rounded only where a function's comment
 * says so.
 */
#include "mx_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------------------------------
 * Element and scale formats
 * ------------------------------------------------------------------------------------------- */

/* E2M1 [EN "What MXFP4 Is"; ZH "MXFP4 是什么"; FR "Quantification MXFP4"]: a 4-bit float with one
 * sign bit (bit 3), two exponent bits (bits 2..1) and one mantissa bit (bit 0). Reading of the
 * open points: exponent bias 1, exponent field 0 holds the subnormals 0 and 0.5, no Inf or NaN
 * codes -- the usual E2M1 definition, whose magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double mxo_e2m1_value(unsigned code) {
  unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
  double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return s ? -mag : mag;
}

/* Shared block scale [EN "What MXFP4 Is": 32-element blocks share a scale]. Reading: the scale is
 * an E8M0 byte, a bare power of two 2^(b-127); b = 255 is NaN. */
double mxo_e8m0_value(unsigned b) {
  if (b == 255u) return NAN;
  return ldexp(1.0, (int)b - 127);
}

/* bf16 = the top 16 bits of an fp32 pattern: 8 significant bits, fp32's exponent range.
 * Single rounding from fp64, to nearest, ties to even (the default FP rounding mode). */
uint16_t mxo_bf16_from_double(double d) {
  if (isnan(d)) return 0x7fc0;
  uint16_t sign = signbit(d) ? 0x8000 : 0;
  double a = fabs(d);
  if (isinf(a)) return sign | 0x7f80;
  if (a == 0.0) return sign;
  int q;
  frexp(a, &q);                /* a = f * 2^q, f in [0.5, 1): leading bit has weight 2^(q-1) */
  int lead = q - 1;
  if (lead < -126) lead = -126;    /* below the normal range the quantum stays 2^-133 */
  double quantum = ldexp(1.0, lead - 7);
  double r = nearbyint(a / quantum) * quantum;   /* exact division by a power of two */
  float rf = (float)r;         /* r has at most 8 significant bits: exact, or +Inf past the max */
  uint32_t bits;
  memcpy(&bits, &rf, 4);
  return sign | (uint16_t)(bits >> 16);
}

double mxo_double_from_bf16(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

static double g_e2m1[16];
static double g_e8m0[256];
/* Value a weight element takes in the matrix products, by (scale byte, code):
 *  - g_dq_exact: code * 2^(b-127) exactly (fp64 holds every such value; byte 255 gives NaN).
 *    The activation variant multiplies MXFP4 by MXFP4 as they are, so its weights are these.
 *  - g_dq_bf16: the same value as the bf16 operand of a bf16 matrix product, rounded to nearest
 *    even. Reading of the open point: the pages describe the de-quantized model as the bf16 one
 *    [EN "Memory Savings"; "Native Support in transformers"], so the weight entering a bf16
 *    product is the bf16 value of code * 2^(b-127). It is the exact value for every byte and
 *    code except where the value lies past bf16's largest finite number (bytes 253 and 254 with
 *    the larger codes), which becomes +-Inf; subnormal values are kept. */
static double g_dq_exact[256][16];
static double g_dq_bf16[256][16];
static pthread_once_t g_tables_once = PTHREAD_ONCE_INIT;

/* Decode tables, filled from the two definitions above (not typed in). */
static void build_tables(void) {
  for (unsigned c = 0; c < 16; ++c) g_e2m1[c] = mxo_e2m1_value(c);
  for (unsigned b = 0; b < 256; ++b) g_e8m0[b] = mxo_e8m0_value(b);
  for (unsigned b = 0; b < 256; ++b)
    for (unsigned c = 0; c < 16; ++c) {
      g_dq_exact[b][c] = g_e2m1[c] * g_e8m0[b];
      g_dq_bf16[b][c] = mxo_double_from_bf16(mxo_bf16_from_double(g_dq_exact[b][c]));
    }
}

/* Once per process, whatever thread gets here first (calls may come from several threads). */
static void ensure_tables(void) { pthread_once(&g_tables_once, build_tables); }

/* Code of element k of a packed row: element 2j is the low nibble of byte j. */
static inline unsigned elem_code(const uint8_t* prow, int64_t k) {
  uint8_t byte = prow[k >> 1];
  return (k & 1) ? (byte >> 4) : (byte & 0xfu);
}

/* Exact value of element k of a packed row. */
static inline double decode_elem(const uint8_t* prow, const uint8_t* srow, int64_t k) {
  return g_dq_exact[srow[k >> 5]][elem_code(prow, k)];
}

/* Value of weight element k in a matrix product: the bf16 operand (bf16_operand != 0: bf16
 * activations on bf16 matrix cores), else the exact value (the activation variant). */
static inline double weight_elem(const uint8_t* prow, const uint8_t* srow, int64_t k,
                                 int bf16_operand) {
  const unsigned b = srow[k >> 5], c = elem_code(prow, k);
  return bf16_operand ? g_dq_bf16[b][c] : g_dq_exact[b][c];
}

double mxo_weight_operand(unsigned code, unsigned b, int mx_act) {
  ensure_tables();
  return mx_act ? g_dq_exact[b & 255u][code & 15u] : g_dq_bf16[b & 255u][code & 15u];
}

/* ---------------------------------------------------------------------------------------------
 * Quantization of one 32-element block.
 *
 * Reading of the open points (the pages give only E2M1 and the shared 32-block scale):
 *  1. amax = max |x_i|. A block holding NaN or +-Inf gets scale byte 255 and all codes 0.
 *  2. Scale exponent s = floor(log2 amax) - 2, clamped to [-127, 127]; amax = 0 gives s = -127.
 *     floor(log2) is read from the binary exponent (frexp), so it is exact for every input.
 *     The minus 2 puts the block maximum at 4 <= amax/2^s < 8, i.e. at the top of the E2M1 range.
 *  3. v_i = x_i / 2^s (exact). Its magnitude goes to the nearest E2M1 magnitude; a tie goes to the
 *     code whose mantissa bit is 0 (round half to even). Beyond 6 the nearest value is 6, so
 *     magnitudes in (6, 8) saturate to 6.
 *  4. The sign bit copies x_i's sign bit (so -0 and small negatives become code 8).
 *  5. Packing: element 2j in the low nibble of byte j; one scale byte per block.
 * ------------------------------------------------------------------------------------------- */
static void quantize_block(const double* x, uint8_t* packed16, uint8_t* scale) {
  double amax = 0.0;
  int finite = 1;
  for (int i = 0; i < 32; ++i) {
    if (!isfinite(x[i])) finite = 0;
    else if (fabs(x[i]) > amax) amax = fabs(x[i]);
  }
  if (!finite) {
    *scale = 255;
    memset(packed16, 0, 16);
    return;
  }
  int s;
  if (amax == 0.0) {
    s = -127;
  } else {
    int q;
    frexp(amax, &q);            /* amax = f * 2^q with f in [0.5, 1), so floor(log2 amax) = q-1 */
    s = (q - 1) - 2;
    if (s < -127) s = -127;
    if (s > 127) s = 127;
  }
  *scale = (uint8_t)(s + 127);

  uint8_t codes[32];
  for (int i = 0; i < 32; ++i) {
    double a = fabs(ldexp(x[i], -s));
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c < 8; ++c) {           /* nearest magnitude; ties to mantissa bit 0 */
      double d = fabs(a - g_e2m1[c]);
      if (d < best_d || (d == best_d && (c & 1) == 0)) {
        best = c;
        best_d = d;
      }
    }
    codes[i] = (uint8_t)(best | (signbit(x[i]) ? 8 : 0));
  }
  for (int j = 0; j < 16; ++j) packed16[j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
}

static void quantize_rows_f64(const double* src, int64_t rows, int64_t K, uint8_t* packed,
                              uint8_t* scales) {
  ensure_tables();
  int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b)
      quantize_block(src + r * K + b * 32, packed + r * (K / 2) + b * 16, scales + r * nb + b);
}

void mxo_quantize_f32(const float* src, int64_t rows, int64_t K, uint8_t* packed, uint8_t* scales) {
  ensure_tables();
  int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double blk[32];
    for (int64_t b = 0; b < nb; ++b) {
      for (int i = 0; i < 32; ++i) blk[i] = (double)src[r * K + b * 32 + i];
      quantize_block(blk, packed + r * (K / 2) + b * 16, scales + r * nb + b);
    }
  }
}

void mxo_quantize_bf16(const uint16_t* src, int64_t rows, int64_t K, uint8_t* packed,
                       uint8_t* scales) {
  ensure_tables();
  int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double blk[32];
    for (int64_t b = 0; b < nb; ++b) {
      for (int i = 0; i < 32; ++i) blk[i] = mxo_double_from_bf16(src[r * K + b * 32 + i]);
      quantize_block(blk, packed + r * (K / 2) + b * 16, scales + r * nb + b);
    }
  }
}

/* Dequantization: code value times scale, exact in fp64 [EN "Memory Savings": the de-quantized
 * model is the bf16 one]. */
void mxo_dequantize(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t K,
                    double* dst) {
  ensure_tables();
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < K; ++k)
      dst[r * K + k] = decode_elem(packed + r * (K / 2), scales + r * (K / 32), k);
}

/* ---------------------------------------------------------------------------------------------
 * Router. The pages name a top-k expert selection kernel for MoE models (GGUF page, section on
 * ggml Metal kernels) but define no router. Reading: a linear router with optional bias, top-k by
 * logit (ties to the lower expert index, outputs in rank order), softmax over only the k chosen.
 * ------------------------------------------------------------------------------------------- */
void mxo_router_logits(const uint16_t* x, const uint16_t* wr, const float* br, int T, int H, int E,
                       float* logits) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += mxo_double_from_bf16(x[(int64_t)t * H + h]) * mxo_double_from_bf16(wr[(int64_t)e * H + h]);
      if (br) acc += (double)br[e];
      logits[(int64_t)t * E + e] = (float)acc;
    }
}

void mxo_topk_softmax(const float* logits, int T, int E, int k, int32_t* idx, float* w) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (int64_t)t * E;
    char* taken = (char*)calloc((size_t)E, 1);
    double sel[256] = {0};  /* k <= 256 */
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {  /* strictly greater: equal logits keep the lower index */
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      taken[best] = 1;
      idx[(int64_t)t * k + j] = best;
      sel[j] = (double)l[best];
    }
    double mx = sel[0], sum = 0.0;
    for (int j = 1; j < k; ++j)
      if (sel[j] > mx) mx = sel[j];
    for (int j = 0; j < k; ++j) sum += exp(sel[j] - mx);
    for (int j = 0; j < k; ++j) w[(int64_t)t * k + j] = (float)(exp(sel[j] - mx) / sum);
    free(taken);
  }
}

/* ---------------------------------------------------------------------------------------------
 * Permutation by expert: histogram, exclusive prefix sum, scatter in (token, slot) order.
 * perm[row] = t*k + j for the pair stored at permuted row `row`; inv[t*k + j] = row.
 * ------------------------------------------------------------------------------------------- */
int mxo_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets, int32_t* perm,
                int32_t* inv) {
  int64_t P = (int64_t)T * k;
  int32_t* fill = (int32_t*)calloc((size_t)E + 1, sizeof(int32_t));
  for (int e = 0; e <= E; ++e) offsets[e] = 0;
  for (int64_t p = 0; p < P; ++p) {
    if (idx[p] < 0 || idx[p] >= E) {
      free(fill);
      return -1;
    }
    offsets[idx[p] + 1] += 1;
  }
  for (int e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
  for (int64_t p = 0; p < P; ++p) {
    int e = idx[p];
    int32_t row = offsets[e] + fill[e]++;
    perm[row] = (int32_t)p;
    inv[p] = row;
  }
  free(fill);
  return 0;
}

/* ---------------------------------------------------------------------------------------------
 * Dense weight-only linear: Y = X W^T with W stored [N][K] (output-major, K contiguous).
 * ------------------------------------------------------------------------------------------- */
static void activation_row(const uint16_t* xrow, int K, int mx_act, double* out) {
  if (!mx_act) {
    for (int i = 0; i < K; ++i) out[i] = mxo_double_from_bf16(xrow[i]);
    return;
  }
  /* Activation variant: the bf16 row is quantized with the same block rule, then decoded. */
  uint8_t* p = (uint8_t*)malloc((size_t)K / 2);
  uint8_t* s = (uint8_t*)malloc((size_t)K / 32);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)K);
  for (int i = 0; i < K; ++i) tmp[i] = mxo_double_from_bf16(xrow[i]);
  quantize_rows_f64(tmp, 1, K, p, s);
  for (int i = 0; i < K; ++i) out[i] = decode_elem(p, s, i);
  free(tmp);
  free(s);
  free(p);
}

void mxo_linear(const uint16_t* x, int M, int K, const uint8_t* packed, const uint8_t* scales, int N,
                int mx_act, double* y) {
  ensure_tables();
  for (int m = 0; m < M; ++m) {
    double* xr = (double*)malloc(sizeof(double) * (size_t)K);
    activation_row(x + (int64_t)m * K, K, mx_act, xr);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
      const uint8_t* prow = packed + (int64_t)n * (K / 2);
      const uint8_t* srow = scales + (int64_t)n * (K / 32);
      double acc = 0.0;
      for (int kk = 0; kk < K; ++kk) acc += xr[kk] * weight_elem(prow, srow, kk, !mx_act);
      y[(int64_t)m * N + n] = acc;
    }
    free(xr);
  }
}

/* ---------------------------------------------------------------------------------------------
 * MoE MLP. Reading of the open points: each expert is a SwiGLU MLP without biases; gate_up rows
 * [0, F) are the gate, rows [F, 2F) the up projection; h = silu(g) * u with silu(g) = g/(1+e^-g);
 * h is rounded to bf16 (it is the next matrix product's bf16 input); the expert output is scaled
 * by the token's routing weight and the k scaled outputs are summed.
 * Precision: fp64 throughout except the bf16 rounding of h (and, in the activation variant, the
 * MXFP4 quantization of x along H and of the bf16 h along F).
 * ------------------------------------------------------------------------------------------- */

/* Adjacent bf16 patterns (one step towards +inf / -inf in value); NaN and Inf never get here. */
static uint16_t bf16_step(uint16_t b, int up) {
  const int neg = (b & 0x8000) != 0;
  const uint16_t mag = b & 0x7fff;
  if (mag == 0) return up ? 0x0001 : 0x8001;
  if (up != neg) return (uint16_t)(b + 1); /* magnitude grows */
  return (uint16_t)(b - 1);
}

/* The other bf16 a value v could have been rounded to when it is known only to within +-dv:
 * the neighbour of hb whose midpoint with hb lies within dv of v. Returns 0 if there is none. */
static int bf16_alternative(double v, uint16_t hb, double dv, uint16_t* alt) {
  const double d = mxo_double_from_bf16(hb);
  int found = 0;
  double best = INFINITY;
  for (int up = 0; up < 2; ++up) {
    const uint16_t nb = bf16_step(hb, up);
    const double dn = mxo_double_from_bf16(nb);
    if (!isfinite(dn)) continue;
    const double dist = fabs(v - 0.5 * (d + dn));
    if (dist <= dv && dist < best) {
      best = dist;
      *alt = nb;
      found = 1;
    }
  }
  return found;
}

/* The expert MLP's activation, by the reading stated with mxo_act_params (mx_oracle.h): gate and
 * up values of output column f are pre-activations gate_row(f) and up_row(f) of the gate_up
 * product (bias included); h = g' * sigmoid(alpha g') * (u' + shift) with g' = min(g, limit) and
 * u' = clamp(u, -limit, limit) when limit > 0. With NULL parameters: alpha 1, no clamp, shift 0,
 * rows [0, F) gate and [F, 2F) up -- h = silu(g) * u. */
static double act_alpha(const mxo_act_params* act) {
  return (act && act->alpha != 0.0) ? act->alpha : 1.0;
}

int mxo_moe_mlp_act(int T, int H, int F, int E, int k, int mx_act, const uint16_t* x,
                    const int32_t* topk_idx, const float* topk_w,
                    const uint8_t* gu_packed, const uint8_t* gu_scales,
                    const uint8_t* dn_packed, const uint8_t* dn_scales,
                    const int32_t* tokens, int n_tokens, double* out, uint16_t* h_out,
                    double acc_c, uint16_t* h_alt_out, double* slack_out,
                    const mxo_act_params* act) {
  ensure_tables();
  const double alpha = act_alpha(act);
  const double limit = act ? act->limit : 0.0;
  const double shift = act ? act->up_shift : 0.0;
  const int interleaved = act ? act->interleaved : 0;
  const float* gu_bias = act ? act->gu_bias : NULL;
  const float* dn_bias = act ? act->dn_bias : NULL;
  if (!tokens) n_tokens = T;
  for (int i = 0; i < n_tokens; ++i) {
    int t = tokens ? tokens[i] : i;
    for (int j = 0; j < k; ++j) {
      int e = topk_idx[(int64_t)t * k + j];
      if (e < 0 || e >= E) return -1;
    }
  }
  const int fragility = (h_alt_out != NULL || slack_out != NULL);
  const double u32 = ldexp(1.0, -24);
  const int64_t gu_row = H / 2, gu_srow = H / 32, dn_row = F / 2, dn_srow = F / 32;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < n_tokens; ++i) {
    int t = tokens ? tokens[i] : i;
    double* xr = (double*)malloc(sizeof(double) * (size_t)H);
    double* a = (double*)malloc(sizeof(double) * 2 * (size_t)F);
    double* a2 = (double*)malloc(sizeof(double) * 2 * (size_t)F);
    double* hv = (double*)malloc(sizeof(double) * (size_t)F);
    double* h = (double*)malloc(sizeof(double) * (size_t)F);
    uint16_t* hb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)F);
    double* o = out + (int64_t)i * H;
    double* sl = slack_out ? slack_out + (int64_t)i * H : NULL;
    activation_row(x + (int64_t)t * H, H, mx_act, xr);
    for (int m = 0; m < H; ++m) o[m] = 0.0;
    if (sl)
      for (int m = 0; m < H; ++m) sl[m] = 0.0;
    for (int j = 0; j < k; ++j) {
      int e = topk_idx[(int64_t)t * k + j];
      double wt = (double)topk_w[(int64_t)t * k + j];
      /* gate_up: a = x W_gu[e]^T */
      for (int n = 0; n < 2 * F; ++n) {
        const uint8_t* prow = gu_packed + ((int64_t)e * 2 * F + n) * gu_row;
        const uint8_t* srow = gu_scales + ((int64_t)e * 2 * F + n) * gu_srow;
        double acc = 0.0, sq = 0.0;
        for (int kk = 0; kk < H; ++kk) {
          const double term = xr[kk] * weight_elem(prow, srow, kk, !mx_act);
          acc += term;
          if (fragility) sq += term * term;
        }
        if (gu_bias) acc += (double)gu_bias[(int64_t)e * 2 * F + n];
        a[n] = acc;
        a2[n] = sq;
      }
      /* the activation (SwiGLU or its clamped, scaled form), then bf16 rounding of h */
      for (int f = 0; f < F; ++f) {
        const int gi = interleaved ? 2 * f : f, ui = interleaved ? 2 * f + 1 : F + f;
        double g = a[gi], u = a[ui];
        if (limit > 0.0) {
          g = fmin(g, limit);
          u = fmax(fmin(u, limit), -limit);
        }
        hv[f] = g / (1.0 + exp(-alpha * g)) * (u + shift);
        hb[f] = mxo_bf16_from_double(hv[f]);
      }
      if (h_out)
        memcpy(h_out + ((int64_t)i * k + j) * F, hb, sizeof(uint16_t) * (size_t)F);
      activation_row(hb, F, mx_act, h);
      /* Fragile decisions of the activation variant (test aid, no effect on `out`): an
       * implementation that forms g and u in fp32 knows h only to within
       *   dv = |silu'(g) u| dg + |silu(g)| du + 16 u32 |h|,   dg = acc_c u32 sqrt(H sum terms^2),
       * so its bf16 h may be the other neighbour of the exact value; where that alternative changes
       * the block's MXFP4 quantization, the down product may legitimately differ by
       *   wt * sum_i |dq'_i - dq_i| |W_dn[m][i]|  on output m, which is added to slack[m]. */
      if (fragility) {
        uint16_t* halt = h_alt_out ? h_alt_out + ((int64_t)i * k + j) * F : NULL;
        if (halt) memcpy(halt, hb, sizeof(uint16_t) * (size_t)F);
        if (mx_act) {
          for (int f = 0; f < F; ++f) {
            const int gi = interleaved ? 2 * f : f, ui = interleaved ? 2 * f + 1 : F + f;
            double g = a[gi], u = a[ui];
            /* a clamped input does not move h: its derivative is 0 there */
            const int g_clamped = limit > 0.0 && g > limit;
            const int u_clamped = limit > 0.0 && fabs(u) > limit;
            if (g_clamped) g = limit;
            if (u_clamped) u = u > 0 ? limit : -limit;
            const double sg = 1.0 / (1.0 + exp(-alpha * g));
            const double dact = sg * (1.0 + alpha * g * (1.0 - sg));  /* d(g sigma(alpha g))/dg */
            const double dg = g_clamped ? 0.0 : acc_c * u32 * sqrt((double)H * a2[gi]);
            const double du = u_clamped ? 0.0 : acc_c * u32 * sqrt((double)H * a2[ui]);
            const double dv = fabs(dact * (u + shift)) * dg + fabs(g * sg) * du +
                              16.0 * u32 * fabs(hv[f]);
            uint16_t alt;
            if (!bf16_alternative(hv[f], hb[f], dv, &alt)) continue;
            const int b0 = f & ~31;
            double blk[32], dq1[32];
            uint8_t p1[16], s1;
            for (int q = 0; q < 32; ++q) blk[q] = mxo_double_from_bf16(b0 + q == f ? alt : hb[b0 + q]);
            quantize_block(blk, p1, &s1);
            int differs = 0;
            for (int q = 0; q < 32; ++q) {
              dq1[q] = decode_elem(p1, &s1, q);
              if (dq1[q] != h[b0 + q]) differs = 1;
            }
            if (!differs) continue;
            if (halt) halt[f] = alt;
            if (sl)
              for (int m = 0; m < H; ++m) {
                const uint8_t* wrow = dn_packed + ((int64_t)e * H + m) * dn_row;
                const uint8_t* wsrow = dn_scales + ((int64_t)e * H + m) * dn_srow;
                double d = 0.0;
                for (int q = 0; q < 32; ++q)
                  d += fabs(dq1[q] - h[b0 + q]) * fabs(decode_elem(wrow, wsrow, b0 + q));
                sl[m] += wt * d;
              }
          }
        }
      }
      /* down, scaled by the routing weight, summed over the k selected experts */
      for (int m = 0; m < H; ++m) {
        const uint8_t* prow = dn_packed + ((int64_t)e * H + m) * dn_row;
        const uint8_t* srow = dn_scales + ((int64_t)e * H + m) * dn_srow;
        double acc = 0.0;
        for (int f = 0; f < F; ++f) acc += h[f] * weight_elem(prow, srow, f, !mx_act);
        if (dn_bias) acc += (double)dn_bias[(int64_t)e * H + m];
        o[m] += wt * acc;
      }
    }
    free(hb);
    free(h);
    free(hv);
    free(a2);
    free(a);
    free(xr);
  }
  return 0;
}

int mxo_moe_mlp_ex(int T, int H, int F, int E, int k, int mx_act, const uint16_t* x,
                   const int32_t* topk_idx, const float* topk_w,
                   const uint8_t* gu_packed, const uint8_t* gu_scales,
                   const uint8_t* dn_packed, const uint8_t* dn_scales,
                   const int32_t* tokens, int n_tokens, double* out, uint16_t* h_out,
                   double acc_c, uint16_t* h_alt_out, double* slack_out) {
  return mxo_moe_mlp_act(T, H, F, E, k, mx_act, x, topk_idx, topk_w, gu_packed, gu_scales,
                         dn_packed, dn_scales, tokens, n_tokens, out, h_out, acc_c, h_alt_out,
                         slack_out, NULL);
}

int mxo_moe_mlp(int T, int H, int F, int E, int k, int mx_act, const uint16_t* x,
                const int32_t* topk_idx, const float* topk_w,
                const uint8_t* gu_packed, const uint8_t* gu_scales,
                const uint8_t* dn_packed, const uint8_t* dn_scales,
                const int32_t* tokens, int n_tokens, double* out, uint16_t* h_out) {
  return mxo_moe_mlp_ex(T, H, F, E, k, mx_act, x, topk_idx, topk_w, gu_packed, gu_scales,
                        dn_packed, dn_scales, tokens, n_tokens, out, h_out, 0.0, NULL, NULL);
}

int mxo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
