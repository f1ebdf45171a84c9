// mx_device.h -- device-side building blocks for gfx950 (CDNA4): vector types, MFMA and FP4
// conversion wrappers, wait counters and barriers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace mx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------------
// Scalar helpers
// ---------------------------------------------------------------------------------------------
// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Eight E2M1 codes (one dword, element 0 in the low nibble) times a scale -> eight bf16 in the
// element order, as one MFMA operand register group.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t w, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ bf16x8 u32x4_as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// 16x16x32 bf16 MFMA, fp32 accumulate. Lane l supplies A[row l%16][8 k-values of group l/16] and
// B[same 8 k-values][col l%16]; D lane l holds rows 4*(l/16)+i, col l%16.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16 MFMA, fp32 accumulate. Lane l supplies A[row l%32][8 k-values of group l/32] and
// B[same 8 k-values][col l%32]; D value v of lane l is row 8*(v/4) + 4*(l/32) + v%4, col l%32.
// On gfx950 it issues at about twice the flops per cycle of the 16x16x32 form (measured: one
// 32x32x16 per ~33 cycles and SIMD against one 16x16x32 per ~29).
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x128 MXFP4 x MXFP4 MFMA with E8M0 block scales (v_mfma_scale_f32_16x16x128_f8f6f4, both
// operands in format 4 = E2M1). Lane l supplies 32 codes (16 bytes) of A row l%16 and of B column
// l%16 for K block l/16, and one scale byte for each (the low byte of the scale register).
__device__ __forceinline__ f32x4 mfma_fp4_16x16x128(u32x4 a, u32x4 b, uint32_t sa, uint32_t sb,
                                                    f32x4 c) {
  const i32x8 av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const i32x8 bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// ---------------------------------------------------------------------------------------------
// MXFP4 quantization (the library's rule, on integer bit patterns only: the results do not
// depend on the denormal mode). Used by the codec kernels and by the epilogue that quantizes the
// SwiGLU output of the activation variant.
// ---------------------------------------------------------------------------------------------
// Bit pattern of (1 + mant23 / 2^23) * 2^e2 as fp32, exact (normal or subnormal) for the
// decision points used below (their mantissas have at least 21 trailing zero bits and
// e2 >= -129 keeps the subnormal shift <= 3).
__device__ __forceinline__ uint32_t pow2_times(uint32_t mant23, int e2) {
  int be = e2 + 127;
  if (be >= 1) return ((uint32_t)be << 23) | mant23;
  return (0x800000u | mant23) >> (1 - be);
}

// E2M1 magnitude code (0..7) of |x| / 2^s for |x| given as fp32 bits u (sign cleared), using
// the seven decision points 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 (times 2^s). A value exactly at a
// decision point goes to the code whose mantissa bit is 0: strict ">" where the lower neighbour
// is even, ">=" where the upper neighbour is even.
struct Thresholds {
  uint32_t t[7];
  __device__ __forceinline__ explicit Thresholds(int s) {
    t[0] = pow2_times(0x000000u, s - 2);  // 0.25
    t[1] = pow2_times(0x400000u, s - 1);  // 0.75
    t[2] = pow2_times(0x200000u, s);      // 1.25
    t[3] = pow2_times(0x600000u, s);      // 1.75
    t[4] = pow2_times(0x200000u, s + 1);  // 2.5
    t[5] = pow2_times(0x600000u, s + 1);  // 3.5
    t[6] = pow2_times(0x200000u, s + 2);  // 5
  }
  __device__ __forceinline__ uint32_t code(uint32_t u) const {
    return (uint32_t)(u > t[0]) + (uint32_t)(u >= t[1]) + (uint32_t)(u > t[2]) +
           (uint32_t)(u >= t[3]) + (uint32_t)(u > t[4]) + (uint32_t)(u >= t[5]) +
           (uint32_t)(u > t[6]);
  }
};

// Scale exponent s from the largest |x| bit pattern of the block (m < 0x7f800000: finite).
__device__ __forceinline__ int scale_exponent(uint32_t m) {
  uint32_t be = m >> 23;                // biased exponent of amax; 0 for zero or subnormal
  if (be == 0) return -127;             // floor(log2 amax) <= -127, clamped
  int s = (int)be - 127 - 2;
  return s < -127 ? -127 : s;
}

// Quantizes one 32-element block given as fp32 bit patterns u[0..31] (bf16 inputs: their bits
// shifted up by 16). Returns the scale byte and sets the 16 packed bytes (element 2j in the low
// nibble of byte j) as four dwords. A block holding NaN or Inf gets byte 255 and codes 0.
__device__ __forceinline__ uint32_t quantize_block32(const uint32_t (&u)[32], uint32_t (&q)[4]) {
  uint32_t m = 0;  // integer max of |x| orders finite values by magnitude, Inf/NaN above all
#pragma unroll
  for (int i = 0; i < 32; ++i) m = max(m, u[i] & 0x7fffffffu);
#pragma unroll
  for (int j = 0; j < 4; ++j) q[j] = 0;
  if (m >= 0x7f800000u) return 255u;
  const int s = scale_exponent(m);
  const Thresholds th(s);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t c = th.code(u[i] & 0x7fffffffu) | ((u[i] >> 28) & 8u);
    q[i >> 3] |= c << (4 * (i & 7));
  }
  return (uint32_t)(s + 127);
}

// The same for a block of 32 bf16 values given as 16 dwords (element 2j in the low half of dword
// j), on the hardware conversion: v_cvt_scalef32_pk_fp4_bf16 with scale 2^s divides by the scale,
// rounds to the nearest E2M1 value with ties to the even code, saturates at 6 and keeps the sign
// bit (zeros included) -- the rule above exactly: on gfx950 it gives the integer rule's code for
// every one of the 65 536 bf16 values at every scale exponent s in [-127, 127] (NaN and Inf, which
// never reach it, aside). Two codes per instruction instead of about 36 integer operations.
__device__ __forceinline__ uint32_t quantize_block32_bf16(const uint32_t (&w)[16],
                                                          uint32_t (&q)[4]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = max(m, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
#pragma unroll
  for (int j = 0; j < 4; ++j) q[j] = 0;
  if (m >= 0x7f80u) return 255u;
  const int s = scale_exponent(m << 16);
  const float scale = __builtin_amdgcn_ldexpf(1.0f, s);  // exact, 2^-127 included
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // byte b of dword j: elements 8j + 2b, 8j + 2b + 1
    uint32_t d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2, w[4 * j]), scale, 0);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, __builtin_bit_cast(bf16x2, w[4 * j + 1]), scale, 1);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, __builtin_bit_cast(bf16x2, w[4 * j + 2]), scale, 2);
    q[j] = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, __builtin_bit_cast(bf16x2, w[4 * j + 3]), scale, 3);
  }
  return (uint32_t)(s + 127);
}

// ---------------------------------------------------------------------------------------------
// Memory helpers
// ---------------------------------------------------------------------------------------------
// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the full memory fence of __syncthreads(): outstanding prefetches
// stay in flight. Callers wait for the counters they need first.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ u32x4 lds_read_b128(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace mx
