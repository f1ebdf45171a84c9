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

// ---- top-k selection (router and the fused selection in the permutation) ----
// (value desc, index asc) ordering: true if (va, ia) ranks before (vb, ib).
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// One wave ranks the E logits of token t (logit_of(e) for e < E; lane l holds experts l, l+64,
// l+128, l+192): k rounds of a wave-wide argmax under (logit desc, expert index asc), then the
// softmax of the k selected logits; lane j < k writes entry j and returns its expert index.
template <class LogitOf>
__device__ __forceinline__ int select_topk_wave(LogitOf logit_of, int lane, int t, int E, int k,
                                                int32_t* __restrict__ idx_out,
                                                float* __restrict__ w_out) {
  float cv[4];
  int ci[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    ci[q] = e;
    cv[q] = (e < E) ? logit_of(e) : -INFINITY;
  }
  bool used[4] = {false, false, false, false};
  float sel_v[8];
  int sel_i[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (!used[q] && ci[q] < E && (bi == 0x7fffffff || ranks_before(cv[q], ci[q], bv, bi))) {
        bv = cv[q];
        bi = ci[q];
      }
    // wave-wide best: DPP exchanges inside each 16-lane row (partners lane^1, lane^2, then the
    // mirrored lane in the half row and in the row), then the four rows' bests combined
    // uniformly from lanes 0, 16, 32 and 48
    auto take = [&](float ov, int oi) {
      if (oi != 0x7fffffff && (bi == 0x7fffffff || ranks_before(ov, oi, bv, bi))) {
        bv = ov;
        bi = oi;
      }
    };
    auto dpp_step = [&](auto ctrl) {
      constexpr int C = decltype(ctrl)::value;
      const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), C, 0xf, 0xf, false));
      const int oi = __builtin_amdgcn_update_dpp(0, bi, C, 0xf, 0xf, false);
      take(ov, oi);
    };
    dpp_step(std::integral_constant<int, 0xb1>{});   // quad_perm [1,0,3,2]: lane ^ 1
    dpp_step(std::integral_constant<int, 0x4e>{});   // quad_perm [2,3,0,1]: lane ^ 2
    dpp_step(std::integral_constant<int, 0x141>{});  // row_half_mirror: 7 - lane in 8
    dpp_step(std::integral_constant<int, 0x140>{});  // row_mirror: 15 - lane in 16
#pragma unroll
    for (int row = 1; row < 4; ++row)
      take(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * row)),
           __builtin_amdgcn_readlane(bi, 16 * row));
    {  // row 0 last, so that every lane ends with the same (uniform) result
      const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
      const int i0 = __builtin_amdgcn_readlane(bi, 0);
      take(v0, i0);
    }
    sel_v[j] = bv;
    sel_i[j] = bi;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (ci[q] == bi) used[q] = true;
  }
  float sum = 0.f, mine = 0.f;
  int mine_i = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    const float ev = expf(sel_v[j] - sel_v[0]);
    sum += ev;
    if (lane == j) {
      mine = ev;
      mine_i = sel_i[j];
    }
  }
  if (lane < k) {
    idx_out[(int64_t)t * k + lane] = mine_i;
    w_out[(int64_t)t * k + lane] = mine / sum;
  }
  return mine_i;
}


}  // namespace mx
