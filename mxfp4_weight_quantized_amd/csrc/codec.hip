// codec.hip -- MXFP4 pack / unpack kernels for gfx950.
//
// Format: E2M1 elements (1 sign, 2 exponent, 1 mantissa bit) sharing one scale per 32-element
// block -- "Transformers 4.40 performance upgrades for OpenAI GPT-OSS ..." (agentlenshq.com,
// English page), section "MXFP4 4-Bit Quantization > What MXFP4 Is". The scale is an E8M0 byte
// b = clamp(floor(log2 amax) - 2, -127, 127) + 127 and elements round to the nearest E2M1 value
// with ties to the even code (the library's reading of what the page leaves open).
//
// Both kernels work on integer bit patterns only, so the results do not depend on the
// denormal mode: floor(log2 amax) is the exponent field of amax, the rounding is a comparison of
// |x|'s bit pattern with the bit patterns of the seven E2M1 decision points times 2^s, and
// decoding assembles sign, exponent and mantissa fields directly.
//
// Mapping: eight lanes per 32-element block, four consecutive elements per lane, so a wave reads
// 1 KB (fp32) of contiguous input per instruction and writes 128 contiguous packed bytes.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {
namespace {

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

template <bool BF16_IN>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ src,
                                                       int64_t nblocks,
                                                       uint8_t* __restrict__ packed,
                                                       uint8_t* __restrict__ scales) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = gid >> 3;
  const int sub = (int)(gid & 7);
  const bool active = blk < nblocks;
  uint32_t u[4] = {0, 0, 0, 0};
  if (active) {
    const int64_t e0 = blk * 32 + sub * 4;
    if (BF16_IN) {
      uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(src) + e0);
      u[0] = v.x << 16; u[1] = v.x & 0xffff0000u; u[2] = v.y << 16; u[3] = v.y & 0xffff0000u;
    } else {
      uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(src) + e0);
      u[0] = v.x; u[1] = v.y; u[2] = v.z; u[3] = v.w;
    }
  }
  // Largest magnitude bit pattern of the block: integer max of |x| patterns orders finite values
  // by magnitude and puts Inf/NaN above them all.
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, u[i] & 0x7fffffffu);
  m = max(m, (uint32_t)__shfl_xor((int)m, 1));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2));
  m = max(m, (uint32_t)__shfl_xor((int)m, 4));
  if (!active) return;

  uint32_t sbyte, codes = 0;
  if (m >= 0x7f800000u) {
    sbyte = 255;                        // NaN or Inf in the block
  } else {
    const int s = scale_exponent(m);
    sbyte = (uint32_t)(s + 127);
    const Thresholds th(s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t c = th.code(u[i] & 0x7fffffffu) | ((u[i] >> 28) & 8u);
      codes |= c << (4 * i);
    }
  }
  *reinterpret_cast<uint16_t*>(packed + blk * 16 + sub * 2) = (uint16_t)codes;
  if (sub == 0) scales[blk] = (uint8_t)sbyte;
}

// fp32 bit pattern of E2M1 code c times 2^(b-127), built field by field.
__device__ __forceinline__ uint32_t decode_f32_bits(uint32_t c, uint32_t b) {
  const uint32_t sign = (c & 8u) << 28;
  const uint32_t m3 = c & 7u;
  if (b == 255u) return sign | 0x7fc00000u;
  if (m3 == 0) return sign;
  const int e = (int)(m3 >> 1) - 1;            // 0.5 -> -1; 1, 1.5 -> 0; 2, 3 -> 1; 4, 6 -> 2
  const uint32_t mant = (m3 >= 2) ? ((m3 & 1u) << 22) : 0u;
  const int be = e + (int)b;                   // biased exponent of the product
  if (be >= 255) return sign | 0x7f800000u;
  if (be >= 1) return sign | ((uint32_t)be << 23) | mant;
  return sign | ((0x800000u | mant) >> (1 - be));
}

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ packed,
                                                         const uint8_t* __restrict__ scales,
                                                         int64_t nblocks, void* __restrict__ dst) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = gid >> 3;
  const int sub = (int)(gid & 7);
  if (blk >= nblocks) return;
  const uint32_t two = *reinterpret_cast<const uint16_t*>(packed + blk * 16 + sub * 2);
  const uint32_t b = scales[blk];
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = decode_f32_bits((two >> (4 * i)) & 15u, b);
  const int64_t e0 = blk * 32 + sub * 4;
  if (BF16_OUT) {
    // every decoded value has at most two significant bits: the top half is exact
    uint2 v = make_uint2((r[0] >> 16) | (r[1] & 0xffff0000u), (r[2] >> 16) | (r[3] & 0xffff0000u));
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(dst) + e0) = v;
  } else {
    *reinterpret_cast<uint4*>(reinterpret_cast<float*>(dst) + e0) = make_uint4(r[0], r[1], r[2], r[3]);
  }
}

inline unsigned grid_for(int64_t nblocks) { return (unsigned)((nblocks * 8 + 255) / 256); }

// Tiled weight layout of G matrices [R][K] (R % 16 == 0): codes [G][R/16][K/32][16][16 bytes]
// (the 16-byte block b of rows 16q..16q+15 as one 256-byte run), scales [G][K/32][R]. One thread
// per 16-byte code block, in source order (coalesced reads, 16-byte scattered writes).
__global__ __launch_bounds__(256) void tile_codes_kernel(const uint4* __restrict__ src, int64_t rows,
                                                         int nb, int R, uint4* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (matrix row, block)
  if (i >= rows * nb) return;
  const int64_t row = i / nb;                                   // over all G * R rows
  const int b = (int)(i - row * nb);
  const int64_t g = row / R;
  const int r = (int)(row - g * R);
  dst[((g * (R >> 4) + (r >> 4)) * nb + b) * 16 + (r & 15)] = src[i];
}
// One thread per scale byte, in destination order (coalesced writes).
__global__ __launch_bounds__(256) void tile_scales_kernel(const uint8_t* __restrict__ src, int64_t rows,
                                                          int nb, int R, uint8_t* __restrict__ dst) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (matrix, block, row)
  if (o >= rows * nb) return;
  const int64_t gb = o / R;
  const int r = (int)(o - gb * R);
  const int64_t g = gb / nb;
  const int b = (int)(gb - g * nb);
  dst[o] = src[(g * R + r) * nb + b];
}

}  // namespace

hipError_t launch_quantize(const void* src, bool bf16_in, int64_t nblocks, uint8_t* packed,
                           uint8_t* scales, hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;
  if (bf16_in)
    hipLaunchKernelGGL(quantize_kernel<true>, dim3(grid_for(nblocks)), dim3(256), 0, stream, src,
                       nblocks, packed, scales);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, dim3(grid_for(nblocks)), dim3(256), 0, stream, src,
                       nblocks, packed, scales);
  return hipGetLastError();
}

hipError_t launch_tile_weights(const uint8_t* packed, const uint8_t* scales, int64_t G, int R,
                               int K, uint8_t* packed_t, uint8_t* scales_t, hipStream_t stream) {
  const int64_t rows = G * R;
  const int nb = K >> 5;
  if (rows == 0 || nb == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows * nb + 255) / 256);
  hipLaunchKernelGGL(tile_codes_kernel, dim3(grid), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(packed), rows, nb, R, reinterpret_cast<uint4*>(packed_t));
  hipLaunchKernelGGL(tile_scales_kernel, dim3(grid), dim3(256), 0, stream, scales, rows, nb, R,
                     scales_t);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* packed, const uint8_t* scales, int64_t nblocks,
                             void* dst, bool bf16_out, hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;
  if (bf16_out)
    hipLaunchKernelGGL(dequantize_kernel<true>, dim3(grid_for(nblocks)), dim3(256), 0, stream,
                       packed, scales, nblocks, dst);
  else
    hipLaunchKernelGGL(dequantize_kernel<false>, dim3(grid_for(nblocks)), dim3(256), 0, stream,
                       packed, scales, nblocks, dst);
  return hipGetLastError();
}

}  // namespace mx
