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
// Mapping: the quantizer takes one 32-element block per thread; the decoder eight lanes per block,
// four consecutive elements per lane.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {
namespace {

// One thread per 32-element block (bf16 inputs: quantize_block32_bf16, the function the
// activation variant's gate_up epilogue uses too; fp32 inputs: the integer quantize_block32):
// a wave reads 4 KB (bf16) or 8 KB (fp32) of contiguous input and writes 1 KB of packed codes and
// 64 scale bytes.
template <bool BF16_IN>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ src,
                                                       int64_t nblocks,
                                                       uint8_t* __restrict__ packed,
                                                       uint8_t* __restrict__ scales) {
  const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= nblocks) return;
  uint32_t q[4], sb;
  if (BF16_IN) {  // 8-byte aligned rows of bf16
    const uint2* p = reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(src) + blk * 32);
    uint32_t w[16];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const uint2 d = p[v];
      w[2 * v] = d.x;
      w[2 * v + 1] = d.y;
    }
    sb = quantize_block32_bf16(w, q);
  } else {        // 16-byte aligned rows of fp32
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(src) + blk * 32);
    uint32_t u[32];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const uint4 d = p[v];
      u[4 * v] = d.x; u[4 * v + 1] = d.y; u[4 * v + 2] = d.z; u[4 * v + 3] = d.w;
    }
    sb = quantize_block32(u, q);
  }
  *reinterpret_cast<uint4*>(packed + blk * 16) = make_uint4(q[0], q[1], q[2], q[3]);
  scales[blk] = (uint8_t)sb;
}

// The MoE MLP's activation variant, decode-shaped calls: x [T][H] bf16 quantized along H (one
// thread per block, as above), codes in token order (the GEMM gathers their rows), and each
// block's scale byte written to every pair of its token that the permutation kept, block-major
// in pair order: scales_bm[b * pitch + inv[t * k + j]]. A stage's scale loads are then one
// contiguous run per block, where the rows of a tile (consecutive pairs) are scattered tokens.
__global__ __launch_bounds__(256) void quantize_x_scatter_kernel(const uint16_t* __restrict__ x,
                                                                 int64_t nblocks, int nb,
                                                                 const int32_t* __restrict__ inv,
                                                                 int k, int P, int64_t pitch,
                                                                 uint8_t* __restrict__ packed,
                                                                 uint8_t* __restrict__ scales_bm) {
  const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= nblocks) return;
  const uint2* src = reinterpret_cast<const uint2*>(x + blk * 32);
  uint32_t w[16], q[4];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const uint2 d = src[v];
    w[2 * v] = d.x;
    w[2 * v + 1] = d.y;
  }
  const uint32_t sb = quantize_block32_bf16(w, q);
  *reinterpret_cast<uint4*>(packed + blk * 16) = make_uint4(q[0], q[1], q[2], q[3]);
  const int64_t t = blk / nb;
  const int b = (int)(blk - t * nb);
  for (int j = 0; j < k; ++j) {
    const int r = inv[t * k + j];
    if (r >= 0 && r < P) scales_bm[b * pitch + r] = (uint8_t)sb;
  }
}

// Prefill-shaped calls: x's codes and scales, quantized in token order ([T][nb] blocks), copied
// into pair order in the layout the prefill GEMM stages read: for pair row p (token perm[p] / k)
// and block b, the 16 code bytes at ((p / 16) * nb + b) * 256 + (p % 16) * 16 (block b of 16
// consecutive pairs as one 256-byte run) and the scale byte at b * pitch + p. One thread per
// (pair, block), consecutive threads on consecutive pairs of one block: whole runs stored, the
// packed token rows read k times (a quarter of the bytes of re-reading x).
__global__ __launch_bounds__(256) void x_pair_copy_kernel(const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ scales,
                                                          int nb, const int32_t* __restrict__ perm,
                                                          int k, int P, int64_t pitch,
                                                          uint8_t* __restrict__ packed,
                                                          uint8_t* __restrict__ scales_bm) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t g = i / (16 * nb);
  const int rem = (int)(i - g * 16 * nb);
  const int b = rem >> 4;
  const int64_t pr = g * 16 + (rem & 15);
  if (pr >= P) return;
  const int64_t tb = (int64_t)(perm[pr] / k) * nb + b;
  *reinterpret_cast<uint4*>(packed + (g * nb + b) * 256 + (rem & 15) * 16) =
      *reinterpret_cast<const uint4*>(codes + tb * 16);
  scales_bm[b * pitch + pr] = scales[tb];
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
// deint: source row r goes to row r/2 (even r) or R/2 + r/2 (odd r) of the tiled matrix.
__global__ __launch_bounds__(256) void tile_codes_kernel(const uint4* __restrict__ src, int64_t rows,
                                                         int nb, int R, int deint,
                                                         uint4* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (matrix row, block)
  if (i >= rows * nb) return;
  const int64_t row = i / nb;                                   // over all G * R rows
  const int b = (int)(i - row * nb);
  const int64_t g = row / R;
  const int r0 = (int)(row - g * R);
  const int r = deint ? ((r0 & 1) ? (R >> 1) + (r0 >> 1) : (r0 >> 1)) : r0;
  dst[((g * (R >> 4) + (r >> 4)) * nb + b) * 16 + (r & 15)] = src[i];
}
// One thread per scale byte, in destination order (coalesced writes).
__global__ __launch_bounds__(256) void tile_scales_kernel(const uint8_t* __restrict__ src, int64_t rows,
                                                          int nb, int R, int deint,
                                                          uint8_t* __restrict__ dst) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (matrix, block, row)
  if (o >= rows * nb) return;
  const int64_t gb = o / R;
  const int r = (int)(o - gb * R);
  const int64_t g = gb / nb;
  const int b = (int)(gb - g * nb);
  const int rs = deint ? (r < (R >> 1) ? 2 * r : 2 * (r - (R >> 1)) + 1) : r;  // source row
  dst[o] = src[(g * R + rs) * nb + b];
}

}  // namespace

hipError_t launch_quantize_x_scatter(const uint16_t* x, int T, int H, const int32_t* inv, int k,
                                     int64_t pitch, uint8_t* packed, uint8_t* scales_bm,
                                     hipStream_t stream) {
  const int64_t nblocks = (int64_t)T * (H / 32);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_x_scatter_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256),
                     0, stream, x, nblocks, H / 32, inv, k, T * k, pitch, packed, scales_bm);
  return hipGetLastError();
}

hipError_t launch_x_pair_copy(const uint8_t* codes, const uint8_t* scales, int H,
                              const int32_t* perm, int k, int P, int64_t pitch, uint8_t* packed,
                              uint8_t* scales_bm, hipStream_t stream) {
  const int64_t n = (int64_t)(P + 15) / 16 * 16 * (H / 32);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(x_pair_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     codes, scales, H / 32, perm, k, P, pitch, packed, scales_bm);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* src, bool bf16_in, int64_t nblocks, uint8_t* packed,
                           uint8_t* scales, hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;
  const unsigned grid = (unsigned)((nblocks + 255) / 256);
  if (bf16_in)
    hipLaunchKernelGGL(quantize_kernel<true>, dim3(grid), dim3(256), 0, stream, src, nblocks,
                       packed, scales);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, dim3(grid), dim3(256), 0, stream, src, nblocks,
                       packed, scales);
  return hipGetLastError();
}

hipError_t launch_tile_weights(const uint8_t* packed, const uint8_t* scales, int64_t G, int R,
                               int K, bool deinterleave, uint8_t* packed_t, uint8_t* scales_t,
                               hipStream_t stream) {
  const int64_t rows = G * R;
  const int nb = K >> 5;
  if (rows == 0 || nb == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows * nb + 255) / 256);
  const int di = deinterleave ? 1 : 0;
  hipLaunchKernelGGL(tile_codes_kernel, dim3(grid), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(packed), rows, nb, R, di,
                     reinterpret_cast<uint4*>(packed_t));
  hipLaunchKernelGGL(tile_scales_kernel, dim3(grid), dim3(256), 0, stream, scales, rows, nb, R, di,
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
