// gemm_tile.h -- one output tile of the MXFP4 weight-only matrix products on gfx950 (the MoE
// MLP's gate_up with fused SwiGLU, its down projection, and the dense linear), the tile
// configurations, and the per-token combine; shared by the kernels launched one per product
// (gemm.hip) and the single-launch decode pipeline (single.hip).
//
// The packed weights are never expanded in memory: they stream from HBM into LDS as 16-byte
// chunks (direct global->LDS loads, several stages in flight) and are decoded in registers right
// before the bf16 MFMA (v_cvt_scalef32_pk_bf16_fp4: two E2M1 codes times the block's E8M0 scale
// per instruction). That is the design the pages point at: quantized matmuls that read the packed
// weights without expanding them ("Hugging Face Transformers GGUF 지원", section "ggml Metal 커널
// 통합") and dedicated MXFP4 kernels instead of a bf16 fallback ("Transformers 4.40 performance
// upgrades for OpenAI GPT-OSS ...", section "MXFP4 4-Bit Quantization").
//
// Operand mapping (v_mfma_f32_16x16x32_bf16, or v_mfma_f32_32x32x16_bf16 for 32 x 32 fragments).
// The reduction order inside a product does not matter, so the K axis is assigned to lanes in
// whole 32-element blocks: in one "super-step" of four MFMAs, lane group g owns one block of the
// K tile (g = lane/16 and block 4j+g for 16 x 16 fragments; g = lane/32 and block 2j+g for
// 32 x 32), and MFMA s uses elements [8s, 8s+8) of it. A lane therefore reads one whole 16-byte
// packed block (one scale byte) per super-step and 64 contiguous bytes of the bf16 activation row.
//
// LDS layout per stage: A [BM rows][KT*64 B], B [BN rows][KT*16 B], 16-byte chunks XOR-swizzled
// by row so that the per-lane 16-byte reads of 8 consecutive rows hit distinct bank groups. The
// swizzle is applied on the load side by choosing which global chunk each lane fetches (the LDS
// destination of a direct load is fixed: lane i writes base + 16*i).
#pragma once
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {
namespace {

enum { MODE_LINEAR = 0, MODE_GATE_UP = 1, MODE_DOWN = 2 };
enum { SCM_BYTE = 0, SCM_STAGE = 1, SCM_RESIDENT = 2 };  // how weight scales reach LDS
constexpr int kResidentNb = 96;  // resident scales hold up to K = 3072 (32-blocks per row)

struct GemmKArgs {
  const uint16_t* A;          // bf16 activation rows of length K; MXFP4 codes: [a_rows][K/2] in
                              // the dense linear, tiled in pair order [a_rows/16][K/32][16][16]
                              // in the MoE products
  int64_t a_rows;             // rows in A (bounds the buffer view of A)
  const uint8_t* Asc;         // A scales when A is MXFP4 (else unused): [a_rows][K/32] in the
                              // linear, block-major in pair order [K/32][sc_pitch] in the MoE
  int64_t sc_pitch;           // FP4 x and h scales, block-major (rows of P, rounded up to 4)
  const int32_t* a_gather;    // A row of permuted row r = a_gather[r] / a_div (NULL: r)
  int a_div;
  const uint8_t* Bp;          // packed weights, expert-major
  const uint8_t* Bs;          // scales, expert-major
  int64_t b_rows_per_expert;  // weight rows per expert (2F gate_up, H down, N linear)
  int n_tiles;                // column tiles
  int N;                      // output columns (F for gate_up)
  int K;
  const int2* tiles;          // grouped: (expert, first permuted row); NULL = dense
  const int32_t* num_tiles;
  const int32_t* offsets;     // grouped: expert row offsets [E+1]
  int M;                      // dense rows
  int rows_total;             // rows of the (permuted) row space: P grouped, M dense
  int F;                      // gate_up: up rows start at F
  void* out;                  // gate_up with FP4 activations: packed codes of h, tiled in pair
                              // order [rows/16][F/32][16][16]
  uint8_t* out_scales;        //   and their scale bytes, block-major [F/32][sc_pitch]
  int out_bf16;
  // expert activation of the gate_up epilogue (act_custom = 0: h = silu(g) * u) with its bias
  // [E][2F] in the caller's row order, interleaved or not (NULL = none). (The down bias is added
  // by the combine.)
  const float* bias;
  int act_custom, bias_interleaved;
  float act_alpha, act_limit, act_shift;
  int gn;                     // column tiles per XCD super-tile (set by the launcher)
  int k_splits;               // linear only: K range split over blockIdx.z (<= 1: none); out
  int64_t part_stride;        //   then takes fp32 partial sums, split z at z * part_stride
};

// LDS swizzles, by the number of 16-byte chunks per LDS row (CH). Chunk c of row r is stored at
// slot c ^ swz(r). The per-lane 16-byte reads of one MFMA operand cover 16 (or 32) consecutive
// rows at the same chunk; with 256-byte bank rows a chunk's bank group is (r % (16/CH))*CH + slot
// for CH < 16, so the pattern must give distinct slots to the rows that share r % (16/CH) within
// any 16 consecutive rows. Measured conflict-free on gfx950 for that access where CH >= 4
// (SQ_LDS_BANK_CONFLICT = 0 for ds_read_b128 over 16 rows x 4 lane groups; e.g. "r & 15" on
// 256-byte rows costs 2x):
//   CH >= 16 (bf16 A rows of 4+ blocks): ((r & 7) << 1) | ((r >> 3) & 1)
//   CH = 8 (128-byte rows): (r ^ (r >> 3)) & 7     CH = 4: ((r >> 2) ^ (r >> 1)) & 3
//   CH = 2 (32-byte rows: rows r and r + 8 share a bank group): (r >> 3) & 1
template <int CH>
__device__ __forceinline__ int swz_rows(int row) {
  static_assert(CH == 2 || CH == 4 || CH == 8 || CH >= 16, "LDS row size");
  if constexpr (CH == 2) return (row >> 3) & 1;
  else if constexpr (CH == 4) return ((row >> 2) ^ (row >> 1)) & 3;
  else if constexpr (CH == 8) return (row ^ (row >> 3)) & 7;
  else return ((row & 7) << 1) | ((row >> 3) & 1);
}

// Buffer views. Loads go through buffer resources (base address, byte size): each lane keeps a
// fixed 32-bit offset and the stage's K offset is a scalar, so issuing a stage costs no vector
// ALU work; an offset at or past the size reads zeros, which is how blocks past the end of K are
// filled (zero codes and zero activations contribute nothing, so the MFMA loop needs no masks).
constexpr uint32_t kBufWord3 = 0x00020000u;   // raw, untyped buffer (gfx9 family)
constexpr uint32_t kOutOfRange = 0xfffffff0u;
// A resource as the four scalar dwords: base[31:0]; base[47:32] with stride 0; size; word 3.
__device__ __forceinline__ i32x4 make_res(const void* base, int64_t bytes) {
  const int nrec = bytes > 0x7ffffff0LL ? 0x7ffffff0 : (int)bytes;  // host checks keep it below
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
               __builtin_amdgcn_readfirstlane(nrec), (int)kBufWord3};
}

// LDS offset of a pointer into a __shared__ object: the low 32 bits of its generic address (the
// shared aperture base has zero low bits), without the null check of an address-space cast.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

// Direct global -> LDS loads (buffer_load ... lds): lane i writes lds + 16*i (16-byte form),
// lds + 4*i (dword form) or the first byte of the dword at lds + 4*i (byte form); lds must be
// wave-uniform. They are written as
// inline asm on purpose: the compiler orders each LDS read after every direct-to-LDS load it
// cannot prove disjoint, and it does not tell the pipeline's stage buffers apart, so with the
// builtin every LDS read of the current stage would also wait for the loads in flight into the
// next ones. The callers wait for these loads themselves (s_waitcnt vmcnt, then a barrier)
// before reading what they wrote. The s_nop covers the M0-write -> LDS-DMA hazard.
// NT: the load carries the non-temporal cache hint (data read once: it need not stay cached).
template <bool NT = false>
__device__ __forceinline__ void dma_b128(const i32x4& res, uint32_t voff, uint32_t soff,
                                         const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds"
                 :: "v"(voff), "s"(res), "s"(__builtin_amdgcn_readfirstlane(soff)), "s"(m0)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(res), "s"(__builtin_amdgcn_readfirstlane(soff)), "s"(m0)
                 : "memory", "m0");
}
// The 16-byte load as device-coherent (sc1): it reads the device's point of coherence, never a
// line of this XCD's L2 that predates another workgroup's write -- for data that workgroups of
// the same launch write (with device-coherent stores, store_coherent) before the reader runs.
__device__ __forceinline__ void dma_b128_coherent(const i32x4& res, uint32_t voff, uint32_t soff,
                                                  const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen sc1 lds"
               :: "v"(voff), "s"(res), "s"(__builtin_amdgcn_readfirstlane(soff)), "s"(m0)
               : "memory", "m0");
}
// 16 bytes as four device-coherent dword stores (sc1: written through to the device's point of
// coherence, so a device-coherent read elsewhere sees them once this wave's stores complete).
__device__ __forceinline__ void store_coherent(void* dst, const uint4& v) {
  uint32_t* d = reinterpret_cast<uint32_t*>(dst);
  __hip_atomic_store(d, v.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(d + 1, v.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(d + 2, v.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(d + 3, v.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void dma_b8(const i32x4& res, uint32_t voff, uint32_t soff,
                                       const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_ubyte %0, %1, %2 offen lds"
               :: "v"(voff), "s"(res), "s"(__builtin_amdgcn_readfirstlane(soff)), "s"(m0)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(const i32x4& res, uint32_t voff, uint32_t soff,
                                        const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(res), "s"(__builtin_amdgcn_readfirstlane(soff)), "s"(m0)
               : "memory", "m0");
}

// E8M0 byte -> fp32 scale operand 2^(b-127), without branches: 2^-127 * 2^b is exact for every
// b (b = 0 gives the subnormal 2^-127), b = 255 overflows to +Inf, and s - (s - s) keeps every
// finite s and turns Inf into NaN, the value of that byte.
__device__ __forceinline__ float e8m0_scale(uint32_t b) {
  const float s = __builtin_amdgcn_ldexpf(0x1p-127f, (int)b);
  return s - (s - s);
}

// Lane offset plus a stage offset, saturating: the out-of-range marker stays out of range.
__device__ __forceinline__ uint32_t off_add(uint32_t voff, uint32_t add) {
  return __builtin_elementwise_add_sat(voff, add);
}

// 32-bit lane offsets of the direct loads of one LDS region. A region of `bytes` bytes is filled
// by bytes/1024 wave-instructions of 64 x 16 bytes (or bytes/256 of 64 x 1 byte for scale
// regions, one byte per dword); wave w issues instructions w*I .. w*I+I-1 (mod the count). When a
// region is smaller than one instruction per wave, several waves load the same bytes to the same
// place, which is harmless and keeps every wave's count of memory ops the same.
template <int REGION_INSTRS, int NW>
struct DmaPlan {
  static constexpr int I = (REGION_INSTRS + NW - 1) / NW;  // instructions per wave
  static __device__ __forceinline__ int instr(int wave, int q) { return (wave * I + q) % REGION_INSTRS; }
};

// An int of the launch's own outputs: plain, or (COH) device-coherent.
template <bool COH>
__device__ __forceinline__ int ld_int(const int* p) {
  if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

// Weight row (within the expert) of local tile row lrow; gate_up tiles hold BN/2 gate rows then
// the matching BN/2 up rows. Rows past the end repeat the last one (their results are dropped).
template <int MODE, int BN>
__device__ __forceinline__ int weight_row_of(const GemmKArgs& p, int nt, int lrow) {
  constexpr int BNH = BN / 2;
  if (MODE == MODE_GATE_UP)
    return lrow < BNH ? min(nt * BNH + lrow, p.F - 1) : p.F + min(nt * BNH + lrow - BNH, p.F - 1);
  return min(nt * BN + lrow, p.N - 1);
}

// Local tile row of fragment f (MF columns) of wave column wn (lane row ln): gate_up waves take
// FN/2 gate fragments and the FN/2 up fragments of the same output columns.
template <int MODE, int BN, int WN, int FN, int MF>
__device__ __forceinline__ int frag_row(int wn, int f, int ln) {
  constexpr int BNH = BN / 2, TN = BN / WN;
  if (MODE == MODE_GATE_UP)
    return ((f < FN / 2) ? wn * (BNH / WN) + f * MF : BNH + wn * (BNH / WN) + (f - FN / 2) * MF) + ln;
  return wn * TN + f * MF + ln;
}

// Row within an MF x MF accumulator fragment of value v of lane group g (the lane's column is
// lane % MF): 16 x 16 -> 4g + v (v < 4); 32 x 32 -> 8(v/4) + 4g + v%4 (v < 16).
template <int MF>
__device__ __forceinline__ int acc_row(int g, int v) {
  return MF == 32 ? 8 * (v >> 2) + 4 * g + (v & 3) : 4 * g + v;
}
template <int MF>
using AccT = std::conditional_t<MF == 32, f32x16, f32x4>;

// Epilogue of a wave's FM x FN fragments (rows r0 + wm*TM + MF*i + acc_row(g, v), column lane
// ln): down -> fp32 at the permuted row (the combine applies the routing weights: the epilogue
// needs no index or weight loads); linear -> fp32 or bf16. (gate_up stores through LDS, below.)
template <int MODE, int FM, int FN, int TM, int BN, int WN, int MF>
__device__ __forceinline__ void store_tile(const GemmKArgs& p, const AccT<MF> (&acc)[FM][FN], int r0,
                                           int row_end, int nt, int wm, int wn, int g, int ln) {
  constexpr int TN = BN / WN;
  constexpr int NV = MF == 32 ? 16 : 4;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int r = r0 + wm * TM + i * MF + acc_row<MF>(g, q);
      if (r >= row_end) continue;
      if constexpr (MODE == MODE_DOWN) {
        float* y = reinterpret_cast<float*>(p.out);
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int col = nt * BN + wn * TN + f * MF + ln;
          if (col < p.N) y[(int64_t)r * p.N + col] = acc[i][f][q];
        }
      } else {
        const int64_t zoff = p.k_splits > 1 ? (int64_t)blockIdx.z * p.part_stride : 0;
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int col = nt * BN + wn * TN + f * MF + ln;
          if (col >= p.N) continue;
          if (p.out_bf16)
            reinterpret_cast<uint16_t*>(p.out)[(int64_t)r * p.N + col] =
                (uint16_t)f32_to_bf16_bits(acc[i][f][q]);
          else
            reinterpret_cast<float*>(p.out)[zoff + (int64_t)r * p.N + col] = acc[i][f][q];
        }
      }
    }
  }
}

// Grouped / dense MXFP4 GEMM tile: out[BM rows x BN cols] = A times the weights (decoded).
//   BM x BN workgroup tile, WM x WN waves, each wave a (BM/WM) x (BN/WN) tile of MF x MF MFMA
//   fragments; KT 32-element blocks per pipeline stage; STAGES (2 to 4) stages in flight.
//   AFP4 = false: A is bf16 and the weights are decoded to bf16 for v_mfma_f32_16x16x32_bf16
//                 (MF = 16) or v_mfma_f32_32x32x16_bf16 (MF = 32).
//   AFP4 = true:  A is MXFP4 too (packed codes + E8M0 scales, same layout as the weights) and
//                 each 16 x 16 x 128 slice is one v_mfma_scale_f32_16x16x128_f8f6f4 with both
//                 operands' block scales, so nothing is decoded.
// Per stage a workgroup moves A chunks and B chunks straight into LDS. The weight scale bytes
// come one of three ways (SCM):
//   SCM_RESIDENT: all K/32 scale bytes of the tile's rows, once per tile. A tile's rows are one
//     (two for gate_up) contiguous byte ranges, loaded as the aligned dwords that cover them:
//     few, coalesced requests, which matters where streaming the weights is the bound.
//   SCM_STAGE: per stage, each row's KT bytes as the SD = ceil(KT/4) + 1 aligned dwords that cover
//     them (the first byte sits at a fixed shift, as stages advance by KT, a multiple of 4).
//   SCM_BYTE: per stage, one byte per lane into its own dword (4x the LDS, exact at any size).
// The dword forms may read past a row's last block (next row, or past K in the last stage):
// those blocks have zero codes and their scale is read as 1.0. A dword the buffer size cuts
// reads as zero, so weights whose scale array is not a whole number of dwords take SCM_BYTE.
// Rows of the tile past its expert's last row are loaded as out-of-range (zeros, no traffic).
// LDS of one GEMM tile: the pipeline stages, the resident weight scales and the tile's activation
// rows. The pipeline stages are filled by direct loads written as inline asm the compiler does
// not see, so it neither orders LDS reads after them nor tracks them: the kernel waits itself.
// 1 KiB-aligned elements: the swizzles and 16-byte reads assume every stage starts on one.
template <int BM, int BN, int WM, int WN, int KT, int STAGES, int MODE, bool AFP4, int SCM, bool TW>
struct GemmLds {
  static constexpr int NW = WM * WN;
  static constexpr bool SWIGLU = (MODE == MODE_GATE_UP);
  static constexpr int BNH = BN / 2;
  static constexpr int A_ROW = AFP4 ? KT * 16 : KT * 64, B_ROW = KT * 16;
  static constexpr int A_STAGE = BM * A_ROW, B_STAGE = BN * B_ROW;
  static constexpr int SD = (KT + 3) / 4 + 1;  // scale dwords per row and stage
  // (stage scale dwords padded to a whole number of instructions per wave: no repeated loads)
  static constexpr int S_DW = SCM == SCM_STAGE ? ((TW ? KT * BN / 4 : BN * SD) + 64 * NW - 1) / (64 * NW) * (64 * NW)
                                               : SCM == SCM_BYTE ? BN * KT : 64;
  // FP4 activation scales of a stage: row-major rows' SD dwords each (the dense linear), or (SBM:
  // the MoE products, whose tile rows are consecutive pairs; the gate_up epilogue writes h's
  // scales block-major in pair order, and the x quantizer writes x's so for every pair of each
  // token) per block the SW aligned dwords that cover the tile's BM bytes of that block's row of
  // the block-major array
  static constexpr bool SBM = AFP4 && MODE != MODE_LINEAR;
  // FP4 activation codes of the prefill-shaped MoE products (tiles of 64 rows or more) in the
  // tiled layout, in pair order: [P/16][K/32][16 rows][16 bytes] (block b of rows 16q..16q+15
  // as one 256-byte run; the x pair copy and the gate_up epilogue write them so), so a stage's A
  // loads are whole 256-byte runs. Decode-shaped tiles (16 rows, weight streaming) keep
  // row-major codes: x in token order, gathered, and h in pair order (the tiled form measured
  // 6 % slower there).
  static constexpr bool ATW = AFP4 && MODE != MODE_LINEAR && BM >= 64;
  static constexpr int SW = BM / 4 + 1;
  static constexpr int SA_DW = ((SBM ? KT * SW : BM * SD) + 63) / 64 * 64;  // activation scale dwords
  // resident scales: region 1 (up rows of gate_up) starts at dword R1; whole instructions
  static constexpr int R1 = (BNH * kResidentNb + 8) / 4;
  static constexpr int RS_DW = ((TW ? kResidentNb * BN / 4 : SWIGLU ? 2 * R1 : (BN * kResidentNb + 8) / 4) + 63) / 64 * 64;
  struct __attribute__((aligned(1024))) Stage {
    uint8_t A[A_STAGE];
    uint8_t B[B_STAGE];
    uint32_t Sc[SCM == SCM_RESIDENT ? 0 : S_DW];  // weight scale bytes of the stage
    uint32_t Sa[AFP4 ? SA_DW : 0];     // activation scale bytes (FP4 A), same layout
  };
  static_assert(sizeof(Stage) % 1024 == 0, "stage alignment");
  struct Storage {
    Stage stg[STAGES];
    uint32_t sRes[SCM == SCM_RESIDENT ? RS_DW : 1];  // resident weight scales (4 B if unused)
    int sArow[BM];
  };
};

// gemm_tile computes output tile (expert e, permuted rows [r0, min(r0 + BM, row_end)), column
// tile nt) in the LDS sm; gemm_body, below, is the launch-grid form (tile from blockIdx).
// STREAMW: the weight loads carry the non-temporal hint (see issue_w). COH: for a launch whose own
// workgroups wrote the tile's inputs: the gather indices and, in the down product, the activation
// rows (h) are loaded device-coherent, and the tile's output (h or the down rows) is stored
// device-coherent.
template <int BM, int BN, int WM, int WN, int KT, int STAGES, int MODE, bool AFP4, int SCM,
          bool TW, int MF, bool STREAMW, bool COH = false>
__device__ __forceinline__ void gemm_tile(
    const GemmKArgs& p, typename GemmLds<BM, BN, WM, WN, KT, STAGES, MODE, AFP4, SCM, TW>::Storage& sm,
    int e, int r0, int row_end, int nt) {
  using LD = GemmLds<BM, BN, WM, WN, KT, STAGES, MODE, AFP4, SCM, TW>;
  constexpr int NW = WM * WN;
  constexpr int NT = NW * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / MF, FN = TN / MF;
  constexpr int LG = 64 / MF;  // lane groups: each owns one 32-element K block per super-step
  constexpr int NV = MF == 32 ? 16 : 4;  // accumulator values per lane and fragment
  constexpr bool SWIGLU = (MODE == MODE_GATE_UP);
  constexpr int BNH = BN / 2;
  constexpr int A_ROW = LD::A_ROW, B_ROW = LD::B_ROW;
  constexpr int A_STAGE = LD::A_STAGE, B_STAGE = LD::B_STAGE;
  using PA = DmaPlan<A_STAGE / 1024, NW>;
  using PB = DmaPlan<B_STAGE / 1024, NW>;
  constexpr int SD = LD::SD, S_DW = LD::S_DW;
  // LDS bytes between a row's consecutive block scales (tiled weights: [block][row] bytes)
  constexpr int SBS = TW ? BN : SCM == SCM_BYTE ? 4 : 1;
  constexpr int B_KB = TW ? 256 : 16;                      // weight bytes between blocks of a row
  constexpr int SA_DW = LD::SA_DW, R1 = LD::R1, RS_DW = LD::RS_DW;
  using PS = DmaPlan<S_DW / 64, NW>;
  using PSA = DmaPlan<AFP4 ? SA_DW / 64 : 1, NW>;
  using PR = DmaPlan<RS_DW / 64, NW>;
  constexpr int IA = PA::I, IB = PB::I, IS = SCM == SCM_RESIDENT ? 0 : PS::I, ISA = AFP4 ? PSA::I : 0;
  constexpr int SS = KT / LG;                              // super-steps per stage
  constexpr int LPS = IS + ISA + IA + IB;                  // vector-memory ops per wave per stage
  static_assert(A_STAGE % 1024 == 0 && B_STAGE % 1024 == 0, "stage split");
  static_assert(FM * MF * WM == BM && FN * MF * WN == BN, "wave tile");
  static_assert(MF == 16 || (MF == 32 && !AFP4), "32 x 32 fragments: bf16 activations only");
  static_assert(!SWIGLU || FN % 2 == 0, "gate/up fragment pairs");
  static_assert(KT % LG == 0 && KT % 2 == 0 && STAGES >= 2 && STAGES <= 4, "pipeline");
  constexpr int ACH = A_ROW / 16, BCH = B_ROW / 16;       // 16-byte chunks per LDS row
  static_assert((STAGES - 1) * LPS < 64, "vmcnt range");
  static_assert(BM <= NT, "one gathered row per thread");
  static_assert(!TW || (SCM != SCM_BYTE && BNH % 16 == 0), "tiled weights: dword scales, row groups");
  // row-major dword stage scales keep a row's first byte at a fixed shift only if stages advance
  // by a multiple of 4 blocks
  static_assert(SCM != SCM_STAGE || TW || KT % 4 == 0, "row-major stage scales: 4-block stages");
  static_assert(!COH || (!AFP4 && MODE != MODE_LINEAR), "coherent tiles: bf16 MoE products");

  using Stage = typename LD::Stage;
  Stage* stg = sm.stg;
  uint32_t* sRes = sm.sRes;
  int* sArow = sm.sArow;
  const int K = p.K;
  const int nb = K >> 5;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS targets go in M0
  const int wm = wave / WN, wn = wave % WN;
  const int ln = lane % MF, g = lane / MF;

  // ---- weight rows (within the expert) ----
  auto weight_row = [&](int lrow) -> int { return weight_row_of<MODE, BN>(p, nt, lrow); };
  // Tiled weights: tile rows map to whole 16-row groups; rows past the matrix are not clamped
  // (gate rows past F read up rows, rows past the end are out of range: zeros, dropped).
  auto weight_row_u = [&](int lrow) -> int {
    if constexpr (SWIGLU) return lrow < BNH ? nt * BNH + lrow : p.F + nt * BNH + lrow - BNH;
    else return nt * BN + lrow;
  };
  const int64_t rpe = p.b_rows_per_expert;
  const i32x4 rB = make_res(p.Bp + (int64_t)e * rpe * (K >> 1), rpe * (K >> 1));
  const i32x4 rS = make_res(p.Bs, (int64_t)(e + 1) * rpe * nb);  // absolute, 4-aligned offsets
  const int n_valid = min(BM, row_end - r0);                      // tile rows of this expert
  const i32x4 rA = make_res(p.A, (LD::ATW ? (p.a_rows + 15) / 16 * 16 : p.a_rows) * (AFP4 ? (K >> 1) : K * 2));
  // activation scales live in the library's workspace, padded past a whole dword
  const i32x4 rSA = make_res(p.Asc, !AFP4 ? 0 : LD::SBM ? (int64_t)nb * p.sc_pitch : (p.a_rows * nb + 3) / 4 * 4);
  uint32_t voffB[IB];
  int bblk[IB];
#pragma unroll
  for (int q = 0; q < IB; ++q) {
    const int off = PB::instr(wave, q) * 1024 + lane * 16;
    const int lrow = off / B_ROW;
    const int chunk = ((off % B_ROW) >> 4) ^ swz_rows<BCH>(lrow);
    bblk[q] = chunk;
    if constexpr (TW) {  // 16-row group gr/16, block chunk: 256 bytes, row gr%16 at 16 * (gr%16)
      const uint32_t gr = (uint32_t)weight_row_u(lrow);
      voffB[q] = (gr >> 4) * (uint32_t)(nb * 256) + (gr & 15u) * 16u + chunk * 256;
    } else {
      voffB[q] = (uint32_t)weight_row(lrow) * (uint32_t)(K >> 1) + chunk * 16;
    }
  }
  // scale dword idx of a stage's scale area is dword idx % SD covering row idx / SD
  auto row_scale_off = [&](int lrow) -> uint32_t {
    return ((uint32_t)e * (uint32_t)rpe + (uint32_t)weight_row(lrow)) * (uint32_t)nb;
  };
  // (byte mode: dword idx holds block idx % KT of row idx / KT)
  uint32_t voffS[IS > 0 ? IS : 1];
  int sblk[IS > 0 ? IS : 1];
#pragma unroll
  for (int q = 0; q < IS; ++q) {
    const int idx = PS::instr(wave, q) * 64 + lane;
    if constexpr (TW) {  // dword idx of [KT][BN]: rows 4*idx % BN .. +3 of block 4*idx / BN
      sblk[q] = 4 * idx / BN;
      voffS[q] = idx < KT * BN / 4
                     ? (uint32_t)(e * nb + sblk[q]) * (uint32_t)rpe + (uint32_t)weight_row_u(4 * idx % BN)
                     : kOutOfRange;
    } else if constexpr (SCM == SCM_STAGE) {
      sblk[q] = 0;
      voffS[q] = idx < BN * SD ? (row_scale_off(idx / SD) & ~3u) + 4 * (idx % SD) : kOutOfRange;
    } else {
      sblk[q] = idx % KT;
      voffS[q] = row_scale_off(idx / KT) + sblk[q];
    }
  }
  // resident scales: the tile's rows as one range (two for gate_up: gate rows, then up rows)
  int rg_rows[2] = {0, 0};
  uint32_t rg_start[2] = {0u, 0u};
  if constexpr (SCM == SCM_RESIDENT && !TW) {
    if (SWIGLU) {
      rg_rows[0] = rg_rows[1] = min(BNH, p.F - nt * BNH);
      rg_start[0] = row_scale_off(0);
      rg_start[1] = row_scale_off(BNH);
    } else {
      rg_rows[0] = min(BN, p.N - nt * BN);
      rg_start[0] = row_scale_off(0);
    }
  }
  int brow[FN], bsh[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    brow[f] = frag_row<MODE, BN, WN, FN, MF>(wn, f, ln);
    // LDS byte of the row's block 0 (of the stage, or of K for resident scales)
    if constexpr (TW) {
      bsh[f] = brow[f];
    } else if constexpr (SCM == SCM_RESIDENT) {
      const int rg = (SWIGLU && brow[f] >= BNH) ? 1 : 0;
      const int rr = min(brow[f] - rg * BNH, rg_rows[rg] - 1);
      bsh[f] = rg * R1 * 4 + (int)(rg_start[rg] & 3u) + rr * nb;
    } else if constexpr (SCM == SCM_STAGE) {
      bsh[f] = brow[f] * SD * 4 + (int)(row_scale_off(brow[f]) & 3u);
    } else {
      bsh[f] = brow[f] * KT * 4;
    }
  }

  // ---- activation rows, weight prefetch ----
  // The activation rows of a gathered tile depend on a chain of loads (tile -> perm -> row). The
  // row indices are read first, with scalar loads (uniform addresses, so they count on lgkmcnt),
  // and the first stages' weight loads go out right behind them: the weights stream while the
  // chain resolves. Rows past the tile's expert read some valid row; their results are dropped.
  int gv[BM];  // perm is padded by the tile height: BM entries from r0 exist
  if (p.a_gather != nullptr) {
#pragma unroll
    for (int q = 0; q < BM; ++q) gv[q] = ld_int<COH>(p.a_gather + r0 + q);
  }
  auto issue_w = [&](Stage& sg, int kt) {
    const int kb = kt * KT;
#pragma unroll
    for (int q = 0; q < IS; ++q) {
      if constexpr (TW)  // blocks past K (last stage only) are out of range: zero scales
        dma_b32(rS, kb + sblk[q] < nb ? off_add(voffS[q], (uint32_t)(kb * rpe)) : kOutOfRange, 0,
                &sg.Sc[PS::instr(wave, q) * 64]);
      else if constexpr (SCM == SCM_STAGE)
        dma_b32(rS, off_add(voffS[q], (uint32_t)kb), 0, &sg.Sc[PS::instr(wave, q) * 64]);
      else
        dma_b8(rS, kb + sblk[q] < nb ? voffS[q] + kb : kOutOfRange, 0, &sg.Sc[PS::instr(wave, q) * 64]);
    }
    // STREAMW where each weight tile serves one row tile alone (grouped-GEMM super-tiles of one
    // row tile: decode-shaped and few-pair tiles, GM = 1): its loads carry the non-temporal hint (20B-shaped
    // decode, T = 64: gate_up 59.0 -> 54.4 us, down 32.3 -> 30.5 us; 120B-shaped T = 256: gate_up
    // 209 -> 198 us). Prefill super-tiles share each weight tile between their row tiles through
    // L2, where the hint measured 14 % slower, and so do the dense linear's row tiles (M = 32:
    // 17.8 -> 19.5 us with it).
    if ((kt + 1) * KT <= nb) {  // full stage: the K offset goes in the scalar offset
#pragma unroll
      for (int q = 0; q < IB; ++q) dma_b128<STREAMW>(rB, voffB[q], kb * B_KB, &sg.B[PB::instr(wave, q) * 1024]);
    } else {
#pragma unroll
      for (int q = 0; q < IB; ++q)
        dma_b128<STREAMW>(rB, kb + bblk[q] < nb ? voffB[q] + kb * B_KB : kOutOfRange, 0,
                           &sg.B[PB::instr(wave, q) * 1024]);
    }
  };
  // K stages of this workgroup: all of them, or (split linear) split blockIdx.z's share
  int kt0 = 0, ntk = (nb + KT - 1) / KT;
  if constexpr (MODE == MODE_LINEAR) {
    if (p.k_splits > 1) {
      const int all = ntk, z = blockIdx.z;
      kt0 = z * all / p.k_splits;
      ntk = (z + 1) * all / p.k_splits - kt0;
    }
  }
  if constexpr (SCM == SCM_RESIDENT) {  // first of all loads: every stage wait covers it
#pragma unroll
    for (int q = 0; q < PR::I; ++q) {
      const int idx = PR::instr(wave, q) * 64 + lane;
      if constexpr (TW) {  // [block][row] bytes of the tile, blocks below nb
        const int blk = 4 * idx / BN;
        const uint32_t vo = (uint32_t)(e * nb + blk) * (uint32_t)rpe + (uint32_t)weight_row_u(4 * idx % BN);
        dma_b32(rS, blk < nb ? vo : kOutOfRange, 0, &sRes[PR::instr(wave, q) * 64]);
        continue;
      }
      const int rg = (SWIGLU && idx >= R1) ? 1 : 0;
      const int d = idx - rg * R1;
      const uint32_t a0 = rg_start[rg] & ~3u;
      const uint32_t end = rg_start[rg] + (uint32_t)(rg_rows[rg] * nb);
      const uint32_t vo = a0 + 4u * (uint32_t)d;
      dma_b32(rS, (d >= 0 && vo < end) ? vo : kOutOfRange, 0, &sRes[PR::instr(wave, q) * 64]);
    }
  }
  for (int q = 0; q < STAGES - 1 && q < ntk; ++q) issue_w(stg[q], kt0 + q);
  if (p.a_gather != nullptr) {  // consumed only now, after the weight loads went out
    int gathered = gv[0];
#pragma unroll
    for (int q = 1; q < BM; ++q) gathered = (tid == q) ? gv[q] : gathered;
    if (tid < BM) sArow[tid] = gathered / p.a_div;
  } else if (tid < BM) {
    sArow[tid] = min(r0 + tid, p.rows_total - 1);
  }
  barrier_lds();
  uint32_t voffA[IA];
  int ablk[IA];
#pragma unroll
  for (int q = 0; q < IA; ++q) {
    const int off = PA::instr(wave, q) * 1024 + lane * 16;
    const int lrow = off / A_ROW;
    if constexpr (AFP4) {
      const int chunk = ((off % A_ROW) >> 4) ^ swz_rows<ACH>(lrow);
      ablk[q] = chunk;
      if constexpr (LD::ATW) {  // row r0 + lrow of the pair-ordered tiled codes
        const uint32_t pr = (uint32_t)(r0 + lrow);
        voffA[q] = ((pr >> 4) * (uint32_t)nb + (uint32_t)chunk) * 256u + (pr & 15u) * 16u;
      } else {
        voffA[q] = (uint32_t)sArow[lrow] * (uint32_t)(K >> 1) + chunk * 16;
      }
    } else {
      const int chunk = ((off % A_ROW) >> 4) ^ swz_rows<ACH>(lrow);
      ablk[q] = chunk >> 2;
      voffA[q] = (uint32_t)sArow[lrow] * (uint32_t)(K * 2) + chunk * 16;
    }
    if (lrow >= n_valid) voffA[q] = kOutOfRange;
  }
  uint32_t voffSA[ISA > 0 ? ISA : 1];
#pragma unroll
  for (int q = 0; q < ISA; ++q) {
    const int idx = PSA::instr(wave, q) * 64 + lane;
    if constexpr (LD::SBM)  // block j of the stage: dwords d of the window over rows r0 ..
      voffSA[q] = idx < KT * LD::SW ? (uint32_t)(idx / LD::SW) * (uint32_t)p.sc_pitch +
                                          ((uint32_t)r0 & ~3u) + 4u * (uint32_t)(idx % LD::SW)
                                    : kOutOfRange;
    else
      voffSA[q] = idx < n_valid * SD
                      ? (((uint32_t)sArow[idx / SD] * (uint32_t)nb) & ~3u) + 4 * (idx % SD)
                      : kOutOfRange;
  }
  int ash[AFP4 ? FM : 1];  // FP4 A: byte of block 0 of each fragment row's scales
#pragma unroll
  for (int i = 0; i < (AFP4 ? FM : 0); ++i) {
    const int r = wm * TM + i * MF + ln;
    if constexpr (LD::SBM) ash[i] = (r0 & 3) + r;
    else ash[i] = r * SD * 4 + (int)(((uint32_t)sArow[r] * (uint32_t)nb) & 3u);
  }
  auto issue_a = [&](Stage& sg, int kt) {
    const int kb = kt * KT;
#pragma unroll
    for (int q = 0; q < ISA; ++q)
      dma_b32(rSA, off_add(voffSA[q], LD::SBM ? (uint32_t)kb * (uint32_t)p.sc_pitch : (uint32_t)kb), 0,
              &sg.Sa[PSA::instr(wave, q) * 64]);
    constexpr int A_KB = LD::ATW ? 256 : AFP4 ? 16 : 64;  // bytes between a row's 32-element blocks
    auto load_a = [&](uint32_t voff, const void* lds) {
      if constexpr (COH && MODE == MODE_DOWN) dma_b128_coherent(rA, voff, 0, lds);
      else dma_b128(rA, voff, 0, lds);
    };
    if ((kt + 1) * KT <= nb) {
#pragma unroll
      for (int q = 0; q < IA; ++q)
        load_a(off_add(voffA[q], (uint32_t)(kb * A_KB)), &sg.A[PA::instr(wave, q) * 1024]);
    } else {
#pragma unroll
      for (int q = 0; q < IA; ++q)
        load_a(kb + ablk[q] < nb ? off_add(voffA[q], (uint32_t)(kb * A_KB)) : kOutOfRange,
               &sg.A[PA::instr(wave, q) * 1024]);
    }
  };
  for (int q = 0; q < STAGES - 1 && q < ntk; ++q) issue_a(stg[q], kt0 + q);

  AccT<MF> acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[i][j][v] = 0.f;

  // One stage of MFMAs. A super-step covers LG K blocks, lane group g owning block LG*j + g.
  //   bf16 A: per super-step, read the wave's A fragments and packed B blocks; decode B fragment
  //   f+1 (two codes per cvt, other register set) while the 4 x FM MFMAs of fragment f run
  //   (16 x 16 x 32, or 32 x 32 x 16 when MF = 32: MFMA s takes elements [8s, 8s+8) of the
  //   lane's block either way).
  //   FP4 A: per super-step and fragment pair, one scaled MFMA on the raw blocks and scale bytes.
  // A wave whose output columns all lie past N (in the last column tile), or whose rows all lie
  // past the tile's last valid row, skips its fragment reads and MFMAs; it still loads its share
  // of every stage and meets every barrier. Where the valid rows fit in the first half of the
  // wave's row fragments (an expert's last, mostly empty row tile), the main loop runs a copy
  // that computes only that half (the other accumulators stay zero; their rows are dropped).
  const int wave_rows = n_valid - wm * TM;
  const bool wave_live = (SWIGLU ? nt * BNH + wn * (BNH / WN) : nt * BN + wn * TN) < p.N && wave_rows > 0;
  constexpr int FMH = (FM % 2 == 0) ? FM / 2 : FM;
  auto compute = [&](const Stage& sg, int kt, auto fl) {
    constexpr int FL = decltype(fl)::value;
    if (!wave_live) return;
    const uint8_t* As = sg.A;
    const uint8_t* Bsm = sg.B;
    const uint8_t* Scb = SCM == SCM_RESIDENT ? reinterpret_cast<const uint8_t*>(sRes) + kt * KT * SBS
                                             : reinterpret_cast<const uint8_t*>(sg.Sc);
    const uint8_t* Sab = reinterpret_cast<const uint8_t*>(sg.Sa);
    const bool partial = (kt + 1) * KT > nb;  // blocks past K: zero codes, scale read as 1.0
#pragma unroll
    for (int j = 0; j < SS; ++j) {
      const bool past = partial && kt * KT + LG * j + g >= nb;
      u32x4 w[FN];
      uint32_t scb[FN];
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const int r = brow[f];
        w[f] = lds_read_b128(Bsm + r * B_ROW + (((LG * j + g) ^ swz_rows<BCH>(r)) << 4));
        // (tiled weights: blocks past K hold zero codes and zero scales, 0 * 2^-127 = 0)
        scb[f] = (!TW && past) ? 127u : (uint32_t)Scb[bsh[f] + (LG * j + g) * SBS];
      }
      if constexpr (AFP4) {
        u32x4 a[FL];
        uint32_t sca[FL];
#pragma unroll
        for (int i = 0; i < FL; ++i) {
          const int r = wm * TM + i * MF + ln;
          a[i] = lds_read_b128(As + r * A_ROW + (((LG * j + g) ^ swz_rows<ACH>(r)) << 4));
          sca[i] = past ? 127u : (uint32_t)Sab[ash[i] + (LG * j + g) * (LD::SBM ? 4 * LD::SW : 1)];
        }
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int i = 0; i < FL; ++i)
            acc[i][f] = mfma_fp4_16x16x128(a[i], w[f], sca[i], scb[f], acc[i][f]);
      } else {
        bf16x8 a[FL][4];
#pragma unroll
        for (int i = 0; i < FL; ++i) {
          const int r = wm * TM + i * MF + ln;
#pragma unroll
          for (int s = 0; s < 4; ++s)
            a[i][s] = u32x4_as_bf16x8(
                lds_read_b128(As + r * A_ROW + ((((LG * j + g) * 4 + s) ^ swz_rows<ACH>(r)) << 4)));
        }
        float sc[FN];
#pragma unroll
        for (int f = 0; f < FN; ++f) sc[f] = e8m0_scale(scb[f]);
        if constexpr (MF == 32) {
          // 32 x 32 fragments are few (FM x FN = 4 for a 64 x 64 wave tile) and a 32x32x16 MFMA
          // has about twice the latency of the 16x16x32 form: go round all accumulators per
          // slice s (each MFMA then has the other FM*FN - 1 between it and its predecessor) and
          // decode slice s+1 of every fragment while slice s's MFMAs run.
          bf16x8 b[FN][4];
#pragma unroll
          for (int f = 0; f < FN; ++f) b[f][0] = fp4x8_to_bf16x8(w[f][0], sc[f]);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            if (s + 1 < 4) {
#pragma unroll
              for (int f = 0; f < FN; ++f) b[f][s + 1] = fp4x8_to_bf16x8(w[f][s + 1], sc[f]);
            }
#pragma unroll
            for (int f = 0; f < FN; ++f)
#pragma unroll
              for (int i = 0; i < FL; ++i) acc[i][f] = mfma32x32x16(a[i][s], b[f][s], acc[i][f]);
          }
        } else {
          bf16x8 b[2][4];
#pragma unroll
          for (int s = 0; s < 4; ++s) b[0][s] = fp4x8_to_bf16x8(w[0][s], sc[0]);
#pragma unroll
          for (int f = 0; f < FN; ++f) {
            if (f + 1 < FN) {
#pragma unroll
              for (int s = 0; s < 4; ++s) b[(f + 1) & 1][s] = fp4x8_to_bf16x8(w[f + 1][s], sc[f + 1]);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
              for (int i = 0; i < FL; ++i) acc[i][f] = mfma16x16x32(a[i][s], b[f & 1][s], acc[i][f]);
          }
        }
      }
    }
  };

  // Pipeline: stage kt+STAGES-1 is issued in iteration kt, weights and activations of a stage
  // back to back (LPS vector-memory ops per wave). The prologue issued the weights of stages
  // 0..STAGES-2, then their activations (LA ops each). At iteration kt the loads of stage kt must
  // have landed; outstanding(kt) counts the loads issued after its last one, which may stay in
  // flight (loads retire in issue order). The wait takes the largest fixed count not above it.
  constexpr int LA = ISA + IA;
  auto outstanding = [&](int kt) -> int {
    const int P = min(STAGES - 1, ntk);
    if (kt < P) return (P - 1 - kt) * LA + max(0, min(kt, ntk - STAGES + 1)) * LPS;
    return max(0, min(STAGES - 2, ntk - kt - 1)) * LPS;
  };
  auto wait_stage = [&](int kt) {
    const int n = outstanding(kt);
    if (STAGES >= 4 && n >= 2 * LPS) wait_vmcnt<(STAGES >= 4 ? 2 * LPS : 0)>();
    else if (STAGES >= 4 && n >= LA + LPS) wait_vmcnt<(STAGES >= 4 ? LA + LPS : 0)>();
    else if (STAGES >= 3 && n >= LPS) wait_vmcnt<(STAGES >= 3 ? LPS : 0)>();
    else if (STAGES >= 4 && n >= 2 * LA) wait_vmcnt<(STAGES >= 4 ? 2 * LA : 0)>();
    else if (STAGES >= 3 && n >= LA) wait_vmcnt<(STAGES >= 3 ? LA : 0)>();
    else wait_vmcnt<0>();
  };
  auto main_loop = [&](auto fl) {
    int st = 0;
    for (int kt = 0; kt < ntk; ++kt) {
      wait_stage(kt);
      barrier_lds();
      if (kt + STAGES - 1 < ntk) {
        Stage& sn = stg[st == 0 ? STAGES - 1 : st - 1];
        issue_w(sn, kt0 + kt + STAGES - 1);
        issue_a(sn, kt0 + kt + STAGES - 1);
      }
      // a wave in its compute phase (LDS reads, weight decoding, MFMAs) takes issue priority over
      // the CU's waves that are waiting or issuing loads (20B-shaped prefill gate_up 850 ->
      // 839 us, FP4 activations 446 -> 440 us; priority 3 measured the same as 1)
      __builtin_amdgcn_s_setprio(1);
      compute(stg[st], kt0 + kt, fl);
      __builtin_amdgcn_s_setprio(0);
      st = st == STAGES - 1 ? 0 : st + 1;
    }
  };
  if (FMH < FM && wave_rows <= FMH * MF) main_loop(std::integral_constant<int, FMH>{});
  else main_loop(std::integral_constant<int, FM>{});

  if constexpr (MODE == MODE_GATE_UP) {
    // h goes out through LDS: SwiGLU into a BM x BN/2 bf16 tile (rows padded by 16 bytes: the
    // four row groups of a fragment land on different banks) in the now idle stage buffers,
    // then whole 16-byte chunks to global, so every store instruction writes full lines instead
    // of 2-byte pieces of 16 columns x 4 rows.
    constexpr int LDH = BNH + 8;
    constexpr int CPR = BNH / 8;  // 16-byte chunks per row
    static_assert(BM * LDH * 2 <= STAGES * (int)sizeof(Stage), "h tile fits the stage buffers");
    uint16_t* sh = reinterpret_cast<uint16_t*>(&stg[0]);
    barrier_lds();  // every wave is done reading the last stage (no loads are in flight)
    if (p.act_custom) {
      // the clamped, scaled form: biases (per output column: gate and up rows of the expert, in
      // the caller's order), gate clamped above and up on both sides at the limit, sigmoid scale
      // alpha, shift added to up
      float bg[FN / 2], bu[FN / 2];
#pragma unroll
      for (int f = 0; f < FN / 2; ++f) {
        const int col = min(nt * BNH + wn * (BNH / WN) + f * MF + ln, p.F - 1);
        const float* b = p.bias + (int64_t)e * 2 * p.F;
        bg[f] = p.bias ? b[p.bias_interleaved ? 2 * col : col] : 0.f;
        bu[f] = p.bias ? b[p.bias_interleaved ? 2 * col + 1 : p.F + col] : 0.f;
      }
      const float lim = p.act_limit, alpha = p.act_alpha, shift = p.act_shift;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < NV; ++q)
#pragma unroll
          for (int f = 0; f < FN / 2; ++f) {
            float gt = acc[i][f][q] + bg[f], up = acc[i][FN / 2 + f][q] + bu[f];
            if (lim > 0.f) {
              gt = fminf(gt, lim);
              up = fmaxf(fminf(up, lim), -lim);
            }
            const float hv = gt * __builtin_amdgcn_rcpf(1.f + __expf(-alpha * gt)) * (up + shift);
            sh[(wm * TM + i * MF + acc_row<MF>(g, q)) * LDH + wn * (BNH / WN) + f * MF + ln] =
                (uint16_t)f32_to_bf16_bits(hv);
          }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < NV; ++q)
#pragma unroll
          for (int f = 0; f < FN / 2; ++f) {
            const float gt = acc[i][f][q], up = acc[i][FN / 2 + f][q];
            const float hv = gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt)) * up;
            sh[(wm * TM + i * MF + acc_row<MF>(g, q)) * LDH + wn * (BNH / WN) + f * MF + ln] =
                (uint16_t)f32_to_bf16_bits(hv);
          }
    }
    barrier_lds();
    if constexpr (AFP4) {
      // FP4 activations: the down product takes h as MXFP4, so each 32-column block of the bf16
      // tile is quantized here (the codec's bf16 quantizer, the same function) and only its 16
      // code bytes and scale byte leave the chip
      // (prefill tiles: codes in the tiled layout, [P/16][F/32][16 rows][16 bytes], consecutive
      // threads on consecutive rows of one block, so 16 of them store one 256-byte run; decode
      // tiles: row-major [P][F/2])
      constexpr int BPR = BNH / 32;  // 32-element blocks per tile row
      uint8_t* hq = reinterpret_cast<uint8_t*>(p.out);
      const int nbf = p.F >> 5;
      for (int c = tid; c < BM * BPR; c += NT) {
        const int lr = LD::ATW ? c % BM : c / BPR, cb = LD::ATW ? c / BM : c % BPR;
        const int r = r0 + lr, col = nt * BNH + cb * 32;
        if (r >= row_end || col >= p.F) continue;
        const uint4* src = reinterpret_cast<const uint4*>(sh + lr * LDH + cb * 32);
        uint32_t w[16];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 w8 = src[v];
          w[4 * v] = w8.x; w[4 * v + 1] = w8.y; w[4 * v + 2] = w8.z; w[4 * v + 3] = w8.w;
        }
        uint32_t q[4];
        const uint32_t sb = quantize_block32_bf16(w, q);
        const int64_t at = LD::ATW ? ((int64_t)(r >> 4) * nbf + (col >> 5)) * 256 + (r & 15) * 16
                                   : (int64_t)r * (p.F >> 1) + (col >> 1);
        *reinterpret_cast<uint4*>(hq + at) = make_uint4(q[0], q[1], q[2], q[3]);
        p.out_scales[(int64_t)(col >> 5) * p.sc_pitch + r] = (uint8_t)sb;  // block-major
      }
    } else {
      uint16_t* h = reinterpret_cast<uint16_t*>(p.out);
      for (int c = tid; c < BM * CPR; c += NT) {
        const int lr = c / CPR, cc = c % CPR;
        const int r = r0 + lr, col = nt * BNH + cc * 8;
        if (r < row_end && col < p.F) {
          const uint4 v = *reinterpret_cast<const uint4*>(sh + lr * LDH + cc * 8);
          if constexpr (COH) store_coherent(h + (int64_t)r * p.F + col, v);
          else *reinterpret_cast<uint4*>(h + (int64_t)r * p.F + col) = v;
        }
      }
    }
  } else if constexpr (MODE == MODE_DOWN && BM * (BN + 4) * 4 <= STAGES * (int)sizeof(Stage)) {
    // Y the same way: the fp32 tile (rows padded by 16 bytes) in the stage buffers, then whole
    // 16-byte chunks of each row to its permuted position
    constexpr int LDY = BN + 4;
    constexpr int CPR = BN / 4;
    float* sy = reinterpret_cast<float*>(&stg[0]);
    barrier_lds();
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < NV; ++q)
#pragma unroll
        for (int f = 0; f < FN; ++f)
          sy[(wm * TM + i * MF + acc_row<MF>(g, q)) * LDY + wn * TN + f * MF + ln] = acc[i][f][q];
    barrier_lds();
    float* y = reinterpret_cast<float*>(p.out);
    for (int c = tid; c < BM * CPR; c += NT) {
      const int lr = c / CPR, cc = c % CPR;
      const int r = r0 + lr, col = nt * BN + cc * 4;
      if (r < row_end && col < p.N) {
        const uint4 v = *reinterpret_cast<const uint4*>(sy + lr * LDY + cc * 4);
        if constexpr (COH) store_coherent(y + (int64_t)r * p.N + col, v);
        else *reinterpret_cast<uint4*>(y + (int64_t)r * p.N + col) = v;
      }
    }
  } else {
    static_assert(!COH, "coherent down tiles store through LDS");
    store_tile<MODE, FM, FN, TM, BN, WN, MF>(p, acc, r0, row_end, nt, wm, wn, g, ln);
  }
}

// out[t][c .. c+8) = sum_{j < k} w[t][j] * Y[inv[t*k + j]][c ..] in slot order (each product
// rounded to fp32, then summed); pairs with inv outside [0, P) (skipped routing indices)
// contribute nothing. Two 16-byte loads per row in flight. Each Y element is read once: the loads
// carry the non-temporal hint (20B-shaped prefill, T = 8192: 82 -> 79 us). With a down bias
// (bias [E][H], idx the pairs' experts) each row is w * (Y + bias of its expert), the bias added
// in fp32 before the weight.
// COH: the rows and the routing are loaded device-coherent (written by other workgroups of the
// same launch).
template <bool BF16_OUT, bool COH = false>
__device__ __forceinline__ void combine8(const float* __restrict__ Y, const int32_t* __restrict__ inv,
                                         const float* __restrict__ w, int t, int c, int H, int k,
                                         int P, void* __restrict__ out,
                                         const int32_t* __restrict__ idx,
                                         const float* __restrict__ bias) {
#pragma clang fp contract(off)  // each product rounded before it is added (no fused multiply-add)
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int r = ld_int<COH>(inv + (int64_t)t * k + j);
    if (r < 0 || r >= P) continue;
    const float wj = COH ? __hip_atomic_load(w + (int64_t)t * k + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : w[(int64_t)t * k + j];
    f32x4 v0, v1;
    if constexpr (COH) {
      const float* yr = Y + (int64_t)r * H + c;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v0[u] = __hip_atomic_load(yr + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v1[u] = __hip_atomic_load(yr + 4 + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      v0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Y + (int64_t)r * H + c));
      v1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Y + (int64_t)r * H + c + 4));
    }
    if (bias != nullptr) {
      const float* b = bias + (int64_t)ld_int<COH>(idx + (int64_t)t * k + j) * H + c;
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(b), b1 = *reinterpret_cast<const f32x4*>(b + 4);
      v0 += b0;
      v1 += b1;
    }
    s[0] += __fmul_rn(v0[0], wj); s[1] += __fmul_rn(v0[1], wj);
    s[2] += __fmul_rn(v0[2], wj); s[3] += __fmul_rn(v0[3], wj);
    s[4] += __fmul_rn(v1[0], wj); s[5] += __fmul_rn(v1[1], wj);
    s[6] += __fmul_rn(v1[2], wj); s[7] += __fmul_rn(v1[3], wj);
  }
  if (BF16_OUT) {
    uint32_t q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = f32_to_bf16_bits(s[2 * u]) | (f32_to_bf16_bits(s[2 * u + 1]) << 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + (int64_t)t * H + c) =
        make_uint4(q[0], q[1], q[2], q[3]);
  } else {
    float* o = reinterpret_cast<float*>(out) + (int64_t)t * H + c;
    *reinterpret_cast<float4*>(o) = make_float4(s[0], s[1], s[2], s[3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(s[4], s[5], s[6], s[7]);
  }
}

// at most min(T*k, E) experts touched: with 128-column tiles fewer than two workgroups per CU
bool use_tiny_tiles(int T, int k, int E, int N) {
  return (int64_t)std::min(T * k, E) * ((N + 127) / 128) < 512;
}

// Tile arguments of the MoE GEMMs (host side).
GemmKArgs gate_up_args(const MoeGemmArgs& m) {
  // A = x rows gathered through perm / k, B = W_gu[e] (2F rows), out = h [P][F]
  GemmKArgs g{};
  g.A = m.x;
  g.a_rows = m.T;
  g.a_gather = m.perm;
  g.a_div = m.k;
  g.Bp = m.gu_packed;
  g.Bs = m.gu_scales;
  g.b_rows_per_expert = 2LL * m.F;
  g.N = m.F;
  g.K = m.H;
  g.tiles = m.tiles;
  g.num_tiles = m.num_tiles;
  g.offsets = m.offsets;
  g.rows_total = m.T * m.k;
  g.F = m.F;
  g.out = m.h;
  g.sc_pitch = m.hqs_pitch;
  if (m.act_custom) {
    g.act_custom = 1;
    g.bias = m.gu_bias;
    g.bias_interleaved = m.gu_interleaved ? 1 : 0;
    g.act_alpha = m.act_alpha;
    g.act_limit = m.act_limit;
    g.act_shift = m.act_shift;
  }
  return g;
}

GemmKArgs down_args(const MoeGemmArgs& m) {
  // A = h rows (permuted order), B = W_dn[e] (H rows), out = Y rows (permuted order)
  GemmKArgs d{};
  d.A = m.h;
  d.a_rows = (int64_t)m.T * m.k;
  d.a_gather = nullptr;
  d.a_div = 1;
  d.Bp = m.dn_packed;
  d.Bs = m.dn_scales;
  d.b_rows_per_expert = m.H;
  d.N = m.H;
  d.K = m.F;
  d.tiles = m.tiles;
  d.num_tiles = m.num_tiles;
  d.offsets = m.offsets;
  d.rows_total = m.T * m.k;
  d.F = m.F;
  d.out = m.y;
  d.sc_pitch = m.hqs_pitch;
  return d;
}

// ---- tile configurations ----
// Prefill-shaped (many rows per expert): 64 x 256 workgroup tiles, four waves of 64 x 64 in
// 32 x 32 fragments, 2-block (64-element) stages, 2 stages, four workgroups per CU. Measured on
// the 20B prefill shape (T = 8192, tiled weights): the mainloop alone (no loads) runs at about
// 70% of the bf16 peak and the loads alone take longer than that, so what pays is hiding load
// latency with more resident workgroups, not more MFMA throughput. Small stages buy the
// residency: 17 KB per stage lets four workgroups share a CU's LDS (0.97 -> 0.88 ms for gate_up
// against 4-block stages of 16 x 16 fragments at two per CU; three per CU with 3 stages 0.91 ms;
// 2-block stages need the 32 x 32 form, whose two lane groups split a stage's two blocks). The
// 16 x 16 form with 4-block stages at two per CU, 128 x 256 tiles of eight waves and GM 2 or 8
// measured slower.
// Decode-shaped (few rows per expert): 16-row tiles, four waves side by side in N, the tile's
// weight scales resident, 4-block stages x 3, three workgroups per CU. Weight streaming
// dominates: a copy of the kernel without its MFMA work and activation loads runs within 5% of
// it (measured on the 20B decode shapes, tiled weights rotated through copies larger than the
// last-level cache: three workgroups per CU beat two; 8-block x 2 stages, 4 stages, four
// workgroups per CU, 256-column tiles, 64-column down tiles and per-stage scales measured no
// better).
// OCC: workgroups per CU the register allocation must leave room for (the second launch bound
// is in waves per SIMD).
// SCM: how the weight scales reach LDS (resident per tile where weight streaming is the bound).
// MF: MFMA fragment size, 32 (v_mfma_f32_32x32x16_bf16) or 16; FP4 activations always take 16.
struct CfgPreGU { static constexpr int BM = 64, BN = 256, WM = 1, WN = 4, KT = 2, ST = 2, GM = 4, OCC = 4, SCM = SCM_STAGE, MF = 32; };
struct CfgPreDn { static constexpr int BM = 64, BN = 256, WM = 1, WN = 4, KT = 2, ST = 2, GM = 4, OCC = 4, SCM = SCM_STAGE, MF = 32; };
struct CfgDecGU { static constexpr int BM = 16, BN = 128, WM = 1, WN = 4, KT = 4, ST = 3, GM = 1, OCC = 3, SCM = SCM_RESIDENT, MF = 16; };
struct CfgDecDn { static constexpr int BM = 16, BN = 192, WM = 1, WN = 4, KT = 4, ST = 3, GM = 1, OCC = 2, SCM = SCM_RESIDENT, MF = 16; };
// The single launch's down tiles and the dense linear at decode sizes (its K splits are sized
// for 128-column tiles) keep the 128-column form; the per-step MoE down GEMM takes 192 columns (2880 = 15 x 192: 600 tiles of the
// 20B-shaped T = 64 layer in one round of two workgroups per CU, against 920 128-column tiles in
// 1.2 rounds of three per CU: 27.9 -> 27.0 us; with two stages at three per CU 33.1 us).
struct CfgDecDn128 { static constexpr int BM = 16, BN = 128, WM = 1, WN = 4, KT = 4, ST = 3, GM = 1, OCC = 3, SCM = SCM_RESIDENT, MF = 16; };
// Activation variant, prefill-shaped: FP4 activations take a quarter of the LDS and need no
// decode instructions, so wide wave tiles with fewer bytes per MFMA pay: 128 x 256 workgroup
// tiles of four waves of 64 x 128, 3 stages, two workgroups per CU (the eight waves a CU holds
// as two independent workgroups, whose barriers no longer stall each other: against one
// workgroup of eight waves on 128 x 512, 20B-shaped prefill gate_up 581 -> 482 us, 120B-shaped
// T = 4096 449 -> 391 us), down with row tiles grouped by 2 (311 -> 293 us); with the pair-ordered
// tiled activations, gate_up row tiles grouped by 8 (455 -> 451 us; down by 4: 266 -> 275 us,
// by 1: 310 us; 2 stages: 478 us). Also measured: 64 x
// 256 (about 15% slower), 128 x 384 with 2 or 4 stages, 8-block stages (spills), three
// workgroups per CU with 2 stages (spills: 5x slower), groups of 8 row tiles, and 128 x 256 as
// one wave row of four.
struct CfgPreGU4 { static constexpr int BM = 128, BN = 256, WM = 2, WN = 2, KT = 4, ST = 3, GM = 8, OCC = 2, SCM = SCM_STAGE, MF = 16; };
struct CfgPreDn4 { static constexpr int BM = 128, BN = 256, WM = 2, WN = 2, KT = 4, ST = 3, GM = 2, OCC = 2, SCM = SCM_STAGE, MF = 16; };
// Few pairs (a handful of experts touched): with fewer tiles than CUs each workgroup's own weight
// stream is the bound, so these tiles keep more stages in flight. The down GEMM (2880 columns: 23
// tiles of 128 per expert) also takes 64-column tiles, twice the workgroups. 120B-shaped decode,
// T = 1: down 15.9 -> 14.1 us for the 64-column tiles, -> 12.2 us with 8-block x 4 stages;
// gate_up 16.8 -> 16.1 us with 4 stages (64-column or 8-block gate_up tiles measured slower).
struct CfgTinyDn { static constexpr int BM = 16, BN = 64, WM = 1, WN = 4, KT = 8, ST = 4, GM = 1, OCC = 2, SCM = SCM_RESIDENT, MF = 16; };
struct CfgTinyGU { static constexpr int BM = 16, BN = 128, WM = 1, WN = 4, KT = 4, ST = 4, GM = 1, OCC = 2, SCM = SCM_RESIDENT, MF = 16; };
constexpr int kPrefillRows = 64, kPrefillRows4 = 128;
static_assert(CfgPreGU::BM == kPrefillRows && CfgPreDn::BM == kPrefillRows, "one tile list");
static_assert(CfgPreGU4::BM == kPrefillRows4 && CfgPreDn4::BM == kPrefillRows4, "one tile list");
static_assert(kPrefillRows <= kMaxTileRows && kPrefillRows4 <= kMaxTileRows, "perm padding");

}  // namespace
}  // namespace mx
