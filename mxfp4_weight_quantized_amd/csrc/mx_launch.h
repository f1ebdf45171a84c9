// mx_launch.h -- host-side launchers of the gfx950 kernels (called by the C ABI layer only).
// Every launcher enqueues on `stream`, performs no allocation or synchronization, and returns the
// launch status. Shapes have been validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// codec.hip
hipError_t launch_quantize(const void* src, bool bf16_in, int64_t nblocks, uint8_t* packed,
                           uint8_t* scales, hipStream_t stream);
hipError_t launch_dequantize(const uint8_t* packed, const uint8_t* scales, int64_t nblocks,
                             void* dst, bool bf16_out, hipStream_t stream);
// G matrices [R][K] (R % 16 == 0, K % 32 == 0) into the tiled layout of the grouped GEMMs.
hipError_t launch_tile_weights(const uint8_t* packed, const uint8_t* scales, int64_t G, int R,
                               int K, uint8_t* packed_t, uint8_t* scales_t, hipStream_t stream);

// route.hip
// partials (may be null): fp32 scratch of route_partial_splits(T, H, E) * T * E floats; with it
// small batches split H over more workgroups.
hipError_t launch_route_topk(const uint16_t* x, const uint16_t* wr, const float* br, int T, int H,
                             int E, int k, float* logits, int32_t* idx, float* w, float* partials,
                             hipStream_t stream);
int route_partial_splits(int T, int H, int E);
// Router logits only, when the selection can be left to launch_select_permute (small batches
// whose logits kernel does not select itself); returns false (nothing launched) otherwise.
bool route_logits_defers_select(int T, int E, int k);
hipError_t launch_route_logits(const uint16_t* x, const uint16_t* wr, const float* br, int T,
                               int H, int E, float* logits, hipStream_t stream);

// permute.hip: tiles/num_tiles may be NULL (tile_rows ignored then). With a tile list, perm must
// hold P + tile_rows entries: the padding (and rows past the last valid pair) are set to pair 0.
constexpr int kMaxTileRows = 128;
constexpr int kSelectMaxPairs = 2048;  // launch_select_permute: T * k at most this
constexpr int kSlicePairs = 4096;      // launch_permute_sliced: pairs per workgroup
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets, int32_t* perm,
                          int32_t* inv, int32_t* status, int tile_rows, int2* tiles,
                          int32_t* num_tiles, hipStream_t stream);
// The same over many workgroups (two launches) for large batches: counts is workspace of
// permute_sliced_workspace(T, k, E) bytes (0: use launch_permute).
size_t permute_sliced_workspace(int T, int k, int E);
hipError_t launch_permute_sliced(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                                 int32_t* perm, int32_t* inv, int32_t* status, int tile_rows,
                                 int2* tiles, int32_t* num_tiles, int32_t* counts,
                                 hipStream_t stream);
// The same after the top-k selection from the router logits (writes idx and w [T][k]).
hipError_t launch_select_permute(const float* logits, int T, int k, int E, int32_t* idx, float* w,
                                 int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* status,
                                 int tile_rows, int2* tiles, int32_t* num_tiles,
                                 hipStream_t stream);

// gemm.hip
struct MoeGemmArgs {
  int T, H, F, E, k;
  const uint16_t* x;         // [T][H] bf16
  const int32_t* perm;       // [P]
  const int32_t* inv;        // [P]
  const int32_t* offsets;    // [E+1]
  const int2* tiles;         // [max_tiles]
  const int32_t* num_tiles;  // device
  int max_tiles;
  const float* topk_w;       // [P]
  const uint8_t *gu_packed, *gu_scales, *dn_packed, *dn_scales;
  uint16_t* h;               // [P][F] bf16 workspace
  float* y;                  // [P][H] fp32 workspace
  void* out;                 // [T][H]
  bool out_bf16;
  // activation variant: x and h MXFP4-quantized (packed [rows][K/2], scales [rows][K/32])
  bool mx_act;
  uint8_t *xq, *xqs, *hq, *hqs;
  // expert weights in the tiled layout (codes [E][R/16][K/32][16][16], scales [E][K/32][R])
  bool tiled;
};
// Tile rows (BM) the grouped GEMMs use for this problem; the permutation's tile list must match.
int moe_tile_rows(int T, int k, int E, bool mx_act);
int moe_max_tiles(int T, int k, int E, int tile_rows);
hipError_t launch_moe_gate_up(const MoeGemmArgs& a, hipStream_t stream);
hipError_t launch_moe_down(const MoeGemmArgs& a, hipStream_t stream);
hipError_t launch_moe_combine(const MoeGemmArgs& a, hipStream_t stream);

// Dense linear. Decode-sized M splits K over several workgroups (linear_k_splits > 1): the
// splits' fp32 partial sums go to `partials` (linear_k_splits * M * N floats), then one more
// launch sums them in split order into y; partials may be null when linear_k_splits is 1.
int linear_k_splits(int M, int K, int N);
hipError_t launch_linear(const uint16_t* x, int M, int K, const uint8_t* packed,
                         const uint8_t* scales, int N, void* y, bool y_bf16, float* partials,
                         hipStream_t stream);
// Activation variant: x already MXFP4 (xq [M][K/2], xqs [M][K/32]).
hipError_t launch_linear_mxact(const uint8_t* xq, const uint8_t* xqs, int M, int K,
                               const uint8_t* packed, const uint8_t* scales, int N, void* y,
                               bool y_bf16, float* partials, hipStream_t stream);

// Kernel attributes that must be set once per process before the first launch.
hipError_t gemm_init();

}  // namespace mx
