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
// The MoE MLP's activation variant. Decode-shaped calls: x [T][H] bf16 quantized along H, codes
// [T][H/2] in token order, scale bytes block-major in pair order ([H/32][pitch], pitch >= T * k):
// the scale of (token t, block b) at b * pitch + inv[t * k + j] for every slot j whose inv is in
// [0, T * k).
hipError_t launch_quantize_x_scatter(const uint16_t* x, int T, int H, const int32_t* inv, int k,
                                     int64_t pitch, uint8_t* packed, uint8_t* scales_bm,
                                     hipStream_t stream);
// Prefill-shaped calls: x's codes [T][H/2] and scales [T][H/32] (token order, launch_quantize)
// copied into pair order (row p is token perm[p] / k, p < P): codes tiled [P/16][H/32][16][16
// bytes] (P rounded up to 16 rows), scales block-major [H/32][pitch].
hipError_t launch_x_pair_copy(const uint8_t* codes, const uint8_t* scales, int H,
                              const int32_t* perm, int k, int P, int64_t pitch, uint8_t* packed,
                              uint8_t* scales_bm, hipStream_t stream);
hipError_t launch_dequantize(const uint8_t* packed, const uint8_t* scales, int64_t nblocks,
                             void* dst, bool bf16_out, hipStream_t stream);
// G matrices [R][K] (R % 16 == 0, K % 32 == 0) into the tiled layout of the grouped GEMMs;
// deinterleave: rows 2i -> i, 2i + 1 -> R/2 + i on the way (R % 32 == 0).
hipError_t launch_tile_weights(const uint8_t* packed, const uint8_t* scales, int64_t G, int R,
                               int K, bool deinterleave, uint8_t* packed_t, uint8_t* scales_t,
                               hipStream_t stream);

// route.hip
// partials (may be null): fp32 scratch of route_partial_splits(T, H, E) * T * E floats; with it
// small batches split H over more workgroups, and large ones (with logits, H % 64 == 0) run as
// 64-token tiles over all experts with H split over route_partial_splits workgroups per tile.
// logits may be null (not stored): then every workgroup covers all experts of its tokens and
// makes the selection itself.
hipError_t launch_route_topk(const uint16_t* x, const uint16_t* wr, const float* br, int T, int H,
                             int E, int k, float* logits, int32_t* idx, float* w, float* partials,
                             hipStream_t stream);
int route_partial_splits(int T, int H, int E);
// Router logits only, where the selection is left to launch_select_permute (batches of up to 16
// tokens whose logits kernel does not select itself, T * E <= kSelectMaxLogits).
// With partials (route_partial_splits(T, H, E) * T * E floats) the partial tiles of H split over
// *n_part workgroups are stored there without the bias (else *n_part = 0 and the logits with the
// bias go to logits).
bool route_logits_defers_select(int T, int E, int k);
// zero_word (may be null): an int the launch sets to 0 (the counter of the next launch).
hipError_t launch_route_logits(const uint16_t* x, const uint16_t* wr, const float* br, int T,
                               int H, int E, float* logits, float* partials, int* n_part,
                               hipStream_t stream, int32_t* zero_word = nullptr);
// Decode-sized batches inside the MoE call whose router is the spread launch (more than one
// expert group, selection not deferred to the permutation, T * k <= kSelectPermuteMaxPairs):
// launch_route_logits (with zero_word = counter) then this one launch, which makes the top-k
// selection of every token (as the selection kernel) and the permutation (as launch_permute).
// (up to 512 pairs: the 20B-shaped T = 64 layer, 8.8 + 4.9 -> 4.7 + 7.3 us; with 1024 pairs, the
// 120B-shaped T = 256 layer, the one workgroup's sort on four waves costs what the launch saves:
// 13.0 + 5.1 -> 6.9 + 11.8 us)
constexpr int kSelectPermuteMaxPairs = 512;
bool route_select_permute_fits(int T, int H, int E, int k);
hipError_t launch_route_select_permute(float* logits, const float* partials, int n_part,
                                       const float* br, int T, int E, int k, int32_t* idx,
                                       float* w, int32_t* counter, int32_t* offsets, int32_t* perm,
                                       int32_t* inv, int32_t* status, int tile_rows, int2* tiles,
                                       int32_t* num_tiles, hipStream_t stream);

// Device error word, one per device, owned by the library: kernels OR error codes into it, and
// mx_get_device_error reads and clears it. device_error_word() is its device address on the
// current device (looked up once per device; nullptr if the lookup failed).
constexpr int32_t kDevErrRouting = 1;  // a routing index outside [0, E) was skipped
constexpr int32_t kDevErrSync = 2;     // a wait of the single-launch pipeline gave up
int32_t* device_error_word();

// permute.hip: tiles/num_tiles may be NULL (tile_rows ignored then). With a tile list, perm must
// hold P + tile_rows entries: the padding (and rows past the last valid pair) are set to pair 0.
constexpr int kMaxTileRows = 128;
constexpr int kSelectMaxPairs = 2048;   // launch_select_permute: T * k at most this
constexpr int kSelectMaxLogits = 16384; //   and T * E at most this (its logits stay in LDS)
constexpr int kSlicePairs = 1024;      // launch_permute_sliced: pairs per workgroup
constexpr int kSlicedMinPairs = 8192;  //   used from this many pairs (with a workspace)
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
// The same after the top-k selection (writes idx and w [T][k]) from the router's logits, or from
// its n_part > 0 partial tiles (summed in split order, plus the bias br; the sums are written to
// logits).
hipError_t launch_select_permute(float* logits, const float* partials, int n_part, const float* br,
                                 int T, int k, int E, int32_t* idx, float* w, int32_t* offsets,
                                 int32_t* perm, int32_t* inv, int32_t* status, int tile_rows,
                                 int2* tiles, int32_t* num_tiles, hipStream_t stream);

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
  const int32_t* topk_idx;   // [P] experts of the pairs (read by the combine for the down bias)
  const uint8_t *gu_packed, *gu_scales, *dn_packed, *dn_scales;
  uint16_t* h;               // [P][F] bf16 workspace
  float* y;                  // [P][H] fp32 workspace
  void* out;                 // [T][H]
  bool out_bf16;
  // activation variant: x and h MXFP4-quantized (packed [rows][K/2]; x's scales [T][H/32], h's
  // block-major [F/32][hqs_pitch], hqs_pitch = T*k rounded up to a multiple of 4)
  bool mx_act;
  uint8_t *xq, *xqs, *hq, *hqs;
  int64_t hqs_pitch;
  // expert weights in the tiled layout (codes [E][R/16][K/32][16][16], scales [E][K/32][R])
  bool tiled;
  // expert activation: act_custom = 0 is the plain SwiGLU (the rest unused); else biases (NULL =
  // none; gu_bias in the caller's row order, interleaved or not), clamp limit (<= 0: none),
  // sigmoid scale and up shift
  bool act_custom;
  const float* gu_bias;      // [E][2F]
  const float* dn_bias;      // [E][H]
  bool gu_interleaved;
  float act_alpha, act_limit, act_shift;
};
// Tile rows (BM) the grouped GEMMs use for this problem; the permutation's tile list must match.
int moe_tile_rows(int T, int k, int E, bool mx_act);
int moe_max_tiles(int T, int k, int E, int tile_rows);
hipError_t launch_moe_gate_up(const MoeGemmArgs& a, hipStream_t stream);
hipError_t launch_moe_down(const MoeGemmArgs& a, hipStream_t stream);
hipError_t launch_moe_combine(const MoeGemmArgs& a, hipStream_t stream);

// single.hip: the whole MoE MLP of a decode-sized batch (T * k <= kSingleMaxPairs, bf16
// activations) as one launch on 16-row tiles (tile list of moe_max_tiles(T, k, E, 16) entries).
// Calls on one device must not overlap: they share the library's counters for the launch.
constexpr int kSingleMaxPairs = 2048;
struct SingleRouting {
  const uint16_t* wr;  // router [E][H] bf16; nullptr: the caller's routing (m.topk_idx, m.topk_w)
  const float* br;     // router bias [E] or nullptr
  float* logits;       // [T][E] or nullptr (not stored)
  float* rpart;        // single_route_splits(T, H, E) * T * E floats
  int32_t* tile_ends;  // [max_tiles] workspace
  int32_t* status;     // 1 if a routing index was outside [0, E)
};
// With internal routing m.topk_idx and m.topk_w are where the routing is written.
int single_route_splits(int T, int H, int E);
hipError_t launch_moe_single(const MoeGemmArgs& m, const SingleRouting& r, hipStream_t stream);

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

}  // namespace mx
