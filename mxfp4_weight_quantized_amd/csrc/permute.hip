// permute.hip -- group the T*k (token, slot) pairs by expert: histogram over experts, exclusive
// prefix sum, stable scatter in (token, slot) order, inverse map, and (for the grouped GEMMs) the
// list of row tiles per expert.
//
// One workgroup of 16 waves does it all in one launch, with no global atomics: pair p belongs to
// wave p / C (C = ceil(P / 16)), each wave counts its chunk per expert in LDS, a scan over
// (expert, wave) gives every (wave, expert) its first output row, and each wave then scatters its
// chunk 64 pairs at a time, ranking equal experts among the 64 lanes with ballots. The order is
// the stable (token, slot) order by construction, so the result is deterministic.
//
// Large batches (P >= kSlicePairs * 2, with a workspace) take two launches over many workgroups
// instead: a histogram of every kSlicePairs-pair slice, then per slice the same scan (each
// workgroup derives its slice's first row per expert from all slice histograms) and the same
// ballot-ranked scatter. Slices are contiguous in (token, slot) order, so the result is the same
// stable counting sort, element for element.
//
// For small batches the same launch can first make the top-k selection from the router logits
// (SELECT: one wave per token, the router's selection function), keeping the indices in LDS;
// this saves the separate selection launch of the router in the MoE MLP.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {
namespace {

constexpr int kWaves = 16;
constexpr int kMaxE = 256;

// Exclusive scan of n (<= 256) ints in LDS by one wave; returns the total to every lane.
__device__ int wave_exclusive_scan(int* v, int n, int lane) {
  int carry = 0;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const int x = (i < n) ? v[i] : 0;
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (i < n) v[i] = carry + incl - x;
    carry += __shfl(incl, 63);
  }
  return carry;
}

template <bool SELECT>
__global__ __launch_bounds__(1024) void permute_kernel(int32_t* __restrict__ idx, int P,
                                                       int E, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ inv,
                                                       int32_t* __restrict__ status, int tile_rows,
                                                       int2* __restrict__ tiles,
                                                       int32_t* __restrict__ num_tiles,
                                                       const float* __restrict__ logits, int k,
                                                       float* __restrict__ w_out) {
  __shared__ int cnt[kWaves][kMaxE];
  __shared__ int tot[kMaxE + 1];
  __shared__ int tbase[kMaxE + 1];
  __shared__ int bad;
  __shared__ int sidx[SELECT ? kSelectMaxPairs : 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int chunk = (P + kWaves - 1) / kWaves;
  const int p_begin = min(P, wave * chunk);
  const int p_end = min(P, p_begin + chunk);

  for (int i = threadIdx.x; i < kWaves * kMaxE; i += blockDim.x) (&cnt[0][0])[i] = 0;
  if (threadIdx.x == 0) bad = 0;
  if constexpr (SELECT) {  // 0. top-k of every token (P = T * k <= kSelectMaxPairs)
    const int T = P / k;
    for (int t = wave; t < T; t += kWaves) {
      const int e = select_topk_wave([&](int x) { return logits[(int64_t)t * E + x]; }, lane, t,
                                     E, k, idx, w_out);
      if (lane < k) sidx[t * k + lane] = e;
    }
  }
  __syncthreads();
  auto pair_expert = [&](int p) -> int {
    if constexpr (SELECT) return sidx[p];
    else return idx[p];
  };

  // 1. per-wave histogram
  for (int p = p_begin + lane; p < p_end; p += 64) {
    const int e = pair_expert(p);
    if (e >= 0 && e < E) atomicAdd(&cnt[wave][e], 1);
    else bad = 1;
  }
  __syncthreads();

  // 2. totals per expert, scan -> offsets; first row of every (wave, expert)
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int s = 0;
    for (int w = 0; w < kWaves; ++w) s += cnt[w][e];
    tot[e] = s;
    if (tile_rows > 0) tbase[e] = (s + tile_rows - 1) / tile_rows;
  }
  __syncthreads();
  if (wave == 0) {
    const int total = wave_exclusive_scan(tot, E, lane);
    if (lane == 0) tot[E] = total;
  } else if (wave == 1 && tile_rows > 0) {
    const int total = wave_exclusive_scan(tbase, E, lane);
    if (lane == 0) tbase[E] = total;
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = tot[e];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = tot[e];
    for (int w = 0; w < kWaves; ++w) {
      const int c = cnt[w][e];
      cnt[w][e] = run;
      run += c;
    }
    if (tile_rows > 0) {
      const int n = tot[e + 1] - tot[e];
      const int tb = tbase[e];
      for (int i = 0; i * tile_rows < n; ++i) tiles[tb + i] = make_int2(e, tot[e] + i * tile_rows);
    }
  }
  if (threadIdx.x == 0) {
    if (tile_rows > 0) *num_tiles = tbase[E];
    if (status != nullptr) *status = bad;
  }
  // With a tile list, perm carries tile_rows entries of padding past P: rows past the last valid
  // one (and the padding) hold pair 0, so a tile may read its whole row range of perm.
  if (tile_rows > 0)
    for (int i = tot[E] + threadIdx.x; i < P + tile_rows; i += blockDim.x) perm[i] = 0;
  __syncthreads();

  // 3. stable scatter, 64 pairs per step in (token, slot) order
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int g0 = p_begin; g0 < p_end; g0 += 64) {
    const int p = g0 + lane;
    int e = (p < p_end) ? pair_expert(p) : -1;
    const bool ok = (e >= 0 && e < E);
    if (!ok) {
      if (p < p_end) inv[p] = -1;
      e = 0;
    }
    uint64_t peers = __ballot(ok);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    const int rank = __popcll(peers & lt_mask);
    int pos = 0;
    if (ok) pos = cnt[wave][e] + rank;
    __builtin_amdgcn_wave_barrier();
    if (ok) {
      perm[pos] = p;
      inv[p] = pos;
      if (rank == 0) cnt[wave][e] = pos + __popcll(peers);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Pass 1 of the sliced permutation: counts[s][e] = pairs of slice s routed to expert e; column
// E counts the indices outside [0, E).
__global__ __launch_bounds__(256) void slice_hist_kernel(const int32_t* __restrict__ idx, int P,
                                                         int E, int32_t* __restrict__ counts) {
  __shared__ int h[kMaxE + 1];
  for (int i = threadIdx.x; i <= E; i += blockDim.x) h[i] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kSlicePairs, p1 = min(P, p0 + kSlicePairs);
  for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    const int e = idx[p];
    atomicAdd(&h[(e >= 0 && e < E) ? e : E], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i <= E; i += blockDim.x) counts[(int64_t)blockIdx.x * (E + 1) + i] = h[i];
}

// Pass 2: slice s (one workgroup of 16 waves) places its pairs. Slice 0 also writes the offsets,
// the tile list, the status word and perm's padding.
__global__ __launch_bounds__(1024) void slice_scatter_kernel(
    const int32_t* __restrict__ idx, int P, int E, const int32_t* __restrict__ counts, int n_slices,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ status, int tile_rows, int2* __restrict__ tiles,
    int32_t* __restrict__ num_tiles) {
  __shared__ int cnt[kWaves][kMaxE];
  __shared__ int tot[kMaxE + 1];
  __shared__ int pre[kMaxE];
  __shared__ int tbase[kMaxE + 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slice = blockIdx.x;
  const int s0 = slice * kSlicePairs, s1 = min(P, s0 + kSlicePairs);
  const int chunk = (s1 - s0 + kWaves - 1) / kWaves;
  const int p_begin = min(s1, s0 + wave * chunk);
  const int p_end = min(s1, p_begin + chunk);

  for (int i = threadIdx.x; i < kWaves * kMaxE; i += blockDim.x) (&cnt[0][0])[i] = 0;
  // totals over all slices and this slice's prefix (slices before it), per expert
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int s = 0, before = 0;
    for (int w = 0; w < n_slices; ++w) {
      const int c = counts[(int64_t)w * (E + 1) + e];
      if (w < slice) before += c;
      s += c;
    }
    tot[e] = s;
    pre[e] = before;
    if (tile_rows > 0) tbase[e] = (s + tile_rows - 1) / tile_rows;
  }
  __syncthreads();
  for (int p = p_begin + lane; p < p_end; p += 64) {  // per-wave histogram of the slice
    const int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[wave][e], 1);
  }
  if (wave == 0) {
    const int total = wave_exclusive_scan(tot, E, lane);
    if (lane == 0) tot[E] = total;
  } else if (wave == 1 && tile_rows > 0 && slice == 0) {
    const int total = wave_exclusive_scan(tbase, E, lane);
    if (lane == 0) tbase[E] = total;
  }
  __syncthreads();
  if (slice == 0) {
    for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = tot[e];
    if (tile_rows > 0)
      for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int n = tot[e + 1] - tot[e];
        for (int i = 0; i * tile_rows < n; ++i) tiles[tbase[e] + i] = make_int2(e, tot[e] + i * tile_rows);
      }
    if (threadIdx.x == 0) {
      if (tile_rows > 0) *num_tiles = tbase[E];
      if (status != nullptr) {
        int bad = 0;
        for (int w = 0; w < n_slices; ++w) bad |= counts[(int64_t)w * (E + 1) + E] != 0;
        *status = bad;
      }
    }
    if (tile_rows > 0)
      for (int i = tot[E] + threadIdx.x; i < P + tile_rows; i += blockDim.x) perm[i] = 0;
  }
  // first row of every (wave, expert) of this slice
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = tot[e] + pre[e];
    for (int w = 0; w < kWaves; ++w) {
      const int c = cnt[w][e];
      cnt[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int g0 = p_begin; g0 < p_end; g0 += 64) {
    const int p = g0 + lane;
    int e = (p < p_end) ? idx[p] : -1;
    const bool ok = (e >= 0 && e < E);
    if (!ok) {
      if (p < p_end) inv[p] = -1;
      e = 0;
    }
    uint64_t peers = __ballot(ok);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    const int rank = __popcll(peers & lt_mask);
    int pos = 0;
    if (ok) pos = cnt[wave][e] + rank;
    __builtin_amdgcn_wave_barrier();
    if (ok) {
      perm[pos] = p;
      inv[p] = pos;
      if (rank == 0) cnt[wave][e] = pos + __popcll(peers);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

size_t permute_sliced_workspace(int T, int k, int E) {
  const int64_t P = (int64_t)T * k;
  if (P < 2LL * kSlicePairs) return 0;
  return (size_t)((P + kSlicePairs - 1) / kSlicePairs) * (E + 1) * 4;
}

hipError_t launch_permute_sliced(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                                 int32_t* perm, int32_t* inv, int32_t* status, int tile_rows,
                                 int2* tiles, int32_t* num_tiles, int32_t* counts,
                                 hipStream_t stream) {
  const int P = T * k;
  if (tiles == nullptr || num_tiles == nullptr) tile_rows = 0;
  const int n_slices = (P + kSlicePairs - 1) / kSlicePairs;
  hipLaunchKernelGGL(slice_hist_kernel, dim3(n_slices), dim3(256), 0, stream, idx, P, E, counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(slice_scatter_kernel, dim3(n_slices), dim3(64 * kWaves), 0, stream, idx, P, E,
                     counts, n_slices, offsets, perm, inv, status, tile_rows, tiles, num_tiles);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets, int32_t* perm,
                          int32_t* inv, int32_t* status, int tile_rows, int2* tiles,
                          int32_t* num_tiles, hipStream_t stream) {
  const int P = T * k;
  if (tiles == nullptr || num_tiles == nullptr) tile_rows = 0;
  hipLaunchKernelGGL(permute_kernel<false>, dim3(1), dim3(64 * kWaves), 0, stream,
                     const_cast<int32_t*>(idx), P, E, offsets, perm, inv, status, tile_rows, tiles,
                     num_tiles, nullptr, k, nullptr);
  return hipGetLastError();
}

hipError_t launch_select_permute(const float* logits, int T, int k, int E, int32_t* idx, float* w,
                                 int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* status,
                                 int tile_rows, int2* tiles, int32_t* num_tiles,
                                 hipStream_t stream) {
  const int P = T * k;
  if (tiles == nullptr || num_tiles == nullptr) tile_rows = 0;
  hipLaunchKernelGGL(permute_kernel<true>, dim3(1), dim3(64 * kWaves), 0, stream, idx, P, E,
                     offsets, perm, inv, status, tile_rows, tiles, num_tiles, logits, k, w);
  return hipGetLastError();
}

}  // namespace mx
