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
// Large batches (P >= kSlicedMinPairs, with a workspace) take two launches over many workgroups
// instead: a histogram of every kSlicePairs-pair slice, then per slice the same scan (each
// workgroup derives its slice's first row per expert from all slice histograms, staged through
// LDS with every count loaded at once) and the same ballot-ranked scatter. Slices are contiguous
// in (token, slot) order, so the result is the same stable counting sort, element for element.
// Both kernels are latency chains: small slices keep them short (4096-pair slices with the
// counts read one slice after another: 17.5 us for 32768 pairs; 1024-pair slices: see the
// results of the library's benchmark).
//
// For small batches the same launch can first make the top-k selection from the router logits
// (SELECT: all logits staged in LDS -- summed from the router's partial tiles where H was split
// over workgroups -- then one wave per token, the router's selection function), keeping the
// indices in LDS; this saves the separate selection launch of the router in the MoE MLP.
#include "route_device.h"

#include <atomic>

namespace mx {

// The library's device error word (one copy per device; see device_error_word).
__device__ int32_t g_device_error;

int32_t* device_error_word() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int32_t*> addr[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  int32_t* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(g_device_error)) != hipSuccess) return nullptr;
    p = static_cast<int32_t*>(a);
    addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

namespace {

constexpr int kWaves = 16;
constexpr int kMaxE = kPermuteMaxE;
constexpr int kCountLds = 8192;  // ints of slice histograms staged at once (>= 31 slices of E + 1)

template <bool SELECT>
__global__ __launch_bounds__(1024) void permute_kernel(int32_t* __restrict__ idx, int P,
                                                       int E, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ inv,
                                                       int32_t* __restrict__ status,
                                                       int32_t* __restrict__ dev_err, int tile_rows,
                                                       int2* __restrict__ tiles,
                                                       int32_t* __restrict__ num_tiles,
                                                       float* __restrict__ logits, int k,
                                                       float* __restrict__ w_out,
                                                       const float* __restrict__ partials,
                                                       int n_part, const float* __restrict__ br) {
  __shared__ int cnt[kWaves][kMaxE];
  __shared__ int tot[kMaxE + 1];
  __shared__ int tbase[kMaxE + 1];
  __shared__ int bad;
  __shared__ int sidx[SELECT ? kSelectMaxPairs : 1];
  __shared__ float slog[SELECT ? kSelectMaxLogits : 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  if constexpr (SELECT) {  // 0. top-k of every token (P = T * k <= kSelectMaxPairs)
    // all T x E logits into LDS with coalesced loads (from the partial tiles: summed in split
    // order, plus the bias, and stored as the logits), then one wave per token ranks them there
    const int T = P / k;
    const int TE = T * E;
    for (int i = threadIdx.x; i < TE; i += blockDim.x) {
      float v;
      if (n_part > 0) {
        v = partials[i];
        for (int q = 1; q < n_part; ++q) v += partials[(int64_t)q * TE + i];
        v += (br != nullptr) ? br[i % E] : 0.f;
        logits[i] = v;
      } else {
        v = logits[i];
      }
      slog[i] = v;
    }
    __syncthreads();
    for (int t = wave; t < T; t += kWaves) {
      const int e = select_topk_wave([&](int x) { return slog[t * E + x]; }, lane, t, E, k, idx,
                                     w_out);
      if (lane < k) sidx[t * k + lane] = e;
    }
    __syncthreads();
  }
  auto pair_expert = [&](int p) -> int {
    if constexpr (SELECT) return sidx[p];
    else return idx[p];
  };
  permute_pairs<kWaves>(pair_expert, P, E, offsets, perm, inv, status, dev_err, tile_rows, tiles,
                        num_tiles, &cnt[0][0], tot, tbase, &bad);
}

// Pass 1 of the sliced permutation: counts[s][e] = pairs of slice s routed to expert e; column
// E counts the indices outside [0, E).
__global__ __launch_bounds__(256) void slice_hist_kernel(const int32_t* __restrict__ idx, int P,
                                                         int E, int32_t* __restrict__ counts) {
  __shared__ int h[kMaxE + 1];
  for (int i = threadIdx.x; i <= E; i += blockDim.x) h[i] = 0;
  const int p0 = blockIdx.x * kSlicePairs, p1 = min(P, p0 + kSlicePairs);
  constexpr int kPer = kSlicePairs / 256;
  int ev[kPer];  // every load of the thread first, then the LDS counts
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int p = p0 + threadIdx.x + 256 * u;
    ev[u] = p < p1 ? idx[p] : 0;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (p0 + (int)threadIdx.x + 256 * u < p1) atomicAdd(&h[(ev[u] >= 0 && ev[u] < E) ? ev[u] : E], 1);
  __syncthreads();
  for (int i = threadIdx.x; i <= E; i += blockDim.x) counts[(int64_t)blockIdx.x * (E + 1) + i] = h[i];
}

// Pass 2: slice s (one workgroup of 16 waves) places its pairs. Slice 0 also writes the offsets,
// the tile list, the status word and perm's padding.
__global__ __launch_bounds__(1024) void slice_scatter_kernel(
    const int32_t* __restrict__ idx, int P, int E, const int32_t* __restrict__ counts, int n_slices,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ status, int32_t* __restrict__ dev_err, int tile_rows,
    int2* __restrict__ tiles, int32_t* __restrict__ num_tiles) {
  __shared__ int cnt[kWaves][kMaxE];
  __shared__ int tot[kMaxE + 1];
  __shared__ int pre[kMaxE];
  __shared__ int tbase[kMaxE + 1];
  __shared__ int cst[kCountLds];
  __shared__ int sbad;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slice = blockIdx.x;
  const int s0 = slice * kSlicePairs, s1 = min(P, s0 + kSlicePairs);
  const int chunk = (s1 - s0 + kWaves - 1) / kWaves;
  const int p_begin = min(s1, s0 + wave * chunk);
  const int p_end = min(s1, p_begin + chunk);

  for (int i = threadIdx.x; i < kWaves * kMaxE; i += blockDim.x) (&cnt[0][0])[i] = 0;
  // totals over all slices and this slice's prefix (slices before it), per expert (thread e < E),
  // and (thread E) whether any slice skipped an index outside [0, E): the slice histograms go
  // through LDS in chunks of whole slices, all of a chunk's counts loaded at once
  const int per = kCountLds / (E + 1);
  int s_all = 0, before = 0;
  for (int w0 = 0; w0 < n_slices; w0 += per) {
    const int n = min(per, n_slices - w0) * (E + 1);
    for (int i0 = 0; i0 < n; i0 += 4 * 64 * kWaves) {
      int v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + threadIdx.x + 64 * kWaves * u;
        v[u] = i < n ? counts[(int64_t)w0 * (E + 1) + i] : 0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + threadIdx.x + 64 * kWaves * u;
        if (i < n) cst[i] = v[u];
      }
    }
    __syncthreads();
    if (threadIdx.x <= E) {
      const int e = threadIdx.x;
      for (int w = 0; w * (E + 1) < n; ++w) {
        const int c = cst[w * (E + 1) + e];
        if (w0 + w < slice) before += c;
        s_all += c;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x < E) {
    const int e = threadIdx.x;
    tot[e] = s_all;
    pre[e] = before;
    if (tile_rows > 0) tbase[e] = (s_all + tile_rows - 1) / tile_rows;
  } else if (threadIdx.x == E) {
    sbad = s_all != 0;
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
      if (status != nullptr) *status = sbad;
      if (sbad && dev_err != nullptr) atomicOr(dev_err, kDevErrRouting);
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
  if (P < kSlicedMinPairs) return 0;
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
                     counts, n_slices, offsets, perm, inv, status, device_error_word(), tile_rows,
                     tiles, num_tiles);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets, int32_t* perm,
                          int32_t* inv, int32_t* status, int tile_rows, int2* tiles,
                          int32_t* num_tiles, hipStream_t stream) {
  const int P = T * k;
  if (tiles == nullptr || num_tiles == nullptr) tile_rows = 0;
  hipLaunchKernelGGL(permute_kernel<false>, dim3(1), dim3(64 * kWaves), 0, stream,
                     const_cast<int32_t*>(idx), P, E, offsets, perm, inv, status,
                     device_error_word(), tile_rows, tiles, num_tiles, nullptr, k, nullptr, nullptr,
                     0, nullptr);
  return hipGetLastError();
}

hipError_t launch_select_permute(float* logits, const float* partials, int n_part, const float* br,
                                 int T, int k, int E, int32_t* idx, float* w, int32_t* offsets,
                                 int32_t* perm, int32_t* inv, int32_t* status, int tile_rows,
                                 int2* tiles, int32_t* num_tiles, hipStream_t stream) {
  const int P = T * k;
  if (tiles == nullptr || num_tiles == nullptr) tile_rows = 0;
  hipLaunchKernelGGL(permute_kernel<true>, dim3(1), dim3(64 * kWaves), 0, stream, idx, P, E,
                     offsets, perm, inv, status, device_error_word(), tile_rows, tiles, num_tiles,
                     logits, k, w, partials, n_part, br);
  return hipGetLastError();
}

}  // namespace mx
