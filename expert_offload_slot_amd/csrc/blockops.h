// Workgroup-wide scans for the single-workgroup control kernels (1024 threads,
// 16 wavefronts): ballot + popcount inside a wavefront, then an ordered pass
// over the 16 wavefront totals.  Results are in thread order.
#pragma once

#include "internal.h"

namespace moe {

constexpr int kBlock = 1024;  // one workgroup, 16 wavefronts
constexpr int kWaves = kBlock / 64;

// Exclusive rank of `flag` among the block's threads in thread order, and the
// total.  All threads of the block must call it.  Uses s_wave[kWaves].
__device__ __forceinline__ int block_rank(bool flag, int* s_wave, int* total) {
  const unsigned long long m = __ballot(flag);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int below = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) s_wave[wid] = __popcll(m);
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = s_wave[w];
    base += w < wid ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + below;
}

// block_rank for four flags at once; s_wave needs 4 * kWaves entries.
__device__ __forceinline__ void block_rank4(const bool f[4], int* s_wave, int rank[4], int total[4]) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  unsigned long long m[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = __ballot(f[i]);
    if (lane == 0) s_wave[i * kWaves + wid] = __popcll(m[i]);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = s_wave[i * kWaves + w];
      base += w < wid ? c : 0;
      tot += c;
    }
    rank[i] = base + __popcll(m[i] & ((1ull << lane) - 1ull));
    total[i] = tot;
  }
  __syncthreads();
}

// Exclusive prefix sum of v over the block's threads; *total = sum.  All
// threads of the block must call it.  Uses s_wave[kWaves].
__device__ __forceinline__ int block_excl_sum(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o);
    if (lane >= o) inc += n;
  }
  if (lane == 63) s_wave[wid] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = s_wave[w];
    base += w < wid ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

}  // namespace moe
