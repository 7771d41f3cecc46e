// Top-k of one token's router logits by one wavefront, with the renormalised
// softmax weights of the chosen experts.
//
// Order: logit descending, expert id ascending on equal logits; a NaN logit is
// reported and ranked as -inf.  Lane l holds experts l, l + 64, ... in
// registers (J per lane); each of the k rounds takes the lane-local best of the
// experts not yet chosen and an xor butterfly over the 64 lanes, after which
// every lane holds the round's winner.  Weights: w_j = exp(l_j - l_0) / sum,
// the sum taken by an xor butterfly in a fixed order.
#pragma once

#include <math.h>

#include "internal.h"

namespace moe {

// registers per lane that hold E logits
inline int topk_lanes(int E) { return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16; }

__device__ __forceinline__ bool logit_before(float va, int ea, float vb, int eb) {
  return va > vb || (va == vb && ea < eb);
}

// Lane j < k gets choice j in *id / *w; returns true (in every lane) if any
// logit was NaN.  J * 64 >= E.
template <int J>
__device__ __forceinline__ bool wave_topk(const float* __restrict__ l, int E, int k, int* id, float* w) {
  const int lane = threadIdx.x & 63;
  float v[J];
  bool nan = false;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    float x = -INFINITY;
    if (e < E) {
      x = l[e];
      if (x != x) {
        nan = true;
        x = -INFINITY;
      }
    }
    v[j] = x;
  }
  uint32_t taken = 0;
  int my_id = 0;
  float my_v = 0.f, v0 = 0.f;
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r) {
    if (r < k) {
      float bv = -INFINITY;
      int be = 0x7fffffff;  // loses to every real expert, -inf logits included
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int e = lane + 64 * j;
        if (e < E && !((taken >> j) & 1u) && logit_before(v[j], e, bv, be)) {
          bv = v[j];
          be = e;
        }
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oe = __shfl_xor(be, o);
        if (logit_before(ov, oe, bv, be)) {
          bv = ov;
          be = oe;
        }
      }
      if (be < E && (be & 63) == lane) taken |= 1u << (be >> 6);
      if (lane == r) {
        my_id = be;
        my_v = bv;
      }
      if (r == 0) v0 = bv;
    }
  }
  const float ex = lane < k ? expf(my_v - v0) : 0.f;
  float sum = ex;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  *id = my_id;
  *w = ex / sum;
  return __any(nan);
}

}  // namespace moe
