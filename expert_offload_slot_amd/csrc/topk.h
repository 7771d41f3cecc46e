// Top-k of router logits by one wavefront per token (radix select), with the
// renormalised softmax weights of the chosen experts.
//
// Order: logit descending, expert id ascending on equal logits; a NaN logit is
// reported and ranked as -inf, and -0 counts as +0.  Each logit becomes a
// 32-bit key that orders like the number:
//     key = bits ^ 0xffffffff (negative),  bits | 0x80000000 (otherwise)
// Lane l holds the keys of experts l, l + 64, ... (J per lane).  Radix select
// over the 32 key bits (one ballot per held key and bit, MSB first) finds the
// k-th largest key theta; every key above theta is chosen, and of the keys
// equal to theta the ones of lowest id.  The k chosen experts are then sorted
// by (key desc, id asc) in a few LDS entries of the wavefront.  Weights:
//     w_j = exp(l_j - l_0) / (exp(l_0 - l_0) + ... + exp(l_{k-1} - l_0))
// with the sum taken in j order.
#pragma once

#include <math.h>

#include "internal.h"

namespace moe {

// registers per lane that hold E logits
__host__ __device__ inline int topk_lanes(int E) {
  return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16;
}

// LDS of one wavefront
struct TopkScratch {
  uint64_t chosen[kMaxTopK];  // (key, ~id) of the chosen experts, unordered
  uint64_t sorted[kMaxTopK];  // the same, by rank
};

// orders the wavefront's LDS accesses around it (LDS runs a wavefront's
// instructions in order; this keeps the compiler from moving them)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t logit_key(float v) {
  if (v == 0.f) v = 0.f;  // -0 == +0
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Top-k of one token's E logits l[0..E) by the calling wavefront (all 64
// lanes, wave-uniform arguments).  Lane j < k gets choice j in *id and *w.
// Returns (in every lane) whether any logit was NaN.  k <= E, J * 64 >= E.
template <int J>
__device__ __forceinline__ bool wave_topk(const float* __restrict__ l, int E, int k, TopkScratch& s, int* id,
                                          float* w) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t key[J];
  bool nan = false;
  float lv[J];
#pragma unroll
  for (int j = 0; j < J; ++j) lv[j] = lane + 64 * j < E ? l[lane + 64 * j] : 0.f;  // every load issued first
#pragma unroll
  for (int j = 0; j < J; ++j) {
    key[j] = 0;  // below every real key (-inf maps to 0x007fffff)
    if (lane + 64 * j < E) {
      float v = lv[j];
      if (v != v) {
        nan = true;
        v = -INFINITY;
      }
      key[j] = logit_key(v);
    }
  }
  // theta: the largest value with at least k keys >= it
  uint32_t theta = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = theta | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) cnt += __popcll(__ballot(key[j] >= cand));
    if (cnt >= k) theta = cand;
  }
  int n_gt = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) n_gt += __popcll(__ballot(key[j] > theta));
  const int need = k - n_gt;  // keys equal to theta to take, lowest ids first
  int eq_before = 0, placed = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const bool eq = key[j] == theta;
    const unsigned long long meq = __ballot(eq);
    const bool sel = key[j] > theta || (eq && eq_before + __popcll(meq & below) < need);
    const unsigned long long msel = __ballot(sel);
    if (sel) s.chosen[placed + __popcll(msel & below)] = ((uint64_t)key[j] << 32) | (0xffffffffu - (uint32_t)(lane + 64 * j));
    placed += __popcll(msel);
    eq_before += __popcll(meq);
  }
  wave_lds_sync();
  if (lane < k) {
    const uint64_t mine = s.chosen[lane];
    int rank = 0;
    for (int i = 0; i < k; ++i) rank += s.chosen[i] > mine ? 1 : 0;
    s.sorted[rank] = mine;
  }
  wave_lds_sync();
  if (lane < k) {
    const float l0 = key_logit((uint32_t)(s.sorted[0] >> 32));
    float sum = 0.f;
    for (int j = 0; j < k; ++j) sum = sum + expf(key_logit((uint32_t)(s.sorted[j] >> 32)) - l0);
    const uint64_t m = s.sorted[lane];
    *id = (int)(0xffffffffu - (uint32_t)m);
    *w = expf(key_logit((uint32_t)(m >> 32)) - l0) / sum;
  }
  wave_lds_sync();  // scratch free for the wavefront's next token
  return __any(nan);
}

}  // namespace moe
