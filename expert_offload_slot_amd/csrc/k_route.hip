// Router: logits, top-k, renormalised softmax weights.
//
// The pages only say experts are "routed" (xinfer-ai 0.14.6 docs/moe_offload.md,
// opening paragraph: placement never changes routing).  The logit is taken in
// binary32 in one fixed order so the integer top-k decision is reproducible:
// a wavefront's 64 lanes each own every 64th chunk of 8 inputs and run an FMA
// chain over them, then an xor-butterfly (offsets 32..1) combines the lanes,
// then the bias is added.  This maps one (token, expert) dot product onto one
// wavefront with 16-byte loads.
//
// Grid: (ceil(E/4), ceil(T/4)) workgroups of 4 wavefronts; a wavefront owns one
// expert and up to 4 tokens (the router row is loaded once for them).  The last
// workgroup of a token group to finish (device-scope counter, reset by that
// workgroup) selects top-k for its tokens, one wavefront per token.
#include <math.h>

#include "internal.h"

namespace moe {
namespace {

__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

__device__ __forceinline__ void load8(const uint16_t* p, float v[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
  v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
}

// Top-k of one token's E logits by one wavefront: k rounds of a (value desc,
// id asc) arg-max; NaN is reported and ranked as -inf.
__device__ void topk_wave(const float* __restrict__ l, int E, int k, int32_t* __restrict__ ids,
                          float* __restrict__ w, int32_t* err) {
  const int lane = threadIdx.x & 63;
  float v[kMaxExperts / 64];
  bool nan = false;
#pragma unroll
  for (int i = 0; i < kMaxExperts / 64; ++i) {
    const int e = lane + 64 * i;
    float x = e < E ? l[e] : -INFINITY;
    if (x != x) {
      nan = true;
      x = -INFINITY;
    }
    v[i] = x;
  }
  if (__any(nan) && lane == 0) atomicOr(err, MOE_DEV_ERR_NAN);
  uint32_t taken = 0;
  float my_l = 0.f, l0 = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxExperts / 64; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < be))) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oe = __shfl_xor(be, o);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (j == 0) l0 = bv;
    if (lane == j) {
      my_l = bv;
      my_e = be;
    }
  }
  const float ex = lane < k ? expf(my_l - l0) : 0.f;
  float sum = ex;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  if (lane < k) {
    ids[lane] = my_e;
    w[lane] = ex / sum;
  }
}

template <typename A>
__global__ __launch_bounds__(256) void k_route(const A* __restrict__ x, const A* __restrict__ wr,
                                               const float* __restrict__ bias, int T, int E, int H, int k,
                                               float* __restrict__ logits, uint32_t* __restrict__ ctr,
                                               int32_t* __restrict__ ids, float* __restrict__ w, int32_t* err) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = blockIdx.x * 4 + wv;
  const int t0 = blockIdx.y * kRouteTokens;
  const int nt = min(kRouteTokens, T - t0);
  if (e < E) {
    float acc[kRouteTokens] = {0.f, 0.f, 0.f, 0.f};
    const A* wrow = wr + (size_t)e * H;
    for (int c = lane; c * 8 < H; c += 64) {
      float wv8[8];
      load8(wrow + c * 8, wv8);
#pragma unroll
      for (int tt = 0; tt < kRouteTokens; ++tt) {
        if (tt < nt) {
          float xv[8];
          load8(x + (size_t)(t0 + tt) * H + c * 8, xv);
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[tt] = __builtin_fmaf(xv[q], wv8[q], acc[tt]);
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < kRouteTokens; ++tt) {
      float p = acc[tt];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) p = p + __shfl_xor(p, o);
      if (lane == 0 && tt < nt) logits[(size_t)(t0 + tt) * E + e] = p + bias[e];
    }
  }
  // the last workgroup of this token group selects top-k
  __threadfence();
  __syncthreads();
  __shared__ int s_last;
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(&ctr[blockIdx.y], 1u);
    s_last = prev == gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (threadIdx.x == 0) ctr[blockIdx.y] = 0;
  if (wv < nt) {
    const int t = t0 + wv;
    topk_wave(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k, err);
  }
}

}  // namespace

hipError_t launch_route(moe_offload* h, const void* x, const void* wr, const float* bias, int T, int32_t* ids,
                        float* w, hipStream_t s) {
  dim3 grid((h->E + 3) / 4, (T + kRouteTokens - 1) / kRouteTokens);
  if (h->dtype == MOE_F32)
    hipLaunchKernelGGL(k_route<float>, grid, dim3(256), 0, s, (const float*)x, (const float*)wr, bias, T, h->E,
                       h->H, h->k, h->logits, h->route_ctr, ids, w, h->cache.err);
  else
    hipLaunchKernelGGL(k_route<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)x, (const uint16_t*)wr, bias, T,
                       h->E, h->H, h->k, h->logits, h->route_ctr, ids, w, h->cache.err);
  return hipGetLastError();
}

}  // namespace moe
