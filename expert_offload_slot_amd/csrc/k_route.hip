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
// Two kernels, no communication between workgroups inside a kernel:
//   k_logits  grid (ceil(E/4), ceil(T/4), routers); a wavefront owns one expert
//             and up to 4 tokens, so the router row is loaded once for them.
//             A second router (the next layer's, for the lookahead) can ride
//             in the same launch.
//   k_topk    one wavefront per token: radix select of the k largest keys,
//             then the softmax over the k chosen logits (topk.h; the fused
//             decode control kernel runs the same code).
#include <math.h>

#include <algorithm>

#include "prof.h"
#include "topk.h"

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

// One router's logits: weights [E][H], bias [E], output [T][E].
template <typename A>
struct RouterJob {
  const A* wr;
  const float* bias;
  float* logits;
  int E;
};

// blockIdx.z picks the router (a layer's own, or the next layer's for the
// lookahead prediction on the same input).
template <typename A>
__global__ __launch_bounds__(256) void k_logits(const A* __restrict__ x, RouterJob<A> j0, RouterJob<A> j1, int T,
                                                int H) {
  const RouterJob<A> j = blockIdx.z == 0 ? j0 : j1;
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t0 = blockIdx.y * kRouteTokens;
  const int nt = min(kRouteTokens, T - t0);
  if (e >= j.E) return;
  float acc[kRouteTokens] = {0.f, 0.f, 0.f, 0.f};
  const A* wrow = j.wr + (size_t)e * H;
#pragma unroll 4
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
    if (lane == 0 && tt < nt) j.logits[(size_t)(t0 + tt) * j.E + e] = p + j.bias[e];
  }
}

// Top-k (topk.h): one wavefront per token, 4 tokens per workgroup.
template <int J>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ w, int32_t* err) {
  __shared__ TopkScratch s[4];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;  // wave-uniform; no workgroup barrier below
  int id;
  float wt;
  const bool nan = wave_topk<J>(logits + (size_t)t * E, E, k, s[wv], &id, &wt);
  if (nan && lane == 0) atomicOr(err, MOE_DEV_ERR_NAN);
  if (lane < k) {
    ids[(size_t)t * k + lane] = id;
    w[(size_t)t * k + lane] = wt;
  }
}

}  // namespace

namespace {
template <typename A>
void logits_jobs(moe_offload* h, const void* x, const void* wr, const float* bias, moe_offload* hn,
                 const void* wrn, const float* biasn, int T, hipStream_t s) {
  RouterJob<A> j0{(const A*)wr, bias, h->logits, h->E};
  RouterJob<A> j1 = hn ? RouterJob<A>{(const A*)wrn, biasn, hn->logits, hn->E} : j0;
  const int E = hn ? std::max(h->E, hn->E) : h->E;
  dim3 grid((E + 3) / 4, (T + kRouteTokens - 1) / kRouteTokens, hn ? 2 : 1);
  launch_k(h, MOE_K_LOGITS, k_logits<A>, grid, dim3(256), 0, s, (const A*)x, j0, j1, T, h->H);
}
}  // namespace

hipError_t launch_logits(moe_offload* h, const void* x, const void* wr, const float* bias, int T, hipStream_t s,
                         moe_offload* hn, const void* wrn, const float* biasn) {
  if (h->dtype == MOE_F32)
    logits_jobs<float>(h, x, wr, bias, hn, wrn, biasn, T, s);
  else
    logits_jobs<uint16_t>(h, x, wr, bias, hn, wrn, biasn, T, s);
  return hipGetLastError();
}

hipError_t launch_route(moe_offload* h, const void* x, const void* wr, const float* bias, int T, int32_t* ids,
                        float* w, hipStream_t s) {
  hipError_t e = launch_logits(h, x, wr, bias, T, s);
  if (e != hipSuccess) return e;
  const int J = topk_lanes(h->E);
  auto kt = J == 1 ? k_topk<1> : J == 2 ? k_topk<2> : J == 4 ? k_topk<4> : J == 8 ? k_topk<8> : k_topk<16>;
  launch_k(h, MOE_K_TOPK, kt, dim3((T + 3) / 4), dim3(256), 0, s, h->logits, T, h->E, h->k, ids, w, h->cache.err);
  return hipGetLastError();
}

}  // namespace moe
