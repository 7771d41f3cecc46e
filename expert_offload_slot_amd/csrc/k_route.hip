// Router: logits, top-k, renormalised softmax weights.
//
// The pages only say experts are "routed" (xinfer-ai 0.14.6 docs/moe_offload.md,
// opening paragraph: where experts sit does not alter which ones are chosen).
// The logit is taken in binary32 in one fixed order so the integer top-k
// decision is reproducible:
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
#include "rownorm.h"
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
  const float be = j.bias[e];  // requested with the first loads, not after the sum
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
    if (lane == 0 && tt < nt) j.logits[(size_t)(t0 + tt) * j.E + e] = p + be;
  }
}

// Decode chain: the previous layer's combine taken into this layer's router
// launch.  Workgroup (x, t, z) recomputes token t's combine exactly as the
// combine kernel does (thread i owns the chunks i, i + 256, ...; y and x_next
// rounded once each; the row norm in rownorm.h's order), keeps the normalised
// row in LDS, and its four wavefronts take the logits of experts 4x .. 4x+3 of
// router z in the canonical order above.  The router rows are requested before
// the combine so both loads are in flight together.
constexpr int kRowChunks = kFusedCombineMaxH / (8 * kRowThreads);  // combine chunks per thread
constexpr int kRouterChunks = kFusedCombineMaxH / (8 * 64);         // router chunks per lane

__global__ __launch_bounds__(kRowThreads) void k_combine_logits(CombineSrc cb, RouterJob<uint16_t> j0,
                                                                RouterJob<uint16_t> j1, int H) {
  __shared__ float s_wave[4];
  __shared__ __align__(16) uint16_t xs[kFusedCombineMaxH];
  const RouterJob<uint16_t> j = blockIdx.z == 0 ? j0 : j1;
  const int t = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int e = blockIdx.x * 4 + (tid >> 6);
  const bool ev = e < j.E;
  const bool lead = blockIdx.x == 0 && blockIdx.z == 0;
  uint4 wr[kRouterChunks];
  const float be = ev ? j.bias[e] : 0.f;  // requested with the router rows, not after the sum
#pragma unroll
  for (int i = 0; i < kRouterChunks; ++i) {
    const int c = lane + 64 * i;
    if (ev && c * 8 < H) wr[i] = *reinterpret_cast<const uint4*>(j.wr + (size_t)e * H + c * 8);
  }
  // combine of token t
  const int k = cb.k, routed = cb.T * cb.k;
  const size_t roff = (size_t)t * H * 2;
  void* yrow = lead ? (uint8_t*)cb.y + roff : nullptr;
  void* xrow = lead ? (uint8_t*)cb.x_next + roff : nullptr;
  void* xnrow = lead ? (uint8_t*)cb.xn_next + roff : nullptr;
  const void* rrow = (const uint8_t*)cb.residual + roff;
  float xv[kRowChunks][8];
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < kRowChunks; ++q) {
    const int c = tid + kRowThreads * q;
    if (c * 8 < H) {
      float acc[8], res[8];
      combine_chunk<false>(cb.part + (uint64_t)t * k * H, cb.w + (size_t)t * k, k, H, c,
                           cb.shared ? cb.part + (uint64_t)(routed + t) * H : nullptr, rrow, acc, res);
      chunk_store<false>(yrow, c, acc);  // acc now holds y as stored
#pragma unroll
      for (int qq = 0; qq < 8; ++qq) xv[q][qq] = res[qq] + acc[qq];
      chunk_store<false>(xrow, c, xv[q]);  // x_next as stored
      ss = chunk_sumsq(xv[q], ss);
    }
  }
  const float inv = row_inv_rms(row_block_sum(ss, s_wave), H, cb.eps);
#pragma unroll
  for (int q = 0; q < kRowChunks; ++q) {
    const int c = tid + kRowThreads * q;
    if (c * 8 < H) {
      float v[8];
#pragma unroll
      for (int qq = 0; qq < 8; ++qq) v[qq] = xv[q][qq] * inv;
      chunk_store<false>(xnrow, c, v);
      chunk_store<false>(xs, c, v);
    }
  }
  __syncthreads();
  if (!ev) return;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kRouterChunks; ++i) {
    const int c = lane + 64 * i;
    if (c * 8 < H) {
      float xv8[8], wv8[8];
      load8(xs + c * 8, xv8);
      const uint4 a4 = wr[i];
      wv8[0] = bf16_lo(a4.x); wv8[1] = bf16_hi(a4.x); wv8[2] = bf16_lo(a4.y); wv8[3] = bf16_hi(a4.y);
      wv8[4] = bf16_lo(a4.z); wv8[5] = bf16_hi(a4.z); wv8[6] = bf16_lo(a4.w); wv8[7] = bf16_hi(a4.w);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc = __builtin_fmaf(xv8[q], wv8[q], acc);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc = acc + __shfl_xor(acc, o);
  if (lane == 0) j.logits[(size_t)t * j.E + e] = acc + be;
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

hipError_t launch_combine_logits(moe_offload* h, const CombineSrc& cb, const void* wr, const float* bias, int T,
                                 hipStream_t s, moe_offload* hn, const void* wrn, const float* biasn) {
  if (h->dtype == MOE_F32 || h->H > kFusedCombineMaxH || (hn && hn->dtype == MOE_F32)) return hipErrorInvalidValue;
  RouterJob<uint16_t> j0{(const uint16_t*)wr, bias, h->logits, h->E};
  RouterJob<uint16_t> j1 = hn ? RouterJob<uint16_t>{(const uint16_t*)wrn, biasn, hn->logits, hn->E} : j0;
  const int E = hn ? std::max(h->E, hn->E) : h->E;
  launch_k(h, MOE_K_LOGITS, k_combine_logits, dim3((E + 3) / 4, T, hn ? 2 : 1), dim3(kRowThreads), 0, s, cb, j0, j1,
           h->H);
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
