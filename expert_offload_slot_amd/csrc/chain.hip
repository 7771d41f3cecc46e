// Decode-step chain: L layers of (route, ensure, copy, ffn + residual) issued
// on one compute stream and captured once into a HIP graph; optionally the
// router-lookahead prefetch variant with a predictor stream and a copy stream.
// Per layer on the compute stream: router logits; one control workgroup (top-k,
// ensure, FFN grouping); the miss copy; the FFN kernels with the combine,
// residual and the next layer's norm.  For small bf16/fp8 batches the combine
// of layer l is instead recomputed by every workgroup of layer l+1's router
// launch, which also writes y_l, x_{l+1} and xn_{l+1} (same bits).  In the lookahead variant the logits
// launch also runs the next layer's router on this layer's input, and the
// control workgroup also installs the predicted experts into the next layer;
// only the prefetch copy runs on a side stream.  (Calls with more than
// kDecideMaxPairs (t, j) pairs use the separate kernels and a predictor stream.)
//
// Layers in cold or split mode join the chain too (npu-offload README,
// "Architecture": per layer the accelerator computes the resident experts while
// the host CPU computes the cold ones from host DRAM): after the control step a
// one-workgroup kernel publishes the call's record indices and activations into
// pinned host memory and bumps the layer's request number; a host server thread
// (host_ffn.cpp) computes the pairs whose record index is S + E + e into the
// layer's host rows and stores the request number as the layer's done number;
// after the GPU's own FFN launches, a one-workgroup kernel waits for that number
// (bounded: past half a second or so it sets MOE_DEV_ERR_HOST_TIMEOUT and goes on)
// and a workgroup per host-computed pair copies its row into the layer's fp32
// outputs before the combine.
// A call without such pairs publishes nothing and waits for nothing.
//
// xinfer-ai 0.14.6 docs/moe_offload.md, "How it works", Decode (the step stays
// inside a captured graph, no host sync); FreeToken issue #677, "Proposal"
// (Lookahead, Install, Correctness constraint: every slot-table writer on the
// compute stream, only reads and byte copies on the other streams).
#include <string.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "host_ffn.h"
#include "internal.h"

struct moe_chain {
  std::vector<moe_offload*> layers;
  std::vector<const void*> wr;
  std::vector<const float*> bias;
  std::vector<const void*> shared;
  int L = 0, T = 0, k = 0, H = 0, prefetch_n = 0, device = 0;
  int read_through = 1;  // decode steps (up to 64 tokens, 256 pairs): the FFN fills missed slots from the host store
  size_t act = 2;
  void* block = nullptr;
  uint8_t* x = nullptr;
  uint8_t* xn = nullptr;
  uint8_t* y = nullptr;
  int32_t* ids = nullptr;
  float* w = nullptr;
  int32_t* sid = nullptr;
  int32_t* pred = nullptr;
  float* wpred = nullptr;
  hipStream_t cs = nullptr, sp = nullptr, sf = nullptr;  // capture/compute, predictor, prefetch copy
  std::vector<hipEvent_t> ev_x, ev_pred, ev_demand, ev_pf;
  hipEvent_t ev_sp_done = nullptr, ev_sf_done = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  // host-computed experts: per layer, whether the issued step publishes its calls to the host
  // (the state the graph was captured with); the pinned buffers shared with the server thread
  std::vector<char> cold;
  void* cold_block = nullptr;  // pinned, mapped, coherent host memory
  int32_t* pub_sid = nullptr;  // [L][T*k] (device addresses of the same bytes: *_d)
  uint8_t* pub_x = nullptr;    // [L][T][H]
  float* cold_out = nullptr;   // [L][T*k][H]
  uint32_t* req = nullptr;     // [L]
  uint32_t* done = nullptr;    // [L]
  int32_t* pub_sid_d = nullptr;
  uint8_t* pub_x_d = nullptr;
  float* cold_out_d = nullptr;
  uint32_t* req_d = nullptr;
  uint32_t* done_d = nullptr;
  uint32_t* seq = nullptr;     // device [L + 1]: each layer's last request number, then the publish count
  moe::ColdServer* server = nullptr;
};

namespace {

int cfail(int code, const char* msg) { return moe::set_error(code, msg); }

#define CHK(call)                                      \
  do {                                                 \
    hipError_t e_ = (call);                            \
    if (e_ != hipSuccess) return e_;                   \
  } while (0)

// ------------------------------------------------------------------ host-computed experts
constexpr uint32_t kColdMaxPolls = 1u << 19;  // half a second or more of polls of the done number

__device__ __forceinline__ bool is_cold(int r, int S, int E) { return r >= S + E && r < S + 2 * E; }

// A workgroup per token: when the call has a host-computed pair, copies the activation row of its
// token if that token has such a pair (workgroup 0 also the call's record indices) into the pinned
// host buffers.  Every thread then fences at system scope, and the last workgroup to count itself
// in (an acquire-release count at system scope in device memory) stores the next request number,
// also kept in seq for the wait, and clears the count for the next launch.  The rows cross the
// host link from T workgroups at once: a single workgroup wrote them at about 4 GB/s.
__global__ __launch_bounds__(256) void k_cold_publish(const int32_t* __restrict__ sid, int T, int k, int S, int E,
                                                      const uint4* __restrict__ x, int row16, int32_t* pub_sid,
                                                      uint4* pub_x, uint32_t* req, uint32_t* seq, uint32_t* arrive) {
  const int n = T * k, t = blockIdx.x;
  bool mine = false;
  for (int i = threadIdx.x; i < n; i += blockDim.x) mine |= is_cold(sid[i], S, E);
  if (!__syncthreads_or(mine)) return;  // the same in every workgroup: nothing for the host, nothing published
  if (t == 0)
    for (int i = threadIdx.x; i < n; i += blockDim.x) pub_sid[i] = sid[i];
  bool row = false;
  for (int j = 0; j < k; ++j) row |= is_cold(sid[t * k + j], S, E);  // uniform
  if (row)
    for (int i = threadIdx.x; i < row16; i += blockDim.x) pub_x[(size_t)t * row16 + i] = x[(size_t)t * row16 + i];
  __threadfence_system();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t a = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_SYSTEM);
    if (a == gridDim.x - 1) {  // every workgroup's rows are out
      __hip_atomic_store(arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t r = *seq + 1;
      *seq = r;
      __hip_atomic_store(req, r, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

// One workgroup: when the call has a host-computed pair, waits until the host's done number equals
// the request number (bounded).  The polls are relaxed system-scope loads, which read memory
// without invalidating the caches each time.
__global__ __launch_bounds__(256) void k_cold_wait(const int32_t* __restrict__ sid, int n, int S, int E,
                                                   const uint32_t* done, const uint32_t* __restrict__ seq,
                                                   int32_t* err) {
  bool mine = false;
  for (int i = threadIdx.x; i < n; i += blockDim.x) mine |= is_cold(sid[i], S, E);
  if (!__syncthreads_or(mine) || threadIdx.x != 0) return;
  const uint32_t r = *seq;
  uint32_t polls = 0;
  while (__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != r) {
    if (++polls == kColdMaxPolls) {
      atomicOr(err, MOE_DEV_ERR_HOST_TIMEOUT);
      break;
    }
    __builtin_amdgcn_s_sleep(8);
  }
}

// 16 bytes of host memory with two relaxed system-scope loads: read from memory, past any cached copy
__device__ __forceinline__ float4 load_host16(const float4* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  return make_float4(__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                     __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32)));
}

// After k_cold_wait (stream order: the host's rows were stored before its done number): a workgroup
// per host-computed pair copies its host row into part.
__global__ __launch_bounds__(256) void k_cold_rows(const int32_t* __restrict__ sid, int n, int S, int E, int H,
                                                   const float4* rows, float4* __restrict__ part) {
  const int h4 = H / 4;
  for (int p = blockIdx.x; p < n; p += gridDim.x) {
    if (!is_cold(sid[p], S, E)) continue;  // workgroup-uniform
    for (int i = threadIdx.x; i < h4; i += blockDim.x) part[(size_t)p * h4 + i] = load_host16(rows + (size_t)p * h4 + i);
  }
}

// whether layer h's calls of T tokens may have host-computed pairs: cold mode, or split mode for calls
// that can overflow (more pairs than the slots they may claim)
bool needs_host(const moe_offload* h, int T) {
  return h->cold_on && !(h->cold_split && (int64_t)T * h->k <= h->S - h->n_pinned);
}

uint8_t* X(moe_chain* c, int l) { return c->x + (size_t)l * c->T * c->H * c->act; }
uint8_t* XN(moe_chain* c, int l) { return c->xn + (size_t)l * c->T * c->H * c->act; }
uint8_t* Y(moe_chain* c, int l) { return c->y + (size_t)l * c->T * c->H * c->act; }
constexpr float kRmsEps = 1e-6f;
size_t R(moe_chain* c, int l) { return (size_t)l * c->T * c->k; }

// Issues one decode step with `cs` as the compute stream.
hipError_t issue(moe_chain* c, hipStream_t cs) {
  const int T = c->T, n = c->T * c->k;
  const bool pf = c->prefetch_n > 0;
  const bool fused = n <= moe::kDecideMaxPairs;
  // the previous layer's combine rides in the next router launch (small bf16 / fp8 decode batches)
  const moe_offload* l0 = c->layers[0];
  const bool fuse_cl = fused && l0->dtype != MOE_F32 && c->H <= moe::kFusedCombineMaxH && T <= 8;
  for (int l = 0; l < c->L; ++l) {
    moe_offload* h = c->layers[l];
    const bool look = pf && l + 1 < c->L;
    // layer 0 normalises the step input; every later input is normalised by the
    // previous layer's combine, in the same order (identical bits)
    if (l == 0) CHK(moe::launch_rmsnorm(X(c, 0), XN(c, 0), T, c->H, h->dtype, kRmsEps, cs));
    moe_offload* hn = look ? c->layers[l + 1] : nullptr;
    if (fused) {
      // router logits (and, for the lookahead, the next layer's router on the same
      // input in the same launch), then one control workgroup: top-k, ensure, FFN
      // grouping (and the next layer's prediction and install)
      if (fuse_cl && l > 0) {  // with layer l-1's combine, which forms this layer's input xn_l
        moe::CombineSrc cb;
        cb.part = c->layers[l - 1]->part;
        cb.w = c->w + R(c, l - 1);
        cb.T = T;
        cb.k = c->k;
        cb.shared = c->shared[l - 1] != nullptr;
        cb.y = Y(c, l - 1);
        cb.residual = X(c, l - 1);
        cb.x_next = X(c, l);
        cb.xn_next = XN(c, l);
        cb.eps = kRmsEps;
        CHK(moe::launch_combine_logits(h, cb, c->wr[l], c->bias[l], T, cs, hn, look ? c->wr[l + 1] : nullptr,
                                       look ? c->bias[l + 1] : nullptr));
      } else {
        CHK(moe::launch_logits(h, XN(c, l), c->wr[l], c->bias[l], T, cs, hn, look ? c->wr[l + 1] : nullptr,
                               look ? c->bias[l + 1] : nullptr));
      }
      CHK(moe::launch_decide(h, T, c->ids + R(c, l), c->w + R(c, l), c->sid + R(c, l), cs, hn,
                             look ? c->pred + R(c, l + 1) : nullptr, look ? c->prefetch_n : 0));
    } else {
      if (look) {  // fork: layer l+1's router on layer l's router input
        CHK(hipEventRecord(c->ev_x[l], cs));
        CHK(hipStreamWaitEvent(c->sp, c->ev_x[l], 0));
        CHK(moe::launch_route(hn, XN(c, l), c->wr[l + 1], c->bias[l + 1], T, c->pred + R(c, l + 1),
                              c->wpred + R(c, l + 1), c->sp));
        CHK(hipEventRecord(c->ev_pred[l + 1], c->sp));
      }
      CHK(moe::launch_route(h, XN(c, l), c->wr[l], c->bias[l], T, c->ids + R(c, l), c->w + R(c, l), cs));
      CHK(moe::launch_ensure(h, c->ids + R(c, l), n, c->sid + R(c, l), cs));
      if (look) {  // join, then install into layer l+1 on the compute stream
        CHK(hipStreamWaitEvent(cs, c->ev_pred[l + 1], 0));
        CHK(moe::launch_install(hn, c->pred + R(c, l + 1), T, c->prefetch_n, cs));
      }
    }
    const bool cold = c->cold[l] != 0;
    if (cold) {  // the call's host-computed pairs go to the server thread
      const size_t xrow = (size_t)c->H * c->act;
      hipLaunchKernelGGL(k_cold_publish, dim3(T), dim3(256), 0, cs, (const int32_t*)(c->sid + R(c, l)), T, c->k,
                         h->S, h->E, (const uint4*)XN(c, l), (int)(xrow / 16), c->pub_sid_d + R(c, l),
                         (uint4*)(c->pub_x_d + (size_t)l * T * xrow), c->req_d + l, c->seq + l, c->seq + c->L);
      CHK(hipGetLastError());
    }
    if (pf && l >= 1) CHK(hipStreamWaitEvent(cs, c->ev_pf[l], 0));  // this layer's prefetch copy first
    // a decode step's misses are read through by its FFN launches instead of a copy launch
    const bool fill = c->read_through && moe::ffn_reads_through(h, T);
    if (!fill) CHK(moe::launch_copy(h, h->cache.copy_list, cs));
    if (look) {  // prefetch copy for layer l+1, after layer l's copy launch (read-through: after its control step)
      CHK(hipEventRecord(c->ev_demand[l], cs));
      CHK(hipStreamWaitEvent(c->sf, c->ev_demand[l], 0));
      CHK(moe::launch_copy(hn, hn->cache.pf_list, c->sf));
      CHK(hipEventRecord(c->ev_pf[l + 1], c->sf));
    }
    const bool combine = !(fuse_cl && l + 1 < c->L);
    void* xn_next = l + 1 < c->L ? XN(c, l + 1) : nullptr;
    CHK(moe::launch_ffn(h, XN(c, l), c->sid + R(c, l), c->w + R(c, l), T, c->shared[l], Y(c, l), X(c, l), X(c, l + 1),
                        xn_next, kRmsEps, cs, fused, combine && !cold, fill));
    if (cold) {  // the host's rows join the GPU's before the combine
      hipLaunchKernelGGL(k_cold_wait, dim3(1), dim3(256), 0, cs, (const int32_t*)(c->sid + R(c, l)), n, h->S, h->E,
                         (const uint32_t*)(c->done_d + l), (const uint32_t*)(c->seq + l), h->cache.err);
      CHK(hipGetLastError());
      hipLaunchKernelGGL(k_cold_rows, dim3(std::min(n, 256)), dim3(256), 0, cs, (const int32_t*)(c->sid + R(c, l)), n,
                         h->S, h->E, c->H, (const float4*)(c->cold_out_d + R(c, l) * c->H), (float4*)h->part);
      CHK(hipGetLastError());
      if (combine)
        CHK(moe::launch_combine(h, XN(c, l), c->w + R(c, l), T, c->shared[l], Y(c, l), X(c, l), X(c, l + 1), xn_next,
                                kRmsEps, cs));
    }
  }
  if (pf && c->L > 1) {  // rejoin the side streams (the predictor stream is used only without fusion)
    if (!fused) {
      CHK(hipEventRecord(c->ev_sp_done, c->sp));
      CHK(hipStreamWaitEvent(cs, c->ev_sp_done, 0));
    }
    CHK(hipEventRecord(c->ev_sf_done, c->sf));
    CHK(hipStreamWaitEvent(cs, c->ev_sf_done, 0));
  }
  return hipSuccess;
}

void release(moe_chain* c) {
  if (c->server) moe::cold_server_stop(c->server);  // after the device drained (the callers synchronise first)
  c->server = nullptr;
  if (c->cold_block) (void)hipHostFree(c->cold_block);
  if (c->exec) (void)hipGraphExecDestroy(c->exec);
  if (c->graph) (void)hipGraphDestroy(c->graph);
  for (auto* v : {&c->ev_x, &c->ev_pred, &c->ev_demand, &c->ev_pf})
    for (hipEvent_t e : *v)
      if (e) (void)hipEventDestroy(e);
  if (c->ev_sp_done) (void)hipEventDestroy(c->ev_sp_done);
  if (c->ev_sf_done) (void)hipEventDestroy(c->ev_sf_done);
  if (c->cs) (void)hipStreamDestroy(c->cs);
  if (c->sp) (void)hipStreamDestroy(c->sp);
  if (c->sf) (void)hipStreamDestroy(c->sf);
  if (c->block) (void)hipFree(c->block);
}

}  // namespace

extern "C" {

int moe_chain_create(moe_offload* const* layers, int32_t L, const void* const* w_router, const float* const* bias,
                     const void* const* shared_records, int32_t T, int32_t prefetch_n, moe_chain** out) {
  if (!out || !layers || !w_router || !bias || L < 1) return cfail(MOE_EINVAL, "moe_chain_create: bad arguments");
  *out = nullptr;
  const moe_offload* l0 = layers[0];
  if (!l0) return cfail(MOE_EINVAL, "moe_chain_create: null layer");
  for (int l = 0; l < L; ++l) {
    const moe_offload* h = layers[l];
    if (!h || h->H != l0->H || h->k != l0->k || h->dtype != l0->dtype || h->device != l0->device ||
        T < 1 || T > h->max_tokens || !w_router[l] || !bias[l])
      return cfail(MOE_EINVAL, "moe_chain_create: layers differ in H/k/dtype/device, T out of range, or null router");
    if (prefetch_n < 0 || prefetch_n > h->S) return cfail(MOE_EINVAL, "moe_chain_create: prefetch_n outside [0, S]");
  }
  moe_chain* c = new (std::nothrow) moe_chain();
  if (!c) return cfail(MOE_ENOMEM, "moe_chain_create: host allocation");
  c->layers.assign(layers, layers + L);
  c->wr.assign(w_router, w_router + L);
  c->bias.assign(bias, bias + L);
  c->shared.assign(L, nullptr);
  if (shared_records)
    for (int l = 0; l < L; ++l) c->shared[l] = shared_records[l];
  c->L = L;
  c->T = T;
  c->k = l0->k;
  c->H = l0->H;
  c->prefetch_n = prefetch_n;
  c->device = l0->device;
  c->act = l0->dtype == MOE_F32 ? 4 : 2;
  c->cold.assign(L, 0);
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(c->device);
  const size_t xa = (size_t)(L + 1) * T * c->H * c->act, ya = (size_t)L * T * c->H * c->act;
  const size_t ra = (size_t)L * T * c->k * 4;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t total = al(xa) + 2 * al(ya) + 5 * al(ra) + al(4 * ((size_t)L + 1));
  hipError_t e = hipMalloc(&c->block, total);
  if (e == hipSuccess) e = hipMemset(c->block, 0, total);
  if (e == hipSuccess) {
    uint8_t* b = (uint8_t*)c->block;
    c->x = b;
    c->xn = b + al(xa);
    c->y = c->xn + al(ya);
    uint8_t* r = c->y + al(ya);
    c->ids = (int32_t*)r;
    c->w = (float*)(r + al(ra));
    c->sid = (int32_t*)(r + 2 * al(ra));
    c->pred = (int32_t*)(r + 3 * al(ra));
    c->wpred = (float*)(r + 4 * al(ra));
    c->seq = (uint32_t*)(r + 5 * al(ra));
    e = hipStreamCreateWithFlags(&c->cs, hipStreamNonBlocking);
  }
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->sp, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->sf, hipStreamNonBlocking);
  for (auto* v : {&c->ev_x, &c->ev_pred, &c->ev_demand, &c->ev_pf}) {
    v->assign(L, nullptr);
    for (int l = 0; l < L && e == hipSuccess; ++l) e = hipEventCreateWithFlags(&(*v)[l], hipEventDisableTiming);
  }
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_sp_done, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_sf_done, hipEventDisableTiming);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  (void)hipSetDevice(prev);
  if (e != hipSuccess) {
    release(c);
    delete c;
    return cfail(e == hipErrorOutOfMemory ? MOE_ENOMEM : MOE_EHIP, hipGetErrorString(e));
  }
  *out = c;
  return MOE_OK;
}

int moe_chain_get_buffers(const moe_chain* c, moe_chain_buffers* out) {
  if (!c || !out) return cfail(MOE_EINVAL, "moe_chain_get_buffers: null argument");
  out->x = c->x;
  out->xn = c->xn;
  out->y = c->y;
  out->ids = c->ids;
  out->w = c->w;
  out->slot_ids = c->sid;
  out->pred = c->pred;
  out->act_bytes = c->act;
  return MOE_OK;
}

// Which layers publish their calls to the host now (cold mode, or split mode with calls that can
// overflow); on the first such layer, the pinned buffers and the server thread.  *changed: the
// set differs from the one the chain was last issued with (a captured graph is then stale).
static int prepare_cold(moe_chain* c, const char* who, bool* changed) {
  std::vector<char> now(c->L, 0);
  bool any = false;
  for (int l = 0; l < c->L; ++l) {
    now[l] = needs_host(c->layers[l], c->T);
    any = any || now[l];
  }
  if (any && c->prefetch_n > 0)
    return moe::set_error(MOE_EINVAL, (std::string(who) + ": lookahead prefetch with a layer in cold or split mode")
                                          .c_str());
  *changed = now != c->cold;
  if (any && !c->cold_block) {
    const size_t L = c->L, n = (size_t)c->T * c->k;
    auto al = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t flags = al(8 * L), sid = al(4 * L * n), xb = al(L * c->T * c->H * c->act), ob = 4 * L * n * c->H;
    hipError_t e = hipHostMalloc(&c->cold_block, flags + sid + xb + ob, hipHostMallocMapped | hipHostMallocCoherent);
    uint8_t* d = nullptr;
    if (e == hipSuccess) {
      memset(c->cold_block, 0, flags + sid + xb + ob);
      e = hipHostGetDevicePointer((void**)&d, c->cold_block, 0);
    }
    if (e != hipSuccess) {
      if (c->cold_block) (void)hipHostFree(c->cold_block);
      c->cold_block = nullptr;
      return moe::set_error(e == hipErrorOutOfMemory ? MOE_ENOMEM : MOE_EHIP, hipGetErrorString(e));
    }
    uint8_t* b = (uint8_t*)c->cold_block;
    c->req = (uint32_t*)b;
    c->done = c->req + L;
    c->pub_sid = (int32_t*)(b + flags);
    c->pub_x = b + flags + sid;
    c->cold_out = (float*)(b + flags + sid + xb);
    c->req_d = (uint32_t*)d;
    c->done_d = c->req_d + L;
    c->pub_sid_d = (int32_t*)(d + flags);
    c->pub_x_d = d + flags + sid;
    c->cold_out_d = (float*)(d + flags + sid + xb);
  }
  if (any && !c->server) {
    // the device request counters restart with the host's numbers
    hipError_t e = hipMemset(c->seq, 0, 4 * ((size_t)c->L + 1));
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return moe::set_error(MOE_EHIP, hipGetErrorString(e));
    memset(c->cold_block, 0, 8 * (size_t)c->L);
    std::vector<moe::ColdChainLayer> ls(c->L);
    for (int l = 0; l < c->L; ++l) {
      const moe_offload* h = c->layers[l];
      ls[l] = {h->host, (uint64_t)h->record_stride, h->dtype, h->H, h->F, h->k, h->S, h->E};
    }
    moe::ColdChainIo io;
    io.sid = c->pub_sid;
    io.x = c->pub_x;
    io.out = c->cold_out;
    io.req = c->req;
    io.done = c->done;
    c->server = moe::cold_server_start(ls.data(), c->L, c->T, (uint64_t)c->H * c->act, io);
    if (!c->server) return moe::set_error(MOE_ENOMEM, (std::string(who) + ": cannot start the host thread").c_str());
  }
  c->cold = now;
  return MOE_OK;
}

int moe_chain_run(moe_chain* c, void* stream) {
  if (!c) return cfail(MOE_EINVAL, "moe_chain_run: null chain");
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(c->device);
  bool changed = false;
  if (int rc = prepare_cold(c, "moe_chain_run", &changed)) {
    (void)hipSetDevice(prev);
    return rc;
  }
  hipError_t e = hipSuccess;
  if (changed && c->exec) {  // the graph was captured with another set of host-computed layers
    e = hipDeviceSynchronize();
    (void)hipGraphExecDestroy(c->exec);
    (void)hipGraphDestroy(c->graph);
    c->exec = nullptr;
    c->graph = nullptr;
  }
  if (e == hipSuccess && !c->exec) {
    e = hipStreamBeginCapture(c->cs, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
      hipError_t ei = issue(c, c->cs);
      e = hipStreamEndCapture(c->cs, &c->graph);
      if (ei != hipSuccess) e = ei;
    }
    if (e == hipSuccess) e = hipGraphInstantiate(&c->exec, c->graph, nullptr, nullptr, 0);
  }
  if (e == hipSuccess) e = hipGraphLaunch(c->exec, (hipStream_t)stream);
  (void)hipSetDevice(prev);
  if (e != hipSuccess) return cfail(MOE_EHIP, hipGetErrorString(e));
  return MOE_OK;
}

int moe_chain_set_read_through(moe_chain* c, int on) {
  if (!c) return cfail(MOE_EINVAL, "moe_chain_set_read_through: null chain");
  if ((on != 0) == (c->read_through != 0)) return MOE_OK;
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(c->device);
  hipError_t e = hipDeviceSynchronize();  // no replay of the old graph may still run
  if (c->exec) (void)hipGraphExecDestroy(c->exec);
  if (c->graph) (void)hipGraphDestroy(c->graph);
  c->exec = nullptr;
  c->graph = nullptr;
  c->read_through = on != 0;
  (void)hipSetDevice(prev);
  if (e != hipSuccess) return cfail(MOE_EHIP, hipGetErrorString(e));
  return MOE_OK;
}

int moe_chain_run_eager(moe_chain* c, void* stream) {
  if (!c) return cfail(MOE_EINVAL, "moe_chain_run_eager: null chain");
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(c->device);
  bool changed = false;
  if (int rc = prepare_cold(c, "moe_chain_run_eager", &changed)) {
    (void)hipSetDevice(prev);
    return rc;
  }
  if (changed && c->exec) {  // the captured graph is stale: it is recaptured at the next moe_chain_run
    (void)hipDeviceSynchronize();
    (void)hipGraphExecDestroy(c->exec);
    (void)hipGraphDestroy(c->graph);
    c->exec = nullptr;
    c->graph = nullptr;
  }
  hipError_t e = issue(c, (hipStream_t)stream);
  (void)hipSetDevice(prev);
  if (e != hipSuccess) return cfail(MOE_EHIP, hipGetErrorString(e));
  return MOE_OK;
}

void moe_chain_destroy(moe_chain* c) {
  if (!c) return;
  (void)hipSetDevice(c->device);
  (void)hipDeviceSynchronize();
  release(c);
  delete c;
}

}  // extern "C"
