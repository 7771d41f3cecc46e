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
// xinfer-ai 0.14.6 docs/moe_offload.md, "How it works", Decode (the step stays
// inside a captured graph, no host sync); FreeToken issue #677, "Proposal"
// (Lookahead, Install, Correctness constraint: every slot-table writer on the
// compute stream, only reads and byte copies on the other streams).
#include <string.h>

#include <new>
#include <vector>

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
};

namespace {

int cfail(int code, const char* msg) { return moe::set_error(code, msg); }

#define CHK(call)                                      \
  do {                                                 \
    hipError_t e_ = (call);                            \
    if (e_ != hipSuccess) return e_;                   \
  } while (0)

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
    CHK(moe::launch_ffn(h, XN(c, l), c->sid + R(c, l), c->w + R(c, l), T, c->shared[l], Y(c, l), X(c, l), X(c, l + 1),
                        l + 1 < c->L ? XN(c, l + 1) : nullptr, kRmsEps, cs, fused, !(fuse_cl && l + 1 < c->L),
                        fill));
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
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(c->device);
  const size_t xa = (size_t)(L + 1) * T * c->H * c->act, ya = (size_t)L * T * c->H * c->act;
  const size_t ra = (size_t)L * T * c->k * 4;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t total = al(xa) + 2 * al(ya) + 5 * al(ra);
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

// the decode chain runs without a host round trip: a layer in cold mode cannot join it
static bool any_cold(const moe_chain* c) {
  for (const moe_offload* h : c->layers)
    if (h->cold_on) return true;
  return false;
}

int moe_chain_run(moe_chain* c, void* stream) {
  if (!c) return cfail(MOE_EINVAL, "moe_chain_run: null chain");
  if (any_cold(c)) return cfail(MOE_EINVAL, "moe_chain_run: a layer is in cold mode (host-computed experts)");
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(c->device);
  hipError_t e = hipSuccess;
  if (!c->exec) {
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
  if (any_cold(c)) return cfail(MOE_EINVAL, "moe_chain_run_eager: a layer is in cold mode (host-computed experts)");
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(c->device);
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
