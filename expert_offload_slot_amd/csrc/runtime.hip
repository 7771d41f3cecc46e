// Handle lifetime, argument checks, error convention and the C entry points.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <new>

#include "host_ffn.h"
#include "prof.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(e == hipErrorOutOfMemory ? MOE_ENOMEM : MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(call)                              \
  do {                                             \
    hipError_t e_ = (call);                        \
    if (e_ != hipSuccess) return hip_fail(e_, #call); \
  } while (0)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t record_bytes_of(int dtype, int H, int F) {
  size_t n = 3 * (size_t)H * (size_t)F;
  if (dtype == MOE_F32) return 4 * n;
  if (dtype == MOE_BF16) return 2 * n;
  if (dtype == MOE_MXFP4) return n / 2 + n / 32;  // codes + one scale byte per 32
  return n + 3 * (size_t)(H / 128) * (size_t)(F / 128) * 4;
}

bool known_dtype(int dtype) {
  return dtype == MOE_F32 || dtype == MOE_BF16 || dtype == MOE_FP8_E4M3_B128 || dtype == MOE_MXFP4;
}

bool same_shape(const moe_offload* a, const moe_offload_desc* d) {
  return a->E == d->num_experts && a->H == d->hidden && a->F == d->ffn && a->dtype == d->dtype;
}

// RAII device guard: every entry point runs on the handle's device.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

void free_all(moe_offload* h) {
  if (h->own_host && h->host) (void)hipHostFree(h->host);
  if (h->slots) (void)hipFree(h->slots);
  if (h->own_staging && h->staging) (void)hipFree(h->staging);
  if (h->state_block) (void)hipFree(h->state_block);
  if (h->pinned_i32) (void)hipHostFree(h->pinned_i32);
  if (h->cold_sid) (void)hipHostFree(h->cold_sid);
  if (h->cold_x) (void)hipHostFree(h->cold_x);
  if (h->cold_out) (void)hipHostFree(h->cold_out);
  if (h->cold_ev) (void)hipEventDestroy(h->cold_ev);
  if (h->ens_ev) (void)hipEventDestroy(h->ens_ev);
  if (h->cold_stream) (void)hipStreamDestroy(h->cold_stream);
  if (h->prof) {
    for (auto& pair : h->prof->ev)
      for (hipEvent_t e : pair)
        if (e) (void)hipEventDestroy(e);
    delete h->prof;
    h->prof = nullptr;
  }
}

int check_desc(const moe_offload_desc* d) {
  if (!known_dtype(d->dtype)) return fail(MOE_EUNSUPPORTED, "unsupported dtype %d", d->dtype);
  if (d->num_experts < 1 || d->num_experts > moe::kMaxExperts)
    return fail(MOE_EINVAL, "num_experts=%d outside [1, %d]", d->num_experts, moe::kMaxExperts);
  if (d->top_k < 1 || d->top_k > moe::kMaxTopK || d->top_k > d->num_experts)
    return fail(MOE_EINVAL, "top_k=%d outside [1, min(%d, E)]", d->top_k, moe::kMaxTopK);
  if (d->num_slots < d->top_k || d->num_slots > d->num_experts)
    return fail(MOE_EINVAL, "num_slots=%d outside [top_k=%d, E=%d]", d->num_slots, d->top_k, d->num_experts);
  // decode kernels: a K block is 16 lanes x 8 weights (16 x 16 MXFP4 weights); fp32: 64-row tiles
  int mult = d->dtype == MOE_F32 ? 64 : (d->dtype == MOE_MXFP4 ? 256 : 128);
  if (d->hidden < mult || d->hidden % mult || d->ffn < mult || d->ffn % mult)
    return fail(MOE_EUNSUPPORTED, "hidden=%d / ffn=%d must be positive multiples of %d for this dtype", d->hidden,
                d->ffn, mult);
  if (d->hidden > 65536 || d->ffn > 65536) return fail(MOE_EINVAL, "hidden/ffn above 65536");
  if (d->max_tokens < 1 || d->max_tokens > 65536) return fail(MOE_EINVAL, "max_tokens=%d outside [1, 65536]", d->max_tokens);
  if ((d->flags & MOE_FLAG_SCORED) && (d->flags & MOE_FLAG_FREQ))
    return fail(MOE_EINVAL, "MOE_FLAG_SCORED and MOE_FLAG_FREQ are exclusive");
  if (d->share_host && !same_shape(d->share_host, d)) return fail(MOE_EINVAL, "share_host handle has another shape");
  if (d->share_staging && !same_shape(d->share_staging, d))
    return fail(MOE_EINVAL, "share_staging handle has another shape");
  return MOE_OK;
}

// Offsets of everything in a handle's state block (one device allocation);
// sets h->gl.  Depends on E, S, H, F, k, dtype and max_tokens only.
struct StateLayout {
  size_t o_slot_of, o_expert_of, o_last, o_score, o_pinned, o_act, o_tick, o_list, o_pf, o_cnt, o_err, o_logits,
      o_grp, o_h, o_part, o_scr, o_cold, total;
};

StateLayout state_layout(moe_offload* h) {
  const int maxSE = std::max(h->S, h->E);
  const int max_pairs = h->max_tokens * h->k;
  h->gl.max_pairs = max_pairs;
  h->gl.max_recs = std::min(max_pairs, h->S + h->E) + 1;
  const int rows = max_pairs + h->max_tokens;  // routed pairs + shared-expert rows
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  StateLayout l;
  l.o_slot_of = take(4 * (size_t)h->E);
  l.o_expert_of = take(4 * (size_t)h->S);
  l.o_last = take(8 * (size_t)h->S);
  l.o_score = take(4 * (size_t)h->S);
  l.o_pinned = take(4 * (size_t)h->S);
  l.o_act = take(4 * (size_t)h->E);
  l.o_tick = take(8);
  l.o_list = take(4 * (2 + 2 * (size_t)maxSE));
  l.o_pf = take(4 * (2 + 2 * (size_t)h->S));
  l.o_cnt = take(8 * moe::C_N);
  l.o_err = take(4);
  l.o_logits = take(4 * (size_t)h->max_tokens * h->E);
  l.o_grp = take(4 * (size_t)h->gl.words());
  l.o_h = take((h->dtype == MOE_F32 ? 4 : 2) * (size_t)rows * h->F);
  l.o_part = take(4 * (size_t)rows * h->H);
  l.o_scr = take(64);
  l.o_cold = take(4);
  l.total = off;
  return l;
}

int check_handle(const moe_offload* h) {
  if (!h) return fail(MOE_EINVAL, "null handle");
  return MOE_OK;
}

int check_T(const moe_offload* h, int32_t T) {
  if (T < 1 || T > h->max_tokens) return fail(MOE_EINVAL, "T=%d outside [1, max_tokens=%d]", T, h->max_tokens);
  return MOE_OK;
}

}  // namespace

int moe::set_error(int code, const char* msg) { return fail(code, "%s", msg); }

extern "C" {

const char* moe_offload_last_error(void) { return g_err; }

int moe_offload_create(const moe_offload_desc* d, moe_offload** out) {
  g_err[0] = 0;
  if (!d || !out) return fail(MOE_EINVAL, "null argument");
  *out = nullptr;
  if (int rc = check_desc(d)) return rc;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || d->device < 0 || d->device >= ndev)
    return fail(MOE_EINVAL, "device %d not available (%d devices)", d->device, ndev);
  DeviceGuard g(d->device);
  if (!g.ok) return fail(MOE_EHIP, "hipSetDevice(%d) failed", d->device);

  moe_offload* h = new (std::nothrow) moe_offload();
  if (!h) return fail(MOE_ENOMEM, "host allocation of the handle failed");
  memset(h, 0, sizeof *h);
  h->E = d->num_experts;
  h->S = d->num_slots;
  h->H = d->hidden;
  h->F = d->ffn;
  h->k = d->top_k;
  h->dtype = d->dtype;
  h->max_tokens = d->max_tokens;
  h->device = d->device;
  h->flags = d->flags;
  h->record_bytes = record_bytes_of(h->dtype, h->H, h->F);
  h->record_stride = align_up(h->record_bytes, 4096);

  int rc = MOE_OK;
  auto bail = [&](int code) {
    free_all(h);
    delete h;
    return code;
  };
  hipError_t e;
  const size_t store = (size_t)h->E * h->record_stride;
  if (d->share_host) {
    h->host = d->share_host->host;
    h->host_dev = d->share_host->host_dev;
    h->own_host = false;
  } else {
    unsigned hf = hipHostMallocMapped | ((h->flags & MOE_FLAG_HOST_COHERENT) ? hipHostMallocCoherent
                                                                               : hipHostMallocNonCoherent);
    e = hipHostMalloc((void**)&h->host, store, hf);
    if (e != hipSuccess) {
      rc = fail(MOE_ENOMEM, "pinned host store of %zu bytes: %s", store, hipGetErrorString(e));
      return bail(rc);
    }
    h->own_host = true;
    e = hipHostGetDevicePointer((void**)&h->host_dev, h->host, 0);
    if (e != hipSuccess) return bail(hip_fail(e, "hipHostGetDevicePointer"));
  }
  e = hipMalloc((void**)&h->slots, (size_t)h->S * h->record_stride);
  if (e != hipSuccess) return bail(hip_fail(e, "slot tensor"));
  if (d->share_staging) {
    h->staging = d->share_staging->staging;
    h->own_staging = false;
  } else {
    e = hipMalloc((void**)&h->staging, store);
    if (e != hipSuccess) return bail(hip_fail(e, "staging buffer"));
    h->own_staging = true;
  }

  // one allocation for the table, lists, counters and workspaces
  const StateLayout sl = state_layout(h);
  const size_t o_slot_of = sl.o_slot_of, o_expert_of = sl.o_expert_of, o_last = sl.o_last, o_score = sl.o_score,
               o_pinned = sl.o_pinned, o_act = sl.o_act, o_tick = sl.o_tick, o_list = sl.o_list, o_pf = sl.o_pf,
               o_cnt = sl.o_cnt, o_err = sl.o_err, o_logits = sl.o_logits, o_grp = sl.o_grp, o_h = sl.o_h,
               o_part = sl.o_part, o_scr = sl.o_scr, off = sl.total;
  e = hipMalloc(&h->state_block, off);
  if (e != hipSuccess) return bail(hip_fail(e, "state block"));
  uint8_t* b = (uint8_t*)h->state_block;
  h->cache.slot_of = (int32_t*)(b + o_slot_of);
  h->cache.expert_of = (int32_t*)(b + o_expert_of);
  h->cache.last_use = (uint64_t*)(b + o_last);
  h->cache.score = (uint32_t*)(b + o_score);
  h->cache.pinned = (int32_t*)(b + o_pinned);
  h->cache.act = (uint32_t*)(b + o_act);
  h->cache.policy = (h->flags & MOE_FLAG_SCORED) ? moe::kPolicyScored
                                                 : ((h->flags & MOE_FLAG_FREQ) ? moe::kPolicyFreq : moe::kPolicyLru);
  h->cache.tick = (uint64_t*)(b + o_tick);
  h->cache.copy_list = (int32_t*)(b + o_list);
  h->cache.pf_list = (int32_t*)(b + o_pf);
  h->cache.counters = (uint64_t*)(b + o_cnt);
  h->cache.err = (int32_t*)(b + o_err);
  h->cache.cold = (int32_t*)(b + sl.o_cold);
  h->cache.E = h->E;
  h->cache.S = h->S;
  h->cache.record_bytes = h->record_bytes;
  h->logits = (float*)(b + o_logits);
  h->grp = (int32_t*)(b + o_grp);
  h->hbuf = (void*)(b + o_h);
  h->part = (float*)(b + o_part);
  h->scratch_i32 = (int32_t*)(b + o_scr);
  e = hipHostMalloc((void**)&h->pinned_i32, 64, hipHostMallocDefault);
  if (e != hipSuccess) return bail(hip_fail(e, "pinned scratch"));
  e = moe::scratch_init(h->device);  // once per device: the no-allocation FFN's workspace address
  if (e != hipSuccess) return bail(hip_fail(e, "device scratch address"));
  // zero everything (counters, workspaces), then set the empty-cache state
  e = hipMemset(h->state_block, 0, off);
  if (e != hipSuccess) return bail(hip_fail(e, "hipMemset"));
  e = moe::launch_reset(h, nullptr);
  if (e != hipSuccess) return bail(hip_fail(e, "reset kernel"));
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return bail(hip_fail(e, "hipDeviceSynchronize"));
  *out = h;
  return MOE_OK;
}

int moe_offload_auto_slots(const moe_offload_desc* d, int32_t layers, int32_t share_staging, uint64_t reserve_bytes,
                           uint64_t free_bytes, int32_t* slots_out) {
  g_err[0] = 0;
  if (!d || !slots_out) return fail(MOE_EINVAL, "moe_offload_auto_slots: null argument");
  if (layers < 1) return fail(MOE_EINVAL, "moe_offload_auto_slots: layers=%d < 1", layers);
  moe_offload_desc dk = *d;  // num_slots is the result: validate the rest with the smallest legal value
  dk.num_slots = d->top_k;
  dk.share_host = dk.share_staging = nullptr;
  if (int rc = check_desc(&dk)) return rc;
  if (free_bytes == 0) {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || d->device < 0 || d->device >= ndev)
      return fail(MOE_EINVAL, "device %d not available (%d devices)", d->device, ndev);
    DeviceGuard g(d->device);
    if (!g.ok) return fail(MOE_EHIP, "hipSetDevice(%d) failed", d->device);
    size_t fr = 0, tot = 0;
    HIP_TRY(hipMemGetInfo(&fr, &tot));
    free_bytes = fr;
  }
  moe_offload probe;  // sizes only: the state block at its largest (S = E)
  memset(&probe, 0, sizeof probe);
  probe.E = d->num_experts;
  probe.S = d->num_experts;
  probe.H = d->hidden;
  probe.F = d->ffn;
  probe.k = d->top_k;
  probe.dtype = d->dtype;
  probe.max_tokens = d->max_tokens;
  const size_t stride = align_up(record_bytes_of(d->dtype, d->hidden, d->ffn), 4096);
  const uint64_t staging = (uint64_t)(share_staging ? 1 : layers) * d->num_experts * stride;
  const uint64_t fixed = staging + (uint64_t)layers * state_layout(&probe).total + reserve_bytes;
  const uint64_t per_slot = (uint64_t)layers * stride;  // one more slot in every layer
  const uint64_t room = free_bytes > fixed ? free_bytes - fixed : 0;
  const uint64_t fit = room / per_slot;
  if (fit < (uint64_t)d->top_k) {
    *slots_out = d->top_k;
    return fail(MOE_ENOMEM, "moe_offload_auto_slots: %llu free bytes minus %llu (reserve, staging, state) hold %llu "
                "slots per layer, fewer than top_k=%d", (unsigned long long)free_bytes, (unsigned long long)fixed,
                (unsigned long long)fit, d->top_k);
  }
  *slots_out = fit > (uint64_t)d->num_experts ? d->num_experts : (int32_t)fit;
  return MOE_OK;
}

void moe_offload_destroy(moe_offload* h) {
  if (!h) return;
  DeviceGuard g(h->device);
  (void)hipDeviceSynchronize();
  free_all(h);
  delete h;
}

int moe_offload_host_records(moe_offload* h, void** host, size_t* record_stride, size_t* record_bytes) {
  if (int rc = check_handle(h)) return rc;
  if (host) *host = h->host;
  if (record_stride) *record_stride = h->record_stride;
  if (record_bytes) *record_bytes = h->record_bytes;
  return MOE_OK;
}

int moe_route_topk(moe_offload* h, const void* x, const void* w_router, const float* bias, int32_t T, int32_t* ids,
                   float* w, void* stream) {
  if (int rc = check_handle(h)) return rc;
  if (int rc = check_T(h, T)) return rc;
  if (!x || !w_router || !bias || !ids || !w) return fail(MOE_EINVAL, "moe_route_topk: null pointer");
  DeviceGuard g(h->device);
  HIP_TRY(moe::launch_route(h, x, w_router, bias, T, ids, w, (hipStream_t)stream));
  return MOE_OK;
}

// Split mode: a call of at most S - (pinned experts) pairs has at most that many distinct experts,
// never more than the slots it may claim, so it cannot overflow and none of its misses goes to the
// host; moe_slot_ffn_host_cold runs it as the plain FFN.
static bool split_call_fits(const moe_offload* h, int T) {
  return (int64_t)T * h->k <= h->S - h->n_pinned;
}

// split mode, after a call's ensure: a call that may overflow records the event its FFN's host
// path waits on before reading the call's indices (on the side stream)
static hipError_t record_split_ensure(moe_offload* h, int T, hipStream_t s) {
  h->ens_recorded = h->cold_split && !split_call_fits(h, T);
  return h->ens_recorded ? hipEventRecord(h->ens_ev, s) : hipSuccess;
}

int moe_slot_ensure(moe_offload* h, const int32_t* ids, int32_t T, int32_t* slot_ids, void* stream) {
  if (int rc = check_handle(h)) return rc;
  if (int rc = check_T(h, T)) return rc;
  if (!ids || !slot_ids) return fail(MOE_EINVAL, "moe_slot_ensure: null pointer");
  DeviceGuard g(h->device);
  HIP_TRY(moe::launch_ensure(h, ids, T * h->k, slot_ids, (hipStream_t)stream));
  HIP_TRY(record_split_ensure(h, T, (hipStream_t)stream));
  return MOE_OK;
}

int moe_copy_misses(moe_offload* h, void* stream) {
  if (int rc = check_handle(h)) return rc;
  DeviceGuard g(h->device);
  HIP_TRY(moe::launch_copy(h, h->cache.copy_list, (hipStream_t)stream));
  return MOE_OK;
}

int moe_slot_ffn(moe_offload* h, const void* x, const int32_t* slot_ids, const float* w, int32_t T,
                 const void* shared_record, void* y, const void* residual, void* x_next, void* stream) {
  if (int rc = check_handle(h)) return rc;
  if (int rc = check_T(h, T)) return rc;
  if (!x || !slot_ids || !w || !y) return fail(MOE_EINVAL, "moe_slot_ffn: null pointer");
  if (h->cold_on) return fail(MOE_EINVAL, "moe_slot_ffn: the layer is in cold mode; use moe_slot_ffn_host_cold");
  DeviceGuard g(h->device);
  HIP_TRY(moe::launch_ffn(h, x, slot_ids, w, T, shared_record, y, residual, x_next, nullptr, 0.f,
                          (hipStream_t)stream));
  return MOE_OK;
}

int moe_slot_ffn_host_cold(moe_offload* h, const void* x, const int32_t* slot_ids, const float* w, int32_t T,
                           const void* shared_record, void* y, const void* residual, void* x_next, void* stream) {
  if (int rc = check_handle(h)) return rc;
  if (int rc = check_T(h, T)) return rc;
  if (!x || !slot_ids || !w || !y) return fail(MOE_EINVAL, "moe_slot_ffn_host_cold: null pointer");
  if (!h->cold_out) return fail(MOE_EINVAL, "moe_slot_ffn_host_cold: the cold mode was never switched on");
  DeviceGuard g(h->device);
  hipStream_t s = (hipStream_t)stream;
  // split mode, a call that cannot overflow: the plain FFN, with no host round trip (the same
  // kernels as moe_slot_ffn)
  if (h->cold_split && split_call_fits(h, T)) {
    HIP_TRY(moe::launch_ffn(h, x, slot_ids, w, T, shared_record, y, residual, x_next, nullptr, 0.f, s));
    return MOE_OK;
  }
  const size_t es = h->dtype == MOE_F32 ? 4 : 2;
  // the call's record indices and activations to the host, then the GPU's share of the FFN; in split
  // mode on a stream of their own from the ensure on, so the host's share runs beside the copy kernel
  // (on the side stream only after an ensure that recorded its event; otherwise in stream order)
  hipStream_t ds = h->cold_split && h->ens_recorded ? h->cold_stream : s;
  if (ds != s) HIP_TRY(hipStreamWaitEvent(ds, h->ens_ev, 0));
  h->ens_recorded = false;
  HIP_TRY(hipMemcpyAsync(h->cold_sid, slot_ids, 4 * (size_t)T * h->k, hipMemcpyDeviceToHost, ds));
  HIP_TRY(hipMemcpyAsync(h->cold_x, x, es * (size_t)T * h->H, hipMemcpyDeviceToHost, ds));
  HIP_TRY(hipEventRecord(h->cold_ev, ds));
  HIP_TRY(moe::launch_ffn(h, x, slot_ids, w, T, shared_record, y, residual, x_next, nullptr, 0.f, s, false, false));
  HIP_TRY(hipEventSynchronize(h->cold_ev));
  // the host's share meanwhile, into the mapped output rows
  moe::HostFfnJob job;
  job.host = h->host;
  job.stride = h->record_stride;
  job.dtype = h->dtype;
  job.H = h->H;
  job.F = h->F;
  job.x = h->cold_x;
  job.T = T;
  job.k = h->k;
  job.sid = h->cold_sid;
  job.S = h->S;
  job.E = h->E;
  job.out = h->cold_out;
  moe::host_cold_ffn(job);
  HIP_TRY(moe::launch_cold_combine(h, x, slot_ids, w, T, shared_record, y, residual, x_next, s));
  return MOE_OK;
}

int moe_slot_ffn_noalloc(moe_offload* h, const void* x, const int32_t* slot_ids, const float* w, int32_t T,
                         const void* shared_record, void* y, const void* residual, void* x_next, void* stream) {
  if (int rc = check_handle(h)) return rc;
  if (int rc = check_T(h, T)) return rc;
  if (!x || !slot_ids || !w || !y) return fail(MOE_EINVAL, "moe_slot_ffn_noalloc: null pointer");
  size_t need = 0;
  (void)moe::ffn_work_in(h, T, nullptr, &need);
  if (need > moe::kScratchBytes)
    return fail(MOE_EINVAL, "moe_slot_ffn_noalloc: T=%d needs %zu bytes of workspace, the device scratch holds %zu",
                T, need, (size_t)moe::kScratchBytes);
  void* base = moe::scratch_ptr(h->device);
  if (!base) return fail(MOE_EHIP, "moe_slot_ffn_noalloc: no device scratch address for device %d", h->device);
  DeviceGuard g(h->device);
  const moe::FfnWork ws = moe::ffn_work_in(h, T, base, nullptr);
  HIP_TRY(moe::launch_ffn(h, x, slot_ids, w, T, shared_record, y, residual, x_next, nullptr, 0.f,
                          (hipStream_t)stream, false, true, false, &ws));
  return MOE_OK;
}

int moe_rmsnorm(const void* x, void* out, int32_t T, int32_t H, int32_t dtype, float eps, void* stream) {
  if (!x || !out) return fail(MOE_EINVAL, "moe_rmsnorm: null pointer");
  if (T < 1 || H < 8 || H % 8) return fail(MOE_EINVAL, "moe_rmsnorm: T=%d, H=%d (H must be a multiple of 8)", T, H);
  if (!known_dtype(dtype)) return fail(MOE_EUNSUPPORTED, "moe_rmsnorm: dtype %d", dtype);
  if (!(eps > 0.0f)) return fail(MOE_EINVAL, "moe_rmsnorm: eps must be positive");
  HIP_TRY(moe::launch_rmsnorm(x, out, T, H, dtype, eps, (hipStream_t)stream));
  return MOE_OK;
}

int moe_prefill_stage(moe_offload* h, const int32_t* ids, int32_t T, int32_t* slot_ids, int32_t* staged_out,
                      void* stream) {
  if (int rc = check_handle(h)) return rc;
  if (int rc = check_T(h, T)) return rc;
  if (!ids || !slot_ids) return fail(MOE_EINVAL, "moe_prefill_stage: null pointer");
  DeviceGuard g(h->device);
  hipStream_t s = (hipStream_t)stream;
  const int n = T * h->k;
  HIP_TRY(moe::launch_distinct(h, ids, n, h->scratch_i32, s));
  HIP_TRY(hipMemcpyAsync(h->pinned_i32, h->scratch_i32, 4, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  const int nd = h->pinned_i32[0];
  if (nd < 0) return fail(MOE_EDEVICE, "moe_prefill_stage: expert id outside [0, %d)", h->E);
  if (nd > h->S) {
    HIP_TRY(hipMemcpyAsync(h->staging, h->host, (size_t)h->E * h->record_stride, hipMemcpyHostToDevice, s));
    HIP_TRY(moe::launch_stage_all(h, ids, n, slot_ids, s));
    if (staged_out) *staged_out = 1;
  } else {
    HIP_TRY(moe::launch_ensure(h, ids, n, slot_ids, s));
    HIP_TRY(moe::launch_copy(h, h->cache.copy_list, s));
    if (staged_out) *staged_out = 0;
  }
  HIP_TRY(record_split_ensure(h, T, s));  // the indices are final
  return MOE_OK;
}

int moe_prefetch_install(moe_offload* h, const int32_t* pred_ids, int32_t T, int32_t max_n, void* stream) {
  if (int rc = check_handle(h)) return rc;
  if (int rc = check_T(h, T)) return rc;
  if (!pred_ids) return fail(MOE_EINVAL, "moe_prefetch_install: null pointer");
  if (max_n < 0 || max_n > h->S) return fail(MOE_EINVAL, "max_n=%d outside [0, S=%d]", max_n, h->S);
  DeviceGuard g(h->device);
  HIP_TRY(moe::launch_install(h, pred_ids, T, max_n, (hipStream_t)stream));
  return MOE_OK;
}

int moe_offload_pin(moe_offload* h, const int32_t* experts, int32_t n, void* stream) {
  if (int rc = check_handle(h)) return rc;
  if (n < 0 || n > h->S - h->k) return fail(MOE_EINVAL, "moe_offload_pin: n=%d outside [0, S - k = %d]", n, h->S - h->k);
  if (n > 0 && !experts) return fail(MOE_EINVAL, "moe_offload_pin: null pointer");
  DeviceGuard g(h->device);
  HIP_TRY(moe::launch_pin(h, experts, n, (hipStream_t)stream));
  HIP_TRY(moe::launch_copy(h, h->cache.copy_list, (hipStream_t)stream));
  h->n_pinned = n;
  return MOE_OK;
}

int moe_copy_prefetch(moe_offload* h, void* stream) {
  if (int rc = check_handle(h)) return rc;
  DeviceGuard g(h->device);
  HIP_TRY(moe::launch_copy(h, h->cache.pf_list, (hipStream_t)stream));
  return MOE_OK;
}

int moe_offload_set_ffn_path(moe_offload* h, int32_t path) {
  if (int rc = check_handle(h)) return rc;
  if (path != MOE_FFN_AUTO && path != MOE_FFN_DECODE && path != MOE_FFN_GEMM)
    return fail(MOE_EINVAL, "moe_offload_set_ffn_path: path %d", path);
  h->ffn_path = path;
  return MOE_OK;
}

int moe_offload_set_gemm_waves(moe_offload* h, int32_t waves) {
  if (int rc = check_handle(h)) return rc;
  if (waves != 0 && waves != 4 && waves != 8)
    return fail(MOE_EINVAL, "moe_offload_set_gemm_waves: waves %d (0, 4 or 8)", waves);
  h->gemm_waves = waves;
  return MOE_OK;
}

// the host side's buffers and the split mode's stream and events, once (the device must be current)
static int cold_buffers(moe_offload* h) {
  if (h->cold_stream) return MOE_OK;
  const size_t es = h->dtype == MOE_F32 ? 4 : 2;
  if (!h->cold_sid) HIP_TRY(hipHostMalloc((void**)&h->cold_sid, 4 * (size_t)h->max_tokens * h->k, hipHostMallocDefault));
  if (!h->cold_x) HIP_TRY(hipHostMalloc(&h->cold_x, es * (size_t)h->max_tokens * h->H, hipHostMallocDefault));
  if (!h->cold_out) {
    HIP_TRY(hipHostMalloc((void**)&h->cold_out, 4 * (size_t)h->max_tokens * h->k * h->H,
                          hipHostMallocMapped | hipHostMallocCoherent));
    HIP_TRY(hipHostGetDevicePointer((void**)&h->cold_out_dev, h->cold_out, 0));
  }
  if (!h->cold_ev) HIP_TRY(hipEventCreateWithFlags(&h->cold_ev, hipEventDisableTiming));
  if (!h->ens_ev) HIP_TRY(hipEventCreateWithFlags(&h->ens_ev, hipEventDisableTiming));
  HIP_TRY(hipStreamCreateWithFlags(&h->cold_stream, hipStreamNonBlocking));
  return MOE_OK;
}

int moe_offload_set_cold(moe_offload* h, int32_t mode, void* stream, int32_t* chosen, double* cpu_us,
                         double* link_us) {
  if (int rc = check_handle(h)) return rc;
  if (mode != MOE_COLD_OFF && mode != MOE_COLD_ON && mode != MOE_COLD_AUTO && mode != MOE_COLD_SPLIT)
    return fail(MOE_EINVAL, "moe_offload_set_cold: mode %d", mode);
  DeviceGuard g(h->device);
  hipStream_t s = (hipStream_t)stream;
  if (cpu_us) *cpu_us = 0.0;
  if (link_us) *link_us = 0.0;
  if (mode != MOE_COLD_OFF)
    if (int rc = cold_buffers(h)) return rc;
  int on = mode == MOE_COLD_ON;
  if (mode == MOE_COLD_AUTO || mode == MOE_COLD_SPLIT) {
    // one record's FFN on the host at one token, against one record over the link (a pinned
    // host-to-device copy into staging); the median of three records, each touched once
    HIP_TRY(hipStreamSynchronize(s));
    const int reps = std::min(3, h->E);
    double cpu[3] = {0, 0, 0}, link[3] = {0, 0, 0};
    memset(h->cold_x, 0, (h->dtype == MOE_F32 ? 4 : 2) * (size_t)h->H);
    hipEvent_t a = nullptr, b = nullptr;
    HIP_TRY(hipEventCreate(&a));
    hipError_t e = hipEventCreate(&b);
    for (int r = 0; r < reps && e == hipSuccess; ++r) {
      const int ex = h->E - 1 - r;  // records the calls of this layer are least likely to have touched
      h->cold_sid[0] = h->S + h->E + ex;
      moe::HostFfnJob job;
      job.host = h->host;
      job.stride = h->record_stride;
      job.dtype = h->dtype;
      job.H = h->H;
      job.F = h->F;
      job.x = h->cold_x;
      job.T = 1;
      job.k = 1;
      job.sid = h->cold_sid;
      job.S = h->S;
      job.E = h->E;
      job.out = h->cold_out;
      const auto t0 = std::chrono::steady_clock::now();
      moe::host_cold_ffn(job);
      cpu[r] = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
      e = hipEventRecord(a, s);
      if (e == hipSuccess)
        e = hipMemcpyAsync(h->staging + (size_t)(r % h->E) * h->record_stride, h->host + (size_t)ex * h->record_stride,
                           h->record_bytes, hipMemcpyHostToDevice, s);
      if (e == hipSuccess) e = hipEventRecord(b, s);
      if (e == hipSuccess) e = hipEventSynchronize(b);
      float ms = 0.f;
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
      link[r] = 1e3 * ms;
    }
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    if (e != hipSuccess) return hip_fail(e, "moe_offload_set_cold: calibration");
    std::sort(cpu, cpu + reps);
    std::sort(link, link + reps);
    const double c_us = cpu[reps / 2], l_us = link[reps / 2];
    if (cpu_us) *cpu_us = c_us;
    if (link_us) *link_us = l_us;
    on = c_us < l_us;
    if (mode == MOE_COLD_SPLIT) {
      const int q = (int)std::lround(256.0 * l_us / (c_us + l_us));
      if (chosen) *chosen = q;
      return moe_offload_set_split(h, q, stream);
    }
  }
  HIP_TRY(moe::launch_set_cold(h, on ? moe::kColdAll : 0, s));
  h->cold_on = on != 0;
  h->cold_split = false;
  if (chosen) *chosen = on;
  return MOE_OK;
}

int moe_offload_set_split(moe_offload* h, int32_t q, void* stream) {
  if (int rc = check_handle(h)) return rc;
  if (q < 0 || q > 256) return fail(MOE_EINVAL, "moe_offload_set_split: q=%d outside [0, 256]", q);
  DeviceGuard g(h->device);
  if (int rc = cold_buffers(h)) return rc;
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(moe::launch_set_cold(h, moe::kColdSplit | (q << 8), s));
  HIP_TRY(hipStreamSynchronize(s));
  h->cold_on = true;
  h->cold_split = true;
  return MOE_OK;
}

int moe_offload_stats(moe_offload* h, moe_stats* out) {
  if (int rc = check_handle(h)) return rc;
  if (!out) return fail(MOE_EINVAL, "null stats");
  DeviceGuard g(h->device);
  HIP_TRY(hipDeviceSynchronize());
  uint64_t c[moe::C_N];
  uint64_t tick = 0;
  int32_t err = 0;
  HIP_TRY(hipMemcpy(c, h->cache.counters, sizeof c, hipMemcpyDeviceToHost));
  HIP_TRY(hipMemcpy(&tick, h->cache.tick, 8, hipMemcpyDeviceToHost));
  HIP_TRY(hipMemcpy(&err, h->cache.err, 4, hipMemcpyDeviceToHost));
  int32_t* eo = new (std::nothrow) int32_t[h->S];
  if (!eo) return fail(MOE_ENOMEM, "stats scratch");
  hipError_t e = hipMemcpy(eo, h->cache.expert_of, 4 * (size_t)h->S, hipMemcpyDeviceToHost);
  int resident = 0;
  for (int s = 0; s < h->S; ++s) resident += eo[s] >= 0;
  delete[] eo;
  if (e != hipSuccess) return hip_fail(e, "stats copy");
  out->calls = c[moe::C_CALLS];
  out->hits = c[moe::C_HITS];
  out->misses = c[moe::C_MISSES];
  out->staged_calls = c[moe::C_STAGED_CALLS];
  out->staged_copies = c[moe::C_STAGED_COPIES];
  out->prefetch_installs = c[moe::C_PF_INSTALLS];
  out->prefetch_hits = c[moe::C_PF_HITS];
  out->bytes_copied = c[moe::C_BYTES];
  out->cold_misses = c[moe::C_COLD];
  out->tick = tick;
  out->error = err;
  out->resident = resident;
  return MOE_OK;
}

int moe_offload_reset(moe_offload* h, void* stream) {
  if (int rc = check_handle(h)) return rc;
  DeviceGuard g(h->device);
  HIP_TRY(moe::launch_reset(h, (hipStream_t)stream));
  h->n_pinned = 0;  // the reset unpins every slot
  return MOE_OK;
}

int moe_offload_profile(moe_offload* h, int32_t enable) {
  if (int rc = check_handle(h)) return rc;
  DeviceGuard g(h->device);
  if (!h->prof) {
    if (!enable) return MOE_OK;
    h->prof = new (std::nothrow) moe::Prof();
    if (!h->prof) return fail(MOE_ENOMEM, "moe_offload_profile: host allocation");
    for (auto& pair : h->prof->ev)
      for (hipEvent_t& e : pair) HIP_TRY(hipEventCreate(&e));
  }
  moe::Prof* p = h->prof;
  for (int kd = 0; kd < MOE_K_N; ++kd) HIP_TRY(moe::prof_collect(p, kd));
  if (enable) {
    for (int kd = 0; kd < MOE_K_N; ++kd) {
      p->ms[kd] = 0.0;
      p->n[kd] = 0;
    }
  }
  p->on = enable != 0;
  return MOE_OK;
}

int moe_offload_kernel_times(moe_offload* h, moe_kernel_times* out) {
  if (int rc = check_handle(h)) return rc;
  if (!out) return fail(MOE_EINVAL, "moe_offload_kernel_times: null output");
  DeviceGuard g(h->device);
  for (int kd = 0; kd < MOE_K_N; ++kd) {
    out->ms[kd] = 0.0;
    out->launches[kd] = 0;
  }
  if (!h->prof) return MOE_OK;
  for (int kd = 0; kd < MOE_K_N; ++kd) {
    HIP_TRY(moe::prof_collect(h->prof, kd));
    out->ms[kd] = h->prof->ms[kd];
    out->launches[kd] = h->prof->n[kd];
  }
  return MOE_OK;
}

int moe_offload_query(const moe_offload* h, moe_info* out) {
  if (int rc = check_handle(h)) return rc;
  if (!out) return fail(MOE_EINVAL, "null info");
  out->slot_of = h->cache.slot_of;
  out->expert_of = h->cache.expert_of;
  out->last_use = h->cache.last_use;
  out->score = h->cache.score;
  out->pinned = h->cache.pinned;
  out->act = h->cache.act;
  out->copy_list = h->cache.copy_list;
  out->prefetch_list = h->cache.pf_list;
  out->slots = h->slots;
  out->staging = h->staging;
  out->host = h->host;
  out->host_dev = h->host_dev;
  out->ffn_h = h->hbuf;
  out->ffn_part = h->part;
  out->ffn_groups = h->grp;
  out->record_bytes = h->record_bytes;
  out->record_stride = h->record_stride;
  out->E = h->E;
  out->S = h->S;
  out->H = h->H;
  out->F = h->F;
  out->k = h->k;
  out->dtype = h->dtype;
  out->max_tokens = h->max_tokens;
  out->device = h->device;
  return MOE_OK;
}

}  // extern "C"
