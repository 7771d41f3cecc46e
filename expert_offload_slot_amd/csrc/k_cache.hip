// Per-layer LRU slot table on the GPU: ensure (lookup, victims, id rewrite,
// copy list, counters), prefetch install, the pinned set, whole-layer
// staging, reset, and the copy kernel that moves records from device-mapped
// pinned host memory.
//
// xinfer-ai 0.14.6 docs/moe_offload.md, "How it works" (Decode, Prefill);
// FreeToken issue #677, "Proposal" (Install, Correctness constraint).
//
// The table is only ever written by one workgroup of one kernel at a time,
// on the caller's compute stream: no atomics on shared state, no races.
#include "prof.h"
#include "table.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- ensure
__global__ __launch_bounds__(kBlock) void k_ensure(CacheDev c, const int32_t* __restrict__ ids, int n, int k,
                                                   int32_t* __restrict__ slot_ids, int audit) {
  __shared__ SharedTable t;
  __shared__ uint64_t keys[2 * kMaxExperts];
  load_table(c, t);
  ensure_body(c, t, ids, n, k, slot_ids, nullptr, audit, keys);
}

// ---------------------------------------------------------------- prefetch install
__global__ __launch_bounds__(kBlock) void k_install(CacheDev c, const int32_t* __restrict__ pred, int n, int k,
                                                    int max_n, int audit) {
  __shared__ SharedTable t;
  __shared__ uint64_t ckey[kMaxExperts];
  __shared__ uint64_t vkey[kMaxExperts];
  load_table(c, t);
  install_body(c, t, pred, n, k, max_n, audit, ckey, vkey);
}

// ---------------------------------------------------------------- profile-guided placement
__global__ __launch_bounds__(kBlock) void k_pin(CacheDev c, const int32_t* __restrict__ P, int n) {
  __shared__ SharedTable t;
  __shared__ uint64_t vkey[kMaxExperts];
  load_table(c, t);
  pin_body(c, t, P, n, vkey);
}

// ---------------------------------------------------------------- prefill helpers
// distinct ids of a call; -1 if any id is outside [0, E)
__global__ __launch_bounds__(kBlock) void k_distinct(int E, const int32_t* __restrict__ ids, int n, int32_t* out) {
  __shared__ int flag[kMaxExperts];
  __shared__ int wave[kWaves];
  __shared__ int bad;
  const int tid = threadIdx.x;
  if (tid < E) flag[tid] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kBlock) {
    const int e = ids[i];
    if ((unsigned)e >= (unsigned)E) bad = 1;
    else flag[e] = 1;
  }
  __syncthreads();
  int nd;
  (void)block_rank(tid < E && flag[tid], wave, &nd);
  if (tid == 0) *out = bad ? -1 : nd;
}

// whole-layer staging: ids -> S + id, copy list {STAGED_ALL, E, (e, S+e)}, tick and counters
__global__ void k_stage_all(CacheDev c, const int32_t* __restrict__ ids, int n, int32_t* __restrict__ slot_ids) {
  const int i0 = blockIdx.x * blockDim.x + threadIdx.x, step = gridDim.x * blockDim.x;
  for (int i = i0; i < n; i += step) slot_ids[i] = c.S + ids[i];
  for (int e = i0; e < c.E; e += step) {
    c.copy_list[2 + 2 * e] = e;
    c.copy_list[3 + 2 * e] = c.S + e;
  }
  if (i0 == 0) {
    c.copy_list[0] = MOE_MODE_STAGED_ALL;
    c.copy_list[1] = c.E;
    *c.tick += 1;
    c.counters[C_CALLS] += 1;
    c.counters[C_STAGED_CALLS] += 1;
    c.counters[C_STAGED_COPIES] += (uint64_t)c.E;
    c.counters[C_BYTES] += (uint64_t)c.E * c.record_bytes;
  }
}

// empty cache, zero counters and error, empty lists
__global__ void k_reset(CacheDev c) {
  const int i0 = blockIdx.x * blockDim.x + threadIdx.x, step = gridDim.x * blockDim.x;
  for (int e = i0; e < c.E; e += step) {
    c.slot_of[e] = -1;
    c.act[e] = 0;
  }
  for (int s = i0; s < c.S; s += step) {
    c.expert_of[s] = -1;
    c.last_use[s] = 0;
    c.score[s] = 0;
    c.pinned[s] = 0;
  }
  for (int i = i0; i < C_N; i += step) c.counters[i] = 0;
  if (i0 == 0) {
    *c.tick = 0;
    *c.err = 0;
    c.copy_list[0] = MOE_MODE_SLOTS;
    c.copy_list[1] = 0;
    c.pf_list[0] = MOE_MODE_SLOTS;
    c.pf_list[1] = 0;
  }
}

// the layer's cold-mode word, written in stream order like the table itself
__global__ void k_set_cold(int32_t* cold, int word) {
  if (threadIdx.x == 0) *cold = word;
}

// ---------------------------------------------------------------- copy
// Fixed grid; the list (mode, count, pairs) is read on the device.  Each
// workgroup moves 16 KiB chunks: 256 threads x 4 loads of 16 bytes in flight,
// read from the device-mapped host store over the host link, written to HBM.
__global__ __launch_bounds__(kCopyThreads) void k_copy(const int32_t* __restrict__ list,
                                                      const uint8_t* __restrict__ host, uint8_t* __restrict__ slots,
                                                      uint8_t* __restrict__ staging, uint64_t stride, uint64_t rb16,
                                                      int S, int E, int32_t* err) {
  const int mode = list[0];
  const int count = list[1];
  if (mode == MOE_MODE_STAGED_ALL || mode == MOE_MODE_COLD || count <= 0) return;  // cold experts never move
  constexpr uint64_t CH = (uint64_t)kCopyThreads * kCopyUnroll;
  const uint64_t per = (rb16 + CH - 1) / CH;
  const uint64_t total = (uint64_t)count * per;
  for (uint64_t cidx = blockIdx.x; cidx < total; cidx += gridDim.x) {
    const int m = (int)(cidx / per);
    const uint64_t off = (cidx - (uint64_t)m * per) * CH;
    const int e = list[2 + 2 * m], r = list[3 + 2 * m];
    if (r >= S + E && r < S + 2 * E) continue;  // split mode: computed on the host, never moved
    if ((unsigned)e >= (unsigned)E || (unsigned)r >= (unsigned)(S + E)) {
      if (threadIdx.x == 0) atomicOr(err, MOE_DEV_ERR_AUDIT);
      continue;
    }
    const uint4* src = reinterpret_cast<const uint4*>(host + (uint64_t)e * stride) + off;
    uint8_t* dbase = r < S ? slots + (uint64_t)r * stride : staging + (uint64_t)(r - S) * stride;
    uint4* dst = reinterpret_cast<uint4*>(dbase) + off;
    const uint64_t lim = rb16 - off;
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const uint64_t i = (uint64_t)u * kCopyThreads + threadIdx.x;
      if (i < lim) v[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const uint64_t i = (uint64_t)u * kCopyThreads + threadIdx.x;
      if (i < lim) dst[i] = v[u];
    }
  }
}

}  // namespace

hipError_t launch_ensure(moe_offload* h, const int32_t* ids, int n, int32_t* slot_ids, hipStream_t s) {
  launch_k(h, MOE_K_ENSURE, k_ensure, dim3(1), dim3(kBlock), 0, s, h->cache, ids, n, h->k, slot_ids,
                     (h->flags & MOE_FLAG_AUDIT) ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_install(moe_offload* h, const int32_t* pred, int T, int max_n, hipStream_t s) {
  launch_k(h, MOE_K_INSTALL, k_install, dim3(1), dim3(kBlock), 0, s, h->cache, pred, T * h->k, h->k, max_n,
                     (h->flags & MOE_FLAG_AUDIT) ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_distinct(moe_offload* h, const int32_t* ids, int n, int32_t* out_dev, hipStream_t s) {
  launch_k(h, MOE_K_STAGE, k_distinct, dim3(1), dim3(kBlock), 0, s, h->E, ids, n, out_dev);
  return hipGetLastError();
}

hipError_t launch_stage_all(moe_offload* h, const int32_t* ids, int n, int32_t* slot_ids, hipStream_t s) {
  launch_k(h, MOE_K_STAGE, k_stage_all, dim3(64), dim3(256), 0, s, h->cache, ids, n, slot_ids);
  return hipGetLastError();
}

hipError_t launch_pin(moe_offload* h, const int32_t* experts, int n, hipStream_t s) {
  launch_k(h, MOE_K_ENSURE, k_pin, dim3(1), dim3(kBlock), 0, s, h->cache, experts, n);
  return hipGetLastError();
}

hipError_t launch_set_cold(moe_offload* h, int word, hipStream_t s) {
  hipLaunchKernelGGL(k_set_cold, dim3(1), dim3(64), 0, s, h->cache.cold, word);
  return hipGetLastError();
}

hipError_t launch_reset(moe_offload* h, hipStream_t s) {
  hipLaunchKernelGGL(k_reset, dim3(16), dim3(256), 0, s, h->cache);
  return hipGetLastError();
}

hipError_t launch_copy(moe_offload* h, const int32_t* list, hipStream_t s) {
  launch_k(h, list == h->cache.pf_list ? MOE_K_PF_COPY : MOE_K_COPY, k_copy, dim3(kCopyGrid), dim3(kCopyThreads), 0,
           s, list, h->host_dev, h->slots, h->staging,
           // whole 16-byte units: the record stride is a multiple of 4096, so rounding
           // the record up stays inside its own stride on both sides
           (uint64_t)h->record_stride, (uint64_t)((h->record_bytes + 15) / 16), h->S, h->E, h->cache.err);
  return hipGetLastError();
}

}  // namespace moe
