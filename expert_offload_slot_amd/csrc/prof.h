// Opt-in per-kernel timing.  While a handle's profiling is on, its kernels are
// launched with hipExtLaunchKernelGGL and a start/stop event pair, which the
// runtime records with the kernel's own dispatch (no separate marker packets);
// launches on a stream that is being captured into a graph are not timed.
#pragma once

#include <hip/hip_ext.h>

#include "internal.h"

namespace moe {

struct Prof {
  bool on = false;
  hipEvent_t ev[MOE_K_N][2] = {};
  bool pending[MOE_K_N] = {};
  double ms[MOE_K_N] = {};
  uint64_t n[MOE_K_N] = {};
};

// adds the kind's pending pair to the sums (waits for its stop event)
inline hipError_t prof_collect(Prof* p, int kind) {
  if (!p->pending[kind]) return hipSuccess;
  p->pending[kind] = false;
  hipError_t e = hipEventSynchronize(p->ev[kind][1]);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, p->ev[kind][0], p->ev[kind][1]);
  if (e == hipSuccess) {
    p->ms[kind] += ms;
    p->n[kind] += 1;
  }
  return e;
}

// true: time this launch with the kind's event pair
inline bool prof_begin(moe_offload* h, int kind, hipStream_t s) {
  Prof* p = h->prof;
  if (!p || !p->on) return false;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess || st != hipStreamCaptureStatusNone) return false;
  return prof_collect(p, kind) == hipSuccess;
}

// Launches kern<<<g, b, shm, s>>>(args...) for handle h as kernel kind `kind`.
template <typename F, typename... Args>
inline void launch_k(moe_offload* h, int kind, F kern, dim3 g, dim3 b, uint32_t shm, hipStream_t s, Args... args) {
  if (prof_begin(h, kind, s)) {
    hipExtLaunchKernelGGL(kern, g, b, shm, s, h->prof->ev[kind][0], h->prof->ev[kind][1], 0, args...);
    h->prof->pending[kind] = true;
  } else {
    hipLaunchKernelGGL(kern, g, b, shm, s, args...);
  }
}

}  // namespace moe
