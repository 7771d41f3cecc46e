// Test shim: exposes the library's host-CPU expert FFN (csrc/host_ffn.cpp, built
// from the same source by the CPU tests) to ctypes.  Test infrastructure only.
#include <stdint.h>

#include "host_ffn.h"

extern "C" int shim_host_cold_ffn(const uint8_t* host, uint64_t stride, int dtype, int H, int F, const void* x, int T,
                                  int k, const int32_t* sid, int S, int E, float* out) {
  moe::HostFfnJob j;
  j.host = host;
  j.stride = stride;
  j.dtype = dtype;
  j.H = H;
  j.F = F;
  j.x = x;
  j.T = T;
  j.k = k;
  j.sid = sid;
  j.S = S;
  j.E = E;
  j.out = out;
  moe::host_cold_ffn(j);
  return moe::host_threads();
}
