// Host-CPU expert FFN for cold experts (host_ffn.cpp).  Plain C++ types only, so
// both the host compiler and hipcc can include it.
#pragma once

#include <stdint.h>

namespace moe {

struct HostFfnJob {
  const uint8_t* host;  // host store [E][stride] (host address)
  uint64_t stride;
  int dtype, H, F;
  const void* x;        // host [T][H] activations (fp32 for MOE_F32, bf16 otherwise)
  int T, k;
  const int32_t* sid;   // host [T*k] record indices of the call; S + E + e marks a cold expert e
  int S, E;
  float* out;           // host [T*k][H]: the rows of the cold pairs are written (fp32), others untouched
};

// Computes out[p] = Wd_e (silu(Wg_e x_t) * (Wu_e x_t)) for every pair p = t*k + j whose record
// index is S + E + e, on the library's worker threads; returns when done.
void host_cold_ffn(const HostFfnJob& job);

// Worker threads of the host FFN (the process's CPU affinity set, the caller included).
int host_threads();

}  // namespace moe
