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

// Host side of a decode chain with host-computed experts.  The GPU publishes each
// such layer's call (record indices and activations) into pinned host memory and
// bumps the layer's request number; a server thread computes the layer's cold
// pairs into its output rows and then stores the request number as the layer's
// done number, which the GPU waits for before it reads the rows.
struct ColdChainLayer {
  const uint8_t* host;  // the layer's host store [E][stride]
  uint64_t stride;
  int dtype, H, F, k, S, E;
};
struct ColdChainIo {    // host addresses of the pinned buffers shared with the GPU
  const int32_t* sid;   // [L][T*k] the published record indices
  const uint8_t* x;     // [L][T][H] the published activations (xrow bytes per row)
  float* out;           // [L][T*k][H] the host's rows
  const uint32_t* req;  // [L] request numbers, written by the GPU
  uint32_t* done;       // [L] done numbers, written here
};
class ColdServer;
// Starts the server thread (it polls req; after about 50 ms without a request it
// polls every 100 us).  Returns null if the thread cannot be started.
ColdServer* cold_server_start(const ColdChainLayer* layers, int L, int T, uint64_t xrow, const ColdChainIo& io);
// Stops and joins the thread.
void cold_server_stop(ColdServer* s);

}  // namespace moe
