// Prefetch copy helpers: extra workgroups in the decode chain's own launches
// that copy the next layer's installed (predicted) records while the host link
// would otherwise sit idle.
//
// FreeToken issue #677, "Proposal" (Lookahead, Install): the next layer's
// predicted experts are installed early and their copy overlaps the current
// layer; "Measured": the demand copies that remain are what the step waits for.
// Here the copy does not need a second stream: layer l's control workgroup
// installs into layer l+1 and resets layer l+1's chunk queue; the gate/up and
// down launches of layer l and the router launch of layer l+1 each start
// kPfHelpers helper workgroups ahead of their own work.  A helper claims 16 KiB
// chunks of the queue with an atomic counter, copies each from the
// device-mapped host store into its slot and counts it done for its record.
// Each wavefront of a helper works on its own (no barrier).  It stops when the
// queue is empty, when every workgroup of its launch's own work has finished
// (so a launch ends at most one chunk after its own work), or at once when its
// launch reads missed records through the host link itself.
// Layer l+1's ensure, a kernel boundary later, marks a record valid once all
// its chunks are done; a hit on a record still incomplete is read through
// (refilled) by that call's FFN.  Nothing waits on the device: every loop ends
// when the queue does.
#pragma once

#include "internal.h"

namespace moe {

struct PfHelp {
  const int32_t* list;    // next layer's prefetch list {mode, n, (expert, slot)...}
  uint32_t* claim;        // chunks claimed so far
  uint32_t* done;         // chunks copied per list entry
  const uint8_t* host;    // next layer's host store (device address)
  uint8_t* slots;         // next layer's slot tensor
  uint64_t stride, rb16;  // record stride (bytes), record size (16-byte units)
  int nc, S, E;           // chunks per record, next layer's slots and experts
  const uint32_t* stop;   // workgroups of this launch's own work that have finished
  uint32_t stop_at;       // ... out of
  const int32_t* busy;    // this layer's fill list (null: none): idle while it reads records through
};

// One helper workgroup: each of its wavefronts claims and copies chunks on its
// own.  Every decision is wavefront-uniform by construction (the claim and the
// stop count are read with one atomic per wavefront and broadcast from the
// first lane), so no lane of a wavefront can be left looping on a value another
// lane updates, and there is no barrier: each wavefront's loop ends after at
// most `total` claims.
__device__ __forceinline__ void pf_help(const PfHelp& p) {
  constexpr int kChunk16 = (int)(kCopyChunk / 16);  // 16-byte units per chunk
  constexpr int kU = 4;                             // loads in flight per lane
  const int lane = threadIdx.x & 63;
  if (p.busy && __builtin_amdgcn_readfirstlane(p.busy[1]) > 0) return;  // the launch's own reads use the link
  const uint32_t total =
      (uint32_t)__builtin_amdgcn_readfirstlane(p.list[1]) * (uint32_t)p.nc;
  for (uint32_t guard = 0; guard <= total; ++guard) {
    // one atomic per wavefront: the lanes add 1 (lane 0) or 0, and lane 0's old value is the claim
    const uint32_t stop = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(p.stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (stop >= p.stop_at || total == 0) return;  // wavefront-uniform (scalar)
    const uint32_t c = __builtin_amdgcn_readfirstlane(atomicAdd(p.claim, lane == 0 ? 1u : 0u));
    if (c >= total) return;  // wavefront-uniform (scalar)
    const int i = (int)(c / (uint32_t)p.nc);
    const uint64_t off = (uint64_t)(c - (uint32_t)i * (uint32_t)p.nc) * kChunk16;
    const int e = __builtin_amdgcn_readfirstlane(p.list[2 + 2 * i]);
    const int s = __builtin_amdgcn_readfirstlane(p.list[3 + 2 * i]);
    if ((unsigned)e < (unsigned)p.E && (unsigned)s < (unsigned)p.S) {  // wavefront-uniform
      const uint4* src = reinterpret_cast<const uint4*>(p.host + (uint64_t)e * p.stride) + off;
      uint4* dst = reinterpret_cast<uint4*>(p.slots + (uint64_t)s * p.stride) + off;
      const uint64_t lim = p.rb16 - off < (uint64_t)kChunk16 ? p.rb16 - off : (uint64_t)kChunk16;
      for (int base = 0; base < kChunk16; base += 64 * kU) {
        uint4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const uint64_t j = (uint64_t)base + (uint64_t)u * 64 + lane;
          if (j < lim) v[u] = src[j];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const uint64_t j = (uint64_t)base + (uint64_t)u * 64 + lane;
          if (j < lim) dst[j] = v[u];
        }
      }
    }
    // counted by the next layer's ensure after a kernel boundary, which orders every store above
    atomicAdd(&p.done[i], lane == 0 ? 1u : 0u);
  }
}

// End of one workgroup of a launch's own work (all its threads): lets the helpers stop.
__device__ __forceinline__ void pf_own_done(uint32_t* ctr) {
  __syncthreads();
  if (threadIdx.x == 0) atomicAdd(ctr, 1u);
}

}  // namespace moe
