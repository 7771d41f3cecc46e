// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_offload.h"

namespace moe {

constexpr int kMaxExperts = 1024;   // one ensure thread per expert
constexpr int kMaxTopK = 16;
constexpr int kCopyGrid = 256;      // copy kernel: fixed grid (one workgroup per CU)
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;      // 16-byte loads in flight per thread
constexpr int kRouteTokens = 4;     // tokens per router wave
constexpr int kTile = 16;           // MFMA output rows per work item
constexpr int kChunk = 128;         // K elements per MFMA group (4 x 32)
constexpr int kTokGroup = 64;       // tokens per pass over a weight tile (4 MFMA column groups)
constexpr int kF32Rows = 64;        // rows per work item on the fp32 path

// counters[] layout (device, uint64)
enum { C_CALLS = 0, C_HITS, C_MISSES, C_STAGED_CALLS, C_STAGED_COPIES, C_PF_INSTALLS, C_PF_HITS, C_BYTES, C_N };

// Device view of one layer's slot table and copy lists.
struct CacheDev {
  int32_t* slot_of;     // [E]
  int32_t* expert_of;   // [S]
  uint64_t* last_use;   // [S]
  uint64_t* tick;       // [1]
  int32_t* copy_list;   // [2 + 2*max(S,E)]
  int32_t* pf_list;     // [2 + 2*S]
  uint64_t* counters;   // [C_N]
  int32_t* err;         // [1] sticky MOE_DEV_ERR_* bits
  int E, S;
  uint64_t record_bytes;
};

// FFN group descriptor offsets (int32 words) inside the FFN workspace
struct GroupLayout {
  int max_recs;   // distinct records a call can touch
  int max_pairs;  // max_tokens * k
  int off_list() const { return 2; }
  int off_start() const { return 2 + max_recs; }
  int off_pairs() const { return 2 + max_recs + max_recs + 1; }
  int words() const { return off_pairs() + max_pairs; }
};

}  // namespace moe

struct moe_offload {
  int E, S, H, F, k, dtype, max_tokens, device;
  uint32_t flags;
  size_t record_bytes, record_stride;

  uint8_t* host;       // pinned host store [E, stride]
  uint8_t* host_dev;   // its device address
  bool own_host;
  uint8_t* slots;      // device [S, stride]
  uint8_t* staging;    // device [E, stride]
  bool own_staging;

  void* state_block;   // one allocation holding everything below
  moe::CacheDev cache;
  float* logits;       // [max_tokens, E]
  uint32_t* route_ctr; // [ceil(max_tokens / kRouteTokens)]
  int32_t* grp;        // FFN group descriptor
  moe::GroupLayout gl;
  void* hbuf;          // [max_pairs + max_tokens, F] bf16 (fp32 for MOE_F32)
  float* part;         // [max_pairs + max_tokens, H] fp32 partial expert outputs
  uint32_t* comb_ctr;  // [H / 16] combine counters
  int32_t* scratch_i32;      // small device scratch (distinct count etc.)
  int32_t* pinned_i32;       // small pinned host scratch
};

namespace moe {

// launchers (return hipError_t of the launch)
hipError_t launch_reset(moe_offload* h, hipStream_t s);
hipError_t launch_route(moe_offload* h, const void* x, const void* wr, const float* bias, int T, int32_t* ids,
                        float* w, hipStream_t s);
hipError_t launch_ensure(moe_offload* h, const int32_t* ids, int n, int32_t* slot_ids, hipStream_t s);
hipError_t launch_install(moe_offload* h, const int32_t* pred, int T, int max_n, hipStream_t s);
hipError_t launch_copy(moe_offload* h, const int32_t* list, hipStream_t s);
hipError_t launch_distinct(moe_offload* h, const int32_t* ids, int n, int32_t* out_dev, hipStream_t s);
hipError_t launch_stage_all(moe_offload* h, const int32_t* ids, int n, int32_t* slot_ids, hipStream_t s);
hipError_t launch_ffn(moe_offload* h, const void* x, const int32_t* slot_ids, const float* w, int T,
                      const void* shared, void* y, void* x_next, hipStream_t s);

}  // namespace moe
