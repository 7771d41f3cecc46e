// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_offload.h"

namespace moe {

constexpr int kMaxExperts = 1024;   // one ensure thread per expert
constexpr int kMaxTopK = 16;
constexpr int kCopyGrid = 64;       // copy kernel: fixed grid; 48+ workgroups already fill the host link
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;      // 16-byte loads in flight per thread
constexpr int kRouteTokens = 4;     // tokens per router wave
constexpr int kF32Rows = 64;        // rows per work item on the fp32 path

// victim orders of the slot table (table.h victim_key)
constexpr int kPolicyLru = 0, kPolicyScored = 1, kPolicyFreq = 2;
// the layer's cold-mode word: 0 off; kColdAll: every miss is computed on the host;
// kColdSplit | q << 8: an overflowing call computes min(staged, round(misses * q / 256))
// of its staged misses (the last in ascending id) on the host, the rest crosses the link
constexpr int kColdAll = 1, kColdSplit = 2;

// counters[] layout (device, uint64)
enum { C_CALLS = 0, C_HITS, C_MISSES, C_STAGED_CALLS, C_STAGED_COPIES, C_PF_INSTALLS, C_PF_HITS, C_BYTES, C_COLD, C_N };

// Device view of one layer's slot table and copy lists.
struct CacheDev {
  int32_t* slot_of;     // [E]
  int32_t* expert_of;   // [S]
  uint64_t* last_use;   // [S]
  uint32_t* score;      // [S] usage score (scored eviction)
  uint32_t* act;        // [E] activation count per expert (activation-aware eviction)
  int32_t* pinned;      // [S] 1: never a victim (profile-guided placement)
  uint64_t* tick;       // [1]
  int32_t* copy_list;   // [2 + 2*max(S,E)]
  int32_t* pf_list;     // [2 + 2*S]
  uint64_t* counters;   // [C_N]
  int32_t* err;         // [1] sticky MOE_DEV_ERR_* bits
  int32_t* cold;        // [1] the cold-mode word (kColdAll, kColdSplit | q << 8); host-computed index S + E + e
  int E, S;
  int policy;           // victim order: kPolicyLru, kPolicyScored, kPolicyFreq (table.h)
  uint64_t record_bytes;
};

// FFN group descriptor (int32 words) inside the FFN workspace:
//   [0]                      number of distinct records nr
//   record block r (32 words, 128-byte aligned) at kRecWords * (1 + r):
//     [0] record index, [1] token count n, [2] offset of its pair ids in the
//     pair array, [3 .. 3 + kInline) its first kInline pair ids (t*k + j)
//   pair array at kRecWords * (1 + max_recs): all pair ids grouped by record
//   tile starts at off_tiles(): record r's first prefill-GEMM tile, and the
//     total at index nr (the prefill GEMM's work list)
// so a work item gets its record and (usually all) its tokens in one load trip.
constexpr int kRecWords = 32;
constexpr int kInline = kRecWords - 3;
// A record's n pairs form prefill-GEMM tiles of kGemmTok pairs, except the last,
// which takes up to kGemmTail: a record of 65 to 80 pairs is one tile, not a
// full one and a nearly empty one that reads all its weights again.
constexpr int kGemmTok = 64;
constexpr int kGemmTail = 80;
__host__ __device__ constexpr inline int gemm_tile_count(int n) {
  return n <= 0 ? 0 : (n <= kGemmTail ? 1 : 1 + (n - kGemmTail + kGemmTok - 1) / kGemmTok);
}
struct GroupLayout {
  int max_recs;   // distinct records a call can touch
  int max_pairs;  // max_tokens * k
  int off_rec(int r) const { return kRecWords * (1 + r); }
  int off_pairs() const { return kRecWords * (1 + max_recs); }
  int off_tiles() const { return off_pairs() + max_pairs; }
  int words() const { return off_tiles() + max_recs + 1; }
};

struct Prof;  // prof.h

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
  int32_t* grp;        // FFN group descriptor
  moe::GroupLayout gl;
  void* hbuf;          // [max_pairs + max_tokens, F] bf16 (fp32 for MOE_F32)
  float* part;         // [max_pairs + max_tokens, H] fp32 partial expert outputs
  int32_t* scratch_i32;      // small device scratch (distinct count etc.)
  int32_t* pinned_i32;       // small pinned host scratch
  moe::Prof* prof;           // per-kernel timing, created on first enable
  int ffn_path;              // MOE_FFN_AUTO / DECODE / GEMM (moe_offload_set_ffn_path)
  int gemm_waves;            // 0 (by the call's size), 4 or 8 (moe_offload_set_gemm_waves)
  int n_pinned;              // size of the pinned set (moe_offload_pin)
  // host-computed cold experts (allocated when the cold mode is first switched on)
  bool cold_on;              // host mirror of the device word: nonzero
  bool cold_split;           // ... and in split mode (the copies run beside the host's share)
  hipStream_t cold_stream;   // split mode: the call's indices and activations go to the host on it
  hipEvent_t ens_ev;         // split mode: recorded after an ensure whose call may overflow (the indices are final)
  bool ens_recorded;         // ... and the last ensure did record it (the FFN's host path then waits on it)
  int32_t* cold_sid;         // pinned host [max_tokens * k]: the call's record indices
  void* cold_x;              // pinned host [max_tokens * H]: the call's activations
  float* cold_out;           // pinned, mapped, coherent host [max_tokens * k][H]: cold pairs' outputs
  float* cold_out_dev;       // its device address
  hipEvent_t cold_ev;        // the call's indices and activations have reached the host
};

namespace moe {

// records the message returned by moe_offload_last_error() on this thread; returns code
int set_error(int code, const char* msg);

// launchers (return hipError_t of the launch)
hipError_t launch_reset(moe_offload* h, hipStream_t s);
// h->logits = x . wr^T + bias; with hn, also hn->logits = x . wrn^T + biasn in the same launch
hipError_t launch_logits(moe_offload* h, const void* x, const void* wr, const float* bias, int T, hipStream_t s,
                         moe_offload* hn = nullptr, const void* wrn = nullptr, const float* biasn = nullptr);
// The previous layer's top-k combine (y, residual, next norm), taken into this
// layer's router launch in the decode chain (bf16 activations, H <= 8192, one
// token per workgroup): every workgroup forms its token's normalised input in
// LDS in the combine's own order; workgroup 0 of each token writes y, x_next
// and xn_next.
struct CombineSrc {
  const float* part;     // [T*k (+T)][H] fp32 expert outputs of the previous layer
  const float* w;        // [T][k] its routing weights
  int T, k, shared;      // shared: rows T*k + t hold the shared expert's output
  void* y;               // [T][H] previous layer output
  const void* residual;  // [T][H] its input stream x_l
  void* x_next;          // [T][H] x_{l+1} = round(x_l + y)
  void* xn_next;         // [T][H] rmsnorm(x_{l+1}): this layer's router and expert input
  float eps;
};
constexpr int kFusedCombineMaxH = 8192;
hipError_t launch_combine_logits(moe_offload* h, const CombineSrc& cb, const void* wr, const float* bias, int T,
                                 hipStream_t s, moe_offload* hn = nullptr, const void* wrn = nullptr,
                                 const float* biasn = nullptr);
hipError_t launch_route(moe_offload* h, const void* x, const void* wr, const float* bias, int T, int32_t* ids,
                        float* w, hipStream_t s);
hipError_t launch_ensure(moe_offload* h, const int32_t* ids, int n, int32_t* slot_ids, hipStream_t s);
hipError_t launch_install(moe_offload* h, const int32_t* pred, int T, int max_n, hipStream_t s);
hipError_t launch_pin(moe_offload* h, const int32_t* experts, int n, hipStream_t s);
hipError_t launch_copy(moe_offload* h, const int32_t* list, hipStream_t s);
hipError_t launch_distinct(moe_offload* h, const int32_t* ids, int n, int32_t* out_dev, hipStream_t s);
hipError_t launch_stage_all(moe_offload* h, const int32_t* ids, int n, int32_t* slot_ids, hipStream_t s);
// xn_next (optional, needs x_next): rmsnorm(x_next) with eps, for the next layer of a chain;
// grouped: the group descriptor for slot_ids was already built (launch_decide)
// combine = false: stop after the down projection (the chain takes the combine into the next router launch)
// fill: where ffn_reads_through(h, T), the records of the copy list are read from the host store and
// written to their slots by the FFN itself (the caller then launches no copy for the call)
// The FFN workspace of one call: the group descriptor (layout from GroupLayout),
// the h rows [T*k + T][F] and the fp32 partial outputs [T*k + T][H].  Null in
// launch_ffn: the handle's own workspace (sized for max_tokens at create).
struct FfnWork {
  int32_t* grp;
  void* hbuf;
  float* part;
  GroupLayout gl;
};
hipError_t launch_ffn(moe_offload* h, const void* x, const int32_t* slot_ids, const float* w, int T,
                      const void* shared, void* y, const void* residual, void* x_next, void* xn_next, float eps,
                      hipStream_t s, bool grouped = false, bool combine = true, bool fill = false,
                      const FfnWork* ws = nullptr);

// File-scope device scratch for callers that cannot allocate (k_ffn.hip).
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
// Once per device, with that device current: looks up the scratch array's device
// address (hipGetSymbolAddress) and keeps it; later calls return at once.
hipError_t scratch_init(int device);
// The device address kept by scratch_init (null before it succeeded on `device`).
void* scratch_ptr(int device);
// The FFN workspace of a call of T tokens carved from `base` (any 256-aligned
// device buffer); *bytes gets its size.
FfnWork ffn_work_in(const moe_offload* h, int T, void* base, size_t* bytes);
bool ffn_reads_through(const moe_offload* h, int T);
// true when a call of T tokens runs the grouped GEMM rather than the decode kernels
bool ffn_uses_gemm(const moe_offload* h, int T);
// Decode control step in one workgroup: top-k of h->logits (launch_logits first),
// ensure, and the FFN grouping.  With hn (max_n > 0): also the top-k of
// hn->logits (the lookahead prediction, ids to pred) and the prefetch install
// of up to max_n experts into hn.  Needs T * k <= kDecideMaxPairs.
constexpr int kDecideMaxPairs = 512;
hipError_t launch_decide(moe_offload* h, int T, int32_t* ids, float* w, int32_t* slot_ids, hipStream_t s,
                         moe_offload* hn = nullptr, int32_t* pred = nullptr, int max_n = 0);
hipError_t launch_rmsnorm(const void* x, void* out, int T, int H, int dtype, float eps, hipStream_t s);
// the layer's cold-mode flag on the device (ordered on s with the table's other writers)
hipError_t launch_set_cold(moe_offload* h, int word, hipStream_t s);
// part rows of the call's cold pairs (record index >= S + E) from h->cold_out, then the combine
hipError_t launch_cold_combine(moe_offload* h, const void* x, const int32_t* slot_ids, const float* w, int T,
                               const void* shared, void* y, const void* residual, void* x_next, hipStream_t s);
// the top-k weighted combine of h->part alone (residual, and the next norm when xn_next is given),
// as launch_ffn ends it
hipError_t launch_combine(moe_offload* h, const void* x, const float* w, int T, const void* shared, void* y,
                          const void* residual, void* x_next, void* xn_next, float eps, hipStream_t s);

}  // namespace moe
