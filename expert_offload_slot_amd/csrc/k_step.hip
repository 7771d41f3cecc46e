// Decode control step in one workgroup: top-k, slot ensure and FFN grouping.
//
// xinfer-ai 0.14.6 docs/moe_offload.md, "How it works" (Decode): between the
// router and the expert GEMMs a decode step looks up the chosen experts in the
// layer's slot table, assigns LRU slots to the misses, rewrites ids to slot ids
// and leaves the miss list on the device, all without a host round trip.
//
// The three steps are the ones the separate entry points run (topk.h,
// table.h, grouping.h); here they share one 1024-thread workgroup so a decode
// layer pays one launch and no global round trip between them: wavefront w
// selects for tokens w, w + 16, ..., the ids stay in LDS for the ensure, and
// the record indices stay in LDS for the counting sort.  The slot table load
// is issued first and is in flight during the top-k.  In the lookahead variant
// the same workgroup then selects the next layer's predicted experts (its
// router on this layer's input) and installs them into the next layer's table
// (table.h, install_body): every table write stays on the compute stream.
#include <algorithm>

#include "grouping.h"
#include "prof.h"
#include "table.h"
#include "topk.h"

namespace moe {
namespace {

// key scratch of ensure (victims) and install (candidates, victims) next to the top-k scratch
constexpr int kDecideKeys = 2 * kMaxExperts;

template <int J>
__global__ __launch_bounds__(kBlock) void k_decide(CacheDev c, const float* __restrict__ logits, int T, int k,
                                                   int32_t* __restrict__ ids, float* __restrict__ w,
                                                   int32_t* __restrict__ slot_ids, int32_t* __restrict__ grp,
                                                   int off_pairs, int off_tiles, int do_group, int audit,
                                                   CacheDev nc,
                                                   int audit_next,
                                                   const float* __restrict__ pred_logits,
                                                   int32_t* __restrict__ pred, int max_n) {
  __shared__ SharedTable t;
  __shared__ union {
    GroupShared g;
    TopkScratch tk[kWaves];
    uint64_t keys[kDecideKeys];
  } u;
  __shared__ int ids_l[kDecideMaxPairs];
  __shared__ float w_l[kDecideMaxPairs];
  __shared__ int rec_l[kDecideMaxPairs];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = T * k;
  const TableRegs tr = fetch_table(c);  // in flight while the top-k reads the logits
  for (int tok = wv; tok < T; tok += kWaves) {
    int id;
    float wt;
    const bool nan = wave_topk<J>(logits + (size_t)tok * c.E, c.E, k, u.tk[wv], &id, &wt);
    if (nan && lane == 0) atomicOr(c.err, MOE_DEV_ERR_NAN);
    if (lane < k) {
      ids_l[tok * k + lane] = id;
      w_l[tok * k + lane] = wt;
    }
  }
  // the table's values before any global store (the wait for a load also
  // waits for the stores issued before it); the top-k results are written
  // out after the ensure for the same reason
  put_table(c, tr, t);
  __syncthreads();
  ensure_body(c, t, ids_l, n, k, slot_ids, rec_l, audit, u.keys);
  __syncthreads();
  // host-computed pairs (index S + E + e, cold and split mode) stay out of every record list
  if (do_group) group_body(rec_l, n, c.S + c.E, grp, off_pairs, off_tiles, c.err, u.g, c.S + 2 * c.E);
  for (int i = threadIdx.x; i < n; i += kBlock) {
    ids[i] = ids_l[i];
    w[i] = w_l[i];
  }
  if (max_n <= 0) return;  // uniform
  // lookahead: the next layer's router on this layer's input predicts its experts;
  // up to max_n of them are installed into the next layer's table
  __syncthreads();
  for (int tok = wv; tok < T; tok += kWaves) {
    int id;
    float wt;
    const bool nan = wave_topk<J>(pred_logits + (size_t)tok * nc.E, nc.E, k, u.tk[wv], &id, &wt);
    if (nan && lane == 0) atomicOr(nc.err, MOE_DEV_ERR_NAN);
    if (lane < k) {
      pred[(size_t)tok * k + lane] = id;
      ids_l[tok * k + lane] = id;
    }
  }
  __syncthreads();
  load_table(nc, t);
  install_body(nc, t, ids_l, n, k, max_n, audit_next, u.keys, u.keys + kMaxExperts);
}

}  // namespace

hipError_t launch_decide(moe_offload* h, int T, int32_t* ids, float* w, int32_t* slot_ids, hipStream_t s,
                         moe_offload* hn, int32_t* pred, int max_n) {
  if (T * h->k > kDecideMaxPairs) return hipErrorInvalidValue;
  if (max_n > 0 && (!hn || !pred || hn->k != h->k || T > hn->max_tokens)) return hipErrorInvalidValue;
  const int E = max_n > 0 ? std::max(h->E, hn->E) : h->E;
  const int J = topk_lanes(E);
  auto kd = J == 1 ? k_decide<1> : J == 2 ? k_decide<2> : J == 4 ? k_decide<4> : J == 8 ? k_decide<8> : k_decide<16>;
  const int audit = (h->flags & MOE_FLAG_AUDIT) ? 1 : 0;
  // a single token's FFN reads its k distinct records straight from slot_ids (launch_ffn)
  const int do_group = T == 1 && h->dtype != MOE_F32 ? 0 : 1;
  const CacheDev nc = max_n > 0 ? hn->cache : h->cache;
  const int audit_next = max_n > 0 && (hn->flags & MOE_FLAG_AUDIT) ? 1 : 0;
  launch_k(h, MOE_K_DECIDE, kd, dim3(1), dim3(kBlock), 0, s, h->cache, h->logits, T, h->k, ids, w, slot_ids, h->grp,
           h->gl.off_pairs(), h->gl.off_tiles(), do_group, audit, nc, audit_next, max_n > 0 ? hn->logits : h->logits, pred,
           max_n);
  return hipGetLastError();
}

}  // namespace moe
