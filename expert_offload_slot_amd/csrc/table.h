// The per-layer LRU slot table as one workgroup sees it: the ensure step, the
// prefetch install and the pinned set.
//
// xinfer-ai 0.14.6 docs/moe_offload.md, "How it works" (Decode): look up the
// experts a call needs, pick least-recently-used slots for the misses, rewrite
// expert ids to slot ids and leave the miss list and count in device memory.
// FreeToken issue #677 ("Proposal", "Measured"): installs at usage 0, and the
// scored-eviction baseline (victims by usage score first).  npu-offload README
// (PolyStrata placement): a pinned hot set, never evicted.
// The table is only ever written by one workgroup of one kernel at a time, on
// the caller's compute stream: no atomics on shared state, no races.
#pragma once

#include "blockops.h"

namespace moe {

// victim order as one integer, ascending:
//   LRU              (occupied, last_use, slot);
//   scored           (occupied, score, last_use, slot);
//   activation-aware (occupied, used since install (last_use != 0), activations of the held expert,
//                     last_use, slot).
// last_use is a call count, below 2^32 in any run; scores and activation counts saturate at kScoreMax
// (20 bits).
constexpr uint32_t kScoreMax = (1u << 20) - 1u;
__device__ __forceinline__ uint64_t victim_key(const CacheDev& c, bool occ, uint32_t score, uint32_t act, uint64_t lu,
                                               int slot) {
  const uint64_t o = occ ? (1ull << 63) : 0ull;
  if (c.policy == kPolicyScored)
    return o | ((uint64_t)score << 43) | ((lu & ((1ull << 33) - 1)) << 10) | (uint64_t)slot;
  if (c.policy == kPolicyFreq) {
    if (!occ) return (uint64_t)slot;
    return o | (lu != 0 ? (1ull << 62) : 0ull) | ((uint64_t)act << 42) | ((lu & ((1ull << 32) - 1)) << 10) |
           (uint64_t)slot;
  }
  return o | ((lu & ((1ull << 53) - 1)) << 10) | (uint64_t)slot;
}

struct SharedTable {
  int slot_of[kMaxExperts];
  int expert_of[kMaxExperts];
  uint64_t last_use[kMaxExperts];
  uint32_t score[kMaxExperts];
  uint32_t act[kMaxExperts];  // activation count per expert
  int pinned[kMaxExperts];  // 1: never a victim (profile-guided placement)
  int flag[kMaxExperts];   // ensure: expert in D; install: tokens predicting it
  int aux[kMaxExperts];    // ensure: pairs routed to it; install: best top-k position
  int cand[kMaxExperts];   // ensure: best top-k position; install: candidate by rank
  int vic[kMaxExperts];    // victim slot by rank
  int wave[4 * kWaves];
  int bad;
  int cold;                // the layer's cold-mode word as loaded (kCold*)
  uint64_t tick;           // the table's call counter as loaded
  uint64_t cnt[C_N];       // the counters as loaded
};

// The table as one thread holds it between fetch_table and put_table.
struct TableRegs {
  int s = -1, e = -1, pin = 0;
  uint32_t sc = 0u, ac = 0u;
  uint64_t lu = 0ull, tc = 0ull;
};

// Issues this thread's loads of the table (slot_of, the slot entries, and in the
// last wavefront the call counter and the statistics) without waiting for them,
// so a caller can start other loads before put_table consumes the values.
__device__ __forceinline__ TableRegs fetch_table(const CacheDev& c) {
  const int tid = threadIdx.x, u = tid - 64 * (kWaves - 1);
  TableRegs r;
  if (tid < c.E) {
    r.s = c.slot_of[tid];
    r.ac = c.act[tid];
  }
  if (tid < c.S) {
    r.e = c.expert_of[tid];
    r.lu = c.last_use[tid];
    r.sc = c.score[tid];
    r.pin = c.pinned[tid];
  }
  if (u == 0) r.tc = *c.tick;
  if (u >= 1 && u <= C_N) r.tc = c.counters[u - 1];
  if (u == C_N + 1) r.tc = (uint64_t)(uint32_t)*c.cold;
  return r;
}

// Writes the fetched table to LDS.  Entries outside their range (only possible
// if the table was overwritten from outside) are dropped and flagged, so every
// later index stays in bounds.
__device__ __forceinline__ void put_table(const CacheDev& c, const TableRegs& r, SharedTable& t) {
  const int tid = threadIdx.x, u = tid - 64 * (kWaves - 1);
  if (tid < c.E) {
    int s = r.s;
    if (s < -1 || s >= c.S) {
      atomicOr(c.err, MOE_DEV_ERR_AUDIT);
      s = -1;
    }
    t.slot_of[tid] = s;
    t.act[tid] = r.ac;
  }
  if (tid < c.S) {
    int e = r.e;
    if (e < -1 || e >= c.E) {
      atomicOr(c.err, MOE_DEV_ERR_AUDIT);
      e = -1;
    }
    t.expert_of[tid] = e;
    t.last_use[tid] = r.lu;
    t.score[tid] = r.sc;
    t.pinned[tid] = r.pin;
  }
  if (u == 0) t.tick = r.tc;
  if (u >= 1 && u <= C_N) t.cnt[u - 1] = r.tc;
  if (u == C_N + 1) t.cold = (int)(uint32_t)r.tc;
}

// Loads the table into LDS (fetch_table, then put_table).
__device__ __forceinline__ void load_table(const CacheDev& c, SharedTable& t) { put_table(c, fetch_table(c), t); }

__device__ __forceinline__ void store_table(const CacheDev& c, const SharedTable& t) {
  const int tid = threadIdx.x;
  if (tid < c.E) {
    c.slot_of[tid] = t.slot_of[tid];
    c.act[tid] = t.act[tid];
  }
  if (tid < c.S) {
    c.expert_of[tid] = t.expert_of[tid];
    c.last_use[tid] = t.last_use[tid];
    c.score[tid] = t.score[tid];
    c.pinned[tid] = t.pinned[tid];
  }
}

// Audit: maps mutually inverse (and, for ensure, every expert of D resident).
__device__ __forceinline__ void audit_table(const CacheDev& c, const SharedTable& t, bool check_D) {
  const int tid = threadIdx.x;
  bool bad = false;
  if (tid < c.S) {
    const int e = t.expert_of[tid];
    if (e >= c.E || (e >= 0 && t.slot_of[e] != tid)) bad = true;
  }
  if (tid < c.E) {
    const int s = t.slot_of[tid];
    if (s >= c.S || (s >= 0 && t.expert_of[s] != tid)) bad = true;
    if (check_D && t.flag[tid] && s < 0) bad = true;
  }
  if (bad) atomicOr(c.err, MOE_DEV_ERR_AUDIT);
}

// Ensure for the n = T*k expert ids of a call (ids may live in LDS or global
// memory).  The table must already be in `t` (load_table, then a barrier).
// Writes the record index of every id to slot_ids (global) and, if given, to
// slot_lds.  Record index r < S is slot r; r >= S is staging record r - S.
//   victims:  slots not pinned and not holding an expert of D, in (free
//             first, then least recently used, then lowest slot) order
//             (scored: least used before least recently used; activation-aware:
//             installed-unused, then least activated, before least recently used);
//   misses <= victims: the misses in ascending id take the victims;
//   misses >  victims (no pins: |D| > S): the misses claim the victims in
//             install order (pairs routed to it desc, best top-k position asc,
//             id asc) and the rest are copied to staging record S + e for
//             this call (mode STAGED);
//   every expert of D holding a slot gets last_use = tick; the copy list holds
//   the misses in ascending id with their record index;
//   an id outside [0, E): nothing changes, slot ids are 0, error bit set.
// keys: LDS scratch of 2 * kMaxExperts entries.  All threads of the block must
// call it; it ends with the table stored back.
__device__ __forceinline__ void ensure_body(const CacheDev& c, SharedTable& t, const int32_t* ids, int n, int k,
                                            int32_t* __restrict__ slot_ids, int32_t* slot_lds, int audit,
                                            uint64_t* keys) {
  const int tid = threadIdx.x;
  const int E = c.E, S = c.S;
  uint64_t* vkey = keys;
  uint64_t* ckey = keys + kMaxExperts;
  if (tid < E) t.flag[tid] = 0;
  if (tid == 0) t.bad = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kBlock) {
    const int e = ids[i];
    if ((unsigned)e >= (unsigned)E) t.bad = 1;
    else t.flag[e] = 1;
  }
  __syncthreads();
  if (t.bad) {  // no-op call: table untouched, empty copy list, valid (0) slot ids
    for (int i = tid; i < n; i += kBlock) {
      slot_ids[i] = 0;
      if (slot_lds) slot_lds[i] = 0;
    }
    if (tid == 0) {
      atomicOr(c.err, MOE_DEV_ERR_BAD_ID);
      c.copy_list[0] = MOE_MODE_SLOTS;
      c.copy_list[1] = 0;
    }
    return;  // block-uniform
  }
  if (audit) audit_table(c, t, false);
  const uint64_t tick = t.tick + 1;
  const bool inD = tid < E && t.flag[tid];
  const int sl = tid < E ? t.slot_of[tid] : -1;
  const bool f[4] = {inD, inD && sl < 0, inD && sl >= 0, inD && sl >= 0 && t.last_use[sl] == 0};
  const bool miss = f[1];
  int rk[4], tot[4];
  block_rank4(f, t.wave, rk, tot);
  const int mrank = rk[1], nm = tot[1], nh = tot[2], npf = tot[3];

  if (t.cold == kColdAll) {  // host-computed cold experts: nothing loads, misses are read at S + E + e
    if (inD && sl >= 0) {
      const uint32_t old = t.score[sl];
      t.last_use[sl] = tick;
      t.score[sl] = old < kScoreMax ? old + 1 : old;
    }
    if (inD && t.act[tid] < kScoreMax) t.act[tid] += 1;
    if (miss) {
      c.copy_list[2 + 2 * mrank] = tid;
      c.copy_list[3 + 2 * mrank] = S + E + tid;
    }
    __syncthreads();
    for (int i = tid; i < n; i += kBlock) {
      const int e = ids[i];
      const int r = t.slot_of[e];
      const int v = r >= 0 ? r : S + E + e;
      slot_ids[i] = v;
      if (slot_lds) slot_lds[i] = v;
    }
    store_table(c, t);
    if (audit) audit_table(c, t, false);
    if (tid == 0) {
      c.copy_list[0] = MOE_MODE_COLD;
      c.copy_list[1] = nm;
      *c.tick = tick;
      c.counters[C_CALLS] = t.cnt[C_CALLS] + 1;
      c.counters[C_HITS] = t.cnt[C_HITS] + (uint64_t)nh;
      c.counters[C_PF_HITS] = t.cnt[C_PF_HITS] + (uint64_t)npf;
      c.counters[C_COLD] = t.cnt[C_COLD] + (uint64_t)nm;
    }
    return;  // block-uniform
  }

  // eligible victims by rank: slots not pinned and not holding an expert of D;
  // the call overflows when the misses outnumber them (no pins: when |D| > S)
  bool over = false;
  int ns = 0;      // misses that get a slot
  int n_host = 0;  // split mode: staged misses handed to the host
  if (nm > 0) {
    bool elig = false;
    if (tid < S) {
      const int ex = t.expert_of[tid];
      const bool occ = ex >= 0;
      elig = !t.pinned[tid] && (!occ || !t.flag[ex]);
      vkey[tid] = elig ? victim_key(c, occ, t.score[tid], occ ? t.act[ex] : 0u, t.last_use[tid], tid) : ~0ull;
    }
    int nv;
    (void)block_rank(elig, t.wave, &nv);  // its barriers also publish vkey
    ns = nm < nv ? nm : nv;
    over = nm > nv;  // block-uniform
    if (over) {  // install-order key of each miss: pairs routed to it, best top-k position, id
      if (tid < E) {
        t.aux[tid] = 0;
        t.cand[tid] = k;
      }
      __syncthreads();
      for (int i = tid; i < n; i += kBlock) {
        const int e = ids[i];
        atomicAdd(&t.aux[e], 1);
        atomicMin(&t.cand[e], i % k);
      }
      __syncthreads();
      if (tid < E)
        ckey[tid] = miss ? ((uint64_t)(0xfffffu - (uint32_t)t.aux[tid]) << 40) | ((uint64_t)t.cand[tid] << 20) |
                               (uint64_t)tid
                         : ~0ull;
    }
    if (elig) {
      const uint64_t mine = vkey[tid];
      int rank = 0;
#pragma unroll 8
      for (int s2 = 0; s2 < S; ++s2) rank += vkey[s2] < mine ? 1 : 0;
      t.vic[rank] = tid;  // rank < nv
    }
    __syncthreads();
    int v = -1;
    bool staged = false;
    if (miss) {
      int crank = mrank;  // claim order: ascending id, or install order when over
      if (over) {
        const uint64_t mine = ckey[tid];
        crank = 0;
#pragma unroll 8
        for (int e2 = 0; e2 < E; ++e2) crank += ckey[e2] < mine ? 1 : 0;
      }
      v = S + tid;
      if (crank < ns) {
        v = t.vic[crank];
        const int old = t.expert_of[v];
        if (old >= 0) t.slot_of[old] = -1;
        t.expert_of[v] = tid;
        t.slot_of[tid] = v;
      }
      staged = crank >= ns;
    }
    if (over && (t.cold & 0xff) == kColdSplit) {  // block-uniform
      // the host's share q/256 of all the call's misses, from the staged ones (the last in ascending id)
      int nst;
      const int srank = block_rank(staged, t.wave, &nst);
      n_host = min(nst, (nm * (t.cold >> 8) + 128) >> 8);
      if (staged && srank >= nst - n_host) {
        v = S + E + tid;
        t.flag[tid] = 2;
      }
    }
    if (miss) {
      c.copy_list[2 + 2 * mrank] = tid;
      c.copy_list[3 + 2 * mrank] = v;
    }
    __syncthreads();
  }
  if (inD && t.slot_of[tid] >= 0) {  // used now; a slot just loaded starts from 0
    const int s = t.slot_of[tid];
    const uint32_t old = miss ? 0u : t.score[s];
    t.last_use[s] = tick;
    t.score[s] = old < kScoreMax ? old + 1 : old;
  }
  if (inD && t.act[tid] < kScoreMax) t.act[tid] += 1;  // every routed expert, resident or staged
  __syncthreads();
  for (int i = tid; i < n; i += kBlock) {
    const int e = ids[i];
    const int r = t.slot_of[e];
    const int v = r >= 0 ? r : (t.flag[e] == 2 ? S + E + e : S + e);
    slot_ids[i] = v;
    if (slot_lds) slot_lds[i] = v;
  }
  store_table(c, t);
  if (audit) audit_table(c, t, !over);
  if (tid == 0) {
    c.copy_list[0] = over ? MOE_MODE_STAGED : MOE_MODE_SLOTS;
    c.copy_list[1] = nm;
    *c.tick = tick;
    c.counters[C_CALLS] = t.cnt[C_CALLS] + 1;
    c.counters[C_HITS] = t.cnt[C_HITS] + (uint64_t)nh;
    c.counters[C_MISSES] = t.cnt[C_MISSES] + (uint64_t)ns;
    c.counters[C_PF_HITS] = t.cnt[C_PF_HITS] + (uint64_t)npf;
    c.counters[C_BYTES] = t.cnt[C_BYTES] + (uint64_t)(nm - n_host) * c.record_bytes;
    if (over) {
      c.counters[C_STAGED_CALLS] = t.cnt[C_STAGED_CALLS] + 1;
      c.counters[C_STAGED_COPIES] = t.cnt[C_STAGED_COPIES] + (uint64_t)(nm - ns - n_host);
      if (n_host) c.counters[C_COLD] = t.cnt[C_COLD] + (uint64_t)n_host;
    }
  }
}

// Prefetch install (FreeToken issue #677, "Proposal", Install) for the n = T*k
// predicted ids of a call (pred may live in LDS or global memory).  The table
// must already be in `t` (load_table, then a barrier).
//   candidates: predicted experts that are not resident, in (tokens predicting
//               it desc, best top-k position asc, id asc) order;
//   victims:    slots not holding a predicted expert, in ensure's order;
//   the first min(max_n, candidates, victims) pairs are installed with
//   last_use = 0 (evicted first) and written to the prefetch copy list.
// ckey: LDS scratch of E entries, vkey: of S entries.  All threads of the block
// must call it; it ends with the table stored back.
__device__ __forceinline__ void install_body(const CacheDev& c, SharedTable& t, const int32_t* pred, int n, int k,
                                             int max_n, int audit, uint64_t* ckey, uint64_t* vkey) {
  const int tid = threadIdx.x;
  const int E = c.E, S = c.S;
  if (tid < E) {
    t.flag[tid] = 0;  // tokens predicting the expert
    t.aux[tid] = k;   // best top-k position
  }
  if (tid == 0) t.bad = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kBlock) {
    const int e = pred[i];
    if ((unsigned)e >= (unsigned)E) {
      t.bad = 1;
    } else {
      atomicAdd(&t.flag[e], 1);
      atomicMin(&t.aux[e], i % k);
    }
  }
  __syncthreads();
  if (t.bad) {
    if (tid == 0) {
      atomicOr(c.err, MOE_DEV_ERR_BAD_ID);
      c.pf_list[0] = MOE_MODE_SLOTS;
      c.pf_list[1] = 0;
    }
    return;  // block-uniform
  }
  // candidate key, ascending = install order (count < 2^20, position < 16, id < 1024)
  const bool cand = tid < E && t.flag[tid] > 0 && t.slot_of[tid] < 0;
  if (tid < E)
    ckey[tid] = cand ? ((uint64_t)(0xfffffu - (uint32_t)t.flag[tid]) << 40) | ((uint64_t)t.aux[tid] << 20) |
                           (uint64_t)tid
                     : ~0ull;
  bool elig = false;
  if (tid < S) {
    const int ex = t.expert_of[tid];
    const bool occ = ex >= 0;
    elig = !t.pinned[tid] && (!occ || t.flag[ex] == 0);
    vkey[tid] = elig ? victim_key(c, occ, t.score[tid], occ ? t.act[ex] : 0u, t.last_use[tid], tid) : ~0ull;
  }
  int nc, nv;
  (void)block_rank(cand, t.wave, &nc);  // its barriers also publish ckey / vkey
  (void)block_rank(elig, t.wave, &nv);
  int m = max_n < nc ? max_n : nc;
  m = m < nv ? m : nv;
  if (cand) {
    const uint64_t mine = ckey[tid];
    int crank = 0;
#pragma unroll 8
    for (int e2 = 0; e2 < E; ++e2) crank += ckey[e2] < mine ? 1 : 0;
    if (crank < m) t.cand[crank] = tid;
  }
  if (elig) {
    const uint64_t mine = vkey[tid];
    int vrank = 0;
#pragma unroll 8
    for (int s2 = 0; s2 < S; ++s2) vrank += vkey[s2] < mine ? 1 : 0;
    if (vrank < m) t.vic[vrank] = tid;
  }
  __syncthreads();
  if (tid < m) {
    const int e = t.cand[tid], v = t.vic[tid];
    const int old = t.expert_of[v];
    if (old >= 0) t.slot_of[old] = -1;
    t.expert_of[v] = e;
    t.slot_of[e] = v;
    t.last_use[v] = 0;
    t.score[v] = 0;
    c.pf_list[2 + 2 * tid] = e;
    c.pf_list[3 + 2 * tid] = v;
  }
  __syncthreads();
  store_table(c, t);
  if (audit) audit_table(c, t, false);
  if (tid == 0) {
    c.pf_list[0] = MOE_MODE_SLOTS;
    c.pf_list[1] = m;
    c.counters[C_PF_INSTALLS] = t.cnt[C_PF_INSTALLS] + (uint64_t)m;
    c.counters[C_BYTES] = t.cnt[C_BYTES] + (uint64_t)m * c.record_bytes;
  }
}

// Profile-guided placement: pin the n distinct experts of P (device ids,
// replacing the pinned set).  Members already resident are pinned in place;
// the others, ascending id, take victims in the ensure order among slots not
// pinned and not holding a member, with last_use = the current tick (the clock
// does not advance) and score 0.  The copy list gets {SLOTS, loads, (expert,
// slot)...}.  An id out of range or repeated: nothing changes, empty list,
// error bit.  keys: LDS scratch of kMaxExperts entries.
__device__ __forceinline__ void pin_body(const CacheDev& c, SharedTable& t, const int32_t* P, int n,
                                         uint64_t* vkey) {
  const int tid = threadIdx.x;
  const int E = c.E, S = c.S;
  if (tid < E) t.flag[tid] = 0;
  if (tid == 0) t.bad = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kBlock) {
    const int e = P[i];
    if ((unsigned)e >= (unsigned)E || atomicAdd(&t.flag[e], 1) != 0) t.bad = 1;
  }
  __syncthreads();
  if (t.bad) {
    if (tid == 0) {
      atomicOr(c.err, MOE_DEV_ERR_BAD_ID);
      c.copy_list[0] = MOE_MODE_SLOTS;
      c.copy_list[1] = 0;
    }
    return;  // block-uniform
  }
  if (tid < S) t.pinned[tid] = 0;
  __syncthreads();
  if (tid < E && t.flag[tid] && t.slot_of[tid] >= 0) t.pinned[t.slot_of[tid]] = 1;
  __syncthreads();
  const bool miss = tid < E && t.flag[tid] && t.slot_of[tid] < 0;
  bool elig = false;
  if (tid < S) {
    const int ex = t.expert_of[tid];
    const bool occ = ex >= 0;
    elig = !t.pinned[tid] && (!occ || !t.flag[ex]);
    vkey[tid] = elig ? victim_key(c, occ, t.score[tid], occ ? t.act[ex] : 0u, t.last_use[tid], tid) : ~0ull;
  }
  int nm, nv;
  const int mrank = block_rank(miss, t.wave, &nm);  // its barriers also publish vkey
  (void)block_rank(elig, t.wave, &nv);
  const int nl = nm < nv ? nm : nv;  // nm <= nv for n <= S
  if (elig) {
    const uint64_t mine = vkey[tid];
    int rank = 0;
#pragma unroll 8
    for (int s2 = 0; s2 < S; ++s2) rank += vkey[s2] < mine ? 1 : 0;
    t.vic[rank] = tid;
  }
  __syncthreads();
  if (miss && mrank < nl) {
    const int v = t.vic[mrank];
    const int old = t.expert_of[v];
    if (old >= 0) t.slot_of[old] = -1;
    t.expert_of[v] = tid;
    t.slot_of[tid] = v;
    t.last_use[v] = t.tick;
    t.score[v] = 0;
    t.pinned[v] = 1;
    c.copy_list[2 + 2 * mrank] = tid;
    c.copy_list[3 + 2 * mrank] = v;
  }
  __syncthreads();
  store_table(c, t);
  if (tid == 0) {
    c.copy_list[0] = MOE_MODE_SLOTS;
    c.copy_list[1] = nl;
    c.counters[C_BYTES] = t.cnt[C_BYTES] + (uint64_t)nl * c.record_bytes;
  }
}

}  // namespace moe
