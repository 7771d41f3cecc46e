// Grouping of a call's (token, choice) pairs by record for the expert FFN:
// one workgroup counting-sorts the n = T*k record indices into the group
// descriptor (internal.h, GroupLayout) that the FFN work items read, with each
// record's first prefill-GEMM tile (a prefix sum of gemm_tile_count(count)).
#pragma once

#include "blockops.h"

namespace moe {

struct GroupShared {
  int cnt[2 * kMaxExperts];
  int cur[2 * kMaxExperts];
  int rank_of[2 * kMaxExperts];
  int wave[kWaves];
};

// rec[i] (LDS or global) is the record index of pair i = t*k + j, in [0, nb).
// An index in [nb, cold_hi) names a cold expert computed on the host: the pair
// is left out of every record list.  Any other index outside [0, nb) is flagged
// (audit bit) and treated as record 0.
// All threads of the block must call it.  The order of the pairs inside a
// record's list is not fixed, and nothing downstream depends on it.
__device__ __forceinline__ void group_body(const int32_t* rec, int n, int nb, int32_t* __restrict__ grp,
                                           int off_pairs, int off_tiles, int32_t* err, GroupShared& g,
                                           int cold_hi = 0) {
  const int tid = threadIdx.x;
  for (int b = tid; b < 2 * kMaxExperts; b += kBlock) g.cnt[b] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kBlock) {
    int r = rec[i];
    if (r >= nb && r < cold_hi) continue;  // a cold expert: computed on the host
    if ((unsigned)r >= (unsigned)nb) {
      atomicOr(err, MOE_DEV_ERR_AUDIT);
      r = 0;
    }
    atomicAdd(&g.cnt[r], 1);
  }
  __syncthreads();
  const int c0 = g.cnt[2 * tid], c1 = g.cnt[2 * tid + 1];
  int tot_pairs, nr;
  const int pre = block_excl_sum(c0 + c1, g.wave, &tot_pairs);
  const int pre_nz = block_excl_sum((c0 > 0) + (c1 > 0), g.wave, &nr);
  const int t0 = gemm_tile_count(c0), t1 = gemm_tile_count(c1);
  int tot_tiles;
  const int pre_t = block_excl_sum(t0 + t1, g.wave, &tot_tiles);
  int32_t* tiles = grp + off_tiles;
  if (c0 > 0) tiles[pre_nz] = pre_t;
  if (c1 > 0) tiles[pre_nz + (c0 > 0)] = pre_t + t0;
  if (tid == 0) tiles[nr] = tot_tiles;
  int32_t* pairs = grp + off_pairs;
  // cnt now holds each record's start in the pair array, cur its cursor
  g.cnt[2 * tid] = pre;
  g.cnt[2 * tid + 1] = pre + c0;
  g.cur[2 * tid] = pre;
  g.cur[2 * tid + 1] = pre + c0;
  g.rank_of[2 * tid] = pre_nz;
  g.rank_of[2 * tid + 1] = pre_nz + (c0 > 0);
  if (c0 > 0) {
    int32_t* blk = grp + kRecWords * (1 + pre_nz);
    blk[0] = 2 * tid;
    blk[1] = c0;
    blk[2] = pre;
  }
  if (c1 > 0) {
    int32_t* blk = grp + kRecWords * (1 + pre_nz + (c0 > 0));
    blk[0] = 2 * tid + 1;
    blk[1] = c1;
    blk[2] = pre + c0;
  }
  if (tid == 0) grp[0] = nr;
  // blocks past the last record, up to the most a call of n pairs can have, are
  // marked empty, so decode work items can read their block without nr
  for (int r = nr + tid; r < min(n, nb); r += kBlock) grp[kRecWords * (1 + r) + 1] = 0;
  __syncthreads();
  // each pair goes to its record's list, and the first kInline of a list also
  // into the record block
  for (int i = tid; i < n; i += kBlock) {
    int r = rec[i];
    if (r >= nb && r < cold_hi) continue;
    if ((unsigned)r >= (unsigned)nb) r = 0;
    const int pos = atomicAdd(&g.cur[r], 1);
    pairs[pos] = i;
    const int q = pos - g.cnt[r];
    if (q < kInline) grp[kRecWords * (1 + g.rank_of[r]) + 3 + q] = i;
  }
}

}  // namespace moe
