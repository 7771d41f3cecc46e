// Grouped expert FFN over the slot tensor, with the top-k weighted combine.
//
// xinfer-ai 0.14.6 docs/moe_offload.md, "How it works": the expert GEMMs read a
// [num_slots, N, K] slot tensor instead of [num_experts, N, K]; which slot an
// expert sits in leaves the arithmetic unchanged.  Per (token t, choice j) with record r = slot_ids[t][j]:
//     h = silu(Wg x_t) * (Wu x_t),  o = Wd h,  y_t = sum_j w[t][j] o  (+ shared expert)
//
// Kernels (one launch each, fixed grids, no communication between workgroups):
//   k_group    one workgroup: counting sort of the T*k (t, j) pairs by record
//              index -> distinct records, each with its token list (the first
//              kInline pair ids inline, so one load trip serves a work item).
//              The decode chain builds the same descriptor in its control
//              workgroup instead.  A single token needs none: its k records
//              are distinct, so each (t, j) pair is its own work item.
//   gate/up + SiLU and down, one of three kernel pairs by call size
//   (ffn_uses_gemm):
//     few pairs per record, T <= kDecodeMaxT (decode): k_gateup_vec / k_down_vec, one wavefront per
//              (record, 4 or 8 weight rows); the rows are loaded once, held in
//              registers and met by every token of the record with the bf16
//              pair-dot instruction.  Few tokens per record make this a
//              weight-streaming (HBM) problem, not a matrix-core one.
//              T = 1: k_gateup_one / k_down_one, the same rows per wavefront
//              for one activation row, work item (choice j, rows).
//     larger T (prefill), or many pairs per record: k_gemm<W, GU, WV>, a grouped GEMM whose
//              work items are (tile of up to 80 pairs of one record, weight
//              rows): weights straight into registers, token rows through LDS
//              shared by the workgroup's WV = 4 or 8 wavefronts (gemm_waves),
//              bf16 MFMA 16x16x32 tiles.
//     fp32 records: plain fp32 FMA kernels, work item (record, 64 rows).
//   h is stored in bf16 (fp32 for fp32 records); down writes fp32 partial
//   outputs per (t, j) to the workspace.
//   k_combine  one workgroup per token: sum over j in order (+ shared), round,
//              residual add, and optionally the next block's RMS norm.
// fp8 records: e4m3 codes are widened exactly to bf16 by the hardware pair
// converter and each 128-wide K block is scaled on its fp32 partial sum.
// MXFP4 records: E2M1 codes are widened by the hardware scaled converter with
// their row's E8M0 block scale folded in (a power of two: the bf16 is exact).
//
// Nothing depends on which slot holds an expert, on S, or on the order of the
// tokens inside a record's list: every output element is one fixed-order sum.
#include <math.h>

#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>

#include "grouping.h"
#include "prof.h"
#include "rownorm.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte moves through a native vector: a uint4 struct copy becomes a memcpy,
// which keeps an array of them in private (scratch) memory instead of registers
__device__ __forceinline__ uint4 ld16(const void* p) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(void* p, const uint4& v) {
  *reinterpret_cast<u32x4*>(p) = u32x4{v.x, v.y, v.z, v.w};
}

struct FfnArgs {
  const void* x;
  const int32_t* slot_ids;
  const float* w;
  const uint8_t* slots;
  const uint8_t* staging;
  const uint8_t* shared;
  uint64_t stride;
  int32_t* grp;
  void* hbuf;
  float* part;
  void* y;
  const void* residual;  // stream the output is added to (x if none given)
  void* x_next;
  int32_t* err;
  int T, k, H, F, S, E;
  int off_pairs, off_tiles;
  int max_routed;  // record blocks a call can fill: min(T * k, S + E); unused ones are marked empty
  int pair_items;  // one token: its k records are distinct, so each choice is its own work item (no grouping)
  // single-token read-through: the ensure's copy list, and the device address of the host store
  // (null list: every record is read where slot_ids points)
  const int32_t* fill_list;
  const uint8_t* host;
};

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)rn_to_bf16(f); }
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// ------------------------------------------------------------------ grouping
__global__ __launch_bounds__(kBlock) void k_group(FfnArgs a) {
  __shared__ GroupShared g;
  group_body(a.slot_ids, a.T * a.k, a.S + a.E, a.grp, a.off_pairs, a.off_tiles, a.err, g, a.S + 2 * a.E);
}

// A work item's record (pointer, token count); its pair ids come from the same
// 128-byte record block, so one load trip serves the item.
struct Item {
  const uint8_t* rec;
  int n;    // tokens of the item
  bool sh;  // the always-resident shared expert
};

__device__ __forceinline__ Item item_record(const FfnArgs& a, int nr, int r) {
  Item it;
  if (r < nr) {
    const int32_t* blk = a.grp + kRecWords * (1 + r);
    const int ri = blk[0];
    it.rec = ri < a.S ? a.slots + (uint64_t)ri * a.stride : a.staging + (uint64_t)(ri - a.S) * a.stride;
    it.n = blk[1];
    it.sh = false;
  } else {
    it.rec = a.shared;
    it.n = a.T;
    it.sh = true;
  }
  return it;
}

// Record of decode work item r without the record count: blocks below
// max_routed are real or marked empty (n = 0); r == max_routed is the shared expert.
__device__ __forceinline__ Item item_block(const FfnArgs& a, int r) {
  Item it;
  if (r < a.max_routed) {
    const int32_t* blk = a.grp + kRecWords * (1 + r);
    const int ri = blk[0];
    it.n = blk[1];
    it.rec = it.n == 0 ? nullptr
                       : (ri < a.S ? a.slots + (uint64_t)ri * a.stride : a.staging + (uint64_t)(ri - a.S) * a.stride);
    it.sh = false;
  } else {
    it.rec = a.shared;
    it.n = a.T;
    it.sh = true;
  }
  return it;
}

// pair id (row of h / part) of entry idx of record r
__device__ __forceinline__ int item_pair(const FfnArgs& a, const Item& it, int r, int idx) {
  if (it.sh) return a.T * a.k + idx;
  const int32_t* blk = a.grp + kRecWords * (1 + r);
  return idx < kInline ? blk[3 + idx] : a.grp[a.off_pairs + blk[2] + idx];
}
__device__ __forceinline__ int pair_token(const FfnArgs& a, int p) {
  const int routed = a.T * a.k;
  return p < routed ? p / a.k : p - routed;
}

template <bool HI>
__device__ __forceinline__ uint32_t cvt2(uint32_t d) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d, 1.0f, HI));
}

// 16 e4m3 codes widened exactly to 16 bf16
__device__ __forceinline__ void widen16(uint4 q, uint4& lo, uint4& hi) {
  lo.x = cvt2<false>(q.x);
  lo.y = cvt2<true>(q.x);
  lo.z = cvt2<false>(q.y);
  lo.w = cvt2<true>(q.y);
  hi.x = cvt2<false>(q.z);
  hi.y = cvt2<true>(q.z);
  hi.z = cvt2<false>(q.w);
  hi.w = cvt2<true>(q.w);
}

__device__ __forceinline__ f32x4 fma4(float s, f32x4 v, f32x4 acc) {
  f32x4 r;
  r.x = __builtin_fmaf(s, v.x, acc.x);
  r.y = __builtin_fmaf(s, v.y, acc.y);
  r.z = __builtin_fmaf(s, v.z, acc.z);
  r.w = __builtin_fmaf(s, v.w, acc.w);
  return r;
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ weight formats
// Kernels with bf16 activations take the weight format W (the moe_dtype code):
//   bf16:  2 bytes per weight, no scales;
//   fp8:   e4m3 codes, an fp32 scale per 128 x 128 block of a matrix;
//   MXFP4: E2M1 codes two per byte (element 2i in the low nibble), an E8M0
//          scale (2^(e - 127)) per 32 consecutive weights of a row.
// Record = gate [F][H] | up [F][H] | down [H][F] codes, then the scales of
// gate, up, down.  Codes are widened exactly to bf16 (MXFP4 with its scale
// folded in, a power of two, so the bf16 value is exact); fp8 block scales
// multiply fp32 partial sums.
constexpr int kBf16 = MOE_BF16, kFp8 = MOE_FP8_E4M3_B128, kMx4 = MOE_MXFP4;

template <int W>
__device__ __forceinline__ uint64_t code_bytes(uint64_t n) {
  return W == kBf16 ? 2 * n : (W == kFp8 ? n : n / 2);
}

// scale base of row r of matrix m (0 gate, 1 up, 2 down; C columns):
// fp8: its 128-row block's fp32 scales; MXFP4: the row's E8M0 bytes
template <int W>
__device__ __forceinline__ const uint8_t* scale_row(const uint8_t* rec, uint64_t mat, int F, int H, int m, int r,
                                                    int C) {
  if (W == kFp8)
    return rec + 3 * mat + 4 * ((uint64_t)m * (F / 128) * (H / 128) + (uint64_t)(r / 128) * (C / 128));
  if (W == kMx4) return rec + 3 * mat + (uint64_t)m * ((uint64_t)F * H / 32) + (uint64_t)r * (C / 32);
  return rec;
}

__device__ __forceinline__ float e8m0_scale(uint32_t e) {
  return __uint_as_float(e == 0 ? 0x00400000u : (e == 255 ? 0x7fc00000u : e << 23));
}

template <int B>
__device__ __forceinline__ uint32_t cvt2_fp4(uint32_t d, float s) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, B));
}

// 16 E2M1 codes times scale s, widened to 16 bf16
__device__ __forceinline__ void widen16_fp4(uint2 q, float s, uint4& lo, uint4& hi) {
  lo.x = cvt2_fp4<0>(q.x, s);
  lo.y = cvt2_fp4<1>(q.x, s);
  lo.z = cvt2_fp4<2>(q.x, s);
  lo.w = cvt2_fp4<3>(q.x, s);
  hi.x = cvt2_fp4<0>(q.y, s);
  hi.y = cvt2_fp4<1>(q.y, s);
  hi.z = cvt2_fp4<2>(q.y, s);
  hi.w = cvt2_fp4<3>(q.y, s);
}

// ------------------------------------------------------------------ prefill GEMMs (bf16, fp8, MXFP4)
// Many tokens per record: a call becomes a grouped GEMM over record tiles.
// Work item = (tile of a record's pairs, row tile: 16 WV rows of gate and of
// up, or 32 WV rows of down, for WV wavefronts per workgroup); a record's pairs
// form tiles of kGemmTok, the last one taking up to kGemmTail
// (gemm_tile_count), and the items of a call follow the tile starts of the
// group descriptor (routed records, then the shared expert's tiles).  A
// workgroup of WV wavefronts runs an item: wavefront w owns 16 rows of gate and
// of up (32 rows of down) and every pair of the tile, so its weight fragments
// are loaded straight from memory into registers in the MFMA operand layout
// (fp8 and MXFP4 codes widened exactly to bf16 there) and are read by no other
// wavefront; only the gathered token rows go through LDS, in 128-wide K
// slices, double-buffered, and every wavefront of the workgroup reads them, so
// the more wavefronts share a tile, the fewer times its token rows are fetched
// (once per row tile).  Weights are loaded two slices
// ahead and token rows one slice ahead.  bf16 MFMA 16x16x32, fp32
// accumulation; fp8: one scale per 128 x 128 block, so one per K slice and
// matrix, multiplies the slice's partial sum.  The grid is the number of
// workgroups the device holds at once (gemm_grid_cap).
// MFMA operands: lane l supplies row (l & 15) (token l & 15 for B) and 8 K
// values of a 32-wide step; the result holds rows 4 * (l >> 4) + i and token
// l & 15.  Which 8 K values lane group g = l >> 4 supplies at step s is
// gemm_kmap(g, s), chosen per weight format so that a lane's codes for a
// slice come in whole 16-byte loads and each load instruction covers 64
// contiguous bytes of each of its 16 rows; A and B use the same map, and a
// slice's four steps cover its 128 K values once.
constexpr int kGemmK = 128;           // K per slice
constexpr int kGemmNJ = kGemmTail / 16;
constexpr int kLdsRow = kGemmK + 8;   // LDS row stride in bf16: rows start on different banks
// weight rows per row tile (gate/up: each matrix) with WV wavefronts per workgroup
__host__ __device__ constexpr int gemm_rows(bool gu, int wv) { return gu ? 16 * wv : 32 * wv; }
// LDS rows of a token slice: WV wavefronts stage 4 WV rows per load, so up to 16 rows past the
// tile's last 16-pair block are written (and never read)
constexpr int gemm_lds_rows(int wv) { return kGemmTail + 4 * wv - 16 > kGemmTail ? kGemmTail + 4 * wv - 16 : kGemmTail; }

struct GemmItem {
  Item it;
  int r;   // record block (nr = the shared expert)
  int n0;  // first pair of the tile within the record
  int w;   // pairs in the tile
  int rt;  // row tile
};

__device__ __forceinline__ GemmItem gemm_item(const FfnArgs& a, int nr, int routed_tiles, int row_tiles, int item) {
  GemmItem g;
  const int ti = item / row_tiles;
  g.rt = item - ti * row_tiles;
  int j, nt;
  if (ti < routed_tiles) {
    const int32_t* tiles = a.grp + a.off_tiles;  // strictly increasing: every record has a pair
    int lo = 0, hi = nr - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tiles[mid] <= ti) lo = mid;
      else hi = mid - 1;
    }
    g.r = lo;
    j = ti - tiles[lo];
    nt = tiles[lo + 1] - tiles[lo];
  } else {
    g.r = nr;
    j = ti - routed_tiles;
    nt = gemm_tile_count(a.T);
  }
  g.it = item_record(a, nr, g.r);
  g.n0 = j * kGemmTok;
  g.w = j == nt - 1 ? g.it.n - g.n0 : kGemmTok;
  return g;
}

__device__ __forceinline__ int gemm_tiles(const FfnArgs& a, int nr, int* routed) {
  *routed = a.grp[a.off_tiles + nr];
  return *routed + (a.shared ? gemm_tile_count(a.T) : 0);
}

// Waits until every global load the wavefront has issued has returned (s_waitcnt vmcnt(0),
// the export and LDS counters left alone).  The GEMM loop issues a slice's loads, computes the
// previous slice, and only then needs them: placed where the loop stores them, this keeps any load
// in flight across the back edge, which would make the compiler wait on the loads just issued
// inside the compute on every iteration.
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int W>
__device__ __forceinline__ int gemm_kmap(int g, int s) {
  if (W == kBf16) return 32 * s + 8 * g;                        // 4 x 16 bytes: K 32s + 8g
  if (W == kFp8) return (s & 2) * 32 + 16 * g + 8 * (s & 1);    // 2 x 16 bytes: K 16g and 64 + 16g
  return 32 * g + 8 * s;                                        // MXFP4, 16 bytes: K 32g (one scale group)
}

// one lane's codes of one 16-row weight fragment over a K slice
template <int W>
struct AFrag {
  static constexpr int N = W == kBf16 ? 4 : (W == kFp8 ? 2 : 1);
  u32x4 q[N];
  uint32_t e;  // MXFP4: the E8M0 scale byte of the lane's 32 weights
  float s;     // ... decoded by prep()

  // row: the lane's weight row (codes at K = 0); rs: MXFP4, its scale bytes
  __device__ __forceinline__ void load(const uint8_t* row, const uint8_t* rs, int k0, int g) {
    if (W == kBf16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = *reinterpret_cast<const u32x4*>(row + 2 * (k0 + gemm_kmap<W>(g, i)));
    } else if (W == kFp8) {
      q[0] = *reinterpret_cast<const u32x4*>(row + k0 + 16 * g);
      q[1] = *reinterpret_cast<const u32x4*>(row + k0 + 64 + 16 * g);
    } else {
      q[0] = *reinterpret_cast<const u32x4*>(row + (k0 + 32 * g) / 2);
      e = rs[(k0 + 32 * g) / 32];
    }
  }

  // MXFP4: decodes the scale where the slice is computed.  The empty asm makes the byte opaque up
  // to here, so the decode (and the wait for its load) is not hoisted to where the load is issued,
  // two slices earlier.
  __device__ __forceinline__ void prep() {
    if (W == kMx4) {
      asm volatile("" : "+v"(e));
      s = e8m0_scale(e);
    }
  }

  // the bf16 operand of step st
  __device__ __forceinline__ bf16x8 op(int st) const {
    u32x4 v;
    if (W == kBf16) {
      v = q[st];
    } else if (W == kFp8) {
      const u32x4 c = q[st >> 1];
      const uint32_t d0 = (st & 1) ? c.z : c.x, d1 = (st & 1) ? c.w : c.y;
      v = u32x4{cvt2<false>(d0), cvt2<true>(d0), cvt2<false>(d1), cvt2<true>(d1)};
    } else {
      const uint32_t d = q[0][st];
      v = u32x4{cvt2_fp4<0>(d, s), cvt2_fp4<1>(d, s), cvt2_fp4<2>(d, s), cvt2_fp4<3>(d, s)};
    }
    return __builtin_bit_cast(bf16x8, v);
  }
};

// One work item of NJ 16-pair blocks.  GU: gate/up over x (rows by token) into
// h = silu(gate) * up in bf16; else down over h (rows by pair) into fp32 partial outputs.
template <int W, bool GU, int WV, int NJ, bool B2 = (WV == 8)>
__device__ __forceinline__ void gemm_run(const FfnArgs& a, const GemmItem& g, uint16_t (*Bs)[gemm_lds_rows(WV)][kLdsRow]) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, lg = lane >> 4, lr = lane & 15;
  const int K = GU ? a.H : a.F, nk = K / kGemmK;
  const int m0 = g.rt * gemm_rows(GU, WV);
  const uint64_t mat = code_bytes<W>((uint64_t)a.F * a.H);
  // the wavefront's two fragments: gate and up rows m0 + 16 wv + lr, or down rows m0 + 32 wv + 16 f + lr
  const uint8_t* row[2];
  const uint8_t* rs[2];
  const float* sc[2];  // fp8: the row block's scales of the fragment's matrix, one per K slice
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int m = GU ? f : 2;
    const int r = GU ? m0 + 16 * wv + lr : m0 + 32 * wv + 16 * f + lr;
    row[f] = g.it.rec + m * mat + code_bytes<W>((uint64_t)r * K);
    rs[f] = scale_row<W>(g.it.rec, mat, a.F, a.H, m, r, K);
    // the wavefront's rows lie in one 128-row scale block; so do the tile's, unless it is taller
    const int rw = gemm_rows(GU, WV) <= 128 ? m0 : __builtin_amdgcn_readfirstlane(m0 + (GU ? 16 : 32) * wv);
    sc[f] = reinterpret_cast<const float*>(scale_row<W>(g.it.rec, mat, a.F, a.H, m, rw, K));
  }
  // the tile's token rows: 16 threads per row, 8 activations each, rows tid / 16 + RQ q for
  // the NJ 16-pair blocks.  Rows past the tile's last pair repeat that pair's row: every load is
  // issued unconditionally (the wait counts stay static), and those columns' results are never
  // stored; rows past the last block are staged and never read.
  constexpr int RQ = 4 * WV, NQ = (16 * NJ + RQ - 1) / RQ;
  static_assert(RQ * NQ <= gemm_lds_rows(WV), "token slice rows exceed the LDS buffer");
  const uint16_t* bp[NQ];
  {
    const uint16_t* base = GU ? (const uint16_t*)a.x : (const uint16_t*)a.hbuf;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int p = item_pair(a, g.it, g.r, g.n0 + min(tid / 16 + RQ * q, g.w - 1));
      bp[q] = base + (uint64_t)(GU ? pair_token(a, p) : p) * K + (tid % 16) * 8;
    }
  }
  auto load_b = [&](u32x4(&b)[NQ], int kb) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) b[q] = *reinterpret_cast<const u32x4*>(bp[q] + kb * kGemmK);
  };
  auto store_b = [&](const u32x4(&b)[NQ], int buf) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) *reinterpret_cast<u32x4*>(&Bs[buf][tid / 16 + RQ * q][(tid % 16) * 8]) = b[q];
  };
  f32x4 acc[2][NJ];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[f][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Weights run two slices ahead in three register sets whose roles rotate (the loop is unrolled
  // by three, so no set is copied while its loads are in flight); token rows run one slice ahead
  // in registers and are stored to the other LDS buffer at the end of each slice.  Every slice
  // issues the same loads (past the last slice they repeat it), so the compiler's wait counts are
  // exact: a slice's MFMAs never wait on global memory.
  AFrag<W> AX[2], AY[2], AZ[2];
  float sX[2] = {1.f, 1.f}, sY[2] = {1.f, 1.f}, sZ[2] = {1.f, 1.f};
  auto load_a = [&](AFrag<W>(&A)[2], float(&sc_)[2], int kb) {
#pragma unroll
    for (int f = 0; f < 2; ++f) A[f].load(row[f], rs[f], kb * kGemmK, lg);
    if (W == kFp8) {
      sc_[0] = sc[0][kb];
      sc_[1] = sc[1][kb];
    }
  };
  // Token rows: with B2, two slices ahead like the weights, in three register sets that rotate
  // with them (BX holds the slice that goes to LDS first); else one slice ahead in one set.
  u32x4 BX[NQ], BY[NQ], BZ[NQ];
  load_a(AX, sX, 0);
  load_a(AY, sY, min(1, nk - 1));
  load_b(BX, 0);
  if (B2) load_b(BY, min(1, nk - 1));
  wait_loads();
  __syncthreads();  // the previous item no longer reads either buffer
  store_b(BX, 0);
  __syncthreads();
  // one slice: issue the token rows of slice kb + 2 (B2; else kb + 1) into bl, then slice kb + 2's
  // weights (into ld), run slice kb from A and LDS, then store slice kb + 1's token rows (bs; with
  // B2 loaded a slice ago, else bl) into the other buffer (the one read in slice kb - 1, before the
  // last barrier)
  auto step = [&](int kb, AFrag<W>(&A)[2], const float(&s_)[2], AFrag<W>(&ld)[2], float(&sl)[2],
                  const u32x4(&bs)[NQ], u32x4(&bl)[NQ]) {
    load_b(bl, min(kb + (B2 ? 2 : 1), nk - 1));
    load_a(ld, sl, min(kb + 2, nk - 1));
    // keep the scheduler from pulling the next slice's widening into this one: that would wait on
    // loads issued a slice ago, and in order behind them on this slice's own
    __builtin_amdgcn_sched_barrier(0);
    A[0].prep();
    A[1].prep();
    const uint16_t (*B)[kLdsRow] = Bs[kb & 1];
    f32x4 part[2][NJ];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int j = 0; j < NJ; ++j) part[f][j] = W == kFp8 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[f][j];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kc = gemm_kmap<W>(lg, st);
      bf16x8 bf[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) bf[j] = *reinterpret_cast<const bf16x8*>(&B[16 * j + lr][kc]);
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const bf16x8 af = A[f].op(st);
#pragma unroll
        for (int j = 0; j < NJ; ++j) part[f][j] = mfma(af, bf[j], part[f][j]);
      }
    }
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[f][j] = W == kFp8 ? fma4(s_[f], part[f][j], acc[f][j]) : part[f][j];
    store_b(B2 ? bs : bl, (kb + 1) & 1);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  // the token-row sets in rotation (RY, RZ); without B2 every slice loads and stores the one set BX
  u32x4(&RY)[NQ] = B2 ? BY : BX;
  u32x4(&RZ)[NQ] = B2 ? BZ : BX;
  int kb = 0;
  for (; kb + 3 <= nk; kb += 3) {
    step(kb, AX, sX, AZ, sZ, RY, RZ);
    step(kb + 1, AY, sY, AX, sX, RZ, BX);
    step(kb + 2, AZ, sZ, AY, sY, BX, RY);
  }
  if (kb < nk) step(kb, AX, sX, AZ, sZ, RY, RZ);
  if (kb + 1 < nk) step(kb + 1, AY, sY, AX, sX, RZ, BX);
  wait_loads();  // the repeated loads of the last slices, before the next item reuses the registers
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int idx = 16 * j + lr;
    if (idx < g.w) {
      const int p = item_pair(a, g.it, g.r, g.n0 + idx);
      if (GU) {
        uint16_t hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = f32_to_bf16(silu_mul(acc[0][j][e], acc[1][j][e]));
        uint2 st;
        st.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
        st.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
        *reinterpret_cast<uint2*>((uint16_t*)a.hbuf + (uint64_t)p * a.F + m0 + 16 * wv + 4 * lg) = st;
      } else {
#pragma unroll
        for (int f = 0; f < 2; ++f)
          *reinterpret_cast<float4*>(a.part + (uint64_t)p * a.H + m0 + 32 * wv + 16 * f + 4 * lg) =
              make_float4(acc[f][j][0], acc[f][j][1], acc[f][j][2], acc[f][j][3]);
      }
    }
  }
}

// gate/up (GU: C[f][p] = W[f] . x[token(p)] for gate and up, h = silu(gate) * up in bf16)
// or down (part[p][r] = Wd[r] . h[p], fp32 partial outputs)
template <int W, bool GU, int WV>
__global__ __launch_bounds__(64 * WV) void k_gemm(FfnArgs a) {
  __shared__ uint16_t Bs[2][gemm_lds_rows(WV)][kLdsRow];
  const int nr = a.grp[0];
  int routed;
  const int ntiles = gemm_tiles(a, nr, &routed);
  const int RT = (GU ? a.F : a.H) / gemm_rows(GU, WV);
  for (int item = blockIdx.x; item < ntiles * RT; item += gridDim.x) {
    const GemmItem g = gemm_item(a, nr, routed, RT, item);
    switch ((g.w + 15) >> 4) {
      case 1: gemm_run<W, GU, WV, 1>(a, g, Bs); break;
      case 2: gemm_run<W, GU, WV, 2>(a, g, Bs); break;
      case 3: gemm_run<W, GU, WV, 3>(a, g, Bs); break;
      case 4: gemm_run<W, GU, WV, 4>(a, g, Bs); break;
      default: gemm_run<W, GU, WV, kGemmNJ>(a, g, Bs); break;
    }
  }
}

// ------------------------------------------------------------------ decode path (bf16, fp8, MXFP4)
// Few tokens per record: the weights are streamed once and every byte meets all
// of the record's tokens while it sits in registers.  A wavefront owns a work
// item; each 16-lane quarter owns one weight row per stream and reads it in
// coalesced pieces: lane c takes lane chunk 16*i + c of K block i, a chunk
// being 8 weights (bf16: 16 bytes, fp8: 8 bytes) or 16 MXFP4 weights (8
// bytes), so a quarter covers 256 (bf16) or 128 contiguous bytes per load.
// Products use the hardware bf16 pair dot (fp32 accumulate); fp8 codes are
// widened exactly to bf16 pairs and each 128-wide K block is scaled on its
// fp32 partial sum; MXFP4 codes are widened with their scale folded in.  The
// 16 lanes' partial sums of the (token, stream) pairs are reduced by a
// transposing butterfly that leaves pair v's sum in lane v.  Fixed order
// throughout.  The number of K blocks loaded per pass is a template parameter
// (one_chunks), so a pass is one unbroken run of loads with no bounds tests.
constexpr int kVecTok = 8;   // tokens per pass over the held weights (8 x 2 streams = 16 lanes)
constexpr int kDecodeMaxT = 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// weights per lane chunk; a K block is 16 lane chunks
template <int W>
constexpr int lane_weights() {
  return W == kMx4 ? 16 : 8;
}

// 8 bf16 weights (as 4 pairs) . 8 bf16 activations
__device__ __forceinline__ float dot8(uint4 w, uint4 x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x), __builtin_bit_cast(bf16x2, x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y), __builtin_bit_cast(bf16x2, x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z), __builtin_bit_cast(bf16x2, x.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w), __builtin_bit_cast(bf16x2, x.w), acc, false);
  return acc;
}

// 8 e4m3 weights widened to 4 bf16 pairs
__device__ __forceinline__ uint4 widen8(uint2 d) {
  uint4 u;
  u.x = cvt2<false>(d.x);
  u.y = cvt2<true>(d.x);
  u.z = cvt2<false>(d.y);
  u.w = cvt2<true>(d.y);
  return u;
}

template <int W>
struct WChunk {
  typedef uint2 T;  // fp8, MXFP4: 8 bytes
};
template <>
struct WChunk<kBf16> {
  typedef uint4 T;
};

// Weight chunks are read once per call and never again before the next layer
// has streamed its own: non-temporal loads keep them from displacing other
// lines in L2 (single-token gate/up 11.45 -> 10.79 us, down 5.84 -> 5.70 us).
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_nt __attribute__((ext_vector_type(2)));
template <int W>
__device__ __forceinline__ typename WChunk<W>::T load_w(const uint8_t* row, int kb, int c) {
  const uint8_t* p = row + (uint64_t)(16 * kb + c) * sizeof(typename WChunk<W>::T);
  if constexpr (W == kBf16) {
    const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    const u32x2_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt*>(p));
    return make_uint2(v.x, v.y);
  }
}

// the stored scale lane c applies in K block kb (srow from scale_row), as raw
// bits: fp8 the fp32 word, MXFP4 the E8M0 byte, bf16 none
template <int W>
__device__ __forceinline__ uint32_t load_sr(const uint8_t* srow, int kb, int c) {
  if (W == kFp8) return reinterpret_cast<const uint32_t*>(srow)[kb];
  if (W == kMx4) return srow[8 * kb + (c >> 1)];
  return 0u;
}

template <int W>
__device__ __forceinline__ float scale_of(uint32_t raw) {
  if (W == kFp8) return __uint_as_float(raw);
  if (W == kMx4) return e8m0_scale(raw);
  return 1.f;
}

// the scale lane c applies in K block kb
template <int W>
__device__ __forceinline__ float load_s(const uint8_t* srow, int kb, int c) {
  return scale_of<W>(load_sr<W>(srow, kb, c));
}

// Where a read-through pass writes what it reads: the two rows' codes in the
// slot, and their scales when this row is the one that owns them (fp8: the
// first row of a 128-row block, lane 0 per K block; MXFP4: every row, even
// lanes, one E8M0 byte per 32 weights).
struct Fill {
  uint8_t* w0 = nullptr;
  uint8_t* w1 = nullptr;
  uint8_t* s0 = nullptr;
  uint8_t* s1 = nullptr;
  bool own0 = false, own1 = false;
};

template <int W>
__device__ __forceinline__ void store_w(uint8_t* row, int kb, int c, typename WChunk<W>::T v) {
  *reinterpret_cast<typename WChunk<W>::T*>(row + (uint64_t)(16 * kb + c) * sizeof(typename WChunk<W>::T)) = v;
}

template <int W>
__device__ __forceinline__ void store_sr(uint8_t* srow, int kb, int c, uint32_t raw) {
  if (W == kFp8) {
    if (c == 0) reinterpret_cast<uint32_t*>(srow)[kb] = raw;
  } else if (W == kMx4) {
    if ((c & 1) == 0) srow[8 * kb + (c >> 1)] = (uint8_t)raw;
  }
}

// acc += lane chunk w (K block kb) . the matching activations of row xr
template <int W>
__device__ __forceinline__ float wdot(typename WChunk<W>::T w, const uint4* xr, int kb, int c, float acc, float s) {
  if constexpr (W == kFp8) {
    return __builtin_fmaf(s, dot8(widen8(w), xr[16 * kb + c], 0.f), acc);
  } else if constexpr (W == kMx4) {
    uint4 lo, hi;
    widen16_fp4(w, s, lo, hi);
    acc = dot8(lo, xr[2 * (16 * kb + c)], acc);
    return dot8(hi, xr[2 * (16 * kb + c) + 1], acc);
  } else {
    return dot8(w, xr[16 * kb + c], acc);
  }
}

// v[16] summed over the 16 lanes of a quarter; lane c returns the sum of v[c]
__device__ __forceinline__ float reduce16_scatter(const float v[16], int c) {
  float w8[8], w4[4], w2[2];
  const bool b3 = c & 8, b2 = c & 4, b1 = c & 2, b0 = c & 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float mine = b3 ? v[8 + i] : v[i], give = b3 ? v[i] : v[8 + i];
    w8[i] = mine + __shfl_xor(give, 8);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float mine = b2 ? w8[4 + i] : w8[i], give = b2 ? w8[i] : w8[4 + i];
    w4[i] = mine + __shfl_xor(give, 4);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float mine = b1 ? w4[2 + i] : w4[i], give = b1 ? w4[i] : w4[2 + i];
    w2[i] = mine + __shfl_xor(give, 2);
  }
  const float mine = b0 ? w2[1] : w2[0], give = b0 ? w2[0] : w2[1];
  return mine + __shfl_xor(give, 1);
}

// v summed over the 16 lanes of a quarter, every lane getting the sum: the same
// pairing tree as reduce16_scatter (bit 3, then 2, 1, 0), so the same bits.
__device__ __forceinline__ float reduce16_all(float v) {
  v += __shfl_xor(v, 8);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 2);
  return v + __shfl_xor(v, 1);
}

// Two weight rows (stream 0 at row0 / scales sr0, stream 1 at row1 / sr1) of nk
// K blocks against up to kVecTok activation rows act[t] (bf16), CH K blocks per
// pass (nk a multiple of CH); acc[t][s] gets the lane's partial sums.
template <int W, int CH>
__device__ __forceinline__ void vec_pass(const uint8_t* row0, const uint8_t* row1, const uint8_t* sr0,
                                         const uint8_t* sr1, int nk, int c, const uint16_t* const act[kVecTok],
                                         int nt, float acc[kVecTok][2]) {
  for (int k0 = 0; k0 < nk; k0 += CH) {
    typename WChunk<W>::T w0[CH], w1[CH];
    float s0[CH], s1[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      w0[i] = load_w<W>(row0, k0 + i, c);
      w1[i] = load_w<W>(row1, k0 + i, c);
      s0[i] = load_s<W>(sr0, k0 + i, c);
      s1[i] = load_s<W>(sr1, k0 + i, c);
    }
#pragma unroll
    for (int t = 0; t < kVecTok; ++t) {
      if (t < nt) {
        const uint4* xr = reinterpret_cast<const uint4*>(act[t]);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          acc[t][0] = wdot<W>(w0[i], xr, k0 + i, c, acc[t][0], s0[i]);
          acc[t][1] = wdot<W>(w1[i], xr, k0 + i, c, acc[t][1], s1[i]);
        }
      }
    }
  }
}

// vec_pass reading a missed record from the host store: every chunk and owned
// scale read is also stored to fl (the same bytes the copy kernel would move),
// raw scale bits held for the stores.  Same per-lane order as vec_pass, so the
// same bits.
template <int W, int CH>
__device__ __forceinline__ void vec_pass_fill(const uint8_t* row0, const uint8_t* row1, const uint8_t* sr0,
                                              const uint8_t* sr1, int nk, int c, const uint16_t* const act[kVecTok],
                                              int nt, float acc[kVecTok][2], const Fill& fl) {
  for (int k0 = 0; k0 < nk; k0 += CH) {
    typename WChunk<W>::T w0[CH], w1[CH];
    uint32_t s0[CH], s1[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      w0[i] = load_w<W>(row0, k0 + i, c);
      w1[i] = load_w<W>(row1, k0 + i, c);
      s0[i] = load_sr<W>(sr0, k0 + i, c);
      s1[i] = load_sr<W>(sr1, k0 + i, c);
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      store_w<W>(fl.w0, k0 + i, c, w0[i]);
      store_w<W>(fl.w1, k0 + i, c, w1[i]);
      if (fl.own0) store_sr<W>(fl.s0, k0 + i, c, s0[i]);
      if (fl.own1) store_sr<W>(fl.s1, k0 + i, c, s1[i]);
    }
#pragma unroll
    for (int t = 0; t < kVecTok; ++t) {
      if (t < nt) {
        const uint4* xr = reinterpret_cast<const uint4*>(act[t]);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          acc[t][0] = wdot<W>(w0[i], xr, k0 + i, c, acc[t][0], scale_of<W>(s0[i]));
          acc[t][1] = wdot<W>(w1[i], xr, k0 + i, c, acc[t][1], scale_of<W>(s1[i]));
        }
      }
    }
  }
}

// vec_pass for one activation row: each pass one unbroken run of loads, then
// the pair dots.  Same per-lane order as vec_pass, so the same bits.  With
// FILL every chunk and owned scale read is also stored to fl (the read-through
// of a missed record: the bytes are the same either way).
template <int W, int CH, bool FILL>
__device__ __forceinline__ void one_pass(const uint8_t* row0, const uint8_t* row1, const uint8_t* sr0,
                                         const uint8_t* sr1, int nk, int c, const uint16_t* act, float& acc0,
                                         float& acc1, const Fill& fl) {
  const uint4* xr = reinterpret_cast<const uint4*>(act);
  for (int k0 = 0; k0 < nk; k0 += CH) {
    typename WChunk<W>::T w0[CH], w1[CH];
    uint32_t s0[CH], s1[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      w0[i] = load_w<W>(row0, k0 + i, c);
      w1[i] = load_w<W>(row1, k0 + i, c);
      s0[i] = load_sr<W>(sr0, k0 + i, c);
      s1[i] = load_sr<W>(sr1, k0 + i, c);
    }
    // every load of the pass is issued before the first dot (the compiler otherwise sinks them
    // next to their uses and keeps about nine in flight per lane); no operands, no outputs
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if constexpr (FILL) {
        store_w<W>(fl.w0, k0 + i, c, w0[i]);
        store_w<W>(fl.w1, k0 + i, c, w1[i]);
        if (fl.own0) store_sr<W>(fl.s0, k0 + i, c, s0[i]);
        if (fl.own1) store_sr<W>(fl.s1, k0 + i, c, s1[i]);
      }
      acc0 = wdot<W>(w0[i], xr, k0 + i, c, acc0, scale_of<W>(s0[i]));
      acc1 = wdot<W>(w1[i], xr, k0 + i, c, acc1, scale_of<W>(s1[i]));
    }
  }
}

// K blocks per pass: the largest listed divisor of nk (16 blocks = 2048 bf16 or
// fp8, 4096 MXFP4 weights per stream held in registers)
inline int one_chunks(int nk) {
  for (int ch : {16, 8, 6, 4, 3, 2})
    if (nk % ch == 0) return ch;
  return 1;
}

// K blocks per read-through pass: half of 16 or 8 (still a divisor of nk), so
// that the values held for the stores do not raise the kernel's register count
// above the in-place pass; the summation order is the same for any pass width
template <int CH>
constexpr int kFillChunks = CH >= 8 ? CH / 2 : CH;

// Read-through for 2 to kDecodeMaxT tokens (at most kFillPairs pairs): the copy
// list {mode, count, (expert, record)...} of the call, loaded once per
// wavefront in one round trip, lane l holding pairs l, l + 64, ...  A work item
// whose record index is in the list reads that expert's host record in its
// first token group and stores every byte it reads into the record (slot, or
// staging for the overflow of a call wider than the cache), as the copy kernel
// would have; its later token groups read the weights back from the record,
// each lane the bytes it stored itself, and the scales again from the host
// (another wavefront may own them), so each weight byte crosses the link once.
constexpr int kFillPairs = 256;
constexpr int kFillRegs = kFillPairs / 64;

struct VecHead {
  int mode = 0, n = 0;
  int e[kFillRegs], r[kFillRegs];
};

__device__ __forceinline__ VecHead vec_head(const FfnArgs& a, bool fill) {
  const int lane = threadIdx.x & 63;
  VecHead v;
#pragma unroll
  for (int i = 0; i < kFillRegs; ++i) {
    v.e[i] = 0;
    v.r[i] = -1;
  }
  if (!fill) return v;
  const int32_t* __restrict__ lst = a.fill_list;
  v.mode = lst[0];
  v.n = lst[1];
  const int cap = min(kFillPairs, max(a.S, a.E));  // the list holds max(S, E) pairs
#pragma unroll
  for (int i = 0; i < kFillRegs; ++i) {
    const int p = lane + 64 * i;
    if (p < cap) {
      v.e[i] = lst[2 + 2 * p];
      v.r[i] = lst[3 + 2 * p];
    }
  }
  return v;
}

// host record that work item record index ri reads through, or null; ri is
// wavefront-uniform
__device__ __forceinline__ const uint8_t* vec_source(const FfnArgs& a, const VecHead& v, int ri) {
  const int lane = threadIdx.x & 63;
  if (v.mode == MOE_MODE_STAGED_ALL) return nullptr;
  const int n = min(v.n, kFillPairs);
#pragma unroll
  for (int i = 0; i < kFillRegs; ++i) {
    const uint64_t hit = __ballot(lane + 64 * i < n && v.r[i] == ri);
    if (!hit) continue;
    const int e = __builtin_amdgcn_readlane(v.e[i], __builtin_ctzll(hit));
    if ((unsigned)e >= (unsigned)a.E) {
      atomicOr(a.err, MOE_DEV_ERR_AUDIT);
      return nullptr;
    }
    return a.host + (uint64_t)e * a.stride;
  }
  return nullptr;
}

// record index of grouped record block r (r < max_routed)
__device__ __forceinline__ int block_record(const FfnArgs& a, int r) { return a.grp[kRecWords * (1 + r)]; }

// gate/up: work item = (record, 4 rows of F); quarter q takes row f = 4*g + q of
// gate (stream 0) and up (stream 1); h = silu(gate) * up stored in bf16.
template <int W, int CH, bool FILL>
__global__ __launch_bounds__(256) void k_gateup_vec(FfnArgs a) {
  const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
  const int nrt = a.max_routed + (a.shared ? 1 : 0);
  const int RG = a.F / 4;
  const int H = a.H, F = a.F;
  const int nk = H / (16 * lane_weights<W>());
  const uint64_t mat = code_bytes<W>((uint64_t)F * H);
  const uint16_t* __restrict__ x = (const uint16_t*)a.x;
  uint16_t* __restrict__ hb = (uint16_t*)a.hbuf;
  const int nwave = gridDim.x * 4;
  const VecHead vh = vec_head(a, FILL);
  for (int item = blockIdx.x * 4 + (threadIdx.x >> 6); item < nrt * RG; item += nwave) {
    const int r = item / RG, fg = (item % RG) * 4, f = fg + q;
    const Item it = item_block(a, r);
    if (it.n == 0) continue;
    const uint8_t* src = FILL && !it.sh ? vec_source(a, vh, block_record(a, r)) : nullptr;
    const uint8_t* rd = src ? src : it.rec;  // weights of the first token group, and the scales
    const uint8_t* wg = rd + code_bytes<W>((uint64_t)f * H);
    const uint8_t* wgr = it.rec + code_bytes<W>((uint64_t)f * H);  // weights of later groups
    const uint8_t* sg = scale_row<W>(rd, mat, F, H, 0, f, H);
    const uint8_t* su = scale_row<W>(rd, mat, F, H, 1, f, H);
    for (int tg = 0; tg < it.n; tg += kVecTok) {
      const int nt = min(kVecTok, it.n - tg);
      const uint16_t* act[kVecTok];
#pragma unroll
      for (int t = 0; t < kVecTok; ++t)
        act[t] = x + (uint64_t)(t < nt ? pair_token(a, item_pair(a, it, r, tg + t)) : 0) * H;
      float acc[kVecTok][2];
#pragma unroll
      for (int t = 0; t < kVecTok; ++t) acc[t][0] = acc[t][1] = 0.f;
      if (FILL && src && tg == 0) {  // uniform per wavefront
        uint8_t* dst = const_cast<uint8_t*>(it.rec);
        Fill fl;
        fl.w0 = dst + code_bytes<W>((uint64_t)f * H);
        fl.w1 = fl.w0 + mat;
        fl.s0 = const_cast<uint8_t*>(scale_row<W>(dst, mat, F, H, 0, f, H));
        fl.s1 = const_cast<uint8_t*>(scale_row<W>(dst, mat, F, H, 1, f, H));
        fl.own0 = fl.own1 = W == kMx4 || (f & 127) == 0;
        vec_pass_fill<W, kFillChunks<CH>>(wg, wg + mat, sg, su, nk, c, act, nt, acc, fl);
      } else if (FILL && src) {
        vec_pass<W, CH>(wgr, wgr + mat, sg, su, nk, c, act, nt, acc);
      } else {
        vec_pass<W, CH>(wg, wg + mat, sg, su, nk, c, act, nt, acc);
      }
      float v[16];
#pragma unroll
      for (int t = 0; t < kVecTok; ++t) {
        v[2 * t] = acc[t][0];
        v[2 * t + 1] = acc[t][1];
      }
      const float mine = reduce16_scatter(v, c);  // token c / 2, stream c % 2
      const float up = __shfl_xor(mine, 1);
      const int t = c >> 1;
      if ((c & 1) == 0 && t < nt) {
        const int p = item_pair(a, it, r, tg + t);
        hb[(uint64_t)p * F + f] = f32_to_bf16(silu_mul(mine, up));
      }
    }
  }
}

// down: work item = (record, 8 rows of H); quarter q takes rows 8*g + q (stream 0)
// and 8*g + 4 + q (stream 1) against h of the record's pairs; fp32 partial outputs.
template <int W, int CH, bool FILL>
__global__ __launch_bounds__(256) void k_down_vec(FfnArgs a) {
  const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
  const int nrt = a.max_routed + (a.shared ? 1 : 0);
  const int RG = a.H / 8;
  const int H = a.H, F = a.F;
  const int nk = F / (16 * lane_weights<W>());
  const uint64_t mat = code_bytes<W>((uint64_t)F * H);
  const uint16_t* __restrict__ hb = (const uint16_t*)a.hbuf;
  float* __restrict__ part = a.part;
  const int nwave = gridDim.x * 4;
  const VecHead vh = vec_head(a, FILL);
  for (int item = blockIdx.x * 4 + (threadIdx.x >> 6); item < nrt * RG; item += nwave) {
    const int r = item / RG, hg = (item % RG) * 8, h0 = hg + q;
    const Item it = item_block(a, r);
    if (it.n == 0) continue;
    const uint8_t* src = FILL && !it.sh ? vec_source(a, vh, block_record(a, r)) : nullptr;
    const uint8_t* rd = src ? src : it.rec;  // weights of the first token group, and the scales
    const uint8_t* wd = rd + 2 * mat + code_bytes<W>((uint64_t)h0 * F);
    const uint8_t* wdr = it.rec + 2 * mat + code_bytes<W>((uint64_t)h0 * F);  // weights of later groups
    const uint8_t* s0 = scale_row<W>(rd, mat, F, H, 2, h0, F);
    const uint8_t* s1 = scale_row<W>(rd, mat, F, H, 2, h0 + 4, F);
    for (int tg = 0; tg < it.n; tg += kVecTok) {
      const int nt = min(kVecTok, it.n - tg);
      const uint16_t* act[kVecTok];
#pragma unroll
      for (int t = 0; t < kVecTok; ++t) act[t] = hb + (uint64_t)(t < nt ? item_pair(a, it, r, tg + t) : 0) * F;
      float acc[kVecTok][2];
#pragma unroll
      for (int t = 0; t < kVecTok; ++t) acc[t][0] = acc[t][1] = 0.f;
      if (FILL && src && tg == 0) {  // uniform per wavefront
        uint8_t* dst = const_cast<uint8_t*>(it.rec);
        Fill fl;
        fl.w0 = dst + 2 * mat + code_bytes<W>((uint64_t)h0 * F);
        fl.w1 = fl.w0 + code_bytes<W>(4ull * F);
        fl.s0 = const_cast<uint8_t*>(scale_row<W>(dst, mat, F, H, 2, h0, F));
        fl.s1 = const_cast<uint8_t*>(scale_row<W>(dst, mat, F, H, 2, h0 + 4, F));
        fl.own0 = W == kMx4 || (h0 & 127) == 0;
        fl.own1 = W == kMx4;  // h0 + 4 is never the first row of a 128-row block
        vec_pass_fill<W, kFillChunks<CH>>(wd, wd + code_bytes<W>(4ull * F), s0, s1, nk, c, act, nt, acc, fl);
      } else if (FILL && src) {
        vec_pass<W, CH>(wdr, wdr + code_bytes<W>(4ull * F), s0, s1, nk, c, act, nt, acc);
      } else {
        vec_pass<W, CH>(wd, wd + code_bytes<W>(4ull * F), s0, s1, nk, c, act, nt, acc);
      }
      float v[16];
#pragma unroll
      for (int t = 0; t < kVecTok; ++t) {
        v[2 * t] = acc[t][0];
        v[2 * t + 1] = acc[t][1];
      }
      const float mine = reduce16_scatter(v, c);  // token c / 2, stream c % 2
      const int t = c >> 1;
      if (t < nt) {
        const int p = item_pair(a, it, r, tg + t);
        part[(uint64_t)p * H + h0 + 4 * (c & 1)] = mine;
      }
    }
  }
}

// Single-token calls (T = 1): the k choices are distinct records, so work item
// (choice j, rows) reads record slot_ids[j] (j = k: the shared expert) against
// the one activation row, and its pair id is j.  Same rows per wavefront, same
// per-lane order and the same 16-lane pairing tree as the kernels above, so the
// same bits; the code is a few hundred instructions instead of the 8-token
// unrolled body, which every layer's launch fetches cold.
//
// The call's record indices and the head of its copy list, one entry per lane,
// requested by every wavefront in its first load: lane j < k holds slot_ids[j];
// with read-through, lane i < 2 + 2k holds entry i of the copy list {mode,
// count, (expert, record)...}, which a single token's at most k misses fit.
// The work items read them from those lanes (a wavefront-uniform index), so
// the weight stream waits for one memory round trip instead of one per entry.
struct OneHead {
  int sid = 0, lst = 0;
};

__device__ __forceinline__ OneHead one_head(const FfnArgs& a, bool fill) {
  const int lane = threadIdx.x & 63;
  OneHead o;
  if (lane < a.k) o.sid = a.slot_ids[lane];
  if (fill && lane < 2 + 2 * a.k) o.lst = a.fill_list[lane];
  return o;
}

// record of choice j (j = k: the shared expert), or null for a cold expert
// (index S + E + e: computed on the host); j is wavefront-uniform
__device__ __forceinline__ const uint8_t* one_record(const FfnArgs& a, int j, const OneHead& o) {
  if (j == a.k) return a.shared;
  int ri = __builtin_amdgcn_readlane(o.sid, j);
  if (ri >= a.S + a.E && ri < a.S + 2 * a.E) return nullptr;
  if ((unsigned)ri >= (unsigned)(a.S + a.E)) {
    atomicOr(a.err, MOE_DEV_ERR_AUDIT);
    ri = 0;
  }
  return ri < a.S ? a.slots + (uint64_t)ri * a.stride : a.staging + (uint64_t)(ri - a.S) * a.stride;
}

// Read-through (FILL): choice j's record was assigned to its slot by this
// call's ensure when the copy list pairs slot_ids[j] with an expert e.  Then
// the record is read from e's row of the device-mapped host store and every
// byte is written to the slot as the FFN reads it: the gate/up launch fills
// the gate and up matrices and their scales, the down launch the rest, so at
// the end of the call the slot holds the whole record, as after the copy
// kernel.  Returns e's host record, or null when j reads its record in place.
// j is wavefront-uniform, so the entries are read from their lanes as scalars.
__device__ __forceinline__ const uint8_t* fill_source(const FfnArgs& a, int j, const OneHead& o) {
  if (j == a.k) return nullptr;  // the shared expert is device resident
  if (__builtin_amdgcn_readlane(o.lst, 0) == MOE_MODE_STAGED_ALL) return nullptr;
  const int n = min(__builtin_amdgcn_readlane(o.lst, 1), a.k);  // a single token has at most k misses
  const int r = __builtin_amdgcn_readlane(o.sid, j);
  for (int m = 0; m < n; ++m) {
    if (__builtin_amdgcn_readlane(o.lst, 3 + 2 * m) != r) continue;
    const int e = __builtin_amdgcn_readlane(o.lst, 2 + 2 * m);
    if ((unsigned)e >= (unsigned)a.E) {
      atomicOr(a.err, MOE_DEV_ERR_AUDIT);
      return nullptr;
    }
    return a.host + (uint64_t)e * a.stride;
  }
  return nullptr;
}

template <int W, int CH, bool FILL>
__global__ __launch_bounds__(128) void k_gateup_one(FfnArgs a) {
  const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
  const int RG = a.F / 4;
  const int H = a.H, F = a.F;
  const int nk = H / (16 * lane_weights<W>());
  const uint64_t mat = code_bytes<W>((uint64_t)F * H);
  const int items = (a.k + (a.shared ? 1 : 0)) * RG;
  const uint16_t* __restrict__ x = (const uint16_t*)a.x;
  uint16_t* __restrict__ hb = (uint16_t*)a.hbuf;
  const OneHead o = one_head(a, FILL);
  for (int item = blockIdx.x * 2 + (threadIdx.x >> 6); item < items; item += gridDim.x * 2) {
    const int j = item / RG, f = (item % RG) * 4 + q;
    const uint8_t* rec = one_record(a, j, o);
    if (!rec) continue;  // a cold expert (wavefront-uniform)
    float g = 0.f, up = 0.f;
    bool done = false;
    if constexpr (FILL) {
      if (const uint8_t* src = fill_source(a, j, o)) {  // uniform per wavefront
        uint8_t* dst = const_cast<uint8_t*>(rec);
        Fill fl;
        fl.w0 = dst + code_bytes<W>((uint64_t)f * H);
        fl.w1 = fl.w0 + mat;
        fl.s0 = const_cast<uint8_t*>(scale_row<W>(dst, mat, F, H, 0, f, H));
        fl.s1 = const_cast<uint8_t*>(scale_row<W>(dst, mat, F, H, 1, f, H));
        fl.own0 = fl.own1 = W == kMx4 || (f & 127) == 0;
        const uint8_t* wg = src + code_bytes<W>((uint64_t)f * H);
        one_pass<W, kFillChunks<CH>, true>(wg, wg + mat, scale_row<W>(src, mat, F, H, 0, f, H),
                                           scale_row<W>(src, mat, F, H, 1, f, H), nk, c, x, g, up, fl);
        done = true;
      }
    }
    if (!done) {
      const uint8_t* wg = rec + code_bytes<W>((uint64_t)f * H);
      one_pass<W, CH, false>(wg, wg + mat, scale_row<W>(rec, mat, F, H, 0, f, H),
                             scale_row<W>(rec, mat, F, H, 1, f, H), nk, c, x, g, up, Fill());
    }
    g = reduce16_all(g);
    up = reduce16_all(up);
    if (c == 0) hb[(uint64_t)j * F + f] = f32_to_bf16(silu_mul(g, up));
  }
}

template <int W, int CH, bool FILL>
__global__ __launch_bounds__(128) void k_down_one(FfnArgs a) {
  const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
  const int RG = a.H / 8;
  const int H = a.H, F = a.F;
  const int nk = F / (16 * lane_weights<W>());
  const uint64_t mat = code_bytes<W>((uint64_t)F * H);
  const int items = (a.k + (a.shared ? 1 : 0)) * RG;
  const uint16_t* __restrict__ hb = (const uint16_t*)a.hbuf;
  float* __restrict__ part = a.part;
  const OneHead o = one_head(a, FILL);
  for (int item = blockIdx.x * 2 + (threadIdx.x >> 6); item < items; item += gridDim.x * 2) {
    const int j = item / RG, h0 = (item % RG) * 8 + q;
    const uint8_t* rec = one_record(a, j, o);
    if (!rec) continue;  // a cold expert (wavefront-uniform)
    float s0 = 0.f, s1 = 0.f;
    bool done = false;
    if constexpr (FILL) {
      if (const uint8_t* src = fill_source(a, j, o)) {  // uniform per wavefront
        uint8_t* dst = const_cast<uint8_t*>(rec);
        Fill fl;
        fl.w0 = dst + 2 * mat + code_bytes<W>((uint64_t)h0 * F);
        fl.w1 = fl.w0 + code_bytes<W>(4ull * F);
        fl.s0 = const_cast<uint8_t*>(scale_row<W>(dst, mat, F, H, 2, h0, F));
        fl.s1 = const_cast<uint8_t*>(scale_row<W>(dst, mat, F, H, 2, h0 + 4, F));
        fl.own0 = W == kMx4 || (h0 & 127) == 0;
        fl.own1 = W == kMx4;  // h0 + 4 is never the first row of a 128-row block
        const uint8_t* wd = src + 2 * mat + code_bytes<W>((uint64_t)h0 * F);
        one_pass<W, kFillChunks<CH>, true>(wd, wd + code_bytes<W>(4ull * F), scale_row<W>(src, mat, F, H, 2, h0, F),
                                           scale_row<W>(src, mat, F, H, 2, h0 + 4, F), nk, c, hb + (uint64_t)j * F,
                                           s0, s1, fl);
        done = true;
      }
    }
    if (!done) {
      const uint8_t* wd = rec + 2 * mat + code_bytes<W>((uint64_t)h0 * F);
      one_pass<W, CH, false>(wd, wd + code_bytes<W>(4ull * F), scale_row<W>(rec, mat, F, H, 2, h0, F),
                             scale_row<W>(rec, mat, F, H, 2, h0 + 4, F), nk, c, hb + (uint64_t)j * F, s0, s1,
                             Fill());
    }
    s0 = reduce16_all(s0);
    s1 = reduce16_all(s1);
    if (c < 2) part[(uint64_t)j * H + h0 + 4 * c] = c ? s1 : s0;
  }
}

// kernel instantiation by K blocks per pass
#define MOE_BY_CHUNKS(KERN, NK, ...)        \
  switch (one_chunks(NK)) {                 \
    case 16: return KERN<W, 16, ##__VA_ARGS__>; \
    case 8: return KERN<W, 8, ##__VA_ARGS__>;   \
    case 6: return KERN<W, 6, ##__VA_ARGS__>;   \
    case 4: return KERN<W, 4, ##__VA_ARGS__>;   \
    case 3: return KERN<W, 3, ##__VA_ARGS__>;   \
    case 2: return KERN<W, 2, ##__VA_ARGS__>;   \
    default: return KERN<W, 1, ##__VA_ARGS__>;  \
  }

typedef void (*FfnKernel)(FfnArgs);
template <int W>
FfnKernel gateup_decode(bool one, bool fill, int H) {
  const int nk = H / (16 * lane_weights<W>());
  if (one && fill) { MOE_BY_CHUNKS(k_gateup_one, nk, true) }
  if (one) { MOE_BY_CHUNKS(k_gateup_one, nk, false) }
  if (fill) { MOE_BY_CHUNKS(k_gateup_vec, nk, true) }
  MOE_BY_CHUNKS(k_gateup_vec, nk, false)
}
template <int W>
FfnKernel down_decode(bool one, bool fill, int F) {
  const int nk = F / (16 * lane_weights<W>());
  if (one && fill) { MOE_BY_CHUNKS(k_down_one, nk, true) }
  if (one) { MOE_BY_CHUNKS(k_down_one, nk, false) }
  if (fill) { MOE_BY_CHUNKS(k_down_vec, nk, true) }
  MOE_BY_CHUNKS(k_down_vec, nk, false)
}
#undef MOE_BY_CHUNKS

// ------------------------------------------------------------------ fp32 path
__global__ __launch_bounds__(256) void k_gateup_f32(FfnArgs a) {
  const int nr = a.grp[0];
  const int nrt = nr + (a.shared ? 1 : 0);
  const int FT = a.F / kF32Rows;
  const int H = a.H, F = a.F;
  const float* __restrict__ x = (const float*)a.x;
  float* __restrict__ hb = (float*)a.hbuf;
  for (int item = blockIdx.x; item < nrt * FT; item += gridDim.x) {
    const int r = item / FT, f = (item % FT) * kF32Rows + (threadIdx.x & 63);
    const Item it = item_record(a, nr, r);
    const float* wg = reinterpret_cast<const float*>(it.rec) + (uint64_t)f * H;
    const float* wu = wg + (uint64_t)F * H;
    for (int idx = threadIdx.x >> 6; idx < it.n; idx += 4) {
      const int p = item_pair(a, it, r, idx);
      const float* xt = x + (uint64_t)pair_token(a, p) * H;
      float g = 0.f, u = 0.f;
      for (int i = 0; i < H; ++i) {
        g = __builtin_fmaf(wg[i], xt[i], g);
        u = __builtin_fmaf(wu[i], xt[i], u);
      }
      hb[(uint64_t)p * F + f] = silu_mul(g, u);
    }
  }
}

__global__ __launch_bounds__(256) void k_down_f32(FfnArgs a) {
  const int nr = a.grp[0];
  const int nrt = nr + (a.shared ? 1 : 0);
  const int HT = a.H / kF32Rows;
  const int H = a.H, F = a.F;
  const float* __restrict__ hb = (const float*)a.hbuf;
  for (int item = blockIdx.x; item < nrt * HT; item += gridDim.x) {
    const int r = item / HT, ht = item % HT, hr = ht * kF32Rows + (threadIdx.x & 63);
    const Item it = item_record(a, nr, r);
    const float* wd = reinterpret_cast<const float*>(it.rec) + 2ull * F * H + (uint64_t)hr * F;
    for (int idx = threadIdx.x >> 6; idx < it.n; idx += 4) {
      const int p = item_pair(a, it, r, idx);
      const float* hp = hb + (uint64_t)p * F;
      float o = 0.f;
      for (int f = 0; f < F; ++f) o = __builtin_fmaf(wd[f], hp[f], o);
      a.part[(uint64_t)p * H + hr] = o;
    }
  }
}

// ------------------------------------------------------------------ combine
// One 256-thread workgroup per token; thread i owns the chunks of 8 elements
// c = i, i + 256, ...: y = sum_j w[t][j] * part[t*k + j] in j order (+ the
// shared expert's row), rounded once; x_next = round(residual + y); and, for
// the decode chain, xn_next = rmsnorm(x_next) in the order of rownorm.h (the
// same bits as the norm kernel).  Each thread re-reads only what it wrote.
template <bool F32>
__global__ __launch_bounds__(kRowThreads) void k_combine(FfnArgs a, void* __restrict__ xn_next, float eps) {
  __shared__ float s_wave[4];
  const int t = blockIdx.x;
  const int H = a.H, k = a.k, routed = a.T * a.k;
  const float* __restrict__ part = a.part;
  const float* __restrict__ wt = a.w + (size_t)t * k;
  const size_t roff = (size_t)t * H * (F32 ? 4 : 2);
  void* __restrict__ yrow = (uint8_t*)a.y + roff;
  void* __restrict__ xrow = a.x_next ? (uint8_t*)a.x_next + roff : nullptr;
  const void* __restrict__ rrow = (const uint8_t*)a.residual + roff;
  float ss = 0.f;
  for (int c = threadIdx.x; c * 8 < H; c += kRowThreads) {
    float acc[8], res[8];
    combine_chunk<F32>(part + (uint64_t)t * k * H, wt, k, H, c, a.shared ? part + (uint64_t)(routed + t) * H : nullptr,
                       xrow ? rrow : nullptr, acc, res);
    chunk_store<F32>(yrow, c, acc);  // acc now holds y as stored
    if (xrow) {
#pragma unroll
      for (int q = 0; q < 8; ++q) res[q] = res[q] + acc[q];
      chunk_store<F32>(xrow, c, res);  // res now holds x_next as stored
      ss = chunk_sumsq(res, ss);
    }
  }
  if (xn_next && xrow) {
    const float inv = row_inv_rms(row_block_sum(ss, s_wave), H, eps);
    row_scale_chunks<F32>(xrow, (uint8_t*)xn_next + roff, H, inv);
  }
}

// part rows of the cold pairs (record index in [S + E, S + 2E)) from the host's
// output rows (device-mapped host memory): one workgroup per pair
__global__ __launch_bounds__(256) void k_cold_scatter(const int32_t* __restrict__ slot_ids, int n, int S, int E,
                                                      int H, const float* __restrict__ host_rows,
                                                      float* __restrict__ part) {
  for (int p = blockIdx.x; p < n; p += gridDim.x) {
    const int r = slot_ids[p];
    if (r < S + E || r >= S + 2 * E) continue;  // workgroup-uniform
    const float4* src = reinterpret_cast<const float4*>(host_rows + (uint64_t)p * H);
    float4* dst = reinterpret_cast<float4*>(part + (uint64_t)p * H);
    for (int i = threadIdx.x; i < H / 4; i += blockDim.x) dst[i] = src[i];
  }
}

}  // namespace

hipError_t launch_cold_combine(moe_offload* h, const void* x, const int32_t* slot_ids, const float* w, int T,
                               const void* shared, void* y, const void* residual, void* x_next, hipStream_t s) {
  const int n = T * h->k;
  launch_k(h, MOE_K_COMBINE, k_cold_scatter, dim3(std::min(n, 1024)), dim3(256), 0, s, slot_ids, n, h->S, h->E, h->H,
           (const float*)h->cold_out_dev, h->part);
  return launch_combine(h, x, w, T, shared, y, residual, x_next, nullptr, 0.f, s);
}

hipError_t launch_combine(moe_offload* h, const void* x, const float* w, int T, const void* shared, void* y,
                          const void* residual, void* x_next, void* xn_next, float eps, hipStream_t s) {
  FfnArgs a;
  memset(&a, 0, sizeof a);
  a.x = x;
  a.w = w;
  a.part = h->part;
  a.y = y;
  a.residual = residual ? residual : x;
  a.x_next = x_next;
  a.shared = (const uint8_t*)shared;
  a.T = T;
  a.k = h->k;
  a.H = h->H;
  a.F = h->F;
  if (h->dtype == MOE_F32)
    launch_k(h, MOE_K_COMBINE, k_combine<true>, dim3(T), dim3(kRowThreads), 0, s, a, xn_next, eps);
  else
    launch_k(h, MOE_K_COMBINE, k_combine<false>, dim3(T), dim3(kRowThreads), 0, s, a, xn_next, eps);
  return hipGetLastError();
}

// read-through: one token (a work item per choice), or up to kDecodeMaxT tokens
// with at most kFillPairs pairs (the decode kernels, the copy list in one load
// per wavefront)
bool ffn_reads_through(const moe_offload* h, int T) {
  return h->dtype != MOE_F32 && !ffn_uses_gemm(h, T) && (T == 1 || (T <= kDecodeMaxT && T * h->k <= kFillPairs));
}

// Kernel pair of a multi-token call.  The decode kernels meet each weight row
// once per 8-token group of a record, the grouped GEMM once per tile of up to
// 80 pairs, so with many pairs per record the GEMM streams fewer bytes; the
// crossover was measured per weight format (FFN time per pair of both pairs on
// the same calls, every expert resident), in T * k / E, the fewest pairs per
// record a call can average: bf16 between 4 and 6 (Mixtral shape; Qwen3 shape
// even at 4); MXFP4 about 1 (the GEMM wins from 0.5 on the Qwen3 shape, the
// decode kernels up to 1 on a 32-expert top-4 layer); fp8 below every size
// measured, down to 0.125 (its decode kernels widen every code once per token
// group).  So the GEMM takes a call when 8 * T * k >= c8 * E with c8 = 40, 8
// and 1.  The rule reads only the layer's shape and the call's token count
// (never S or which experts are resident): every output bit stays independent
// of the slot count.
bool ffn_uses_gemm(const moe_offload* h, int T) {
  if (h->dtype == MOE_F32 || T == 1) return false;
  if (T > kDecodeMaxT || h->ffn_path == MOE_FFN_GEMM) return true;
  if (h->ffn_path == MOE_FFN_DECODE) return false;
  const int c8 = h->dtype == MOE_FP8_E4M3_B128 ? 1 : (h->dtype == MOE_MXFP4 ? 8 : 40);
  return 8 * T * h->k >= c8 * h->E;
}

// ------------------------------------------------------------------ scratch workspace
// For callers that cannot allocate (graph capture, serving loops that forbid
// allocation): one FFN workspace per device in a file-scope device array.  Host
// code never passes `scratch` itself to a kernel: its name is a host-side
// stand-in; the device address comes from hipGetSymbolAddress, once per device.
namespace {
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

hipError_t scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[device]) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device) return hipErrorInvalidDevice;  // the caller makes `device` current
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!ptr) return hipErrorInvalidSymbol;
  g_scratch[device] = ptr;
  return hipSuccess;
}

void* scratch_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch[device];
}

// Workgroups of GEMM kernel k the device holds at once (CUs x resident workgroups per CU of
// `block` threads).  The GEMM's grid is no larger: every workgroup then starts at once and strides
// over the work list in step with the others, so the token tiles of one record and row tile (the
// row-tile count apart: on one XCD when that count is a multiple of 8, as workgroup w runs on XCD
// w mod 8) run together and fetch the weight rows into that XCD's L2 once.
template <typename Kern>
int gemm_grid_cap(Kern k, int block, int device) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  std::lock_guard<std::mutex> lk(mu);
  const auto key = std::make_pair(reinterpret_cast<const void*>(k), device);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k, block, 0) != hipSuccess || cus <= 0 || per <= 0) {
    (void)hipGetLastError();
    return 2048;  // not cached: the query is repeated on the next call
  }
  return cache[key] = cus * per;
}

// Wavefronts per grouped-GEMM workgroup for gate/up (gu) or down.  Eight share each token slice
// in LDS across twice the weight rows and load it two slices ahead, but a compute unit holds one
// such workgroup: the call needs at least 1024 of their work items (about four per compute unit),
// counted at T * k / kGemmTok token tiles.  Eight need the rows to divide into their tiles (F and
// H are multiples of 128: gate/up always; down when H is a multiple of 256).  Reads the layer's
// shape, T and the handle's setting only; the outputs are the same bits either way.
int gemm_waves(const moe_offload* h, int T, bool gu) {
  const int rows = gu ? h->F : h->H;
  if (rows % gemm_rows(gu, 8)) return 4;
  if (h->gemm_waves) return h->gemm_waves;
  return (int64_t)(T * h->k / kGemmTok) * (rows / gemm_rows(gu, 8)) >= 1024 ? 8 : 4;
}

FfnWork ffn_work_in(const moe_offload* h, int T, void* base, size_t* bytes) {
  FfnWork w;
  w.gl.max_pairs = T * h->k;
  w.gl.max_recs = std::min(T * h->k, h->S + h->E) + 1;
  const size_t rows = (size_t)T * h->k + T;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t g = al(4 * (size_t)w.gl.words());
  const size_t hb = al((h->dtype == MOE_F32 ? 4 : 2) * rows * h->F);
  const size_t pb = 4 * rows * h->H;
  uint8_t* b = (uint8_t*)base;
  w.grp = (int32_t*)b;
  w.hbuf = b ? (void*)(b + g) : nullptr;
  w.part = b ? (float*)(b + g + hb) : nullptr;
  if (bytes) *bytes = g + hb + pb;
  return w;
}

hipError_t launch_ffn(moe_offload* h, const void* x, const int32_t* slot_ids, const float* w, int T,
                      const void* shared, void* y, const void* residual, void* x_next, void* xn_next, float eps,
                      hipStream_t s, bool grouped, bool combine, bool fill, const FfnWork* ws) {
  FfnArgs a;
  a.x = x;
  a.slot_ids = slot_ids;
  a.w = w;
  a.slots = h->slots;
  a.staging = h->staging;
  a.shared = (const uint8_t*)shared;
  a.stride = h->record_stride;
  a.grp = ws ? ws->grp : h->grp;
  a.hbuf = ws ? ws->hbuf : h->hbuf;
  a.part = ws ? ws->part : h->part;
  a.y = y;
  a.residual = residual ? residual : x;
  a.x_next = x_next;
  a.err = h->cache.err;
  a.T = T;
  a.k = h->k;
  a.H = h->H;
  a.F = h->F;
  a.S = h->S;
  a.E = h->E;
  a.off_pairs = ws ? ws->gl.off_pairs() : h->gl.off_pairs();
  a.off_tiles = ws ? ws->gl.off_tiles() : h->gl.off_tiles();
  a.max_routed = std::min(T * h->k, h->S + h->E);
  a.pair_items = T == 1 && h->dtype != MOE_F32 ? 1 : 0;
  fill = fill && ffn_reads_through(h, T);
  a.fill_list = fill ? h->cache.copy_list : nullptr;
  a.host = h->host_dev;
  // distinct records a call can touch (+ the shared expert)
  const int max_items_r = a.max_routed + (shared ? 1 : 0);
  if (!grouped && !a.pair_items) {
    launch_k(h, MOE_K_GROUP, k_group, dim3(1), dim3(kBlock), 0, s, a);
  }
  const int wf = h->dtype;  // weight format
  // gate/up and down: fp32 FMA kernels, the decode kernels, or the MFMA kernels (ffn_uses_gemm)
  void (*gu)(FfnArgs) = nullptr;
  void (*dn)(FfnArgs) = nullptr;
  dim3 g1, g2, b1, b2;
  if (h->dtype == MOE_F32) {
    gu = k_gateup_f32;
    dn = k_down_f32;
    g1 = dim3(std::min(max_items_r * (h->F / kF32Rows), 2048));
    g2 = dim3(std::min(max_items_r * (h->H / kF32Rows), 2048));
    b1 = b2 = dim3(256);
  } else if (!ffn_uses_gemm(h, T)) {  // one wavefront per work item
    const bool one = a.pair_items != 0;
    gu = wf == kFp8 ? gateup_decode<kFp8>(one, fill, h->H)
                    : (wf == kMx4 ? gateup_decode<kMx4>(one, fill, h->H) : gateup_decode<kBf16>(one, fill, h->H));
    dn = wf == kFp8 ? down_decode<kFp8>(one, fill, h->F)
                    : (wf == kMx4 ? down_decode<kMx4>(one, fill, h->F) : down_decode<kBf16>(one, fill, h->F));
    if (one) {  // 2 per workgroup: a single token's items spread evenly over the CUs (batch-1 step 1 % faster)
      g1 = dim3(std::min((max_items_r * (h->F / 4) + 1) / 2, 16384));
      g2 = dim3(std::min((max_items_r * (h->H / 8) + 1) / 2, 16384));
      b1 = b2 = dim3(128);
    } else {  // 4 per workgroup
      g1 = dim3(std::min((max_items_r * (h->F / 4) + 3) / 4, 8192));
      g2 = dim3(std::min((max_items_r * (h->H / 8) + 3) / 4, 8192));
      b1 = b2 = dim3(256);
    }
  } else {  // grouped GEMM over (record tile, row tile) work items; the grid strides over the call's list
    const int wg = gemm_waves(h, T, true), wd = gemm_waves(h, T, false);
    if (wg == 8)
      gu = wf == kFp8 ? k_gemm<kFp8, true, 8> : (wf == kMx4 ? k_gemm<kMx4, true, 8> : k_gemm<kBf16, true, 8>);
    else
      gu = wf == kFp8 ? k_gemm<kFp8, true, 4> : (wf == kMx4 ? k_gemm<kMx4, true, 4> : k_gemm<kBf16, true, 4>);
    if (wd == 8)
      dn = wf == kFp8 ? k_gemm<kFp8, false, 8> : (wf == kMx4 ? k_gemm<kMx4, false, 8> : k_gemm<kBf16, false, 8>);
    else
      dn = wf == kFp8 ? k_gemm<kFp8, false, 4> : (wf == kMx4 ? k_gemm<kMx4, false, 4> : k_gemm<kBf16, false, 4>);
    // tiles of a call: gemm_tile_count(n) <= ceil(n / kGemmTok), so at most one partial tile per
    // record on top of the full ones
    const int tiles = (T * h->k) / kGemmTok + std::min(T * h->k, h->S + h->E) +
                      (shared ? gemm_tile_count(T) : 0);
    b1 = dim3(64 * wg);
    b2 = dim3(64 * wd);
    g1 = dim3(std::min(tiles * (h->F / gemm_rows(true, wg)), gemm_grid_cap(gu, 64 * wg, h->device)));
    g2 = dim3(std::min(tiles * (h->H / gemm_rows(false, wd)), gemm_grid_cap(dn, 64 * wd, h->device)));
  }
  {
    launch_k(h, MOE_K_GATEUP, gu, g1, b1, 0, s, a);
  }
  {
    launch_k(h, MOE_K_DOWN, dn, g2, b2, 0, s, a);
  }
  if (combine) {
    if (h->dtype == MOE_F32)
      launch_k(h, MOE_K_COMBINE, k_combine<true>, dim3(T), dim3(kRowThreads), 0, s, a, xn_next, eps);
    else
      launch_k(h, MOE_K_COMBINE, k_combine<false>, dim3(T), dim3(kRowThreads), 0, s, a, xn_next, eps);
  }
  return hipGetLastError();
}

}  // namespace moe
