// Grouped expert FFN over the slot tensor, with the top-k weighted combine.
//
// xinfer-ai 0.14.6 docs/moe_offload.md, "How it works": the expert GEMMs read a
// [num_slots, N, K] slot tensor instead of [num_experts, N, K]; placement never
// changes precision.  Per (token t, choice j) with record r = slot_ids[t][j]:
//     h = silu(Wg x_t) * (Wu x_t),  o = Wd h,  y_t = sum_j w[t][j] o  (+ shared expert)
//
// Kernels (one launch each, fixed grids):
//   k_group    one workgroup: counting sort of the T*k (t, j) pairs by record
//              index -> list of distinct records, their token lists.
//   k_gateup   work item = (record, 16 rows of F): gate and up rows streamed
//              once, bf16 MFMA 16x16x32 against up to 64 gathered tokens per
//              pass, K split over the 4 wavefronts of the workgroup and reduced
//              through LDS in a fixed order, SiLU * up fused, h stored in bf16.
//   k_down     work item = (record, 16 rows of H): down rows against h, fp32
//              partial outputs per (t, j).  The last work item of each 16-row
//              tile to finish (device-scope counter) combines that tile for
//              all tokens in j order, rounds to bf16, and adds the residual.
// fp8 records: e4m3 codes are widened exactly to bf16 by the hardware pair
// converter and each 128-wide K block is scaled on the fp32 accumulator.
// fp32 records use plain fp32 FMA kernels with the same structure.
//
// Nothing depends on which slot holds an expert, on S, or on the order of the
// tokens inside a record's list: every output element is one fixed-order sum.
#include <math.h>

#include <algorithm>

#include "internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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
  uint32_t* comb_ctr;
  void* y;
  void* x_next;
  int32_t* err;
  int T, k, H, F, S, E;
  int off_list, off_start, off_pairs;
};

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// ------------------------------------------------------------------ grouping
constexpr int kGrpBlock = 1024;

// inclusive scan of v over the 1024 threads; returns exclusive prefix, *total = sum
__device__ __forceinline__ int block_excl_sum(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o);
    if (lane >= o) inc += n;
  }
  if (lane == 63) s_wave[wid] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kGrpBlock / 64; ++w) {
    const int c = s_wave[w];
    base += w < wid ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

__global__ __launch_bounds__(kGrpBlock) void k_group(FfnArgs a) {
  __shared__ int cnt[2 * kMaxExperts];
  __shared__ int cur[2 * kMaxExperts];
  __shared__ int wave[kGrpBlock / 64];
  const int tid = threadIdx.x;
  const int n = a.T * a.k, nb = a.S + a.E;
  for (int b = tid; b < 2 * kMaxExperts; b += kGrpBlock) cnt[b] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kGrpBlock) {
    int r = a.slot_ids[i];
    if ((unsigned)r >= (unsigned)nb) {
      atomicOr(a.err, MOE_DEV_ERR_AUDIT);
      r = 0;
    }
    atomicAdd(&cnt[r], 1);
  }
  __syncthreads();
  const int c0 = cnt[2 * tid], c1 = cnt[2 * tid + 1];
  int tot_pairs, nr;
  const int pre = block_excl_sum(c0 + c1, wave, &tot_pairs);
  const int pre_nz = block_excl_sum((c0 > 0) + (c1 > 0), wave, &nr);
  int32_t* list = a.grp + a.off_list;
  int32_t* start = a.grp + a.off_start;
  int32_t* pairs = a.grp + a.off_pairs;
  cur[2 * tid] = pre;
  cur[2 * tid + 1] = pre + c0;
  if (c0 > 0) {
    list[pre_nz] = 2 * tid;
    start[pre_nz] = pre;
  }
  if (c1 > 0) {
    list[pre_nz + (c0 > 0)] = 2 * tid + 1;
    start[pre_nz + (c0 > 0)] = pre + c0;
  }
  if (tid == 0) {
    start[nr] = n;
    a.grp[0] = nr;
  }
  __syncthreads();
  for (int i = tid; i < n; i += kGrpBlock) {
    int r = a.slot_ids[i];
    if ((unsigned)r >= (unsigned)nb) r = 0;
    pairs[atomicAdd(&cur[r], 1)] = i;
  }
}

// work item -> record bytes and its token list
struct Item {
  const uint8_t* rec;
  const int32_t* plist;  // pair ids (t*k + j); null for the shared expert
  int n;                 // number of tokens
};

__device__ __forceinline__ Item item_record(const FfnArgs& a, int nr, int r) {
  Item it;
  if (r < nr) {
    const int ri = a.grp[a.off_list + r];
    it.rec = ri < a.S ? a.slots + (uint64_t)ri * a.stride : a.staging + (uint64_t)(ri - a.S) * a.stride;
    const int s0 = a.grp[a.off_start + r];
    it.n = a.grp[a.off_start + r + 1] - s0;
    it.plist = a.grp + a.off_pairs + s0;
  } else {
    it.rec = a.shared;
    it.n = a.T;
    it.plist = nullptr;
  }
  return it;
}

// pair id (row of h / part) and token of entry idx of an item
__device__ __forceinline__ int item_pair(const FfnArgs& a, const Item& it, int idx) {
  return it.plist ? it.plist[idx] : a.T * a.k + idx;
}
__device__ __forceinline__ int pair_token(const FfnArgs& a, int p) {
  const int routed = a.T * a.k;
  return p < routed ? p / a.k : p - routed;
}

// ------------------------------------------------------------------ MFMA operand loads
// Lane l of a 16x16x32 MFMA supplies row (l & 15) and 8 consecutive K values of
// one of 4 K slices.  Over a 128-wide K chunk lane l reads 32 contiguous values
// at K offset 32*(l >> 4) of its row and feeds values [8i, 8i+8) to MFMA i; the
// B operand uses the same mapping, so the 4 MFMAs together cover the chunk.

__device__ __forceinline__ void load_a_bf16(const uint16_t* p, bf16x8 a[4]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = __builtin_bit_cast(bf16x8, q[i]);
}

template <bool HI>
__device__ __forceinline__ uint32_t cvt2(uint32_t d) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d, 1.0f, HI));
}

__device__ __forceinline__ void load_a_fp8(const uint8_t* p, bf16x8 a[4]) {
  const uint4 q0 = reinterpret_cast<const uint4*>(p)[0];
  const uint4 q1 = reinterpret_cast<const uint4*>(p)[1];
  const uint32_t d[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 u;
    u.x = cvt2<false>(d[2 * i]);
    u.y = cvt2<true>(d[2 * i]);
    u.z = cvt2<false>(d[2 * i + 1]);
    u.w = cvt2<true>(d[2 * i + 1]);
    a[i] = __builtin_bit_cast(bf16x8, u);
  }
}

__device__ __forceinline__ void load_b_bf16(const uint16_t* p, bool valid, bf16x8 b[4]) {
  if (valid) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = __builtin_bit_cast(bf16x8, q[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }
}

__device__ __forceinline__ f32x4 mfma4(const bf16x8 a[4], const bf16x8 b[4], f32x4 acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[i], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ f32x4 fma4(float s, f32x4 v, f32x4 acc) {
  f32x4 r;
  r.x = __builtin_fmaf(s, v.x, acc.x);
  r.y = __builtin_fmaf(s, v.y, acc.y);
  r.z = __builtin_fmaf(s, v.z, acc.z);
  r.w = __builtin_fmaf(s, v.w, acc.w);
  return r;
}

// ------------------------------------------------------------------ gate/up (bf16, fp8)
template <bool FP8>
__global__ __launch_bounds__(256) void k_gateup(FfnArgs a) {
  __shared__ float red[4][4][2][4][64];  // [wave][token group][gate/up][row][lane]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nr = a.grp[0];
  const int nrt = nr + (a.shared ? 1 : 0);
  const int FT = a.F / kTile;
  const int H = a.H, F = a.F;
  const uint64_t mat = (uint64_t)F * H * (FP8 ? 1 : 2);
  const int nsc = (F / 128) * (H / 128);
  const int kq = 32 * (lane >> 4);
  const uint16_t* x = (const uint16_t*)a.x;
  uint16_t* hb = (uint16_t*)a.hbuf;
  for (int item = blockIdx.x; item < nrt * FT; item += gridDim.x) {
    const int r = item / FT, f0 = (item % FT) * kTile;
    const Item it = item_record(a, nr, r);
    const int row = f0 + (lane & 15);
    for (int tg0 = 0; tg0 < it.n; tg0 += kTokGroup) {
      const int ng = min(4, (it.n - tg0 + 15) / 16);
      int tok[4];
      bool tv[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int idx = tg0 + 16 * g + (lane & 15);
        tv[g] = g < ng && idx < it.n;
        tok[g] = tv[g] ? pair_token(a, item_pair(a, it, idx)) : 0;
      }
      f32x4 ag[4], au[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        ag[g] = f32x4{0.f, 0.f, 0.f, 0.f};
        au[g] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      for (int kc = wv * kChunk; kc < H; kc += 4 * kChunk) {
        bf16x8 wg[4], wu[4];
        float sg = 1.f, su = 1.f;
        if (FP8) {
          const uint8_t* pg = it.rec + (uint64_t)row * H + kc + kq;
          load_a_fp8(pg, wg);
          load_a_fp8(pg + mat, wu);
          const float* sc = reinterpret_cast<const float*>(it.rec + 3 * mat);
          const int si = (f0 / 128) * (H / 128) + kc / 128;
          sg = sc[si];
          su = sc[nsc + si];
        } else {
          const uint16_t* pg = reinterpret_cast<const uint16_t*>(it.rec) + (uint64_t)row * H + kc + kq;
          load_a_bf16(pg, wg);
          load_a_bf16(pg + (uint64_t)F * H, wu);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (g < ng) {
            bf16x8 b[4];
            load_b_bf16(x + (uint64_t)tok[g] * H + kc + kq, tv[g], b);
            if (FP8) {
              const f32x4 z = {0.f, 0.f, 0.f, 0.f};
              ag[g] = fma4(sg, mfma4(wg, b, z), ag[g]);
              au[g] = fma4(su, mfma4(wu, b, z), au[g]);
            } else {
              ag[g] = mfma4(wg, b, ag[g]);
              au[g] = mfma4(wu, b, au[g]);
            }
          }
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g < ng) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            red[wv][g][0][i][lane] = ag[g][i];
            red[wv][g][1][i][lane] = au[g][i];
          }
        }
      }
      __syncthreads();
      if (wv < ng) {  // wavefront g finishes token group g
        const int g = wv;
        const int idx = tg0 + 16 * g + (lane & 15);
        if (idx < it.n) {
          const int p = item_pair(a, it, idx);
          uint16_t hv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gs = ((red[0][g][0][i][lane] + red[1][g][0][i][lane]) + red[2][g][0][i][lane]) +
                             red[3][g][0][i][lane];
            const float us = ((red[0][g][1][i][lane] + red[1][g][1][i][lane]) + red[2][g][1][i][lane]) +
                             red[3][g][1][i][lane];
            hv[i] = f32_to_bf16(silu_mul(gs, us));
          }
          uint2 st;
          st.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
          st.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
          *reinterpret_cast<uint2*>(hb + (uint64_t)p * F + f0 + 4 * (lane >> 4)) = st;
        }
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ combine
// rows [r0, r0 + nrows) of y for all tokens, in j order, + shared, rounded once
template <typename A>
__device__ void combine_tile(const FfnArgs& a, int r0, int nrows) {
  const int routed = a.T * a.k;
  for (int q = threadIdx.x; q < a.T * nrows; q += blockDim.x) {
    const int t = q / nrows, rr = r0 + q % nrows;
    float acc = 0.f;
    for (int j = 0; j < a.k; ++j)
      acc = __builtin_fmaf(a.w[t * a.k + j], a.part[(uint64_t)(t * a.k + j) * a.H + rr], acc);
    if (a.shared) acc = acc + a.part[(uint64_t)(routed + t) * a.H + rr];
    const uint64_t o = (uint64_t)t * a.H + rr;
    if (sizeof(A) == 2) {
      const uint16_t yb = f32_to_bf16(acc);
      ((uint16_t*)a.y)[o] = yb;
      if (a.x_next)
        ((uint16_t*)a.x_next)[o] = f32_to_bf16(bf16_to_f32(((const uint16_t*)a.x)[o]) + bf16_to_f32(yb));
    } else {
      ((float*)a.y)[o] = acc;
      if (a.x_next) ((float*)a.x_next)[o] = ((const float*)a.x)[o] + acc;
    }
  }
}

// Counts a finished (record, tile) item; the last one for the tile combines it.
template <typename A>
__device__ void finish_tile(const FfnArgs& a, int nrt, int tile, int r0, int nrows) {
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(&a.comb_ctr[tile], 1u) == (uint32_t)(nrt - 1);
  __syncthreads();
  if (s_last) {
    __threadfence();
    if (threadIdx.x == 0) a.comb_ctr[tile] = 0;
    combine_tile<A>(a, r0, nrows);
  }
  __syncthreads();
}

// ------------------------------------------------------------------ down (bf16, fp8)
template <bool FP8>
__global__ __launch_bounds__(256) void k_down(FfnArgs a) {
  __shared__ float red[4][4][4][64];  // [wave][token group][row][lane]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nr = a.grp[0];
  const int nrt = nr + (a.shared ? 1 : 0);
  const int HT = a.H / kTile;
  const int H = a.H, F = a.F;
  const uint64_t mat = (uint64_t)F * H * (FP8 ? 1 : 2);
  const int nsc = (F / 128) * (H / 128);
  const int kq = 32 * (lane >> 4);
  const uint16_t* hb = (const uint16_t*)a.hbuf;
  for (int item = blockIdx.x; item < nrt * HT; item += gridDim.x) {
    const int r = item / HT, ht = item % HT, h0 = ht * kTile;
    const Item it = item_record(a, nr, r);
    const int row = h0 + (lane & 15);
    for (int tg0 = 0; tg0 < it.n; tg0 += kTokGroup) {
      const int ng = min(4, (it.n - tg0 + 15) / 16);
      int pr[4];
      bool tv[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int idx = tg0 + 16 * g + (lane & 15);
        tv[g] = g < ng && idx < it.n;
        pr[g] = tv[g] ? item_pair(a, it, idx) : 0;
      }
      f32x4 acc[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int kc = wv * kChunk; kc < F; kc += 4 * kChunk) {
        bf16x8 wd[4];
        float sd = 1.f;
        if (FP8) {
          load_a_fp8(it.rec + 2 * mat + (uint64_t)row * F + kc + kq, wd);
          const float* sc = reinterpret_cast<const float*>(it.rec + 3 * mat);
          sd = sc[2 * nsc + (h0 / 128) * (F / 128) + kc / 128];
        } else {
          load_a_bf16(reinterpret_cast<const uint16_t*>(it.rec + 2 * mat) + (uint64_t)row * F + kc + kq, wd);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (g < ng) {
            bf16x8 b[4];
            load_b_bf16(hb + (uint64_t)pr[g] * F + kc + kq, tv[g], b);
            if (FP8) {
              const f32x4 z = {0.f, 0.f, 0.f, 0.f};
              acc[g] = fma4(sd, mfma4(wd, b, z), acc[g]);
            } else {
              acc[g] = mfma4(wd, b, acc[g]);
            }
          }
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (g < ng) {
#pragma unroll
          for (int i = 0; i < 4; ++i) red[wv][g][i][lane] = acc[g][i];
        }
      __syncthreads();
      if (wv < ng) {
        const int g = wv;
        const int idx = tg0 + 16 * g + (lane & 15);
        if (idx < it.n) {
          const int p = item_pair(a, it, idx);
          float4 o;
          float* ov = reinterpret_cast<float*>(&o);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ov[i] = ((red[0][g][i][lane] + red[1][g][i][lane]) + red[2][g][i][lane]) + red[3][g][i][lane];
          *reinterpret_cast<float4*>(a.part + (uint64_t)p * H + h0 + 4 * (lane >> 4)) = o;
        }
      }
      __syncthreads();
    }
    finish_tile<uint16_t>(a, nrt, ht, h0, kTile);
  }
}

// ------------------------------------------------------------------ fp32 path
__global__ __launch_bounds__(256) void k_gateup_f32(FfnArgs a) {
  const int nr = a.grp[0];
  const int nrt = nr + (a.shared ? 1 : 0);
  const int FT = a.F / kF32Rows;
  const int H = a.H, F = a.F;
  const float* x = (const float*)a.x;
  float* hb = (float*)a.hbuf;
  for (int item = blockIdx.x; item < nrt * FT; item += gridDim.x) {
    const int r = item / FT, f = (item % FT) * kF32Rows + (threadIdx.x & 63);
    const Item it = item_record(a, nr, r);
    const float* wg = reinterpret_cast<const float*>(it.rec) + (uint64_t)f * H;
    const float* wu = wg + (uint64_t)F * H;
    for (int idx = threadIdx.x >> 6; idx < it.n; idx += 4) {
      const int p = item_pair(a, it, idx);
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
  const float* hb = (const float*)a.hbuf;
  for (int item = blockIdx.x; item < nrt * HT; item += gridDim.x) {
    const int r = item / HT, ht = item % HT, hr = ht * kF32Rows + (threadIdx.x & 63);
    const Item it = item_record(a, nr, r);
    const float* wd = reinterpret_cast<const float*>(it.rec) + 2ull * F * H + (uint64_t)hr * F;
    for (int idx = threadIdx.x >> 6; idx < it.n; idx += 4) {
      const int p = item_pair(a, it, idx);
      const float* hp = hb + (uint64_t)p * F;
      float o = 0.f;
      for (int f = 0; f < F; ++f) o = __builtin_fmaf(wd[f], hp[f], o);
      a.part[(uint64_t)p * H + hr] = o;
    }
    finish_tile<float>(a, nrt, ht, ht * kF32Rows, kF32Rows);
  }
}

}  // namespace

hipError_t launch_ffn(moe_offload* h, const void* x, const int32_t* slot_ids, const float* w, int T,
                      const void* shared, void* y, void* x_next, hipStream_t s) {
  FfnArgs a;
  a.x = x;
  a.slot_ids = slot_ids;
  a.w = w;
  a.slots = h->slots;
  a.staging = h->staging;
  a.shared = (const uint8_t*)shared;
  a.stride = h->record_stride;
  a.grp = h->grp;
  a.hbuf = h->hbuf;
  a.part = h->part;
  a.comb_ctr = h->comb_ctr;
  a.y = y;
  a.x_next = x_next;
  a.err = h->cache.err;
  a.T = T;
  a.k = h->k;
  a.H = h->H;
  a.F = h->F;
  a.S = h->S;
  a.E = h->E;
  a.off_list = h->gl.off_list();
  a.off_start = h->gl.off_start();
  a.off_pairs = h->gl.off_pairs();
  // distinct records a call can touch (+ the shared expert)
  const int max_items_r = std::min(T * h->k, h->E) + (shared ? 1 : 0);
  hipLaunchKernelGGL(k_group, dim3(1), dim3(kGrpBlock), 0, s, a);
  if (h->dtype == MOE_F32) {
    const int g1 = std::min(max_items_r * (h->F / kF32Rows), 2048);
    const int g2 = std::min(max_items_r * (h->H / kF32Rows), 2048);
    hipLaunchKernelGGL(k_gateup_f32, dim3(g1), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_down_f32, dim3(g2), dim3(256), 0, s, a);
  } else {
    const int g1 = std::min(max_items_r * (h->F / kTile), 4096);
    const int g2 = std::min(max_items_r * (h->H / kTile), 4096);
    if (h->dtype == MOE_FP8_E4M3_B128) {
      hipLaunchKernelGGL(k_gateup<true>, dim3(g1), dim3(256), 0, s, a);
      hipLaunchKernelGGL(k_down<true>, dim3(g2), dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL(k_gateup<false>, dim3(g1), dim3(256), 0, s, a);
      hipLaunchKernelGGL(k_down<false>, dim3(g2), dim3(256), 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
