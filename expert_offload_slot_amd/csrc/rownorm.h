// Per-token RMS normalisation helpers shared by every kernel that normalises a
// row, so they all produce the same bits.  One 256-thread workgroup per row:
// thread i owns the chunks of 8 elements c = i, i + 256, ... and accumulates
// their squares with FMAs in element order; each wavefront then combines its
// lanes with an xor-butterfly (offsets 32..1) and the four wavefront sums are
// added in wavefront order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kRowThreads = 256;

__device__ __forceinline__ float rn_bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float rn_bf_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t rn_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// load / store one chunk of 8 activations as floats
template <bool F32>
__device__ __forceinline__ void chunk_load(const void* row, int c, float v[8]) {
  if (F32) {
    const float4* p = reinterpret_cast<const float4*>((const float*)row + c * 8);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 a = *reinterpret_cast<const uint4*>((const uint16_t*)row + c * 8);
    v[0] = rn_bf_lo(a.x); v[1] = rn_bf_hi(a.x); v[2] = rn_bf_lo(a.y); v[3] = rn_bf_hi(a.y);
    v[4] = rn_bf_lo(a.z); v[5] = rn_bf_hi(a.z); v[6] = rn_bf_lo(a.w); v[7] = rn_bf_hi(a.w);
  }
}

// rounds v to the activation type (bf16 RNE; fp32 unchanged) and, if row is not
// null, stores the chunk.  `v` is updated to the rounded values.
template <bool F32>
__device__ __forceinline__ void chunk_store(void* row, int c, float v[8]) {
  if (F32) {
    if (!row) return;
    float4* p = reinterpret_cast<float4*>((float*)row + c * 8);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint32_t b[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      b[q] = rn_to_bf16(v[q]);
      v[q] = __uint_as_float(b[q] << 16);
    }
    if (row)
      *reinterpret_cast<uint4*>((uint16_t*)row + c * 8) =
          make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
  }
}

// Top-k weighted combine of one chunk of 8 outputs of token t:
//   acc = sum over j < k, in j order, of fma(w[j], part[j][8c .. 8c+7]), then + shared[8c ..]
// (part: the token's k fp32 partial-output rows of H; shared: its shared-expert
// row or null), and res = the residual chunk (rrow null: not loaded).  Every
// load of the chunk is issued before the first arithmetic on it (up to eight
// partial rows at a time), so a chunk costs one memory round trip for k <= 8
// instead of one per choice; the operations and their order are those of the
// plain loop.
template <bool F32>
__device__ __forceinline__ void combine_chunk(const float* part, const float* w, int k, int H, int c,
                                              const float* shared, const void* rrow, float acc[8], float res[8]) {
  uint4 rb = make_uint4(0, 0, 0, 0);
  float4 rf0 = make_float4(0.f, 0.f, 0.f, 0.f), rf1 = rf0, s0 = rf0, s1 = rf0;
  if (rrow) {
    if (F32) {
      const float4* p = reinterpret_cast<const float4*>((const float*)rrow + c * 8);
      rf0 = p[0];
      rf1 = p[1];
    } else {
      rb = *reinterpret_cast<const uint4*>((const uint16_t*)rrow + c * 8);
    }
  }
  if (shared) {
    const float4* p = reinterpret_cast<const float4*>(shared + c * 8);
    s0 = p[0];
    s1 = p[1];
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  for (int j0 = 0; j0 < k; j0 += 8) {
    float4 p0[8], p1[8];
    float wj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u < k) {
        wj[u] = w[j0 + u];
        const float4* pr = reinterpret_cast<const float4*>(part + (uint64_t)(j0 + u) * H + c * 8);
        p0[u] = pr[0];
        p1[u] = pr[1];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u < k) {
        acc[0] = __builtin_fmaf(wj[u], p0[u].x, acc[0]); acc[1] = __builtin_fmaf(wj[u], p0[u].y, acc[1]);
        acc[2] = __builtin_fmaf(wj[u], p0[u].z, acc[2]); acc[3] = __builtin_fmaf(wj[u], p0[u].w, acc[3]);
        acc[4] = __builtin_fmaf(wj[u], p1[u].x, acc[4]); acc[5] = __builtin_fmaf(wj[u], p1[u].y, acc[5]);
        acc[6] = __builtin_fmaf(wj[u], p1[u].z, acc[6]); acc[7] = __builtin_fmaf(wj[u], p1[u].w, acc[7]);
      }
    }
  }
  if (shared) {
    acc[0] = acc[0] + s0.x; acc[1] = acc[1] + s0.y; acc[2] = acc[2] + s0.z; acc[3] = acc[3] + s0.w;
    acc[4] = acc[4] + s1.x; acc[5] = acc[5] + s1.y; acc[6] = acc[6] + s1.z; acc[7] = acc[7] + s1.w;
  }
  if (F32) {
    res[0] = rf0.x; res[1] = rf0.y; res[2] = rf0.z; res[3] = rf0.w;
    res[4] = rf1.x; res[5] = rf1.y; res[6] = rf1.z; res[7] = rf1.w;
  } else {
    res[0] = rn_bf_lo(rb.x); res[1] = rn_bf_hi(rb.x); res[2] = rn_bf_lo(rb.y); res[3] = rn_bf_hi(rb.y);
    res[4] = rn_bf_lo(rb.z); res[5] = rn_bf_hi(rb.z); res[6] = rn_bf_lo(rb.w); res[7] = rn_bf_hi(rb.w);
  }
}

__device__ __forceinline__ float chunk_sumsq(const float v[8], float ss) {
#pragma unroll
  for (int q = 0; q < 8; ++q) ss = __builtin_fmaf(v[q], v[q], ss);
  return ss;
}

// sum over the 256 threads of the workgroup in the fixed order above; every
// thread gets the result.  Must be called by all threads of the workgroup.
__device__ __forceinline__ float row_block_sum(float v, float* s_wave /* [4] */) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) s_wave[threadIdx.x >> 6] = v;
  __syncthreads();
  const float tot = ((s_wave[0] + s_wave[1]) + s_wave[2]) + s_wave[3];
  __syncthreads();
  return tot;
}

__device__ __forceinline__ float row_inv_rms(float ss, int H, float eps) { return 1.0f / sqrtf(ss / (float)H + eps); }

// out = round(row * inv) for this thread's chunks (row may have been written by this thread)
template <bool F32>
__device__ __forceinline__ void row_scale_chunks(const void* row, void* out, int H, float inv) {
  for (int c = threadIdx.x; c * 8 < H; c += kRowThreads) {
    float v[8];
    chunk_load<F32>(row, c, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] *= inv;
    chunk_store<F32>(out, c, v);
  }
}

}  // namespace moe
