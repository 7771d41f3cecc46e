// Per-token RMS normalisation of the residual stream, the input of each MoE
// block in the decode-step chain: xn = x / sqrt(mean(x^2) + eps), no learned
// scale, rounded once to the activation dtype.  One 256-thread workgroup per
// token, in the order of rownorm.h (shared with the fused norm of the combine).
#include <math.h>

#include "internal.h"
#include "rownorm.h"

namespace moe {
namespace {

template <bool F32>
__global__ __launch_bounds__(kRowThreads) void k_rmsnorm(const void* __restrict__ x, void* __restrict__ out, int H,
                                                          float eps) {
  __shared__ float s_wave[4];
  const size_t off = (size_t)blockIdx.x * H * (F32 ? 4 : 2);
  const void* row = (const uint8_t*)x + off;
  float ss = 0.f;
  for (int c = threadIdx.x; c * 8 < H; c += kRowThreads) {
    float v[8];
    chunk_load<F32>(row, c, v);
    ss = chunk_sumsq(v, ss);
  }
  const float inv = row_inv_rms(row_block_sum(ss, s_wave), H, eps);
  row_scale_chunks<F32>(row, (uint8_t*)out + off, H, inv);
}

}  // namespace

hipError_t launch_rmsnorm(const void* x, void* out, int T, int H, int dtype, float eps, hipStream_t s) {
  if (dtype == MOE_F32)
    hipLaunchKernelGGL(k_rmsnorm<true>, dim3(T), dim3(kRowThreads), 0, s, x, out, H, eps);
  else
    hipLaunchKernelGGL(k_rmsnorm<false>, dim3(T), dim3(kRowThreads), 0, s, x, out, H, eps);
  return hipGetLastError();
}

}  // namespace moe
