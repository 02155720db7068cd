// norm.hpp -- gated RMSNorm arithmetic on 4 consecutive elements of a head,
// shared by the 16-byte norm kernel and the fused decode kernel so that both
// produce the same bits.
//
// fm_kernel_ssm.h (Foundry), "Gated RMSNorm" section:
// out = ((y * rsqrt(mean(y^2) + eps)) * w) * silu(z), mean over the head.
#pragma once
#include <hip/hip_runtime.h>

#include "wave.hpp"

namespace gdn {

// y.x^2 + y.y^2 + y.z^2 + y.w^2, in that order, with explicit FMAs
__device__ __forceinline__ float sumsq4(const float4 &y) {
  float ss = y.x * y.x;
  ss = __builtin_fmaf(y.y, y.y, ss);
  ss = __builtin_fmaf(y.z, y.z, ss);
  ss = __builtin_fmaf(y.w, y.w, ss);
  return ss;
}

// 1 / sqrt(sum / head_dim + eps) from the head's summed squares
__device__ __forceinline__ float norm_inv(float ss, int hd, float eps) {
  return 1.0f / sqrtf(ss / (float)hd + eps);
}

__device__ __forceinline__ float4 gated_norm4(const float4 &y, const float4 &z, const float4 &w,
                                              float inv) {
  return make_float4(((y.x * inv) * w.x) * silu(z.x), ((y.y * inv) * w.y) * silu(z.y),
                     ((y.z * inv) * w.z) * silu(z.z), ((y.w * inv) * w.w) * silu(z.w));
}

}  // namespace gdn
