// k_norm.hip -- gated RMSNorm, out = ((y * rsqrt(mean(y^2) + eps)) * w) * silu(z)
// per (row, head), with the weight shared by every head.
//
// Math and multiply order: fm_kernel_ssm.h (Foundry), "Gated RMSNorm" section.
// z read from a wider per-token row at an offset: ssm_mamba.rs (spark_model),
// gdn_verify_fused_norm_k2 (the caller passes z already offset).
//
// Thread maps (each lane reads its own y before any lane writes, so out may be
// y itself; the sum of squares is an in-wave xor butterfly):
//   k_gated_rmsnorm_v4 : lane i of the launch owns elements 4i .. 4i+3 of the
//     flattened [rows][H * head_dim] space, one 16-byte access per tensor;
//     a head is head_dim/4 consecutive lanes, so one wave covers 256 elements
//     (possibly of several rows).  Used when every pointer is 16-byte aligned
//     and every row stride is a multiple of 4 elements.
//   k_gated_rmsnorm : any alignment; one wave64 per block of 64*CPL
//     consecutive elements of a row, lane l holding elements l, l+64, ..; a
//     block is one head (head_dim >= 64) or two heads of 32 lanes.
#include <hip/hip_runtime.h>

#include "gdn.h"
#include "launch.hpp"
#include "norm.hpp"
#include "wave.hpp"

namespace gdn {

template <int CPL, int LPH>
__global__ __launch_bounds__(256) void k_gated_rmsnorm(const float *y, int64_t y_row,
                                                       const float *__restrict__ w,
                                                       const float *__restrict__ z, int64_t z_row,
                                                       float *out, int64_t o_row, int rows,
                                                       int row_elems, int waves_per_row, int hd,
                                                       float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t r = wave / waves_per_row;
  if (r >= rows) return;  // uniform per wave
  const int e0 = (int)(wave - r * waves_per_row) * 64 * CPL + lane;
  const float *yr = y + r * y_row;
  const float *zr = z + r * z_row;
  float *orow = out + r * o_row;

  float yv[CPL], zv[CPL];
  bool ok[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int e = e0 + 64 * c;
    ok[c] = e < row_elems;
    yv[c] = ok[c] ? yr[e] : 0.0f;
    zv[c] = ok[c] ? zr[e] : 0.0f;
  }
  float ss = yv[0] * yv[0];
#pragma unroll
  for (int c = 1; c < CPL; ++c) ss = __builtin_fmaf(yv[c], yv[c], ss);
  ss = group_sum<LPH>(ss);
  const float inv = 1.0f / sqrtf(ss / (float)hd + eps);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    if (!ok[c]) continue;
    const int e = e0 + 64 * c;
    const int col = e % hd;  // position inside the head: the shared weight index
    orow[e] = ((yv[c] * inv) * w[col]) * silu(zv[c]);
  }
}

// LPH4 = head_dim / 4 lanes per head.  Lanes past the end load a clamped
// (valid) float4 and store nothing; heads never straddle that boundary, so no
// valid head sums an invalid lane.  y, z and out stream through once, so
// their accesses are non-temporal (at 4096 rows x 32 heads x 128: 36.6 us
// against 39.7 us with ordinary accesses); the shared weight stays cached.
typedef float norm_f4 __attribute__((ext_vector_type(4)));
template <int LPH4>
__global__ __launch_bounds__(256) void k_gated_rmsnorm_v4(const float *y, int64_t y_row,
                                                          const float *__restrict__ w,
                                                          const float *__restrict__ z,
                                                          int64_t z_row, float *out, int64_t o_row,
                                                          unsigned total4, unsigned row4,
                                                          float eps) {
  constexpr int HD = 4 * LPH4;
  const unsigned i4 = blockIdx.x * blockDim.x + threadIdx.x;
  const unsigned ic = i4 < total4 ? i4 : total4 - 1;
  const unsigned r = ic / row4;
  const int e = (int)(ic - r * row4) * 4;
  const int col = e % HD;
  const norm_f4 yn = __builtin_nontemporal_load(reinterpret_cast<const norm_f4 *>(y + r * y_row + e));
  const norm_f4 zn = __builtin_nontemporal_load(reinterpret_cast<const norm_f4 *>(z + r * z_row + e));
  const float4 yv = make_float4(yn.x, yn.y, yn.z, yn.w);
  const float4 zv = make_float4(zn.x, zn.y, zn.z, zn.w);
  const float4 wv = *reinterpret_cast<const float4 *>(w + col);
  const float ss = group_sum<LPH4>(sumsq4(yv));
  const float4 o = gated_norm4(yv, zv, wv, norm_inv(ss, HD, eps));
  if (i4 < total4) {
    const norm_f4 on = {o.x, o.y, o.z, o.w};
    __builtin_nontemporal_store(on, reinterpret_cast<norm_f4 *>(out + r * o_row + e));
  }
}

namespace {
template <int CPL, int LPH>
int run_norm(const NormArgs &a, hipStream_t stream) {
  const int row_elems = a.H * a.hd;
  const int waves_per_row = (row_elems + 64 * CPL - 1) / (64 * CPL);
  const int64_t waves = (int64_t)a.rows * waves_per_row;
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  return launch_kernel(k_gated_rmsnorm<CPL, LPH>, dim3(blocks), dim3(256), 0, stream, a.y,
                       a.y_row, a.w, a.z, a.z_row, a.out, a.o_row, a.rows, row_elems,
                       waves_per_row, a.hd, a.eps);
}
}  // namespace

namespace {
template <int LPH4>
int run_norm_v4(const NormArgs &a, unsigned total4, hipStream_t stream) {
  const unsigned blocks = (total4 + 255) / 256;
  return launch_kernel(k_gated_rmsnorm_v4<LPH4>, dim3(blocks), dim3(256), 0, stream, a.y, a.y_row,
                       a.w, a.z, a.z_row, a.out, a.o_row, total4,
                       (unsigned)(a.H * a.hd / 4), a.eps);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
}  // namespace

int launch_gated_rmsnorm(const NormArgs &a, hipStream_t stream) {
  if (a.rows == 0) return GDN_OK;
  const int64_t total4 = (int64_t)a.rows * a.H * a.hd / 4;
  if (aligned16(a.y) && aligned16(a.z) && aligned16(a.out) && aligned16(a.w) &&
      a.y_row % 4 == 0 && a.z_row % 4 == 0 && a.o_row % 4 == 0 && total4 < (int64_t)1 << 31) {
    switch (a.hd) {
      case 32: return run_norm_v4<8>(a, (unsigned)total4, stream);
      case 64: return run_norm_v4<16>(a, (unsigned)total4, stream);
      case 128: return run_norm_v4<32>(a, (unsigned)total4, stream);
      case 256: return run_norm_v4<64>(a, (unsigned)total4, stream);
      default: break;
    }
  }
  switch (a.hd) {
    case 32: return run_norm<1, 32>(a, stream);
    case 64: return run_norm<1, 64>(a, stream);
    case 128: return run_norm<2, 64>(a, stream);
    case 256: return run_norm<4, 64>(a, stream);
    default: return GDN_ERR_UNSUPPORTED;
  }
}

}  // namespace gdn
