// conv.hpp -- per-lane pieces of the depthwise causal conv1d + SiLU + per-head
// L2 norm (fm_kernel_ssm.h (Foundry), "Causal depthwise conv1d + SiLU"
// section; ssm_mamba.rs (spark_model), conv1d_update_l2norm).  Shared by the
// conv kernels and the fused decode step, so every caller computes a channel
// with the same lane map and the same FMA order and their results agree bit
// for bit.
//
// Lane map: a lane owns CPL = 4 consecutive channels c0 .. c0 + 3; an L2 head
// of head_dim channels is head_dim / 4 consecutive, aligned lanes (LPH4), and
// its sum of squares is an in-wave xor butterfly (wave.hpp), so every lane of
// the wave must be active where conv_step4 runs.
#pragma once
#include <hip/hip_runtime.h>

#include "wave.hpp"

namespace gdn {

constexpr int CPL = 4;   // channels per lane

// SiLU of a conv output, a / (1 + e^-a), on the hardware base-2 exponential
// (of -a log2(e)) and reciprocal, each about 1 ulp: a few instructions where
// the libm exponential and a correctly rounded division take dozens, which
// matters where the conv runs inside a compute-bound kernel.  For a below
// about -88 the exponential overflows and the result is -0 (the exact value
// is below 1e-36 in magnitude).
__device__ __forceinline__ float conv_silu(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * 1.4426950408889634f));
}

// acc = sum_j w[j] * win[j] in tap order, oldest tap first, explicit FMAs.
template <int D>
__device__ __forceinline__ float conv_position(const float (&w)[D], const float (&win)[D]) {
  float acc = w[0] * win[0];
#pragma unroll
  for (int j = 1; j < D; ++j) acc = __builtin_fmaf(w[j], win[j], acc);
  return conv_silu(acc);
}

// 1 / sqrt(x) for the L2 step, the hardware reciprocal square root (about
// 1 ulp; x >= eps > 0 here): one instruction where a correctly rounded square
// root and division take about thirty.
__device__ __forceinline__ float l2_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }

// 1 / sqrt(sum over the lane's L2 head of o^2 + eps); LPH4 lanes per head.
template <int LPH4>
__device__ __forceinline__ float l2_scale(const float (&o)[CPL], float eps) {
  float ss = o[0] * o[0];
#pragma unroll
  for (int c = 1; c < CPL; ++c) ss = __builtin_fmaf(o[c], o[c], ss);
  ss = group_sum<LPH4>(ss);
  return l2_rsqrt(ss + eps);
}

// The lane's channels: chc[c] is channel c0 + c clamped to the last channel
// (lanes past the end compute on valid data and store nothing), ok[c] says
// whether it exists.  c0v is the float4 base of VEC loads: with C a multiple
// of 4 a lane is all valid or all past the end, and c0v is c0 or the last
// group of 4.
struct LaneChans {
  int c0, c0v;
  int chc[CPL];
  bool ok[CPL];
  bool all_ok;
};
__device__ __forceinline__ LaneChans lane_chans(int blk0, int lane, int C) {
  LaneChans L;
  L.c0 = blk0 + 4 * lane;
  L.c0v = min(L.c0, C - 4);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    L.ok[c] = L.c0 + c < C;
    L.chc[c] = min(L.c0 + c, C - 1);
  }
  L.all_ok = L.c0 + CPL - 1 < C;
  return L;
}

// The lane's 4 values of one per-position row.  No load sits behind a branch:
// a branch would make the compiler wait for every load in flight where it
// rejoins.
template <bool VEC>
__device__ __forceinline__ void load_row4(const float *__restrict__ row, const LaneChans &L,
                                          float (&v)[CPL]) {
  if constexpr (VEC) {
    const float4 t = *reinterpret_cast<const float4 *>(row + L.c0v);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else {
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = row[L.chc[c]];
  }
}
template <bool VEC>
__device__ __forceinline__ void store_row4(float *__restrict__ row, const LaneChans &L,
                                           const float (&v)[CPL]) {
  if constexpr (VEC) {
    if (L.all_ok) *reinterpret_cast<float4 *>(row + L.c0) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      if (L.ok[c]) row[L.c0 + c] = v[c];
  }
}

// The lane's 4 channels' records of N floats each ([channel][N] layout: taps,
// history, snapshots): 4N consecutive floats, N 16-byte accesses when VEC.
// The 16-byte form in two halves: the raw loads, and their unpacking into
// [channel][N] order.  A caller that issues other loads in between keeps the
// unpacking (which needs the data) from waiting before those are issued.
typedef float conv_f4 __attribute__((ext_vector_type(4)));
template <int N>
__device__ __forceinline__ void load_recs_raw(const float *__restrict__ p, const LaneChans &L,
                                              conv_f4 (&raw)[N]) {
#pragma unroll
  for (int q = 0; q < N; ++q) raw[q] = *reinterpret_cast<const conv_f4 *>(p + (int64_t)L.c0v * N + 4 * q);
}
template <int N>
__device__ __forceinline__ void unpack_recs(const conv_f4 (&raw)[N], float (&r)[CPL][N]) {
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const float f[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) r[(4 * q + e) / N][(4 * q + e) % N] = f[e];
  }
}

template <int N, bool VEC>
__device__ __forceinline__ void load_recs(const float *__restrict__ p, const LaneChans &L,
                                          float (&r)[CPL][N]) {
  if constexpr (VEC) {
    conv_f4 raw[N];
    load_recs_raw<N>(p, L, raw);
    unpack_recs<N>(raw, r);
  } else {
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int j = 0; j < N; ++j) r[c][j] = p[(int64_t)L.chc[c] * N + j];
  }
}
template <int N, bool VEC>
__device__ __forceinline__ void store_recs(float *__restrict__ p, const LaneChans &L,
                                           const float (&r)[CPL][N]) {
  if constexpr (VEC) {
    if (L.all_ok) {
#pragma unroll
      for (int q = 0; q < N; ++q) {
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = r[(4 * q + e) / N][(4 * q + e) % N];
        *reinterpret_cast<float4 *>(p + (int64_t)L.c0 * N + 4 * q) =
            make_float4(f[0], f[1], f[2], f[3]);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      if (L.ok[c]) {
#pragma unroll
        for (int j = 0; j < N; ++j) p[(int64_t)(L.c0 + c) * N + j] = r[c][j];
      }
  }
}

// Taps and history of the lane's channels (once per wave).
template <int D, bool VEC>
__device__ __forceinline__ void load_taps_hist(const float *__restrict__ w,
                                               const float *__restrict__ hist, const LaneChans &L,
                                               float (&wt)[CPL][D], float (&hv)[CPL][D - 1]) {
  load_recs<D, VEC>(w, L, wt);
  load_recs<D - 1, VEC>(hist, L, hv);
}

// The window's first D-1 slots (the history after the last position).
template <int D>
__device__ __forceinline__ void window_hist(const float (&win)[CPL][D], float (&h)[CPL][D - 1]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int j = 0; j < D - 1; ++j) h[c][j] = win[c][j];
}

// One position: output of the lane's 4 channels from the window, which then
// rolls with the raw input.  LPH4 == 0: SiLU only (no Q/K channel here).
template <int D, int LPH4>
__device__ __forceinline__ void conv_step4(const float (&wt)[CPL][D], float (&win)[CPL][D],
                                           const float (&xv)[CPL], bool qk, float eps,
                                           float (&o)[CPL]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    win[c][D - 1] = xv[c];
    o[c] = conv_position<D>(wt[c], win[c]);
#pragma unroll
    for (int j = 0; j < D - 1; ++j) win[c][j] = win[c][j + 1];
  }
  if constexpr (LPH4 > 0) {
    const float inv = l2_scale<LPH4>(o, eps);
    if (qk) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[c] *= inv;
    }
  }
}

}  // namespace gdn
