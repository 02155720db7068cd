// recur.hpp -- per-row pieces of the token-by-token recurrence, shared by
// the decode kernel and the fused decode kernel.
//
// Math: fm_kernel_ssm.h (Foundry), "Delta-rule recurrence" section.  The
// state is stored transposed, state[j][i] = S[i][j]: a 16-lane DPP row holds
// value row j, lane l holding key elements {64m + 4l + c} (S >= 64) or
// {2l, 2l+1} (S = 32).
#pragma once
#include <hip/hip_runtime.h>

#include "wave.hpp"

namespace gdn {

template <int S>
struct RowMap {
  static constexpr int EPL = S / 16;                // floats per lane per row
  static constexpr int VEC = S >= 64 ? 4 : 2;      // floats per vector access
  static constexpr int NV = EPL / VEC;             // vector accesses per row
  // offset of vector access m of lane l16 within a row
  __device__ static int off(int l16, int m) { return S >= 64 ? 64 * m + 4 * l16 : 2 * l16; }
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// NT selects non-temporal accesses: the state streams through once per call,
// so its lines are not kept in the caches, which leaves them to k, q and v,
// read by every wave of a head.
template <int S, bool NT = false>
__device__ __forceinline__ void load_row(const float *p, int l16, float (&r)[S / 16]) {
  using M = RowMap<S>;
#pragma unroll
  for (int m = 0; m < M::NV; ++m) {
    if constexpr (M::VEC == 4) {
      const f32x4 *a = reinterpret_cast<const f32x4 *>(p + M::off(l16, m));
      const f32x4 t = NT ? __builtin_nontemporal_load(a) : *a;
      r[4 * m] = t.x; r[4 * m + 1] = t.y; r[4 * m + 2] = t.z; r[4 * m + 3] = t.w;
    } else {
      const f32x2 *a = reinterpret_cast<const f32x2 *>(p + M::off(l16, m));
      const f32x2 t = NT ? __builtin_nontemporal_load(a) : *a;
      r[2 * m] = t.x; r[2 * m + 1] = t.y;
    }
  }
}

template <int S, bool NT = false>
__device__ __forceinline__ void store_row(float *p, int l16, const float (&r)[S / 16]) {
  using M = RowMap<S>;
#pragma unroll
  for (int m = 0; m < M::NV; ++m) {
    if constexpr (M::VEC == 4) {
      f32x4 *a = reinterpret_cast<f32x4 *>(p + M::off(l16, m));
      const f32x4 t = {r[4 * m], r[4 * m + 1], r[4 * m + 2], r[4 * m + 3]};
      if constexpr (NT) __builtin_nontemporal_store(t, a); else *a = t;
    } else {
      f32x2 *a = reinterpret_cast<f32x2 *>(p + M::off(l16, m));
      const f32x2 t = {r[2 * m], r[2 * m + 1]};
      if constexpr (NT) __builtin_nontemporal_store(t, a); else *a = t;
    }
  }
}

// One position for RG rows held by this lane.  Shared by every n_tok, so a
// K-position call and K one-position calls execute the same operations.
template <int S, int RG>
__device__ __forceinline__ void recur_position(float (&st)[RG][S / 16], const float (&kv)[S / 16],
                                               const float (&qv)[S / 16], const float (&vj)[RG],
                                               float gamma, float b, float (&yo)[RG]) {
  constexpr int EPL = S / 16;
  float p[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) st[r][e] *= gamma;  // decay
    float acc = st[r][0] * kv[0];
#pragma unroll
    for (int e = 1; e < EPL; ++e) acc = __builtin_fmaf(st[r][e], kv[e], acc);
    p[r] = acc;
  }
#pragma unroll
  for (int r = 0; r < RG; ++r) p[r] = sum16(p[r]);  // p = S^T k, row j
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const float delta = b * (vj[r] - p[r]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) st[r][e] = __builtin_fmaf(kv[e], delta, st[r][e]);
    float acc = st[r][0] * qv[0];
#pragma unroll
    for (int e = 1; e < EPL; ++e) acc = __builtin_fmaf(st[r][e], qv[e], acc);
    yo[r] = acc;
  }
#pragma unroll
  for (int r = 0; r < RG; ++r) yo[r] = sum16(yo[r]);  // S^T q, row j
}

}  // namespace gdn
