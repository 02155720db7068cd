// k_fused.hip -- the decode / K-position verify layer core in one launch:
// decay gate -> gated delta-rule recurrence -> gated RMSNorm.
//
// fm_kernel_ssm.h (Foundry) notes that the decay gate costs only its dispatch
// and should ride with its neighbours rather than run alone; ssm_mamba.rs
// (spark_model), conv1d_update_l2norm, fuses neighbouring ops to save a
// launch per layer.  Here the gate and the norm ride with the recurrence.
//
// Every value is computed by the same device functions as the separate
// kernels (gate.hpp, recur.hpp, norm.hpp) in the same order, so on 16-byte
// aligned buffers the outputs equal, bit for bit, those of gdn_decay_gate ->
// gdn_recurrence_decode -> gdn_gated_rmsnorm (whose norm then takes its
// 16-byte path).
//
// Thread map: one workgroup per (sequence, value head), S / (4 RG) waves; a
// 16-lane DPP row owns a state row as in the decode kernel, 4 RG rows per
// wave, so the workgroup holds the whole head.  Per position, the row leaders
// write y[j] into LDS; after one barrier every wave reads the head's y as
// S/4 lanes of float4 (lanes past S/4 repeat the last group and store
// nothing), forms the same sum of squares as the norm kernel, and wave 0
// stores the normed output.  y is double-buffered in LDS so one barrier per
// position suffices.
//
// When to use it: the single launch replaces three, which dominates at small
// batches (one sequence of 32 heads: 15.3 us against 28.5 us for the three
// calls).  At 64 sequences x 48 heads the two are even (70.2 us against
// 70.9 us): a whole head per workgroup streams the state a little slower than
// the decode kernel's 4-wave blocks, and the per-position barrier holds every
// wave of a head to the slowest.
#include <hip/hip_runtime.h>

#include "gate.hpp"
#include "gdn.h"
#include "launch.hpp"
#include "norm.hpp"
#include "recur.hpp"
#include "wave.hpp"

namespace gdn {

template <int S, int RG>
__global__ __launch_bounds__(16 * S / RG) void k_decode_fused(
    float *__restrict__ state, int64_t st_seq, const float *__restrict__ q,
    const float *__restrict__ k, int64_t qk_tok, int64_t qk_seq, const float *__restrict__ v,
    int64_t v_tok, int64_t v_seq, const float *__restrict__ alpha, const float *__restrict__ dt,
    const float *__restrict__ a, const float *__restrict__ beta, const float *__restrict__ nw,
    const float *__restrict__ z, int64_t z_tok, int64_t z_seq, float *__restrict__ out,
    int64_t o_tok, int64_t o_seq, float *__restrict__ g_out, float *__restrict__ y_out,
    int64_t y_tok, int64_t y_seq, float *__restrict__ snap, int64_t sn_seq, int n_tok, int H,
    int Hk, float scale, float eps) {
  constexpr int EPL = S / 16;
  constexpr int L4 = S / 4;   // lanes of float4 that cover a head
  __shared__ __attribute__((aligned(16))) float ybuf[2][S];
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int wv = threadIdx.x >> 6;
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int hk = h / (H / Hk);
  const int row0 = wv * 4 * RG + (lane >> 4);  // + 4r

  float *st_base = state + s * st_seq + (int64_t)h * S * S;
  float st[RG][EPL];
#pragma unroll
  for (int r = 0; r < RG; ++r) load_row<S, true>(st_base + (int64_t)(row0 + 4 * r) * S, l16, st[r]);

  const float *qs = q + s * qk_seq + (int64_t)hk * S;
  const float *ks = k + s * qk_seq + (int64_t)hk * S;
  const float *vs = v + s * v_seq + (int64_t)h * S;
  const int64_t gb0 = (int64_t)s * n_tok * H + h;   // (s, t, h) = gb0 + t * H
  const float dth = dt[h], ah = a[h];
  // the norm lanes: float4 group e4 of the head (lanes past L4 repeat the last)
  const int e4 = 4 * (lane < L4 ? lane : L4 - 1);
  const float4 w4 = *reinterpret_cast<const float4 *>(nw + e4);

  for (int t = 0; t < n_tok; ++t) {
    float kv[EPL], qv[EPL], vj[RG], yo[RG];
    load_row<S>(ks + t * qk_tok, l16, kv);
    load_row<S>(qs + t * qk_tok, l16, qv);
#pragma unroll
    for (int r = 0; r < RG; ++r) vj[r] = vs[t * v_tok + row0 + 4 * r];
    const float4 z4 = *reinterpret_cast<const float4 *>(z + s * z_seq + t * z_tok +
                                                         (int64_t)h * S + e4);
    const float gval = decay_gate_value(alpha[gb0 + (int64_t)t * H], dth, ah);
    const float b = beta[gb0 + (int64_t)t * H];
    recur_position<S, RG>(st, kv, qv, vj, expf(gval), b, yo);
    float *yb = ybuf[t & 1];
    if (l16 == 0) {
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const float yv = scale * yo[r];
        yb[row0 + 4 * r] = yv;
        if (y_out != nullptr) y_out[s * y_seq + t * y_tok + (int64_t)h * S + row0 + 4 * r] = yv;
      }
    }
    if (g_out != nullptr && threadIdx.x == 0) g_out[gb0 + (int64_t)t * H] = gval;
    if (snap != nullptr && t < n_tok - 1) {
      float *sp = snap + s * sn_seq + (int64_t)t * H * S * S + (int64_t)h * S * S;
#pragma unroll
      for (int r = 0; r < RG; ++r) store_row<S, true>(sp + (int64_t)(row0 + 4 * r) * S, l16, st[r]);
    }
    if (t == n_tok - 1) {
      // the final state is stored before the barrier, so each wave's writes
      // drain while the slower waves of the head finish
#pragma unroll
      for (int r = 0; r < RG; ++r)
        store_row<S, true>(st_base + (int64_t)(row0 + 4 * r) * S, l16, st[r]);
    }
    __syncthreads();
    // gated RMSNorm of position t: every wave forms the (identical) head sum;
    // wave 0 stores
    const float4 y4 = *reinterpret_cast<const float4 *>(yb + e4);
    const float ss = group_sum<L4>(sumsq4(y4));
    const float4 o4 = gated_norm4(y4, z4, w4, norm_inv(ss, S, eps));
    if (wv == 0 && lane < L4)
      *reinterpret_cast<float4 *>(out + s * o_seq + t * o_tok + (int64_t)h * S + e4) = o4;
  }
}

namespace {

template <int S, int RG>
int run_fused(const FusedArgs &a, hipStream_t stream) {
  static_assert(S % (4 * RG) == 0 && S / (4 * RG) <= 16, "a workgroup holds the whole head");
  const dim3 grid((unsigned)a.r.H, (unsigned)a.r.n_seq);
  return launch_kernel(k_decode_fused<S, RG>, grid, dim3(64 * (S / (4 * RG))), 0, stream,
                       a.r.state, a.r.st_seq, a.r.q, a.r.k, a.r.qk_tok, a.r.qk_seq, a.r.v,
                       a.r.v_tok, a.r.v_seq, a.alpha, a.dt, a.a, a.r.beta, a.w, a.z, a.z_tok,
                       a.z_seq, a.r.y, a.r.y_tok, a.r.y_seq, a.g, a.y, a.y_tok, a.y_seq, a.r.snap,
                       a.r.sn_seq, a.r.n_tok, a.r.H, a.r.Hk, a.r.scale, a.eps);
}

}  // namespace

int launch_decode_fused(const FusedArgs &a, hipStream_t stream) {
  // rows per lane: enough that one workgroup (at most 16 waves) holds a head;
  // at S = 128, 4 rows per lane (8 waves) beat 2 (16 waves) from one sequence
  // (15.3 against 16.0 us, 32 heads) to 64 (70.2 against 73.4 us, 48 heads)
  // at S = 256, 8 rows per lane keep the state in registers (with 4 the
  // 16-wave bound of 128 registers spills)
  switch (a.r.S) {
    case 32: return run_fused<32, 1>(a, stream);
    case 64: return run_fused<64, 1>(a, stream);
    case 128: return run_fused<128, 4>(a, stream);
    case 256: return run_fused<256, 8>(a, stream);
    default: return GDN_ERR_UNSUPPORTED;
  }
}

}  // namespace gdn
