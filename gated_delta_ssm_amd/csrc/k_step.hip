// k_step.hip -- the whole decode / K-position verify layer core in one launch:
// conv1d + SiLU + L2 -> decay gate -> gated delta-rule recurrence -> gated
// RMSNorm.
//
// ssm_mamba.rs (spark_model), gdn_verify_fused_conv_k2, runs the conv, its
// rollback snapshot and the recurrence of a K = 2 verify in one launch, and
// conv1d_update_l2norm fuses neighbouring ops to save launches per layer;
// fm_kernel_ssm.h (Foundry) header notes treat the decay gate as dispatch cost
// that should ride with its neighbours.  At 64 sequences the conv on its own
// moves about 21 MB, too little to amortise a launch's ramp and drain; here
// its bytes stream inside the recurrence's launch.
//
// Every value is computed by the same device functions as the separate
// kernels (conv.hpp, gate.hpp, recur.hpp, norm.hpp), with the same lane map
// for each conv head (so the Q/K L2 butterflies pair the same lanes), so the
// results equal, bit for bit, those of gdn_conv1d_silu_l2norm followed by
// gdn_decode_fused.
//
// Thread map: one workgroup per (sequence, value head), laid out as in
// k_decode_fused (a 16-lane DPP row per state row, 4 RG rows per wave, the
// whole head in the workgroup).  The first waves compute the conv of the
// three S-channel heads this value head needs -- its q and k head (query/key
// group hk) and its v head -- with S/4 lanes per head (lanes past the three
// heads compute on clamped channels and store nothing, so every lane of a
// conv wave is active for the L2 butterfly), and leave q, k, v of every
// position in LDS.  They request the conv's inputs before their state rows;
// since loads return in order, the conv then runs while the state is still
// arriving, and its latency hides under the state stream.
//
// Conv history ownership: the v history of head h has one reader and writer,
// this workgroup.  The q/k history of group hk is read by the group's
// G = H / Hk workgroups; each Q/K conv wave takes a ticket from a per-(sequence,
// group, wave) counter in the workspace once its history loads have returned
// (the ticket's operand depends on a conv output), and the holder of the last
// ticket (G - 1) writes the new history at its end and resets the counter.
// Nobody waits for anybody, so the grid needs no co-residency.
#include <hip/hip_runtime.h>

#include "conv.hpp"
#include "gate.hpp"
#include "gdn.h"
#include "launch.hpp"
#include "norm.hpp"
#include "recur.hpp"
#include "wave.hpp"

namespace gdn {

// positions per launch, staged in LDS: up to 32 (16 at S = 256), which keeps
// two workgroups' LDS per CU at S = 128 (about 70 KB each)
template <int S>
constexpr int step_max_tok() { return S <= 128 ? 32 : 16; }

// MT: the positions the LDS staging holds.  A one-position call (decode) at
// S <= 128 runs the MT = 1 instance: n_tok is then the constant 1, its loops
// and snapshot branches fold away, and it holds 6 KB of LDS and fewer
// registers than the K-position instance (measured at 64 sequences x 48
// heads: 73.6 against 74.4 us, the same bits).
template <int S, int RG, int D, int MT>
__global__ __launch_bounds__(16 * S / RG) void k_decode_step(const StepArgs A) {
  constexpr int EPL = S / 16;
  constexpr int L4 = S / 4;                       // lanes of one S-channel head
  constexpr int DH = D - 1;
  constexpr int CONV_WAVES = (3 * L4 + 63) / 64;  // waves holding q, k, v heads
  constexpr int MAXT = MT;
  __shared__ __attribute__((aligned(16))) float cbuf[MAXT][3][S];  // q, k, v
  __shared__ __attribute__((aligned(16))) float ybuf[2][S];
  __shared__ float hstash[2 * L4][CPL * DH];      // q/k windows after the last position
  __shared__ __attribute__((aligned(16))) float zbuf[MAXT][S];   // norm gate z
  __shared__ float gbuf[MAXT], bbuf[MAXT];                       // gate value, beta
  constexpr int NWAVES = S / (4 * RG);
  static_assert(NWAVES > CONV_WAVES, "the last wave stages the per-position inputs");
  const FusedArgs &F = A.f;
  const RecurArgs &R = F.r;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, wv = tid >> 6;
  // (sequence, head) of this workgroup, numbered so that consecutive heads (a
  // query/key group, whose q/k conv inputs they share) land on one XCD: XCD
  // x < r of nwg = 8q + r takes q + 1 consecutive units, the others q
  const int nwg = gridDim.x, q8 = nwg / 8, r8 = nwg % 8;
  const int xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
  const int unit = (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + idx;
  const int H = R.H, Hk = R.Hk, G = H / Hk, n_tok = MT == 1 ? 1 : R.n_tok;
  const int s = unit / H, h = unit - s * H, hk = h / G;
  const int row0 = wv * 4 * RG + (lane >> 4);  // + 4r

  // 1. the conv waves request their taps, history and position 0's inputs
  // first: loads return in order, so the conv can then run while the state
  // is still arriving
  const int C = (2 * Hk + H) * S;
  float *hist = A.hist + s * A.h_seq;
  const float *xs = A.x + s * A.x_seq;
  const bool conv_wave = wv < CONV_WAVES;           // uniform per wave
  const int u_raw = tid / L4;                       // 0: q, 1: k, 2: v; 3 and up: idle lanes
  const bool act = u_raw < 3;
  const int u = act ? u_raw : 2;
  const int ci = tid - u_raw * L4;
  const int base = u == 0 ? hk * S : (u == 1 ? (Hk + hk) * S : (2 * Hk + h) * S);
  const LaneChans L = lane_chans(base, ci, C);
  conv_f4 raw_w[D], raw_h[DH], raw_x;
  if (conv_wave) {
    load_recs_raw<D>(A.cw, L, raw_w);
    load_recs_raw<DH>(hist, L, raw_h);
    raw_x = *reinterpret_cast<const conv_f4 *>(xs + L.c0v);
  }

  // 2. the head's state rows
  float *st_base = R.state + s * R.st_seq + (int64_t)h * S * S;
  float st[RG][EPL];
#pragma unroll
  for (int r = 0; r < RG; ++r) load_row<S, true>(st_base + (int64_t)(row0 + 4 * r) * S, l16, st[r]);

  // the per-position gate value, beta and z, staged in LDS by the last wave
  // (never a conv wave), so the position loop below issues no global loads:
  // a load's wait there would also wait for the conv's ticket
  const int64_t gb0 = (int64_t)s * n_tok * H + h;   // (s, t, h) = gb0 + t * H
  const int e4 = 4 * (lane < L4 ? lane : L4 - 1);
  if (wv == NWAVES - 1) {
    if (lane < n_tok) {
      const float gval = decay_gate_value(F.alpha[gb0 + (int64_t)lane * H], F.dt[h], F.a[h]);
      gbuf[lane] = gval;
      bbuf[lane] = R.beta[gb0 + (int64_t)lane * H];
      if (F.g != nullptr) F.g[gb0 + (int64_t)lane * H] = gval;
    }
    const float *zs = F.z + s * F.z_seq + (int64_t)h * S + e4;
    for (int t = 0; t < n_tok; ++t)
      if (lane < L4) *reinterpret_cast<float4 *>(&zbuf[t][e4]) = *reinterpret_cast<const float4 *>(zs + t * F.z_tok);
  }
  const float4 w4 = *reinterpret_cast<const float4 *>(F.w + e4);

  // 3. the conv of this head's q, k, v channels, every position, into LDS
  const bool qk_wave = G > 1 && wv * 64 < 2 * L4;   // holds Q/K heads shared with the group
  int ticket = 0;
  if (conv_wave) {
    // the raw loads are consumed only from here on (after the state's loads
    // are issued); the empty asm keeps the compiler from unpacking them
    // earlier, inside the branch that issued them
#pragma unroll
    for (int q = 0; q < D; ++q) asm volatile("" : "+v"(raw_w[q]));
#pragma unroll
    for (int q = 0; q < DH; ++q) asm volatile("" : "+v"(raw_h[q]));
    asm volatile("" : "+v"(raw_x));
    float wt[CPL][D], win[CPL][D];
    {
      float hv[CPL][DH];
      unpack_recs<D>(raw_w, wt);
      unpack_recs<DH>(raw_h, hv);
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int j = 0; j < DH; ++j) win[c][j] = hv[c][j];
    }
    const bool qk = u < 2;
    // q/k snapshots are identical in every workgroup of the group: the
    // group's first head writes them
    const bool snap_owner = act && (u == 2 || h == hk * G);
    float o_first = 0.0f;
    for (int t = 0; t < n_tok; ++t) {
      float xv[CPL], o[CPL];
      if (t == 0) {
        xv[0] = raw_x.x; xv[1] = raw_x.y; xv[2] = raw_x.z; xv[3] = raw_x.w;
      } else {
        load_row4<true>(xs + (int64_t)t * A.x_tok, L, xv);
      }
      conv_step4<D, L4>(wt, win, xv, qk, A.l2_eps, o);
      if (t == 0) o_first = o[0];
      if (act) *reinterpret_cast<float4 *>(&cbuf[t][u][4 * ci]) = make_float4(o[0], o[1], o[2], o[3]);
      if (A.csnap != nullptr && t < n_tok - 1 && snap_owner) {
        float hw[CPL][DH];
        window_hist<D>(win, hw);
        store_recs<DH, true>(A.csnap + s * A.cs_seq + t * A.cs_tok, L, hw);
      }
    }
    float hw[CPL][DH];
    window_hist<D>(win, hw);
    if (!(qk && G > 1)) {
      if (act) store_recs<DH, true>(hist, L, hw);   // this workgroup owns these channels
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int j = 0; j < DH; ++j) hstash[tid][c * DH + j] = hw[c][j];
    }
    if (qk_wave) {
      // The ticket's operand depends on position 0's output, which used every
      // history value this wave loaded, so the ticket is issued only after
      // those loads have returned; the clobber keeps the compiler from moving
      // it earlier.
      int one = 1;
      asm volatile("" : "+v"(one) : "v"(o_first) : "memory");
      if (lane == 0) ticket = atomicAdd(A.cnt + ((int64_t)s * Hk + hk) * 2 + wv, one);
    }
  }
  __syncthreads();   // q, k, v of every position are in LDS

  // 4. gate -> recurrence -> norm per position, as k_decode_fused
  for (int t = 0; t < n_tok; ++t) {
    float kv[EPL], qv[EPL], vj[RG], yo[RG];
    load_row<S>(&cbuf[t][1][0], l16, kv);
    load_row<S>(&cbuf[t][0][0], l16, qv);
#pragma unroll
    for (int r = 0; r < RG; ++r) vj[r] = cbuf[t][2][row0 + 4 * r];
    const float4 z4 = *reinterpret_cast<const float4 *>(&zbuf[t][e4]);
    const float gval = gbuf[t];
    recur_position<S, RG>(st, kv, qv, vj, expf(gval), bbuf[t], yo);
    float *yb = ybuf[t & 1];
    if (l16 == 0) {
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const float yv = R.scale * yo[r];
        yb[row0 + 4 * r] = yv;
        if (F.y != nullptr) F.y[s * F.y_seq + t * F.y_tok + (int64_t)h * S + row0 + 4 * r] = yv;
      }
    }
    if (R.snap != nullptr && t < n_tok - 1) {
      float *sp = R.snap + s * R.sn_seq + (int64_t)t * H * S * S + (int64_t)h * S * S;
#pragma unroll
      for (int r = 0; r < RG; ++r) store_row<S, true>(sp + (int64_t)(row0 + 4 * r) * S, l16, st[r]);
    }
    if (t == n_tok - 1) {
#pragma unroll
      for (int r = 0; r < RG; ++r)
        store_row<S, true>(st_base + (int64_t)(row0 + 4 * r) * S, l16, st[r]);
    }
    __syncthreads();
    const float4 y4 = *reinterpret_cast<const float4 *>(yb + e4);
    const float ss = group_sum<L4>(sumsq4(y4));
    const float4 o4 = gated_norm4(y4, z4, w4, norm_inv(ss, S, F.eps));
    if (wv == 0 && lane < L4)
      *reinterpret_cast<float4 *>(R.y + s * R.y_seq + t * R.y_tok + (int64_t)h * S + e4) = o4;
  }

  // 5. the last reader of the group's q/k history writes the new one
  if (qk_wave) {   // uniform per wave
    ticket = __shfl(ticket, 0, 64);
    if (ticket == G - 1) {
      if (tid < 2 * L4) {   // the q/k lanes; L is their channel map
        float hw[CPL][DH];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int j = 0; j < DH; ++j) hw[c][j] = hstash[tid][c * DH + j];
        store_recs<DH, true>(hist, L, hw);
      }
      if (lane == 0) atomicExch(A.cnt + ((int64_t)s * Hk + hk) * 2 + wv, 0);
    }
  }
}

namespace {

template <int S, int RG, int D>
int run_step(const StepArgs &a, hipStream_t stream) {
  if (a.f.r.n_tok > step_max_tok<S>()) return GDN_ERR_SHAPE;
  static_assert(S % (4 * RG) == 0 && S / (4 * RG) <= 16, "a workgroup holds the whole head");
  static_assert((3 * S / 4 + 63) / 64 <= S / (4 * RG), "the conv fits in the workgroup");
  const int64_t units = (int64_t)a.f.r.n_seq * a.f.r.H;
  if (units > INT32_MAX) return GDN_ERR_SHAPE;
  if constexpr (S <= 128) {   // at S = 256 the one-position instance spills
    if (a.f.r.n_tok == 1)
      return launch_kernel(k_decode_step<S, RG, D, 1>, dim3((unsigned)units), dim3(16 * S / RG),
                           0, stream, a);
  }
  return launch_kernel(k_decode_step<S, RG, D, step_max_tok<S>()>, dim3((unsigned)units),
                       dim3(16 * S / RG), 0, stream, a);
}

template <int S, int RG>
int pick_d(const StepArgs &a, hipStream_t stream) {
  switch (a.D) {
    case 2: return run_step<S, RG, 2>(a, stream);
    case 3: return run_step<S, RG, 3>(a, stream);
    case 4: return run_step<S, RG, 4>(a, stream);
    default: return GDN_ERR_UNSUPPORTED;
  }
}

}  // namespace

int launch_decode_step(const StepArgs &a, hipStream_t stream) {
  // rows per lane as k_decode_fused
  switch (a.f.r.S) {
    case 32: return pick_d<32, 1>(a, stream);
    case 64: return pick_d<64, 1>(a, stream);
    case 128: return pick_d<128, 4>(a, stream);
    case 256: return pick_d<256, 8>(a, stream);
    default: return GDN_ERR_UNSUPPORTED;
  }
}

}  // namespace gdn
