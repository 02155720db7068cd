// k_conv.hip -- depthwise causal conv1d + SiLU + per-head L2 norm on the Q/K
// channels, with a rolling history and optional rollback snapshots.
//
// Math: fm_kernel_ssm.h (Foundry), "Causal depthwise conv1d + SiLU" section
// (window = [history oldest..newest, x]; the history appends the RAW input);
// ssm_mamba.rs (spark_model), conv1d_update_l2norm (L2 on channels below
// qk_channels, per head_dim block, after SiLU), gdn_verify_fused_conv_k2
// (snapshot of the window after position 0), conv1d_update_prefill (the
// output depends on inputs only, so positions can run in parallel with the
// same per-position arithmetic).
//
// Thread map (both kernels): one wave64 owns a block of 64*CPL consecutive
// channels; lane l holds channels l, l+64, .., so every per-position load and
// store of x / out is a coalesced 256-byte wave access.  A block is one L2 head
// (head_dim = 64*CPL) or, at head_dim 32, two heads of 32 lanes each; the
// head's sum of squares is an in-wave xor butterfly (wave.hpp), no LDS.
//
//   k_conv_step : one wave walks every position of its sequence in order
//                 (decode, K-position verify with snapshots).
//   k_conv_tp   : one wave per (channel block, tile of TT positions); the
//                 window is preloaded from x (or from the history before
//                 position 0), so long prompts spread over the whole chip.
// Both call conv_position() and l2_scale() below with the same lane map and
// the same FMA order, so their outputs and histories agree bit for bit.
#include <hip/hip_runtime.h>

#include "gdn.h"
#include "launch.hpp"
#include "wave.hpp"

namespace gdn {

// acc = sum_j w[j] * win[j] in tap order, oldest tap first, explicit FMAs.
template <int D>
__device__ __forceinline__ float conv_position(const float (&w)[D], const float (&win)[D]) {
  float acc = w[0] * win[0];
#pragma unroll
  for (int j = 1; j < D; ++j) acc = __builtin_fmaf(w[j], win[j], acc);
  return silu(acc);
}

// Taps of channel ch (clamped to a valid channel by the caller): one 16-byte
// load when there are 4 taps.  Loads are never behind a branch: a branch
// would make the compiler wait for every load in flight where it rejoins.
template <int D>
__device__ __forceinline__ void load_taps(const float *__restrict__ w, int ch, float (&wt)[D]) {
  if constexpr (D == 4) {
    const float4 t = *reinterpret_cast<const float4 *>(w + (int64_t)ch * 4);
    wt[0] = t.x; wt[1] = t.y; wt[2] = t.z; wt[3] = t.w;
  } else {
#pragma unroll
    for (int j = 0; j < D; ++j) wt[j] = w[(int64_t)ch * D + j];
  }
}

// 1 / sqrt(sum over the lane's L2 head of o^2 + eps); LPH lanes per head.
template <int CPL, int LPH>
__device__ __forceinline__ float l2_scale(const float (&o)[CPL], float eps) {
  float ss = o[0] * o[0];
#pragma unroll
  for (int c = 1; c < CPL; ++c) ss = __builtin_fmaf(o[c], o[c], ss);
  ss = group_sum<LPH>(ss);
  return 1.0f / sqrtf(ss + eps);
}

// LPH == 0: SiLU only (no channel of the block is a Q/K channel).
template <int D, int CPL, int LPH>
__global__ __launch_bounds__(256) void k_conv_step(
    const float *__restrict__ x, int64_t x_tok, int64_t x_seq, const float *__restrict__ w,
    float *__restrict__ hist, int64_t h_seq, float *__restrict__ out, int64_t o_tok, int64_t o_seq,
    float *__restrict__ snap, int64_t sn_tok, int64_t sn_seq, int n_tok, int C, int qk_channels,
    float eps) {
  constexpr int DH = D - 1;
  const int lane = threadIdx.x & 63;
  const int blk0 = (blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 64 * CPL;
  if (blk0 >= C) return;  // uniform per wave
  const int s = blockIdx.y;
  x += s * x_seq;
  out += s * o_seq;
  hist += s * h_seq;

  // lanes past the last channel compute on channel C-1 and store nothing
  float wt[CPL][D], win[CPL][D];
  bool ok[CPL];
  int chc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int ch = blk0 + lane + 64 * c;
    ok[c] = ch < C;
    chc[c] = min(ch, C - 1);
    load_taps<D>(w, chc[c], wt[c]);
#pragma unroll
    for (int j = 0; j < DH; ++j) win[c][j] = hist[(int64_t)chc[c] * DH + j];
  }
  const bool qk = LPH > 0 && blk0 + lane < qk_channels;

  for (int t = 0; t < n_tok; ++t) {
    float o[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      win[c][DH] = x[(int64_t)t * x_tok + chc[c]];
      o[c] = conv_position<D>(wt[c], win[c]);
#pragma unroll
      for (int j = 0; j < DH; ++j) win[c][j] = win[c][j + 1];  // roll with the raw input
    }
    if (snap != nullptr && t < n_tok - 1) {
      float *sp = snap + s * sn_seq + t * sn_tok;
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        if (ok[c]) {
          const int ch = blk0 + lane + 64 * c;
#pragma unroll
          for (int j = 0; j < DH; ++j) sp[(int64_t)ch * DH + j] = win[c][j];
        }
    }
    if constexpr (LPH > 0) {
      const float inv = l2_scale<CPL, LPH>(o, eps);
      if (qk) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[c] *= inv;
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      if (ok[c]) out[(int64_t)t * o_tok + blk0 + lane + 64 * c] = o[c];
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c)
    if (ok[c]) {
      const int ch = blk0 + lane + 64 * c;
#pragma unroll
      for (int j = 0; j < DH; ++j) hist[(int64_t)ch * DH + j] = win[c][j];
    }
}

// Token-parallel form: grid (channel-block waves, position tiles, sequences).
// Only the wave of tile 0 reads the old history, and it is also the one that
// writes the new history, so no other wave can observe a half-updated history.
template <int D, int CPL, int LPH, int TT>
__global__ __launch_bounds__(256) void k_conv_tp(
    const float *__restrict__ x, int64_t x_tok, int64_t x_seq, const float *__restrict__ w,
    float *__restrict__ hist, int64_t h_seq, float *__restrict__ out, int64_t o_tok, int64_t o_seq,
    int n_tok, int C, int qk_channels, float eps) {
  constexpr int DH = D - 1;
  const int lane = threadIdx.x & 63;
  const int blk0 = (blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 64 * CPL;
  if (blk0 >= C) return;
  const int s = blockIdx.z;
  const int t0 = blockIdx.y * TT;
  const int t1 = min(t0 + TT, n_tok);
  x += s * x_seq;
  out += s * o_seq;
  hist += s * h_seq;

  // lanes past the last channel compute on channel C-1 and store nothing;
  // both window sources are loaded and one is selected (no load behind a
  // branch)
  float wt[CPL][D], win[CPL][D], old[CPL][DH];
  bool ok[CPL];
  int chc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int ch = blk0 + lane + 64 * c;
    ok[c] = ch < C;
    chc[c] = min(ch, C - 1);
    load_taps<D>(w, chc[c], wt[c]);
#pragma unroll
    for (int j = 0; j < DH; ++j) {
      // window slot j before position t0 holds position p = t0 - DH + j,
      // which is before position 0 only in tile 0 (TT >= DH), where it is
      // history slot j
      const int p = t0 - DH + j;
      old[c][j] = hist[(int64_t)chc[c] * DH + j];
      const float xp = x[(int64_t)max(p, 0) * x_tok + chc[c]];
      win[c][j] = t0 == 0 ? old[c][j] : xp;
    }
  }
  const bool qk = LPH > 0 && blk0 + lane < qk_channels;

  for (int t = t0; t < t1; ++t) {
    float o[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      win[c][DH] = x[(int64_t)t * x_tok + chc[c]];
      o[c] = conv_position<D>(wt[c], win[c]);
#pragma unroll
      for (int j = 0; j < DH; ++j) win[c][j] = win[c][j + 1];
    }
    if constexpr (LPH > 0) {
      const float inv = l2_scale<CPL, LPH>(o, eps);
      if (qk) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[c] *= inv;
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      if (ok[c]) out[(int64_t)t * o_tok + blk0 + lane + 64 * c] = o[c];
  }

  if (t0 == 0) {  // the new history: positions n_tok-DH .. n_tok-1
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      if (ok[c]) {
        const int ch = blk0 + lane + 64 * c;
#pragma unroll
        for (int j = 0; j < DH; ++j) {
          // position p = n_tok - DH + j; before position 0 it is old slot p + DH
          const int p = n_tok - DH + j;
          const float xp = x[(int64_t)max(p, 0) * x_tok + ch];
          float hv = xp;
#pragma unroll
          for (int k2 = 0; k2 < DH; ++k2)
            if (p + DH == k2) hv = old[c][k2];
          hist[(int64_t)ch * DH + j] = hv;
        }
      }
  }
}

namespace {

constexpr int kTileTok = 32;   // positions per wave in the token-parallel kernel
constexpr int kWavesPerBlock = 4;

template <int D, int CPL, int LPH>
int run_conv(const ConvArgs &a, hipStream_t stream) {
  const int blocks_ch = (a.C + 64 * CPL - 1) / (64 * CPL);           // one wave each
  const int grid_x = (blocks_ch + kWavesPerBlock - 1) / kWavesPerBlock;
  const dim3 block(64 * kWavesPerBlock);
  if (a.snap == nullptr && a.n_tok > 8) {
    const dim3 grid(grid_x, (a.n_tok + kTileTok - 1) / kTileTok, a.n_seq);
    return launch_kernel(k_conv_tp<D, CPL, LPH, kTileTok>, grid, block, 0, stream, a.x, a.x_tok,
                         a.x_seq, a.w, a.hist, a.h_seq, a.out, a.o_tok, a.o_seq, a.n_tok, a.C,
                         a.qk_channels, a.eps);
  }
  const dim3 grid(grid_x, a.n_seq);
  return launch_kernel(k_conv_step<D, CPL, LPH>, grid, block, 0, stream, a.x, a.x_tok, a.x_seq,
                       a.w, a.hist, a.h_seq, a.out, a.o_tok, a.o_seq, a.snap, a.sn_tok, a.sn_seq,
                       a.n_tok, a.C, a.qk_channels, a.eps);
}

template <int D>
int dispatch_head(const ConvArgs &a, hipStream_t stream) {
  if (a.qk_channels == 0) return run_conv<D, 2, 0>(a, stream);
  switch (a.head_dim) {
    case 32: return run_conv<D, 1, 32>(a, stream);
    case 64: return run_conv<D, 1, 64>(a, stream);
    case 128: return run_conv<D, 2, 64>(a, stream);
    case 256: return run_conv<D, 4, 64>(a, stream);
    default: return GDN_ERR_UNSUPPORTED;
  }
}

}  // namespace

int launch_conv(const ConvArgs &a, hipStream_t stream) {
  switch (a.D) {
    case 2: return dispatch_head<2>(a, stream);
    case 3: return dispatch_head<3>(a, stream);
    case 4: return dispatch_head<4>(a, stream);
    case 5: return dispatch_head<5>(a, stream);
    case 6: return dispatch_head<6>(a, stream);
    case 7: return dispatch_head<7>(a, stream);
    case 8: return dispatch_head<8>(a, stream);
    default: return GDN_ERR_UNSUPPORTED;
  }
}

}  // namespace gdn
