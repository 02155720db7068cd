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
// Thread map (both kernels): lane l of a wave owns the 4 consecutive channels
// c0 = blk0 + 4l .. c0 + 3, so a wave covers 256 channels and each
// per-position access of x and out is one 16-byte load or store per lane (a
// 1 KiB wave access) when the rows are 16-byte aligned (VEC), or four 4-byte
// accesses otherwise; the lane's taps, history and snapshot records are its 4
// channels' consecutive [channel][tap] entries, likewise 16-byte accesses
// when VEC.  The arithmetic is the same either way.  An L2 head of
// head_dim channels is head_dim/4 consecutive lanes (LPH4); its sum of
// squares is an in-wave xor butterfly (wave.hpp), no LDS.
//
//   k_conv_step : one wave walks every position of its sequence in order
//                 (decode, K-position verify with snapshots).
//   k_conv_tp   : one wave per (channel block, tile of TT positions); the
//                 window is preloaded from x (or from the history before
//                 position 0), so long prompts spread over the whole chip.
// Both call conv_step4() (conv.hpp) with the same lane map and the same FMA order,
// so their outputs and histories agree bit for bit.
#include <hip/hip_runtime.h>

#include "gdn.h"
#include "conv.hpp"
#include "launch.hpp"
#include "wave.hpp"

namespace gdn {

template <int D, int LPH4, bool VEC>
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

  const LaneChans L = lane_chans(blk0, lane, C);
  float wt[CPL][D], win[CPL][D];
  {
    float hv[CPL][DH];
    load_taps_hist<D, VEC>(w, hist, L, wt, hv);
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int j = 0; j < DH; ++j) win[c][j] = hv[c][j];
  }
  const bool qk = LPH4 > 0 && L.c0 < qk_channels;

  for (int t = 0; t < n_tok; ++t) {
    float xv[CPL], o[CPL];
    load_row4<VEC>(x + (int64_t)t * x_tok, L, xv);
    conv_step4<D, LPH4>(wt, win, xv, qk, eps, o);
    if (snap != nullptr && t < n_tok - 1) {
      float h[CPL][DH];
      window_hist<D>(win, h);
      store_recs<DH, VEC>(snap + s * sn_seq + t * sn_tok, L, h);
    }
    store_row4<VEC>(out + (int64_t)t * o_tok, L, o);
  }
  float h[CPL][DH];
  window_hist<D>(win, h);
  store_recs<DH, VEC>(hist, L, h);
}

// Token-parallel form: grid (channel-block waves, position tiles, sequences).
// Only the wave of tile 0 uses the old history, and it is also the one that
// writes the new history, so no other wave can observe a half-updated history
// (the other tiles load it too, unconditionally, and discard it).
template <int D, int LPH4, bool VEC, int TT>
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

  const LaneChans L = lane_chans(blk0, lane, C);
  float wt[CPL][D], win[CPL][D], old[CPL][DH];
  load_taps_hist<D, VEC>(w, hist, L, wt, old);
  // window slot j before position t0 holds position p = t0 - DH + j, which is
  // before position 0 only in tile 0 (TT >= DH), where it is history slot j;
  // both sources are loaded and one is selected
#pragma unroll
  for (int j = 0; j < DH; ++j) {
    float xp[CPL];
    load_row4<VEC>(x + (int64_t)max(t0 - DH + j, 0) * x_tok, L, xp);
#pragma unroll
    for (int c = 0; c < CPL; ++c) win[c][j] = t0 == 0 ? old[c][j] : xp[c];
  }
  const bool qk = LPH4 > 0 && L.c0 < qk_channels;

  // positions in batches of TB, two batches in flight: the next batch's rows
  // are requested before the current batch is computed (rows past the end are
  // clamped to the last position and not used)
  constexpr int TB = 4;
  static_assert(TT % (2 * TB) == 0 && TT >= DH, "whole pairs of batches; a tile covers the history");
  auto load_batch = [&](float (&xv)[TB][CPL], int tb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TB; ++i)
      load_row4<VEC>(x + (int64_t)min(tb + i, n_tok - 1) * x_tok, L, xv[i]);
  };
  auto run_batch = [&](float (&xv)[TB][CPL], int tb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      if (tb + i < t1) {   // uniform per wave
        float o[CPL];
        conv_step4<D, LPH4>(wt, win, xv[i], qk, eps, o);
        store_row4<VEC>(out + (int64_t)(tb + i) * o_tok, L, o);
      }
    }
  };
  float xa[TB][CPL], xb[TB][CPL];
  load_batch(xa, t0);
  for (int tb = t0; tb < t1; tb += 2 * TB) {
    load_batch(xb, tb + TB);
    run_batch(xa, tb);
    load_batch(xa, tb + 2 * TB);
    run_batch(xb, tb + TB);
  }
  if (t0 == 0) {  // the new history: positions n_tok-DH .. n_tok-1
    float h[CPL][DH];
#pragma unroll
    for (int j = 0; j < DH; ++j) {
      // position p = n_tok - DH + j; before position 0 it is old slot p + DH
      const int p = n_tok - DH + j;
      float xp[CPL];
      load_row4<VEC>(x + (int64_t)max(p, 0) * x_tok, L, xp);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        float hv = xp[c];
#pragma unroll
        for (int k2 = 0; k2 < DH; ++k2)
          if (p + DH == k2) hv = old[c][k2];
        h[c][j] = hv;
      }
    }
    store_recs<DH, VEC>(hist, L, h);
  }
}

namespace {

// positions per wave in the token-parallel kernel: at 4096 positions x 8192
// channels, 8-position tiles (8192 waves) took 58 us against 67 us for 32
// (2048 waves, batches of 8 without the prefetch) and 62 us for 16; the extra
// window rows each tile reloads (d_conv - 1) cost less than the waves gain
constexpr int kTileTok = 8;
// tiles for prompts whose 8-position tiles would exceed the grid's y limit
constexpr int kTileTokLong = 64;
constexpr int kMaxGridY = 65535;
constexpr int kWavesPerBlock = 4;

template <int D, int LPH4, bool VEC>
int run_conv(const ConvArgs &a, hipStream_t stream) {
  const int blocks_ch = (a.C + 64 * CPL - 1) / (64 * CPL);           // one wave each
  const int grid_x = (blocks_ch + kWavesPerBlock - 1) / kWavesPerBlock;
  const dim3 block(64 * kWavesPerBlock);
  if (a.snap == nullptr && a.n_tok > 8) {
    const int64_t tiles = ((int64_t)a.n_tok + kTileTok - 1) / kTileTok;
    if (tiles <= kMaxGridY)
      return launch_kernel(k_conv_tp<D, LPH4, VEC, kTileTok>, dim3(grid_x, (unsigned)tiles, a.n_seq),
                           block, 0, stream, a.x, a.x_tok, a.x_seq, a.w, a.hist, a.h_seq, a.out,
                           a.o_tok, a.o_seq, a.n_tok, a.C, a.qk_channels, a.eps);
    const int64_t tiles_long = ((int64_t)a.n_tok + kTileTokLong - 1) / kTileTokLong;
    if (tiles_long > kMaxGridY) return GDN_ERR_UNSUPPORTED;
    return launch_kernel(k_conv_tp<D, LPH4, VEC, kTileTokLong>,
                         dim3(grid_x, (unsigned)tiles_long, a.n_seq), block, 0, stream, a.x,
                         a.x_tok, a.x_seq, a.w, a.hist, a.h_seq, a.out, a.o_tok, a.o_seq, a.n_tok,
                         a.C, a.qk_channels, a.eps);
  }
  // the step kernel is latency-bound (a few loads per wave, then one chain of
  // arithmetic): one-wave blocks spread its waves evenly over the CUs
  const dim3 grid(blocks_ch, a.n_seq);
  return launch_kernel(k_conv_step<D, LPH4, VEC>, grid, dim3(64), 0, stream, a.x, a.x_tok, a.x_seq,
                       a.w, a.hist, a.h_seq, a.out, a.o_tok, a.o_seq, a.snap, a.sn_tok, a.sn_seq,
                       a.n_tok, a.C, a.qk_channels, a.eps);
}

template <int D, bool VEC>
int dispatch_head(const ConvArgs &a, hipStream_t stream) {
  if (a.qk_channels == 0) return run_conv<D, 0, VEC>(a, stream);
  switch (a.head_dim) {
    case 32: return run_conv<D, 8, VEC>(a, stream);
    case 64: return run_conv<D, 16, VEC>(a, stream);
    case 128: return run_conv<D, 32, VEC>(a, stream);
    case 256: return run_conv<D, 64, VEC>(a, stream);
    default: return GDN_ERR_UNSUPPORTED;
  }
}

template <int D>
int dispatch_vec(const ConvArgs &a, hipStream_t stream) {
  // 16-byte accesses need whole groups of 4 channels and 16-byte aligned
  // rows of x, out, the weights, the history and the snapshots
  auto al = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool vec = a.C % 4 == 0 && al(a.x) && al(a.out) && al(a.w) && al(a.hist) &&
                   (a.snap == nullptr || al(a.snap)) && a.x_tok % 4 == 0 && a.x_seq % 4 == 0 &&
                   a.o_tok % 4 == 0 && a.o_seq % 4 == 0 && a.h_seq % 4 == 0 &&
                   a.sn_tok % 4 == 0 && a.sn_seq % 4 == 0;
  return vec ? dispatch_head<D, true>(a, stream) : dispatch_head<D, false>(a, stream);
}

}  // namespace

int launch_conv(const ConvArgs &a, hipStream_t stream) {
  switch (a.D) {
    case 2: return dispatch_vec<2>(a, stream);
    case 3: return dispatch_vec<3>(a, stream);
    case 4: return dispatch_vec<4>(a, stream);
    case 5: return dispatch_vec<5>(a, stream);
    case 6: return dispatch_vec<6>(a, stream);
    case 7: return dispatch_vec<7>(a, stream);
    case 8: return dispatch_vec<8>(a, stream);
    default: return GDN_ERR_UNSUPPORTED;
  }
}

}  // namespace gdn
