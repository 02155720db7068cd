// k_recur.hip -- gated delta-rule recurrence, token by token (decode and
// K-position speculative verify with rollback snapshots).
//
// Math: fm_kernel_ssm.h (Foundry), "Delta-rule recurrence" section.  Per value
// head and position, in this order: S <- exp(g) S; p = S^T k;
// delta = beta (v - p); S <- S + k delta^T; y = scale S^T q.  The state is
// stored transposed, state[j][i] = S[i][j], so the value row j of a head is
// contiguous over the key index i and carries its own scalar delta_j.
// Snapshots follow ssm_mamba.rs (spark_model), gdn_verify_fused_conv_k2: the
// state after position t < n_tok-1 is written aside, the committed state stays
// in place.
//
// Thread map (gfx950, wave64): a 16-lane DPP row owns one state row; lane l of
// the row holds key elements {64m + 4l + c} (S >= 64) or {2l, 2l+1} (S = 32),
// i.e. S/16 floats, loaded and stored as float4 (float2) so a row segment is
// one 256-byte (128-byte) coalesced access.  A wave holds 4*RG rows of one
// (sequence, head) in registers for all positions; both per-position dot
// products are 16-lane DPP butterflies (wave.hpp), with no LDS and no barrier.
// The state is read from HBM once and written once per call.  k and q are
// loaded once per wave per position and shared by its 4*RG rows.
#include <hip/hip_runtime.h>

#include "gdn.h"
#include "launch.hpp"
#include "recur.hpp"
#include "wave.hpp"

namespace gdn {

// grid: x = H * blocks_per_head, y = n_seq; block = 64 * waves_per_block.
template <int S, int RG>
__global__ __launch_bounds__(256) void k_recur_decode(
    float *__restrict__ state, int64_t st_seq, const float *__restrict__ q,
    const float *__restrict__ k, int64_t qk_tok, int64_t qk_seq, const float *__restrict__ v,
    int64_t v_tok, int64_t v_seq, const float *__restrict__ g, const float *__restrict__ beta,
    float *__restrict__ y, int64_t y_tok, int64_t y_seq, float *__restrict__ snap,
    int64_t sn_seq, int n_tok, int H, int Hk, int blocks_per_head, float scale) {
  constexpr int EPL = S / 16;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int wpb = blockDim.x >> 6;
  const int h = blockIdx.x / blocks_per_head;
  const int rb = blockIdx.x - h * blocks_per_head;
  const int s = blockIdx.y;
  const int hk = h / (H / Hk);
  const int row0 = (rb * wpb + (threadIdx.x >> 6)) * 4 * RG + (lane >> 4);  // + 4r

  const int64_t head_off = s * st_seq + (int64_t)h * S * S;
  float *st_base = state + head_off;

  float st[RG][EPL];
#pragma unroll
  for (int r = 0; r < RG; ++r) load_row<S, true>(st_base + (int64_t)(row0 + 4 * r) * S, l16, st[r]);

  const float *qs = q + s * qk_seq + (int64_t)hk * S;
  const float *ks = k + s * qk_seq + (int64_t)hk * S;
  const float *vs = v + s * v_seq + (int64_t)h * S;
  float *ys = y + s * y_seq + (int64_t)h * S;
  const float *gs = g + ((int64_t)s * n_tok) * H + h;
  const float *bs = beta + ((int64_t)s * n_tok) * H + h;

  for (int t = 0; t < n_tok; ++t) {
    float kv[EPL], qv[EPL], vj[RG], yo[RG];
    load_row<S>(ks + t * qk_tok, l16, kv);
    load_row<S>(qs + t * qk_tok, l16, qv);
#pragma unroll
    for (int r = 0; r < RG; ++r) vj[r] = vs[t * v_tok + row0 + 4 * r];
    const float gamma = expf(gs[(int64_t)t * H]);
    const float b = bs[(int64_t)t * H];
    recur_position<S, RG>(st, kv, qv, vj, gamma, b, yo);
    if (l16 == 0) {
#pragma unroll
      for (int r = 0; r < RG; ++r) ys[t * y_tok + row0 + 4 * r] = scale * yo[r];
    }
    if (snap != nullptr && t < n_tok - 1) {
      float *sp = snap + s * sn_seq + (int64_t)t * H * S * S + (int64_t)h * S * S;
#pragma unroll
      for (int r = 0; r < RG; ++r) store_row<S, true>(sp + (int64_t)(row0 + 4 * r) * S, l16, st[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < RG; ++r) store_row<S, true>(st_base + (int64_t)(row0 + 4 * r) * S, l16, st[r]);
}

namespace {

template <int S, int RG>
int run_recur(const RecurArgs &a, hipStream_t stream) {
  // rows of one head split over blocks of `wpb` waves, 4*RG rows per wave
  constexpr int rows_per_wave = 4 * RG;
  static_assert(S % rows_per_wave == 0, "rows per wave must divide S");
  const int waves_per_head = S / rows_per_wave;
  const int wpb = waves_per_head < 4 ? waves_per_head : 4;
  const int bph = waves_per_head / wpb;
  const dim3 grid((unsigned)(a.H * bph), (unsigned)a.n_seq);
  return launch_kernel(k_recur_decode<S, RG>, grid, dim3(64 * wpb), 0, stream, a.state, a.st_seq,
                       a.q, a.k, a.qk_tok, a.qk_seq, a.v, a.v_tok, a.v_seq, a.g, a.beta, a.y,
                       a.y_tok, a.y_seq, a.snap, a.sn_seq, a.n_tok, a.H, a.Hk, bph, a.scale);
}

template <int S>
int pick_rows(const RecurArgs &a, hipStream_t stream) {
  // Two rows per lane once there are enough waves to cover 256 CUs several
  // times over; beyond two, the extra bytes in flight per wave cost more in
  // occupancy than they gain (measured at 64 sequences x 48 heads, S = 128).
  const int64_t rows = (int64_t)a.n_seq * a.H * S;
  if (rows / 8 >= 4096) return run_recur<S, 2>(a, stream);
  return run_recur<S, 1>(a, stream);
}

}  // namespace

int launch_recur_decode(const RecurArgs &a, hipStream_t stream) {
  switch (a.S) {
    case 32: return pick_rows<32>(a, stream);
    case 64: return pick_rows<64>(a, stream);
    case 128: return pick_rows<128>(a, stream);
    case 256: return pick_rows<256>(a, stream);
    default: return GDN_ERR_UNSUPPORTED;
  }
}

}  // namespace gdn
