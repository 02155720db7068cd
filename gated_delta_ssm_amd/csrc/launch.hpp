// launch.hpp -- host-side launchers, one per kernel family.  Each returns a
// gdn_status; arguments reaching them are already validated (validate.cpp).
#pragma once
#include <cstddef>
#include <cstdint>
#include <tuple>
#include <utility>

#include <hip/hip_runtime_api.h>

#include "gdn.h"

namespace gdn {

// Launch `kern` through hipLaunchKernel and return its status, so a refused
// launch is reported by this call itself rather than through the thread's
// last-error slot.  Arguments are converted to the kernel's parameter types.
template <typename... KArgs, typename... Args>
int launch_kernel(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                  Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
  std::tuple<KArgs...> params(static_cast<KArgs>(args)...);
  void *ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
  std::apply([&ptrs](auto &...p) {
    int i = 0;
    ((ptrs[i++] = (void *)&p), ...);
  }, params);
  return hipLaunchKernel((const void *)kern, grid, block, ptrs, shmem, stream) == hipSuccess
             ? GDN_OK
             : GDN_ERR_LAUNCH;
}

int launch_decay_gate(const float *alpha, const float *dt, const float *a, float *g, int rows,
                      int n_heads, hipStream_t stream);

struct ConvArgs {
  const float *x;
  int64_t x_tok, x_seq;
  const float *w;
  float *hist;
  int64_t h_seq;
  float *out;
  int64_t o_tok, o_seq;
  float *snap;
  int64_t sn_tok, sn_seq;
  int n_seq, n_tok, C, D, qk_channels, head_dim;
  float eps;
};
int launch_conv(const ConvArgs &a, hipStream_t stream);

struct RecurArgs {
  float *state;
  int64_t st_seq;
  const float *q, *k;
  int64_t qk_tok, qk_seq;
  const float *v;
  int64_t v_tok, v_seq;
  const float *g, *beta;
  float *y;
  int64_t y_tok, y_seq;
  float *snap;
  int64_t sn_seq;
  int n_seq, n_tok, H, Hk, S;
  float scale;
};
int launch_recur_decode(const RecurArgs &a, hipStream_t stream);

size_t chunked_workspace_bytes(int n_seq, int n_tok, int H, int Hk, int S, int chunk);
int launch_recur_chunked(const RecurArgs &a, int chunk, void *ws, size_t ws_bytes,
                         hipStream_t stream);

// The conv and gate inputs of the fused prefill (gdn_prefill_chunked): the
// RecurArgs' q, k, v and g are unused, its beta, state, y and sizes are used.
struct PrefillConv {
  const float *x;
  int64_t x_tok, x_seq;
  const float *w;
  float *hist;
  int64_t h_seq;
  const float *alpha, *dt, *a;
  int D;
  float eps;
};
int launch_prefill_chunked(const RecurArgs &a, const PrefillConv &pc, int chunk, void *ws,
                           size_t ws_bytes, hipStream_t stream);

// Sequence map of a chunked call, passed to the kernels by value.  NoTab: a
// fixed-length batch (sequence s at s * seq_stride, n_tok positions each).
// VarTab: a packed variable-length batch; sequence s holds token rows
// tok0[s] .. tok0[s+1]-1 and workspace chunks ch0[s] .. ch0[s+1]-1 (its chunk
// count rounded up to even); ch0[n_seq] is the total.
struct NoTab {};
struct VarTab {
  int n_seq;
  int tok0[GDN_VARLEN_MAX_SEQ + 1];
  int ch0[GDN_VARLEN_MAX_SEQ + 1];
};
// Chunk slots a sequence of n_tok positions takes: ceil(n_tok / 64) rounded up
// to even (0 for an empty sequence).
inline int padded_chunks(int n_tok) { return ((n_tok + 63) / 64 + 1) & ~1; }
// Workspace bound of a packed batch of n_seq sequences and total_tok positions.
size_t chunked_varlen_workspace_bytes(int n_seq, int total_tok, int H, int Hk, int S);
// a.n_tok is the packed total; a.qk_seq, a.v_seq, a.y_seq are unused.  With
// bf16_in, a.q, a.k, a.v point at bf16 elements (strides still in elements).
int launch_recur_chunked_varlen(const RecurArgs &a, const VarTab &tab, bool bf16_in, int chunk,
                                void *ws, size_t ws_bytes, hipStream_t stream);
// The chunked form for S = 32 and 64 (fp32, one pass, no workspace).
int launch_chunk_small(const RecurArgs &a, hipStream_t stream);
int launch_chunk_small_varlen(const RecurArgs &a, const VarTab &tab, bool bf16_in,
                              hipStream_t stream);

// The Mamba-2 chunked SSD scan (k_ssd.hip); arguments already validated.
struct SsdLaunch {
  float *state;
  int64_t st_seq;
  const float *x;
  int64_t x_tok, x_seq;
  const float *Bm, *Cm;
  int64_t bc_tok, bc_seq;
  const float *dt_raw;
  int64_t dt_tok, dt_seq;
  const float *A_log, *D, *dt_bias;
  float *y;
  int64_t y_tok, y_seq;
  int n_seq, n_tok, H, G, P, N;
  float dt_min, dt_max;
  void *ws;
};
size_t ssd_workspace_bytes(int n_seq, int n_tok, int H, int P, int N);
int launch_ssd(const SsdLaunch &l, hipStream_t stream);

struct NormArgs {
  const float *y;
  int64_t y_row;
  const float *w, *z;
  int64_t z_row;
  float *out;
  int64_t o_row;
  int rows, H, hd;
  float eps;
};
int launch_gated_rmsnorm(const NormArgs &a, hipStream_t stream);

// Fused decode: r.y / r.y_tok / r.y_seq describe the normed output, r.g is
// unused (the gate is computed from alpha, dt, a); g and y are optional
// outputs (nullptr: not written).
struct FusedArgs {
  RecurArgs r;
  const float *alpha, *dt, *a, *w, *z;
  int64_t z_tok, z_seq;
  float *g, *y;
  int64_t y_tok, y_seq;
  float eps;
};
int launch_decode_fused(const FusedArgs &a, hipStream_t stream);

// Fused decode step: conv -> gate -> recurrence -> norm.  f.r.q, f.r.k, f.r.v
// are unused (the conv produces them on chip); cnt is the ticket workspace.
struct StepArgs {
  FusedArgs f;
  const float *x;
  int64_t x_tok, x_seq;
  const float *cw;
  float *hist;
  int64_t h_seq;
  float *csnap;
  int64_t cs_tok, cs_seq;
  int D;
  float l2_eps;
  int *cnt;
};
int launch_decode_step(const StepArgs &a, hipStream_t stream);

}  // namespace gdn
