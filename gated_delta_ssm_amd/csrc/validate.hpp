// validate.hpp -- host-only argument checks (no HIP runtime calls).
#pragma once
#include <cstddef>
#include <cstdint>

namespace gdn {

int check_decay_gate(const float *alpha, const float *dt, const float *a, const float *g,
                     int rows, int n_heads);

int check_conv(const float *x, int64_t x_tok, int64_t x_seq, const float *w, const float *hist,
               int64_t h_seq, const float *out, int64_t o_tok, int64_t o_seq, const float *snap,
               int64_t sn_tok, int64_t sn_seq, int n_seq, int n_tok, int C, int D, int qk,
               int head_dim);

int check_recur(const float *state, int64_t st_seq, const float *q, const float *k,
                int64_t qk_tok, int64_t qk_seq, const float *v, int64_t v_tok, int64_t v_seq,
                const float *g, const float *beta, const float *y, int64_t y_tok, int64_t y_seq,
                const float *snap, int64_t sn_seq, int n_seq, int n_tok, int H, int Hk, int S);

int check_chunked(const float *state, int64_t st_seq, const float *q, const float *k,
                  int64_t qk_tok, int64_t qk_seq, const float *v, int64_t v_tok, int64_t v_seq,
                  const float *g, const float *beta, const float *y, int64_t y_tok,
                  int64_t y_seq, int n_seq, int n_tok, int H, int Hk, int S, int chunk,
                  const void *ws, size_t ws_bytes, size_t ws_needed);

// A packed batch: cu host array of n_seq + 1 offsets; token tensors are one
// [total_tok] run of rows (q, k, v of the given gdn_dtype), the state n_seq
// rows of st_seq.
int check_chunked_varlen(const float *state, int64_t st_seq, const void *q, const void *k,
                         int64_t qk_tok, const void *v, int64_t v_tok, int dtype, const float *g,
                         const float *beta, const float *y, int64_t y_tok, const int32_t *cu,
                         int n_seq, int total_tok, int H, int Hk, int S, int chunk,
                         const void *ws, size_t ws_bytes, size_t ws_needed);

int check_ssd(const float *state, int64_t st_seq, const float *x, int64_t x_tok, int64_t x_seq,
              const float *B, const float *C, int64_t bc_tok, int64_t bc_seq,
              const float *dt_raw, int64_t dt_tok, int64_t dt_seq, const float *A_log,
              const float *D, const float *dt_bias, const float *y, int64_t y_tok,
              int64_t y_seq, int n_seq, int n_tok, int H, int G, int P, int N, int chunk,
              const void *ws, size_t ws_bytes, size_t ws_needed);

int check_norm(const float *y, int64_t y_row, const float *w, const float *z, int64_t z_row,
               const float *out, int64_t o_row, int rows, int H, int hd);

int check_fused(const float *state, int64_t st_seq, const float *q, const float *k,
                int64_t qk_tok, int64_t qk_seq, const float *v, int64_t v_tok, int64_t v_seq,
                const float *alpha, const float *dt, const float *a, const float *beta,
                const float *w, const float *z, int64_t z_tok, int64_t z_seq, const float *out,
                int64_t o_tok, int64_t o_seq, const float *g, const float *y, int64_t y_tok,
                int64_t y_seq, const float *snap, int64_t sn_seq, int n_seq, int n_tok, int H,
                int Hk, int S);

// The fused prefill: conv input x with (2 Hk + H) S channels, conv taps and
// history, alpha / dt / a of the gate, beta, the state and y.
int check_prefill(const float *state, int64_t st_seq, const float *x, int64_t x_tok,
                  int64_t x_seq, const float *cw, const float *hist, int64_t h_seq,
                  const float *alpha, const float *dt, const float *a, const float *beta,
                  const float *y, int64_t y_tok, int64_t y_seq, int n_seq, int n_tok, int H,
                  int Hk, int S, int D, int chunk, const void *ws, size_t ws_bytes,
                  size_t ws_needed);

size_t step_workspace_bytes(int n_seq, int Hk);

int check_step(const float *state, int64_t st_seq, const float *x, int64_t x_tok, int64_t x_seq,
               const float *cw, const float *hist, int64_t h_seq, const float *csnap,
               int64_t cs_tok, int64_t cs_seq, const float *alpha, const float *dt,
               const float *a, const float *beta, const float *w, const float *z, int64_t z_tok,
               int64_t z_seq, const float *out, int64_t o_tok, int64_t o_seq, const float *g,
               const float *y, int64_t y_tok, int64_t y_seq, const float *snap, int64_t sn_seq,
               int n_seq, int n_tok, int H, int Hk, int S, int D, const void *ws,
               size_t ws_bytes, bool lib_scratch = false);

}  // namespace gdn
