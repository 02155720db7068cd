/*
 * gdn.h -- C ABI of libgdn.so, the MI355X (gfx950) gated-delta SSM layer core.
 *
 * Sources (page title, then the part of the page):
 *   [FM]  fm_kernel_ssm.h, Foundry Metal kernels (git.teamide.dev)
 *   [AT]  ssm_mamba.rs, spark_model layers/ops (atlas-docs)
 *   [SCR] scr_state.hpp, regolith Metal engine scripts (tangled.org)
 *
 * Conventions shared by every entry point:
 *   - Every tensor is fp32 DEVICE memory allocated, owned and freed by the
 *     caller, who keeps it alive until the work on `stream` has finished.
 *   - Strides are in ELEMENTS (floats), not bytes.  Within a row, heads are
 *     packed densely (head stride = head width).
 *   - Every call is asynchronous on `stream` (0 = the null stream), allocates
 *     nothing, never synchronises, and keeps no state between calls.  Calls on
 *     different streams with disjoint buffers may run concurrently.
 *   - Arguments are validated on the host before anything is launched; a
 *     failed check returns a negative gdn_status and launches nothing.  A
 *     launch failure returns GDN_ERR_LAUNCH.  Faults inside a kernel surface at
 *     the caller's next synchronisation on that stream.
 *   - Grouped heads: value head h reads query/key head h / (n_v_heads /
 *     n_qk_heads); n_v_heads must be a multiple of n_qk_heads.  Passing
 *     n_qk_heads == n_v_heads is [FM]'s "already repeated" contract.
 *   - Shape limits ([FM] "Shape limits" block): the state size S is one of
 *     32, 64, 128, 256; the conv kernel width is 2..8; a norm head width
 *     (head_dim) is a multiple of 32, and this library has kernels for
 *     32, 64, 128 and 256 (other multiples return GDN_ERR_UNSUPPORTED).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_NULL = -1,        /* a required pointer is NULL */
  GDN_ERR_SHAPE = -2,       /* a size or stride is out of range or inconsistent */
  GDN_ERR_UNSUPPORTED = -3, /* a valid shape this library has no kernel for */
  GDN_ERR_ALIAS = -4,       /* outputs overlap inputs where that is not allowed */
  GDN_ERR_WORKSPACE = -5,   /* the workspace is missing, too small or misaligned */
  GDN_ERR_LAUNCH = -6,      /* the HIP runtime refused the launch */
  GDN_ERR_SCRATCH = -7      /* the sizes exceed a fixed on-device scratch array */
} gdn_status;

/* Static, NUL-terminated description of a status code. */
const char *gdn_strerror(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int gdn_version(void);

/*
 * Decay gate.  [FM] "Decay gate" section, fm_ssm_decay_gate_at;
 * [SCR] "GDN staleness", log_gate.
 *
 *   g[r][h] = a[h] * softplus(alpha[r][h] + dt[h]),
 *   softplus(v) = v if v > 20, else log1p(exp(v)),
 *
 * with a = -exp(A_log) pre-baked by the caller, so g < 0; g is returned
 * PRE-exp (the recurrence exponentiates it).
 *   alpha [rows][n_heads], row stride n_heads       (in)
 *   dt, a [n_heads]                                (in)
 *   g     [rows][n_heads]                          (out, may alias alpha)
 * rows >= 0 (0 launches nothing), n_heads >= 1.
 */
int gdn_decay_gate(const float *alpha, const float *dt, const float *a, float *g, int rows,
                   int n_heads, hipStream_t stream);

/*
 * Depthwise causal conv1d + SiLU + per-head L2 norm on the Q/K channels, over
 * n_tok consecutive positions of n_seq independent sequences.
 * [FM] "Causal depthwise conv1d + SiLU" section (fm_ssm_conv1d_silu_at,
 * fm_ssm_conv1d_silu_seq_at); [AT] conv1d_update_l2norm,
 * conv1d_update_l2norm_strided, gdn_verify_fused_conv_k2 and
 * conv1d_update_prefill; [SCR] "GDN staleness" for the L2 form.
 *
 * Per sequence s, position t, channel c:
 *   window = [hist[c][0] .. hist[c][d_conv-2], x[t][c]]  (oldest first)
 *   o      = silu(sum_j w[c][j] * window[j])
 *   then hist[c] shifts by one place: its oldest value leaves and the input
 *   x[t][c] itself (not the activated o) becomes its newest value
 *   for c < qk_channels: o /= sqrt(sum over c's head_dim block of o^2 + l2_eps)
 *
 *   x     element x[s][t][c] at x + s*x_seq_stride + t*x_tok_stride + c  (in)
 *   w     [conv_dim][d_conv], row-major; tap d_conv-1 meets the newest input (in)
 *   conv_state [s][conv_dim][d_conv-1] at conv_state + s*state_seq_stride,
 *         oldest tap first, updated in place to the window after the last position
 *   out   element at out + s*out_seq_stride + t*out_tok_stride + c        (out)
 *   snap  NULL, or the rollback snapshots: the history after position t, for
 *         t < n_tok-1, at snap + s*snap_seq_stride + t*snap_tok_stride
 *         ([conv_dim][d_conv-1] each); the committed history stays in conv_state.
 *
 * Requirements: n_seq >= 1, n_tok >= 1, conv_dim >= 1, 2 <= d_conv <= 8,
 * 0 <= qk_channels <= conv_dim, qk_channels % head_dim == 0, head_dim in
 * {32, 64, 128, 256} (ignored when qk_channels == 0), x_tok_stride >= conv_dim
 * when n_tok > 1 and out_tok_stride >= conv_dim when n_tok > 1, sequence strides
 * large enough that sequences do not overlap.  out must not overlap x or
 * conv_state; snap must not overlap conv_state.
 * The result does not depend on which internal kernel runs: the multi-position
 * path and n single-position calls agree bit for bit.
 */
int gdn_conv1d_silu_l2norm(const float *x, int64_t x_tok_stride, int64_t x_seq_stride,
                           const float *w, float *conv_state, int64_t state_seq_stride,
                           float *out, int64_t out_tok_stride, int64_t out_seq_stride,
                           float *snap, int64_t snap_tok_stride, int64_t snap_seq_stride,
                           int n_seq, int n_tok, int conv_dim, int d_conv, int qk_channels,
                           int head_dim, float l2_eps, hipStream_t stream);

/*
 * Gated delta-rule recurrence, token by token (decode and K-position verify).
 * [FM] "Delta-rule recurrence" section (fm_ssm_recurrence_at,
 * fm_ssm_recurrence_seq_at); [AT] gdn_verify_fused_conv_k2 for the rollback
 * snapshot semantics.
 *
 * For each sequence s, value head h and position t, on the S x S state of
 * (s, h), in this order:
 *   S <- exp(g) S;  p = S^T k;  delta = beta (v - p);  S <- S + k delta^T;
 *   y = scale S^T q        (the readout sees the updated state)
 *
 *   state [s][h][j][i] = S[i][j] (TRANSPOSED: row j, value index, is contiguous
 *         over the key index i), sequence stride state_seq_stride >= H*S*S,
 *         updated in place                                              (in/out)
 *   q, k  element [s][t][hk][i] at q + s*qk_seq_stride + t*qk_tok_stride + hk*S + i
 *   v     element [s][t][h][j]  at v + s*v_seq_stride + t*v_tok_stride + h*S + j
 *   g, beta  dense [n_seq][n_tok][n_v_heads]; g pre-exp, beta already sigmoid'd
 *   y     element [s][t][h][j]  at y + s*y_seq_stride + t*y_tok_stride + h*S + j (out)
 *   snap  NULL, or the state after position t for t < n_tok-1, in the state's
 *         layout, at snap + s*snap_seq_stride + t*(n_v_heads*S*S)         (out)
 *
 * Running n_tok positions in one call and n_tok calls of one position give
 * bit-identical y and state.  y must not overlap any input; snap must not
 * overlap state.  S in {32, 64, 128, 256}.
 */
int gdn_recurrence_decode(float *state, int64_t state_seq_stride, const float *q, const float *k,
                          int64_t qk_tok_stride, int64_t qk_seq_stride, const float *v,
                          int64_t v_tok_stride, int64_t v_seq_stride, const float *g,
                          const float *beta, float *y, int64_t y_tok_stride, int64_t y_seq_stride,
                          float *snap, int64_t snap_seq_stride, int n_seq, int n_tok,
                          int n_v_heads, int n_qk_heads, int S, float scale, hipStream_t stream);

/*
 * Workspace bytes gdn_recurrence_chunked needs for these sizes (0 if the
 * sizes are invalid).  [AT] "Mamba-2 SSD chunked prefill scan" comment for
 * the chunked idea; the WY/UT algebra is given with gdn_recurrence_chunked.
 */
size_t gdn_recurrence_chunked_workspace_bytes(int n_seq, int n_tok, int n_v_heads,
                                              int n_qk_heads, int S, int chunk);

/*
 * The same recurrence over a long prompt in chunked (WY / UT-transform) form,
 * one dependent step per chunk of positions instead of one per position ([AT]
 * "Mamba-2 SSD chunked prefill scan" comment); [FM] fm_ssm_recurrence_seq_at is the sequential scan
 * it is validated against.  Per chunk of n <= chunk tokens from state S0, with
 * G_t the inclusive within-chunk cumulative sum of g:
 *   A  = strictly_lower(beta_t e^{G_t-G_s} k_t.k_s),  T = (I + A)^{-1}
 *   W  = T diag(beta e^G) K,   U = T diag(beta) V - W S0
 *   y  = scale [diag(e^G) Q S0 + (L o Q K^T) U],  L[t][s] = e^{G_t-G_s} (s <= t)
 *   S  = e^{G_n} S0 + (diag(e^{G_n-G}) K)^T U
 * Same tensor arguments and layouts as gdn_recurrence_decode (no snapshots).
 *
 * Preconditions (the chunked form's algebra and storage rely on them; the
 * token-by-token entry point needs neither):
 *   - g <= 0 at every position (true for gdn_decay_gate's output): every
 *     exponential the chunked form takes is of a non-positive argument;
 *   - beta_t |k_t|^2 <= 2 at every position (true for unit-length keys and
 *     beta in [0, 1]), so every factor I - beta_t k_t k_t^T has spectral
 *     norm <= 1.  Under these two, |T[t][s]| <= beta_t for s < t, every entry
 *     of W is at most beta_t |k_t| (its rows are products of such
 *     contractions applied to beta_t e^{G_t} k_t), every entry of (L o Q K^T)
 *     at most |q_t| |k_s|, and every entry of Q and K at most 1 for unit-length
 *     queries and keys.
 * Numerics at S = 128: the intra-chunk products (K K^T, Q K^T, W,
 * T diag(beta) V) run on bf16 MFMA with each fp32 operand split into hi + lo
 * and fp32 accumulation; the triangular inverse, cumulative gate,
 * exponentials and the state carry are fp32.  W and Q are stored in the
 * workspace as fp16, K and L o Q K^T as fp16 hi + lo (Q and K once per
 * query/key head); the inter-chunk products use them on fp16 MFMA against the
 * state and U split into fp16 hi + lo after a power-of-two scaling chosen from
 * a running bound on their norms (so no input size can overflow fp16).
 * Agreement with the sequential scan is a tolerance (normwise 2e-3), not bit
 * identity; outside the preconditions the results are not specified.
 *
 * chunk must be 64; S in {32, 64, 128} (256 returns GDN_ERR_UNSUPPORTED).
 * S = 128 runs the two-phase MFMA form above and needs a workspace: device
 * memory of at least gdn_recurrence_chunked_workspace_bytes(...) bytes,
 * 256-byte aligned, owned by the caller and not used by anything else until
 * the call's work on `stream` has finished.  S = 32 and 64 run the same
 * algebra in fp32, one workgroup per (sequence, head) with every chunk tile on
 * chip; the workspace size is 0 and workspace may be NULL.
 */
int gdn_recurrence_chunked(float *state, int64_t state_seq_stride, const float *q, const float *k,
                           int64_t qk_tok_stride, int64_t qk_seq_stride, const float *v,
                           int64_t v_tok_stride, int64_t v_seq_stride, const float *g,
                           const float *beta, float *y, int64_t y_tok_stride,
                           int64_t y_seq_stride, int n_seq, int n_tok, int n_v_heads,
                           int n_qk_heads, int S, float scale, int chunk, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * Workspace bytes gdn_prefill_chunked needs (0 if the sizes are invalid or
 * unsupported); the same amount as gdn_recurrence_chunked at S = 128.
 */
size_t gdn_prefill_chunked_workspace_bytes(int n_seq, int n_tok, int n_v_heads, int n_qk_heads,
                                           int S, int chunk);

/*
 * The prefill layer core up to the norm in two launches: decay gate (as
 * gdn_decay_gate) and depthwise conv1d + SiLU + per-head L2 (as
 * gdn_conv1d_silu_l2norm) computed inside the chunked recurrence's first
 * phase, then the chunked recurrence (as gdn_recurrence_chunked).  [AT]
 * conv1d_update_prefill (the conv of every position depends on inputs only,
 * so it runs token-parallel with the per-position arithmetic unchanged) and
 * conv1d_update_l2norm (fusing neighbouring ops saves launches and memory
 * passes); [AT] "Mamba-2 SSD chunked prefill scan" comment; [FM] "Causal
 * depthwise conv1d + SiLU" and "Decay gate" sections.  The conv outputs and
 * g never go to device memory.
 *
 * The conv row of a position carries conv_dim = (2*n_qk_heads + n_v_heads)*S
 * channels: q heads at [0, Hk*S), k heads at [Hk*S, 2*Hk*S), v heads at
 * [2*Hk*S, conv_dim), i.e. qk_channels = 2*Hk*S and head_dim = S for the
 * conv.
 *   x            element x[s][t][c] at x + s*x_seq_stride + t*x_tok_stride + c (in)
 *   conv_w       [conv_dim][d_conv], tap d_conv-1 meets the newest input  (in)
 *   conv_state   [s][conv_dim][d_conv-1] at conv_state + s*conv_state_seq_stride,
 *                oldest tap first, updated in place to the window after the
 *                last position                                          (in/out)
 *   alpha        [n_seq][n_tok][n_v_heads] dense; dt, a [n_v_heads]: the
 *                decay gate's inputs, g = a*softplus(alpha + dt)         (in)
 *   beta         [n_seq][n_tok][n_v_heads] dense, already sigmoid'd    (in)
 *   state, y     as gdn_recurrence_chunked                    (in/out, out)
 *   workspace    at least gdn_prefill_chunked_workspace_bytes(...) bytes,
 *                256-byte aligned, under gdn_recurrence_chunked's rules
 * Supported: S = 128, d_conv = 4, chunk = 64 (other valid sizes return
 * GDN_ERR_UNSUPPORTED); x, conv_w, conv_state, the state and y 16-byte aligned
 * with strides that are multiples of 4; n_tok >= 1.  The preconditions of
 * gdn_recurrence_chunked apply to the conv outputs and g (the L2 step gives
 * unit-length q and k; a <= 0 gives g <= 0).
 * Results (y, state and conv_state) are bit-identical to gdn_decay_gate into
 * g, gdn_conv1d_silu_l2norm into a buffer, then gdn_recurrence_chunked on the
 * buffer's q, k, v channels.  No output may overlap an input, another output
 * or the workspace.
 */
int gdn_prefill_chunked(float *state, int64_t state_seq_stride, const float *x,
                        int64_t x_tok_stride, int64_t x_seq_stride, const float *conv_w,
                        float *conv_state, int64_t conv_state_seq_stride, const float *alpha,
                        const float *dt, const float *a, const float *beta, float *y,
                        int64_t y_tok_stride, int64_t y_seq_stride, int n_seq, int n_tok,
                        int n_v_heads, int n_qk_heads, int S, int d_conv, float scale,
                        float l2_eps, int chunk, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* Most sequences one gdn_recurrence_chunked_varlen call takes. */
#define GDN_VARLEN_MAX_SEQ 256

/* Element type of the q, k, v inputs of gdn_recurrence_chunked_varlen. */
typedef enum {
  GDN_DTYPE_F32 = 0,  /* IEEE binary32 */
  GDN_DTYPE_BF16 = 1  /* bfloat16: the upper 16 bits of a binary32 */
} gdn_dtype;

/*
 * Workspace bytes gdn_recurrence_chunked_varlen needs for any split of
 * total_tok positions into n_seq sequences (a bound; 0 if the sizes are
 * invalid or S is 32 or 64, which need none).
 */
size_t gdn_recurrence_chunked_varlen_workspace_bytes(int n_seq, int total_tok, int n_v_heads,
                                                     int n_qk_heads, int S, int chunk);

/*
 * The chunked recurrence of gdn_recurrence_chunked over a packed batch of
 * sequences of different lengths, in one call: every sequence runs the
 * chunked form from its own state, its chunks starting at its own first
 * position.  [AT] "Mamba-2 SSD chunked prefill scan" comment (one dependent
 * step per chunk of each sequence); [FM] fm_ssm_recurrence_seq_at is the
 * per-sequence definition.
 *
 *   cu_seqlens  HOST array of n_seq + 1 int32: sequence s holds packed token
 *               rows cu_seqlens[s] .. cu_seqlens[s+1]-1; cu_seqlens[0] = 0,
 *               non-decreasing, cu_seqlens[n_seq] = total_tok.  Empty
 *               sequences are allowed (their state is left as it is).  Read
 *               during the call only.
 *   state       [n_seq][H][S][S] fp32, sequence stride state_seq_stride (in/out)
 *   q, k        [total_tok][Hk][S], row stride qk_tok_stride               (in)
 *   v           [total_tok][H][S],  row stride v_tok_stride                (in)
 *   qkv_dtype   element type of q, k and v (gdn_dtype; strides count
 *               elements of that type).  bf16 values are widened to fp32
 *               exactly on load, so a bf16 call equals, bit for bit, an fp32
 *               call on the same values; everything else stays fp32.  At
 *               S = 128, q, k, v are 16-byte aligned and their row strides a
 *               multiple of 16 bytes.
 *   g, beta     [total_tok][H] dense                                       (in)
 *   y           [total_tok][H][S],  row stride y_tok_stride                (out)
 * 1 <= n_seq <= GDN_VARLEN_MAX_SEQ, total_tok >= 0 (0: nothing to do), chunk
 * 64, S in {32, 64, 128}.  S = 128 needs a workspace of at least
 * gdn_recurrence_chunked_varlen_workspace_bytes(...) bytes, 256-byte aligned,
 * under the same rules as gdn_recurrence_chunked's.  Each sequence's results
 * are bit-identical to a gdn_recurrence_chunked call on that sequence alone.
 * A malformed cu_seqlens returns GDN_ERR_SHAPE before any launch.
 */
int gdn_recurrence_chunked_varlen(float *state, int64_t state_seq_stride, const void *q,
                                  const void *k, int64_t qk_tok_stride, const void *v,
                                  int64_t v_tok_stride, int qkv_dtype, const float *g,
                                  const float *beta, float *y, int64_t y_tok_stride,
                                  const int32_t *cu_seqlens,
                                  int n_seq, int total_tok, int n_v_heads, int n_qk_heads, int S,
                                  float scale, int chunk, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * Workspace bytes gdn_mamba2_ssd_chunked needs (0 if the sizes are invalid).
 */
size_t gdn_mamba2_ssd_workspace_bytes(int n_seq, int n_tok, int n_heads, int head_dim,
                                      int d_state, int chunk);

/*
 * Mamba-2 selective scan over a prompt, chunked (state-space-duality) form.
 * [AT] mamba2_ssm_prefill (its arguments: state, x, B and C projections, raw
 * dt with a per-head bias and dt_min / dt_max limits, A_log, the D skip,
 * n_groups, per-tensor token strides) and its "Mamba-2 SSD chunked prefill
 * scan" comment (one dependent step per 64-position chunk, everything else as
 * dense matrix products).  Per
 * sequence, head h (group h / (n_heads / n_groups)) and token t:
 *   dt = min(max(softplus(dt_raw + dt_bias), dt_min), dt_max)   (softplus
 *        guarded at 20),  A = -exp(A_log)
 *   state <- exp(dt A) state + dt x B^T,   y = state C + D x
 *
 *   state   [n_seq][H][head_dim][d_state] fp32, sequence stride        (in/out)
 *   x       [n_seq][T][H][head_dim], token / sequence strides          (in)
 *   B, C    [n_seq][T][G][d_state], shared token / sequence strides    (in)
 *   dt_raw  [n_seq][T][H], token / sequence strides                    (in)
 *   A_log, D, dt_bias  [H]                                             (in)
 *   y       [n_seq][T][H][head_dim], token / sequence strides          (out)
 * All fp32 device memory, strides in elements.  head_dim in {32, 64},
 * d_state in {64, 128}, chunk 64, n_heads % n_groups == 0, T >= 1.  x, B, C,
 * y, state 16-byte aligned with strides a multiple of 4.  The workspace is
 * device memory of gdn_mamba2_ssd_workspace_bytes(...) bytes, 256-byte
 * aligned, owned by the caller.  fp32 arithmetic throughout; the result
 * matches the token-by-token scan to rounding, not bit for bit.
 */
int gdn_mamba2_ssd_chunked(float *state, int64_t state_seq_stride, const float *x,
                           int64_t x_tok_stride, int64_t x_seq_stride, const float *B,
                           const float *C, int64_t bc_tok_stride, int64_t bc_seq_stride,
                           const float *dt_raw, int64_t dt_tok_stride, int64_t dt_seq_stride,
                           const float *A_log, const float *D, const float *dt_bias, float *y,
                           int64_t y_tok_stride, int64_t y_seq_stride, int n_seq, int n_tok,
                           int n_heads, int n_groups, int head_dim, int d_state, float dt_min,
                           float dt_max, int chunk, void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Gated RMSNorm per (row, head).  [FM] "Gated RMSNorm" section
 * (fm_ssm_gated_norm_at); [AT] gdn_verify_fused_norm_k2 for reading z out of
 * a wider per-token row (pass z already offset to its column).
 *
 *   out = ((y * (1 / sqrt(mean(y^2) + eps))) * w) * silu(z)
 *
 *   y    [rows][n_heads][head_dim] with row stride y_row_stride      (in)
 *   w    [head_dim], shared by every head                             (in)
 *   z    [rows][n_heads][head_dim] with row stride z_row_stride      (in)
 *   out  [rows][n_heads][head_dim] with row stride out_row_stride    (out;
 *        may alias y exactly, i.e. out == y with equal row strides)
 * head_dim in {32, 64, 128, 256}; rows >= 0; n_heads >= 1; row strides >=
 * n_heads*head_dim when rows > 1.
 */
int gdn_gated_rmsnorm(const float *y, int64_t y_row_stride, const float *w, const float *z,
                      int64_t z_row_stride, float *out, int64_t out_row_stride, int rows,
                      int n_heads, int head_dim, float eps, hipStream_t stream);

/*
 * The decode / K-position verify layer core in one launch: decay gate ->
 * recurrence -> gated RMSNorm (the norm's head_dim is S).  [FM] header notes
 * on timing: the decay gate is dispatch cost that should ride with its
 * neighbours; [AT] conv1d_update_l2norm: fusing neighbouring ops saves a
 * launch per layer.
 *
 * Per (s, t, h):  g = a[h] * softplus(alpha[s][t][h] + dt[h])  (as
 * gdn_decay_gate), then the recurrence of gdn_recurrence_decode with that g,
 * then out = gated_rmsnorm(y, norm_w, z) per head (as gdn_gated_rmsnorm).
 * Each value is computed with the same operations in the same order as those
 * three calls; with 16-byte aligned buffers (on which gdn_gated_rmsnorm takes
 * its 16-byte path) the results are bit-identical to them.
 *
 *   state, q, k, v, beta, snap: as gdn_recurrence_decode
 *   alpha  dense [n_seq][n_tok][n_v_heads]; dt, a: [n_v_heads]          (in)
 *   norm_w [S], 16-byte aligned                                          (in)
 *   z      element [s][t][h][j] at z + s*z_seq_stride + t*z_tok_stride + h*S + j,
 *          16-byte aligned, strides multiples of 4                       (in)
 *   out    the normed output, element [s][t][h][j] at
 *          out + s*out_seq_stride + t*out_tok_stride + h*S + j, 16-byte
 *          aligned, strides multiples of 4                              (out)
 *   g      NULL, or dense [n_seq][n_tok][n_v_heads]: the gate values    (out)
 *   y      NULL, or the pre-norm output in the layout of out with its own
 *          strides                                                      (out)
 * No output may overlap an input or another output.  S in {32, 64, 128, 256}.
 */
int gdn_decode_fused(float *state, int64_t state_seq_stride, const float *q, const float *k,
                     int64_t qk_tok_stride, int64_t qk_seq_stride, const float *v,
                     int64_t v_tok_stride, int64_t v_seq_stride, const float *alpha,
                     const float *dt, const float *a, const float *beta, const float *norm_w,
                     const float *z, int64_t z_tok_stride, int64_t z_seq_stride, float *out,
                     int64_t out_tok_stride, int64_t out_seq_stride, float *g, float *y,
                     int64_t y_tok_stride, int64_t y_seq_stride, float *snap,
                     int64_t snap_seq_stride, int n_seq, int n_tok, int n_v_heads,
                     int n_qk_heads, int S, float scale, float norm_eps, hipStream_t stream);

/*
 * Workspace bytes gdn_decode_step needs: n_seq * n_qk_heads * 2 int32
 * counters (0 if the sizes are invalid).
 */
size_t gdn_decode_step_workspace_bytes(int n_seq, int n_qk_heads);

/*
 * The whole decode / K-position verify layer core in one launch: conv1d +
 * SiLU + per-head L2 (as gdn_conv1d_silu_l2norm) -> decay gate -> recurrence
 * -> gated RMSNorm (as gdn_decode_fused).  [AT] gdn_verify_fused_conv_k2
 * (the conv, its rollback snapshot and the recurrence of a K = 2 verify in
 * one launch) and conv1d_update_l2norm (fusing neighbouring ops saves
 * launches per layer); [FM] header notes (the gate rides with its
 * neighbours).
 *
 * The conv row of a position carries conv_dim = (2*n_qk_heads + n_v_heads)*S
 * channels: q heads at [0, Hk*S), k heads at [Hk*S, 2*Hk*S), v heads at
 * [2*Hk*S, conv_dim), i.e. qk_channels = 2*Hk*S and head_dim = S in the terms
 * of gdn_conv1d_silu_l2norm.  The conv outputs feed the recurrence on chip
 * and are not written out.
 *
 *   x, conv_w, conv_state, conv_snap: as gdn_conv1d_silu_l2norm with that
 *          conv_dim; x, conv_w, conv_state and conv_snap 16-byte aligned,
 *          their strides multiples of 4                             (in / in/out)
 *   state, alpha, dt, a, beta, norm_w, z, out, g, y, snap: as gdn_decode_fused
 *   workspace: at least gdn_decode_step_workspace_bytes(n_seq, n_qk_heads)
 *          bytes of device memory, 4-byte aligned, ZERO-FILLED by the caller
 *          before its first use; the work of every call that returns GDN_OK
 *          leaves it zero-filled again.  Calls whose work may overlap in time
 *          (other streams) need workspaces of their own.
 *
 * The value heads of one query/key group all read the group's q/k conv
 * history; each takes a ticket from a workspace counter once it has read it,
 * and the last one writes the new history, so no workgroup waits for another.
 * Results are bit-identical to gdn_conv1d_silu_l2norm into a buffer followed
 * by gdn_decode_fused on its q, k, v channels.  1 <= n_tok <= 32 (<= 16 at
 * S = 256); S in {32, 64, 128, 256}; d_conv in {2, 3, 4} (2..8 are valid
 * widths; the others return GDN_ERR_UNSUPPORTED).  No output may overlap an
 * input, another output or the workspace.
 */
int gdn_decode_step(float *state, int64_t state_seq_stride, const float *x, int64_t x_tok_stride,
                    int64_t x_seq_stride, const float *conv_w, float *conv_state,
                    int64_t conv_state_seq_stride, float *conv_snap,
                    int64_t conv_snap_tok_stride, int64_t conv_snap_seq_stride,
                    const float *alpha, const float *dt, const float *a, const float *beta,
                    const float *norm_w, const float *z, int64_t z_tok_stride,
                    int64_t z_seq_stride, float *out, int64_t out_tok_stride,
                    int64_t out_seq_stride, float *g, float *y, int64_t y_tok_stride,
                    int64_t y_seq_stride, float *snap, int64_t snap_seq_stride, int n_seq,
                    int n_tok, int n_v_heads, int n_qk_heads, int S, int d_conv, float scale,
                    float l2_eps, float norm_eps, void *workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* Bytes of the on-device scratch array of gdn_decode_step_noalloc (per GPU). */
#define GDN_NOALLOC_SCRATCH_BYTES 65536

/*
 * gdn_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and results (bit for bit) as gdn_decode_step, with
 * no workspace argument: the ticket counters live in a file-scope device array
 * of GDN_NOALLOC_SCRATCH_BYTES bytes inside the library, one copy per GPU,
 * held until the process ends.  The call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine).
 *
 *   Limit: gdn_decode_step_workspace_bytes(n_seq, n_qk_heads) must not exceed
 *   GDN_NOALLOC_SCRATCH_BYTES (n_seq * n_qk_heads <= 8192), else
 *   GDN_ERR_SCRATCH before anything is launched.
 *   Set-up: the first call on a device (with that device current) looks up
 *   the array's device address and clears it with a small kernel on `stream`;
 *   every call whose work completes leaves the counters it used at zero.
 *   Sharing: every call on one GPU uses that GPU's one array, so calls whose
 *   work may overlap in time on one GPU (different streams, or concurrent
 *   host threads) race on the counters; serialise them on one stream.
 */
int gdn_decode_step_noalloc(float *state, int64_t state_seq_stride, const float *x,
                            int64_t x_tok_stride, int64_t x_seq_stride, const float *conv_w,
                            float *conv_state, int64_t conv_state_seq_stride, float *conv_snap,
                            int64_t conv_snap_tok_stride, int64_t conv_snap_seq_stride,
                            const float *alpha, const float *dt, const float *a,
                            const float *beta, const float *norm_w, const float *z,
                            int64_t z_tok_stride, int64_t z_seq_stride, float *out,
                            int64_t out_tok_stride, int64_t out_seq_stride, float *g, float *y,
                            int64_t y_tok_stride, int64_t y_seq_stride, float *snap,
                            int64_t snap_seq_stride, int n_seq, int n_tok, int n_v_heads,
                            int n_qk_heads, int S, int d_conv, float scale, float l2_eps,
                            float norm_eps, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
