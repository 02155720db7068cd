// gdn_api.cpp -- the extern "C" entry points declared in include/gdn.h:
// validate on the host, then hand over to the kernel family's launcher.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"

#include "launch.hpp"
#include "validate.hpp"

namespace {

// The argument block of the one-launch decode step (conv -> gate ->
// recurrence -> norm), shared by gdn_decode_step and gdn_decode_step_noalloc;
// cnt is the ticket counter array.
int launch_step(float *state, int64_t state_seq_stride, const float *x, int64_t x_tok_stride,
                int64_t x_seq_stride, const float *conv_w, float *conv_state,
                int64_t conv_state_seq_stride, float *conv_snap, int64_t conv_snap_tok_stride,
                int64_t conv_snap_seq_stride, const float *alpha, const float *dt,
                const float *a, const float *beta, const float *norm_w, const float *z,
                int64_t z_tok_stride, int64_t z_seq_stride, float *out, int64_t out_tok_stride,
                int64_t out_seq_stride, float *g, float *y, int64_t y_tok_stride,
                int64_t y_seq_stride, float *snap, int64_t snap_seq_stride, int n_seq, int n_tok,
                int n_v_heads, int n_qk_heads, int S, int d_conv, float scale, float l2_eps,
                float norm_eps, int *cnt, hipStream_t stream) {
  gdn::StepArgs sa{};
  sa.f.r = gdn::RecurArgs{state,          state_seq_stride, nullptr,     nullptr,
                          0,              0,                nullptr,     0,
                          0,              nullptr,          beta,        out,
                          out_tok_stride, out_seq_stride,   snap,        snap_seq_stride,
                          n_seq,          n_tok,            n_v_heads,   n_qk_heads,
                          S,              scale};
  sa.f.alpha = alpha;
  sa.f.dt = dt;
  sa.f.a = a;
  sa.f.w = norm_w;
  sa.f.z = z;
  sa.f.z_tok = z_tok_stride;
  sa.f.z_seq = z_seq_stride;
  sa.f.g = g;
  sa.f.y = y;
  sa.f.y_tok = y_tok_stride;
  sa.f.y_seq = y_seq_stride;
  sa.f.eps = norm_eps;
  sa.x = x;
  sa.x_tok = x_tok_stride;
  sa.x_seq = x_seq_stride;
  sa.cw = conv_w;
  sa.hist = conv_state;
  sa.h_seq = conv_state_seq_stride;
  sa.csnap = conv_snap;
  sa.cs_tok = conv_snap_tok_stride;
  sa.cs_seq = conv_snap_seq_stride;
  sa.D = d_conv;
  sa.l2_eps = l2_eps;
  sa.cnt = cnt;
  return gdn::launch_decode_step(sa, stream);
}

// ---- the no-allocation decode step's ticket counters
// One array per GPU (each device holds its own copy at its own address).  In
// host code `step_scratch` names a host-side stand-in, never the device
// memory: kernels and memory operations get the address that
// hipGetSymbolAddress returns for the current device, kept per device.
__device__ __align__(256) int step_scratch[GDN_NOALLOC_SCRATCH_BYTES / sizeof(int)];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
int *scratch_dev_ptr[MAX_DEVICES] = {};

__global__ void k_clear_ints(int *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// The current device's scratch address; on the first call on a device, look
// it up and clear the array with a kernel on `stream` (a kernel, not a memset
// node, so the clear is also valid inside a captured graph).
int step_scratch_ptr(hipStream_t stream, int **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return GDN_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(step_scratch)) != hipSuccess || !p)
      return GDN_ERR_LAUNCH;
    constexpr int n = GDN_NOALLOC_SCRATCH_BYTES / sizeof(int);
    const int rc = gdn::launch_kernel(k_clear_ints, dim3((n + 255) / 256), dim3(256), 0, stream,
                                      static_cast<int *>(p), n);
    if (rc != GDN_OK) return rc;
    scratch_dev_ptr[dev] = static_cast<int *>(p);
  }
  *out = scratch_dev_ptr[dev];
  return GDN_OK;
}

}  // namespace

extern "C" {

const char *gdn_strerror(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "a required pointer is NULL";
    case GDN_ERR_SHAPE: return "a size, stride or alignment is out of range or inconsistent";
    case GDN_ERR_UNSUPPORTED: return "valid shape with no kernel in this library";
    case GDN_ERR_ALIAS: return "an output overlaps an input where that is not allowed";
    case GDN_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case GDN_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
    case GDN_ERR_SCRATCH: return "sizes exceed the fixed scratch array of a no-allocation call";
    default: return "unknown gdn status";
  }
}

int gdn_version(void) { return 100; /* 0.1.0 */ }

int gdn_decay_gate(const float *alpha, const float *dt, const float *a, float *g, int rows,
                   int n_heads, hipStream_t stream) {
  const int rc = gdn::check_decay_gate(alpha, dt, a, g, rows, n_heads);
  if (rc != GDN_OK || rows == 0) return rc;
  return gdn::launch_decay_gate(alpha, dt, a, g, rows, n_heads, stream);
}

int gdn_conv1d_silu_l2norm(const float *x, int64_t x_tok_stride, int64_t x_seq_stride,
                           const float *w, float *conv_state, int64_t state_seq_stride,
                           float *out, int64_t out_tok_stride, int64_t out_seq_stride,
                           float *snap, int64_t snap_tok_stride, int64_t snap_seq_stride,
                           int n_seq, int n_tok, int conv_dim, int d_conv, int qk_channels,
                           int head_dim, float l2_eps, hipStream_t stream) {
  const int rc = gdn::check_conv(x, x_tok_stride, x_seq_stride, w, conv_state, state_seq_stride,
                                 out, out_tok_stride, out_seq_stride, snap, snap_tok_stride,
                                 snap_seq_stride, n_seq, n_tok, conv_dim, d_conv, qk_channels,
                                 head_dim);
  if (rc != GDN_OK) return rc;
  gdn::ConvArgs a{x,        x_tok_stride,  x_seq_stride,   w,       conv_state,
                  state_seq_stride, out,   out_tok_stride, out_seq_stride,
                  snap,     snap_tok_stride, snap_seq_stride, n_seq, n_tok,
                  conv_dim, d_conv,        qk_channels,    head_dim, l2_eps};
  return gdn::launch_conv(a, stream);
}

int gdn_recurrence_decode(float *state, int64_t state_seq_stride, const float *q, const float *k,
                          int64_t qk_tok_stride, int64_t qk_seq_stride, const float *v,
                          int64_t v_tok_stride, int64_t v_seq_stride, const float *g,
                          const float *beta, float *y, int64_t y_tok_stride, int64_t y_seq_stride,
                          float *snap, int64_t snap_seq_stride, int n_seq, int n_tok,
                          int n_v_heads, int n_qk_heads, int S, float scale, hipStream_t stream) {
  const int rc = gdn::check_recur(state, state_seq_stride, q, k, qk_tok_stride, qk_seq_stride, v,
                                  v_tok_stride, v_seq_stride, g, beta, y, y_tok_stride,
                                  y_seq_stride, snap, snap_seq_stride, n_seq, n_tok, n_v_heads,
                                  n_qk_heads, S);
  if (rc != GDN_OK) return rc;
  gdn::RecurArgs a{state,        state_seq_stride, q,           k,          qk_tok_stride,
                   qk_seq_stride, v,               v_tok_stride, v_seq_stride, g,
                   beta,         y,                y_tok_stride, y_seq_stride, snap,
                   snap_seq_stride, n_seq,         n_tok,        n_v_heads,  n_qk_heads,
                   S,            scale};
  return gdn::launch_recur_decode(a, stream);
}

size_t gdn_recurrence_chunked_workspace_bytes(int n_seq, int n_tok, int n_v_heads,
                                              int n_qk_heads, int S, int chunk) {
  if (n_seq < 1 || n_tok < 1 || n_v_heads < 1 || n_qk_heads < 1 || n_v_heads % n_qk_heads)
    return 0;
  if ((S != 32 && S != 64 && S != 128) || chunk != 64) return 0;
  return gdn::chunked_workspace_bytes(n_seq, n_tok, n_v_heads, n_qk_heads, S, chunk);
}

int gdn_recurrence_chunked(float *state, int64_t state_seq_stride, const float *q, const float *k,
                           int64_t qk_tok_stride, int64_t qk_seq_stride, const float *v,
                           int64_t v_tok_stride, int64_t v_seq_stride, const float *g,
                           const float *beta, float *y, int64_t y_tok_stride,
                           int64_t y_seq_stride, int n_seq, int n_tok, int n_v_heads,
                           int n_qk_heads, int S, float scale, int chunk, void *workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  const size_t need =
      gdn_recurrence_chunked_workspace_bytes(n_seq, n_tok, n_v_heads, n_qk_heads, S, chunk);
  const int rc = gdn::check_chunked(state, state_seq_stride, q, k, qk_tok_stride, qk_seq_stride,
                                    v, v_tok_stride, v_seq_stride, g, beta, y, y_tok_stride,
                                    y_seq_stride, n_seq, n_tok, n_v_heads, n_qk_heads, S, chunk,
                                    workspace, workspace_bytes, need);
  if (rc != GDN_OK) return rc;
  gdn::RecurArgs a{state,        state_seq_stride, q,           k,          qk_tok_stride,
                   qk_seq_stride, v,               v_tok_stride, v_seq_stride, g,
                   beta,         y,                y_tok_stride, y_seq_stride, nullptr,
                   0,            n_seq,            n_tok,        n_v_heads,  n_qk_heads,
                   S,            scale};
  return gdn::launch_recur_chunked(a, chunk, workspace, workspace_bytes, stream);
}

size_t gdn_prefill_chunked_workspace_bytes(int n_seq, int n_tok, int n_v_heads, int n_qk_heads,
                                           int S, int chunk) {
  if (S != 128 || chunk != 64) return 0;
  return gdn_recurrence_chunked_workspace_bytes(n_seq, n_tok, n_v_heads, n_qk_heads, S, chunk);
}

int gdn_prefill_chunked(float *state, int64_t state_seq_stride, const float *x,
                        int64_t x_tok_stride, int64_t x_seq_stride, const float *conv_w,
                        float *conv_state, int64_t conv_state_seq_stride, const float *alpha,
                        const float *dt, const float *a, const float *beta, float *y,
                        int64_t y_tok_stride, int64_t y_seq_stride, int n_seq, int n_tok,
                        int n_v_heads, int n_qk_heads, int S, int d_conv, float scale,
                        float l2_eps, int chunk, void *workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  const size_t need =
      gdn_prefill_chunked_workspace_bytes(n_seq, n_tok, n_v_heads, n_qk_heads, S, chunk);
  const int rc = gdn::check_prefill(state, state_seq_stride, x, x_tok_stride, x_seq_stride,
                                    conv_w, conv_state, conv_state_seq_stride, alpha, dt, a, beta,
                                    y, y_tok_stride, y_seq_stride, n_seq, n_tok, n_v_heads,
                                    n_qk_heads, S, d_conv, chunk, workspace, workspace_bytes,
                                    need);
  if (rc != GDN_OK) return rc;
  gdn::RecurArgs ra{state,   state_seq_stride, nullptr,      nullptr,      0,
                    0,       nullptr,          0,            0,            nullptr,
                    beta,    y,                y_tok_stride, y_seq_stride, nullptr,
                    0,       n_seq,            n_tok,        n_v_heads,    n_qk_heads,
                    S,       scale};
  const gdn::PrefillConv pc{x, x_tok_stride, x_seq_stride, conv_w, conv_state,
                            conv_state_seq_stride, alpha, dt, a, d_conv, l2_eps};
  return gdn::launch_prefill_chunked(ra, pc, chunk, workspace, workspace_bytes, stream);
}

size_t gdn_recurrence_chunked_varlen_workspace_bytes(int n_seq, int total_tok, int n_v_heads,
                                                     int n_qk_heads, int S, int chunk) {
  if (n_seq < 1 || n_seq > GDN_VARLEN_MAX_SEQ || total_tok < 0 || n_v_heads < 1 ||
      n_qk_heads < 1 || n_v_heads % n_qk_heads)
    return 0;
  if ((S != 32 && S != 64 && S != 128) || chunk != 64) return 0;
  return gdn::chunked_varlen_workspace_bytes(n_seq, total_tok, n_v_heads, n_qk_heads, S);
}

int gdn_recurrence_chunked_varlen(float *state, int64_t state_seq_stride, const void *q,
                                  const void *k, int64_t qk_tok_stride, const void *v,
                                  int64_t v_tok_stride, int qkv_dtype, const float *g,
                                  const float *beta, float *y, int64_t y_tok_stride,
                                  const int32_t *cu_seqlens,
                                  int n_seq, int total_tok, int n_v_heads, int n_qk_heads, int S,
                                  float scale, int chunk, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  const size_t need = gdn_recurrence_chunked_varlen_workspace_bytes(n_seq, total_tok, n_v_heads,
                                                                    n_qk_heads, S, chunk);
  const int rc = gdn::check_chunked_varlen(state, state_seq_stride, q, k, qk_tok_stride, v,
                                           v_tok_stride, qkv_dtype, g, beta, y, y_tok_stride,
                                           cu_seqlens, n_seq, total_tok, n_v_heads, n_qk_heads,
                                           S, chunk,
                                           workspace, workspace_bytes, need);
  if (rc != GDN_OK || total_tok == 0) return rc;
  gdn::VarTab tab;
  tab.n_seq = n_seq;
  tab.tok0[0] = 0;
  tab.ch0[0] = 0;
  for (int s = 0; s < n_seq; ++s) {
    tab.tok0[s + 1] = cu_seqlens[s + 1];
    tab.ch0[s + 1] = tab.ch0[s] + gdn::padded_chunks(cu_seqlens[s + 1] - cu_seqlens[s]);
  }
  // q, k, v travel as untyped pointers; the launcher reinterprets them per dtype
  gdn::RecurArgs a{state,   state_seq_stride, static_cast<const float *>(q),
                   static_cast<const float *>(k), qk_tok_stride,
                   0,       static_cast<const float *>(v), v_tok_stride, 0, g,
                   beta,    y,                y_tok_stride, 0,          nullptr,
                   0,       n_seq,            total_tok,    n_v_heads,  n_qk_heads,
                   S,       scale};
  return gdn::launch_recur_chunked_varlen(a, tab, qkv_dtype == GDN_DTYPE_BF16, chunk, workspace,
                                          workspace_bytes, stream);
}

size_t gdn_mamba2_ssd_workspace_bytes(int n_seq, int n_tok, int n_heads, int head_dim,
                                      int d_state, int chunk) {
  if (n_seq < 1 || n_tok < 1 || n_heads < 1 || chunk != 64) return 0;
  if ((head_dim != 32 && head_dim != 64) || (d_state != 64 && d_state != 128)) return 0;
  return gdn::ssd_workspace_bytes(n_seq, n_tok, n_heads, head_dim, d_state);
}

int gdn_mamba2_ssd_chunked(float *state, int64_t state_seq_stride, const float *x,
                           int64_t x_tok_stride, int64_t x_seq_stride, const float *B,
                           const float *C, int64_t bc_tok_stride, int64_t bc_seq_stride,
                           const float *dt_raw, int64_t dt_tok_stride, int64_t dt_seq_stride,
                           const float *A_log, const float *D, const float *dt_bias, float *y,
                           int64_t y_tok_stride, int64_t y_seq_stride, int n_seq, int n_tok,
                           int n_heads, int n_groups, int head_dim, int d_state, float dt_min,
                           float dt_max, int chunk, void *workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  const size_t need =
      gdn_mamba2_ssd_workspace_bytes(n_seq, n_tok, n_heads, head_dim, d_state, chunk);
  const int rc = gdn::check_ssd(state, state_seq_stride, x, x_tok_stride, x_seq_stride, B, C,
                                bc_tok_stride, bc_seq_stride, dt_raw, dt_tok_stride,
                                dt_seq_stride, A_log, D, dt_bias, y, y_tok_stride, y_seq_stride,
                                n_seq, n_tok, n_heads, n_groups, head_dim, d_state, chunk,
                                workspace, workspace_bytes, need);
  if (rc != GDN_OK) return rc;
  gdn::SsdLaunch l{state,         state_seq_stride, x,      x_tok_stride, x_seq_stride,
                   B,             C,                bc_tok_stride, bc_seq_stride,
                   dt_raw,        dt_tok_stride,    dt_seq_stride, A_log,  D,
                   dt_bias,       y,                y_tok_stride,  y_seq_stride,
                   n_seq,         n_tok,            n_heads,       n_groups, head_dim,
                   d_state,       dt_min,           dt_max,        workspace};
  return gdn::launch_ssd(l, stream);
}

int gdn_gated_rmsnorm(const float *y, int64_t y_row_stride, const float *w, const float *z,
                      int64_t z_row_stride, float *out, int64_t out_row_stride, int rows,
                      int n_heads, int head_dim, float eps, hipStream_t stream) {
  const int rc = gdn::check_norm(y, y_row_stride, w, z, z_row_stride, out, out_row_stride, rows,
                                 n_heads, head_dim);
  if (rc != GDN_OK || rows == 0) return rc;
  gdn::NormArgs a{y, y_row_stride, w, z, z_row_stride, out, out_row_stride, rows, n_heads,
                  head_dim, eps};
  return gdn::launch_gated_rmsnorm(a, stream);
}

int gdn_decode_fused(float *state, int64_t state_seq_stride, const float *q, const float *k,
                     int64_t qk_tok_stride, int64_t qk_seq_stride, const float *v,
                     int64_t v_tok_stride, int64_t v_seq_stride, const float *alpha,
                     const float *dt, const float *a, const float *beta, const float *norm_w,
                     const float *z, int64_t z_tok_stride, int64_t z_seq_stride, float *out,
                     int64_t out_tok_stride, int64_t out_seq_stride, float *g, float *y,
                     int64_t y_tok_stride, int64_t y_seq_stride, float *snap,
                     int64_t snap_seq_stride, int n_seq, int n_tok, int n_v_heads,
                     int n_qk_heads, int S, float scale, float norm_eps, hipStream_t stream) {
  const int rc = gdn::check_fused(state, state_seq_stride, q, k, qk_tok_stride, qk_seq_stride, v,
                                  v_tok_stride, v_seq_stride, alpha, dt, a, beta, norm_w, z,
                                  z_tok_stride, z_seq_stride, out, out_tok_stride,
                                  out_seq_stride, g, y, y_tok_stride, y_seq_stride, snap,
                                  snap_seq_stride, n_seq, n_tok, n_v_heads, n_qk_heads, S);
  if (rc != GDN_OK) return rc;
  gdn::FusedArgs fa{};
  fa.r = gdn::RecurArgs{state,          state_seq_stride, q,           k,
                        qk_tok_stride,  qk_seq_stride,    v,           v_tok_stride,
                        v_seq_stride,   nullptr,          beta,        out,
                        out_tok_stride, out_seq_stride,   snap,        snap_seq_stride,
                        n_seq,          n_tok,            n_v_heads,   n_qk_heads,
                        S,              scale};
  fa.alpha = alpha;
  fa.dt = dt;
  fa.a = a;
  fa.w = norm_w;
  fa.z = z;
  fa.z_tok = z_tok_stride;
  fa.z_seq = z_seq_stride;
  fa.g = g;
  fa.y = y;
  fa.y_tok = y_tok_stride;
  fa.y_seq = y_seq_stride;
  fa.eps = norm_eps;
  return gdn::launch_decode_fused(fa, stream);
}

size_t gdn_decode_step_workspace_bytes(int n_seq, int n_qk_heads) {
  return gdn::step_workspace_bytes(n_seq, n_qk_heads);
}

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
                    hipStream_t stream) {
  const int rc = gdn::check_step(
      state, state_seq_stride, x, x_tok_stride, x_seq_stride, conv_w, conv_state,
      conv_state_seq_stride, conv_snap, conv_snap_tok_stride, conv_snap_seq_stride, alpha, dt, a,
      beta, norm_w, z, z_tok_stride, z_seq_stride, out, out_tok_stride, out_seq_stride, g, y,
      y_tok_stride, y_seq_stride, snap, snap_seq_stride, n_seq, n_tok, n_v_heads, n_qk_heads, S,
      d_conv, workspace, workspace_bytes);
  if (rc != GDN_OK) return rc;
  return launch_step(state, state_seq_stride, x, x_tok_stride, x_seq_stride, conv_w, conv_state,
                     conv_state_seq_stride, conv_snap, conv_snap_tok_stride,
                     conv_snap_seq_stride, alpha, dt, a, beta, norm_w, z, z_tok_stride,
                     z_seq_stride, out, out_tok_stride, out_seq_stride, g, y, y_tok_stride,
                     y_seq_stride, snap, snap_seq_stride, n_seq, n_tok, n_v_heads, n_qk_heads,
                     S, d_conv, scale, l2_eps, norm_eps, static_cast<int *>(workspace), stream);
}

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
                            float norm_eps, hipStream_t stream) {
  // the fixed array's limit first: a clear error for sizes beyond it
  if (n_seq >= 1 && n_qk_heads >= 1 &&
      gdn::step_workspace_bytes(n_seq, n_qk_heads) > GDN_NOALLOC_SCRATCH_BYTES)
    return GDN_ERR_SCRATCH;
  const int rc = gdn::check_step(
      state, state_seq_stride, x, x_tok_stride, x_seq_stride, conv_w, conv_state,
      conv_state_seq_stride, conv_snap, conv_snap_tok_stride, conv_snap_seq_stride, alpha, dt, a,
      beta, norm_w, z, z_tok_stride, z_seq_stride, out, out_tok_stride, out_seq_stride, g, y,
      y_tok_stride, y_seq_stride, snap, snap_seq_stride, n_seq, n_tok, n_v_heads, n_qk_heads, S,
      d_conv, nullptr, 0, /*lib_scratch=*/true);
  if (rc != GDN_OK) return rc;
  int *cnt = nullptr;
  const int src = step_scratch_ptr(stream, &cnt);
  if (src != GDN_OK) return src;
  return launch_step(state, state_seq_stride, x, x_tok_stride, x_seq_stride, conv_w, conv_state,
                     conv_state_seq_stride, conv_snap, conv_snap_tok_stride,
                     conv_snap_seq_stride, alpha, dt, a, beta, norm_w, z, z_tok_stride,
                     z_seq_stride, out, out_tok_stride, out_seq_stride, g, y, y_tok_stride,
                     y_seq_stride, snap, snap_seq_stride, n_seq, n_tok, n_v_heads, n_qk_heads,
                     S, d_conv, scale, l2_eps, norm_eps, cnt, stream);
}

}  // extern "C"
