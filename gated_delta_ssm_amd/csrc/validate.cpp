// validate.cpp -- host-only argument checks for every entry point.  Nothing
// here calls the HIP runtime, so a wrong call is rejected before any launch
// (and the checks are testable on a machine without a GPU).
//
// Shape limits come from fm_kernel_ssm.h (Foundry), "Shape limits" block and
// the per-function preconditions: state size a multiple of 32 and at most 256,
// conv kernel 2..8, norm head width a multiple of 32, at least one position.
#include "validate.hpp"

#include <cstdint>

#include "gdn.h"

namespace gdn {

namespace {

struct Span {
  uintptr_t lo = 0, hi = 0;  // byte range [lo, hi)
  bool empty() const { return hi <= lo; }
};

// Bytes touched by a [n_outer][n_inner][len] view with element strides
// (elements of esz bytes; fp32 unless stated).
Span span_of(const void *p, int64_t n_outer, int64_t s_outer, int64_t n_inner, int64_t s_inner,
             int64_t len, int64_t esz = sizeof(float)) {
  Span r;
  if (!p || n_outer <= 0 || n_inner <= 0 || len <= 0) return r;
  const int64_t last = (n_outer - 1) * s_outer + (n_inner - 1) * s_inner + len;
  r.lo = (uintptr_t)p;
  r.hi = r.lo + (uintptr_t)(last * esz);
  return r;
}

bool overlap(Span a, Span b) { return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void *p, uintptr_t bytes) { return ((uintptr_t)p % bytes) == 0; }

// Rows of an OUTPUT view must not overlap one another.
bool rows_disjoint(int64_t n_outer, int64_t s_outer, int64_t n_inner, int64_t s_inner,
                   int64_t len) {
  if (n_inner > 1 && s_inner < len) return false;
  if (n_outer > 1 && s_outer < (n_inner - 1) * s_inner + len) return false;
  return true;
}

bool supported_head_dim(int hd) { return hd == 32 || hd == 64 || hd == 128 || hd == 256; }

}  // namespace

int check_decay_gate(const float *alpha, const float *dt, const float *a, const float *g,
                     int rows, int n_heads) {
  if (rows < 0 || n_heads < 1) return GDN_ERR_SHAPE;
  if (rows == 0) return GDN_OK;
  if (!alpha || !dt || !a || !g) return GDN_ERR_NULL;
  const Span out = span_of(g, 1, 0, rows, n_heads, n_heads);
  const Span in = span_of(alpha, 1, 0, rows, n_heads, n_heads);
  // g may be alpha itself (elementwise), but not a shifted overlap of it
  if (overlap(out, in) && g != alpha) return GDN_ERR_ALIAS;
  if (overlap(out, span_of(dt, 1, 0, 1, 0, n_heads)) || overlap(out, span_of(a, 1, 0, 1, 0, n_heads)))
    return GDN_ERR_ALIAS;
  return GDN_OK;
}

int check_conv(const float *x, int64_t x_tok, int64_t x_seq, const float *w, const float *hist,
               int64_t h_seq, const float *out, int64_t o_tok, int64_t o_seq, const float *snap,
               int64_t sn_tok, int64_t sn_seq, int n_seq, int n_tok, int C, int D, int qk,
               int head_dim) {
  if (n_seq < 1 || n_tok < 1 || C < 1) return GDN_ERR_SHAPE;
  if (D < 2 || D > 8) return GDN_ERR_SHAPE;
  if (qk < 0 || qk > C) return GDN_ERR_SHAPE;
  if (qk > 0) {
    if (head_dim < 32 || head_dim % 32 != 0 || qk % head_dim != 0) return GDN_ERR_SHAPE;
    if (!supported_head_dim(head_dim)) return GDN_ERR_UNSUPPORTED;
  }
  if (x_tok < 0 || x_seq < 0 || h_seq < 0 || o_tok < 0 || o_seq < 0 || sn_tok < 0 || sn_seq < 0)
    return GDN_ERR_SHAPE;
  if (!x || !w || !hist || !out) return GDN_ERR_NULL;
  const int64_t hlen = (int64_t)C * (D - 1);
  if (!rows_disjoint(n_seq, o_seq, n_tok, o_tok, C)) return GDN_ERR_SHAPE;
  if (!rows_disjoint(n_seq, h_seq, 1, 0, hlen)) return GDN_ERR_SHAPE;
  const int n_snap = n_tok - 1;
  if (snap && n_snap > 0 && !rows_disjoint(n_seq, sn_seq, n_snap, sn_tok, hlen))
    return GDN_ERR_SHAPE;
  const Span sx = span_of(x, n_seq, x_seq, n_tok, x_tok, C);
  const Span sw = span_of(w, 1, 0, 1, 0, (int64_t)C * D);
  const Span sh = span_of(hist, n_seq, h_seq, 1, 0, hlen);
  const Span so = span_of(out, n_seq, o_seq, n_tok, o_tok, C);
  const Span ss = snap ? span_of(snap, n_seq, sn_seq, n_snap, sn_tok, hlen) : Span{};
  if (overlap(so, sx) || overlap(so, sw) || overlap(so, sh) || overlap(so, ss)) return GDN_ERR_ALIAS;
  if (overlap(sh, sx) || overlap(sh, sw) || overlap(ss, sh) || overlap(ss, sx) || overlap(ss, sw))
    return GDN_ERR_ALIAS;
  return GDN_OK;
}

int check_recur(const float *state, int64_t st_seq, const float *q, const float *k,
                int64_t qk_tok, int64_t qk_seq, const float *v, int64_t v_tok, int64_t v_seq,
                const float *g, const float *beta, const float *y, int64_t y_tok, int64_t y_seq,
                const float *snap, int64_t sn_seq, int n_seq, int n_tok, int H, int Hk, int S) {
  if (n_seq < 1 || n_tok < 1 || H < 1 || Hk < 1 || H % Hk != 0) return GDN_ERR_SHAPE;
  if (S < 32 || S % 32 != 0 || S > 256) return GDN_ERR_SHAPE;
  if (S != 32 && S != 64 && S != 128 && S != 256) return GDN_ERR_UNSUPPORTED;
  if (st_seq < 0 || qk_tok < 0 || qk_seq < 0 || v_tok < 0 || v_seq < 0 || y_tok < 0 ||
      y_seq < 0 || sn_seq < 0)
    return GDN_ERR_SHAPE;
  if (!state || !q || !k || !v || !g || !beta || !y) return GDN_ERR_NULL;
  const int64_t head = (int64_t)S * S, st_len = head * H;
  if (!rows_disjoint(n_seq, st_seq, 1, 0, st_len)) return GDN_ERR_SHAPE;
  if (!rows_disjoint(n_seq, y_seq, n_tok, y_tok, (int64_t)H * S)) return GDN_ERR_SHAPE;
  const int n_snap = n_tok - 1;
  if (snap && n_snap > 0 && !rows_disjoint(n_seq, sn_seq, n_snap, st_len, st_len))
    return GDN_ERR_SHAPE;
  // vector accesses: float4 rows (float2 at S = 32)
  const uintptr_t va = S >= 64 ? 16 : 8;
  const int64_t ve = S >= 64 ? 4 : 2;
  if (!aligned(state, va) || !aligned(q, va) || !aligned(k, va) || (snap && !aligned(snap, va)))
    return GDN_ERR_SHAPE;
  if (st_seq % ve || qk_tok % ve || qk_seq % ve || sn_seq % ve) return GDN_ERR_SHAPE;
  const Span sst = span_of(state, n_seq, st_seq, 1, 0, st_len);
  const Span sq = span_of(q, n_seq, qk_seq, n_tok, qk_tok, (int64_t)Hk * S);
  const Span sk = span_of(k, n_seq, qk_seq, n_tok, qk_tok, (int64_t)Hk * S);
  const Span sv = span_of(v, n_seq, v_seq, n_tok, v_tok, (int64_t)H * S);
  const Span sg = span_of(g, 1, 0, 1, 0, (int64_t)n_seq * n_tok * H);
  const Span sb = span_of(beta, 1, 0, 1, 0, (int64_t)n_seq * n_tok * H);
  const Span sy = span_of(y, n_seq, y_seq, n_tok, y_tok, (int64_t)H * S);
  const Span ssn = snap ? span_of(snap, n_seq, sn_seq, n_snap, st_len, st_len) : Span{};
  for (Span in : {sq, sk, sv, sg, sb})
    if (overlap(sst, in) || overlap(sy, in) || overlap(ssn, in)) return GDN_ERR_ALIAS;
  if (overlap(sy, sst) || overlap(ssn, sst) || overlap(ssn, sy)) return GDN_ERR_ALIAS;
  return GDN_OK;
}

int check_chunked(const float *state, int64_t st_seq, const float *q, const float *k,
                  int64_t qk_tok, int64_t qk_seq, const float *v, int64_t v_tok, int64_t v_seq,
                  const float *g, const float *beta, const float *y, int64_t y_tok,
                  int64_t y_seq, int n_seq, int n_tok, int H, int Hk, int S, int chunk,
                  const void *ws, size_t ws_bytes, size_t ws_needed) {
  const int rc = check_recur(state, st_seq, q, k, qk_tok, qk_seq, v, v_tok, v_seq, g, beta, y,
                             y_tok, y_seq, nullptr, 0, n_seq, n_tok, H, Hk, S);
  if (rc != GDN_OK) return rc;
  if (chunk != 64 || (S != 32 && S != 64 && S != 128)) return GDN_ERR_UNSUPPORTED;
  if (S != 128) return GDN_OK;   // the one-pass fp32 form: no workspace, no vector rows
  if (v_tok % 4 || v_seq % 4 || y_tok % 4 || y_seq % 4 || !aligned(v, 16) || !aligned(y, 16))
    return GDN_ERR_SHAPE;
  if (!ws || ws_bytes < ws_needed || !aligned(ws, 256)) return GDN_ERR_WORKSPACE;
  const Span sw{(uintptr_t)ws, (uintptr_t)ws + ws_bytes};
  const int64_t st_len = (int64_t)S * S * H;
  for (Span t : {span_of(state, n_seq, st_seq, 1, 0, st_len),
                 span_of(q, n_seq, qk_seq, n_tok, qk_tok, (int64_t)Hk * S),
                 span_of(k, n_seq, qk_seq, n_tok, qk_tok, (int64_t)Hk * S),
                 span_of(v, n_seq, v_seq, n_tok, v_tok, (int64_t)H * S),
                 span_of(y, n_seq, y_seq, n_tok, y_tok, (int64_t)H * S),
                 span_of(g, 1, 0, 1, 0, (int64_t)n_seq * n_tok * H),
                 span_of(beta, 1, 0, 1, 0, (int64_t)n_seq * n_tok * H)})
    if (overlap(sw, t)) return GDN_ERR_ALIAS;
  return GDN_OK;
}

int check_chunked_varlen(const float *state, int64_t st_seq, const void *q, const void *k,
                         int64_t qk_tok, const void *v, int64_t v_tok, int dtype, const float *g,
                         const float *beta, const float *y, int64_t y_tok, const int32_t *cu,
                         int n_seq, int total_tok, int H, int Hk, int S, int chunk,
                         const void *ws, size_t ws_bytes, size_t ws_needed) {
  if (n_seq < 1 || n_seq > GDN_VARLEN_MAX_SEQ || total_tok < 0) return GDN_ERR_SHAPE;
  if (H < 1 || Hk < 1 || H % Hk != 0) return GDN_ERR_SHAPE;
  if (S < 32 || S % 32 != 0 || S > 256) return GDN_ERR_SHAPE;
  if (chunk != 64 || (S != 32 && S != 64 && S != 128)) return GDN_ERR_UNSUPPORTED;
  if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;
  if (!cu) return GDN_ERR_NULL;
  if (cu[0] != 0 || cu[n_seq] != total_tok) return GDN_ERR_SHAPE;
  for (int s = 0; s < n_seq; ++s)
    if (cu[s + 1] < cu[s]) return GDN_ERR_SHAPE;
  if (!state) return GDN_ERR_NULL;
  if (total_tok == 0) return GDN_OK;   // nothing to compute
  if (!q || !k || !v || !g || !beta || !y) return GDN_ERR_NULL;
  if (st_seq < 0 || qk_tok < 0 || v_tok < 0 || y_tok < 0) return GDN_ERR_SHAPE;
  const int64_t esz = dtype == GDN_DTYPE_BF16 ? 2 : 4;
  const int64_t st_len = (int64_t)S * S * H;
  if (!rows_disjoint(n_seq, st_seq, 1, 0, st_len)) return GDN_ERR_SHAPE;
  if (!rows_disjoint(1, 0, total_tok, y_tok, (int64_t)H * S)) return GDN_ERR_SHAPE;
  // vector accesses: the state and y as float4 (float2 at S = 32); at S = 128
  // q, k, v rows are read 16 bytes at a time
  const uintptr_t va = S >= 64 ? 16 : 8;
  const int64_t ve = S >= 64 ? 4 : 2;
  if (!aligned(state, va) || st_seq % ve) return GDN_ERR_SHAPE;
  if (S == 128) {
    const int64_t in_vec = 16 / esz;   // elements per 16-byte load
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || qk_tok % in_vec ||
        v_tok % in_vec)
      return GDN_ERR_SHAPE;
    if (!aligned(y, 16) || y_tok % 4) return GDN_ERR_SHAPE;
    if (!ws || ws_bytes < ws_needed || !aligned(ws, 256)) return GDN_ERR_WORKSPACE;
  } else {
    if (!aligned(q, esz) || !aligned(k, esz) || !aligned(v, esz)) return GDN_ERR_SHAPE;
    if (dtype == GDN_DTYPE_F32 && (!aligned(q, va) || !aligned(k, va) || qk_tok % ve))
      return GDN_ERR_SHAPE;   // the fp32 rules of the fixed-length entry point
  }
  const Span sst = span_of(state, n_seq, st_seq, 1, 0, st_len);
  const Span sy = span_of(y, 1, 0, total_tok, y_tok, (int64_t)H * S);
  const Span sw = S == 128 ? Span{(uintptr_t)ws, (uintptr_t)ws + ws_bytes} : Span{};
  for (Span in : {span_of(q, 1, 0, total_tok, qk_tok, (int64_t)Hk * S, esz),
                  span_of(k, 1, 0, total_tok, qk_tok, (int64_t)Hk * S, esz),
                  span_of(v, 1, 0, total_tok, v_tok, (int64_t)H * S, esz),
                  span_of(g, 1, 0, 1, 0, (int64_t)total_tok * H),
                  span_of(beta, 1, 0, 1, 0, (int64_t)total_tok * H)})
    if (overlap(sst, in) || overlap(sy, in) || overlap(sw, in)) return GDN_ERR_ALIAS;
  if (overlap(sy, sst) || overlap(sw, sst) || overlap(sw, sy)) return GDN_ERR_ALIAS;
  return GDN_OK;
}

int check_ssd(const float *state, int64_t st_seq, const float *x, int64_t x_tok, int64_t x_seq,
              const float *B, const float *C, int64_t bc_tok, int64_t bc_seq,
              const float *dt_raw, int64_t dt_tok, int64_t dt_seq, const float *A_log,
              const float *D, const float *dt_bias, const float *y, int64_t y_tok,
              int64_t y_seq, int n_seq, int n_tok, int H, int G, int P, int N, int chunk,
              const void *ws, size_t ws_bytes, size_t ws_needed) {
  if (n_seq < 1 || n_tok < 1 || H < 1 || G < 1 || H % G != 0) return GDN_ERR_SHAPE;
  if (P < 32 || P % 32 != 0 || N < 32 || N % 32 != 0) return GDN_ERR_SHAPE;
  if ((P != 32 && P != 64) || (N != 64 && N != 128) || chunk != 64) return GDN_ERR_UNSUPPORTED;
  if (st_seq < 0 || x_tok < 0 || x_seq < 0 || bc_tok < 0 || bc_seq < 0 || dt_tok < 0 ||
      dt_seq < 0 || y_tok < 0 || y_seq < 0)
    return GDN_ERR_SHAPE;
  if (!state || !x || !B || !C || !dt_raw || !A_log || !D || !dt_bias || !y) return GDN_ERR_NULL;
  const int64_t st_len = (int64_t)H * P * N;
  if (!rows_disjoint(n_seq, st_seq, 1, 0, st_len)) return GDN_ERR_SHAPE;
  if (!rows_disjoint(n_seq, y_seq, n_tok, y_tok, (int64_t)H * P)) return GDN_ERR_SHAPE;
  for (const void *p : {(const void *)state, (const void *)x, (const void *)B, (const void *)C,
                        (const void *)y})
    if (!aligned(p, 16)) return GDN_ERR_SHAPE;
  if (st_seq % 4 || x_tok % 4 || x_seq % 4 || bc_tok % 4 || bc_seq % 4 || y_tok % 4 || y_seq % 4)
    return GDN_ERR_SHAPE;
  if (!ws || ws_bytes < ws_needed || !aligned(ws, 256)) return GDN_ERR_WORKSPACE;
  const Span sst = span_of(state, n_seq, st_seq, 1, 0, st_len);
  const Span sy = span_of(y, n_seq, y_seq, n_tok, y_tok, (int64_t)H * P);
  const Span sw{(uintptr_t)ws, (uintptr_t)ws + ws_bytes};
  for (Span in : {span_of(x, n_seq, x_seq, n_tok, x_tok, (int64_t)H * P),
                  span_of(B, n_seq, bc_seq, n_tok, bc_tok, (int64_t)G * N),
                  span_of(C, n_seq, bc_seq, n_tok, bc_tok, (int64_t)G * N),
                  span_of(dt_raw, n_seq, dt_seq, n_tok, dt_tok, H),
                  span_of(A_log, 1, 0, 1, 0, H), span_of(D, 1, 0, 1, 0, H),
                  span_of(dt_bias, 1, 0, 1, 0, H)})
    if (overlap(sst, in) || overlap(sy, in) || overlap(sw, in)) return GDN_ERR_ALIAS;
  if (overlap(sy, sst) || overlap(sw, sst) || overlap(sw, sy)) return GDN_ERR_ALIAS;
  return GDN_OK;
}

int check_norm(const float *y, int64_t y_row, const float *w, const float *z, int64_t z_row,
               const float *out, int64_t o_row, int rows, int H, int hd) {
  if (rows < 0 || H < 1) return GDN_ERR_SHAPE;
  if (hd < 32 || hd % 32 != 0) return GDN_ERR_SHAPE;
  if (!supported_head_dim(hd)) return GDN_ERR_UNSUPPORTED;
  if (y_row < 0 || z_row < 0 || o_row < 0) return GDN_ERR_SHAPE;
  if (rows == 0) return GDN_OK;
  if (!y || !w || !z || !out) return GDN_ERR_NULL;
  const int64_t len = (int64_t)H * hd;
  if (!rows_disjoint(1, 0, rows, o_row, len)) return GDN_ERR_SHAPE;
  const Span sy = span_of(y, 1, 0, rows, y_row, len);
  const Span sz = span_of(z, 1, 0, rows, z_row, len);
  const Span sw = span_of(w, 1, 0, 1, 0, hd);
  const Span so = span_of(out, 1, 0, rows, o_row, len);
  if (overlap(so, sz) || overlap(so, sw)) return GDN_ERR_ALIAS;
  if (overlap(so, sy) && !(out == y && o_row == y_row)) return GDN_ERR_ALIAS;
  return GDN_OK;
}

int check_fused(const float *state, int64_t st_seq, const float *q, const float *k,
                int64_t qk_tok, int64_t qk_seq, const float *v, int64_t v_tok, int64_t v_seq,
                const float *alpha, const float *dt, const float *a, const float *beta,
                const float *w, const float *z, int64_t z_tok, int64_t z_seq, const float *out,
                int64_t o_tok, int64_t o_seq, const float *g, const float *y, int64_t y_tok,
                int64_t y_seq, const float *snap, int64_t sn_seq, int n_seq, int n_tok, int H,
                int Hk, int S) {
  // the recurrence's own rules, with alpha in the place of g and out in the
  // place of y (same shapes)
  const int rc = check_recur(state, st_seq, q, k, qk_tok, qk_seq, v, v_tok, v_seq, alpha, beta,
                             out, o_tok, o_seq, snap, sn_seq, n_seq, n_tok, H, Hk, S);
  if (rc != GDN_OK) return rc;
  if (!dt || !a || !w || !z) return GDN_ERR_NULL;
  if (z_tok < 0 || z_seq < 0 || (y && (y_tok < 0 || y_seq < 0))) return GDN_ERR_SHAPE;
  // the norm reads z and w and writes out as float4
  if (!aligned(out, 16) || !aligned(z, 16) || !aligned(w, 16) || o_tok % 4 || o_seq % 4 ||
      z_tok % 4 || z_seq % 4)
    return GDN_ERR_SHAPE;
  const int64_t row = (int64_t)H * S, st_len = (int64_t)S * S * H;
  if (y && !rows_disjoint(n_seq, y_seq, n_tok, y_tok, row)) return GDN_ERR_SHAPE;
  const int n_snap = n_tok - 1;
  const Span in[] = {span_of(q, n_seq, qk_seq, n_tok, qk_tok, (int64_t)Hk * S),
                     span_of(k, n_seq, qk_seq, n_tok, qk_tok, (int64_t)Hk * S),
                     span_of(v, n_seq, v_seq, n_tok, v_tok, row),
                     span_of(alpha, 1, 0, 1, 0, (int64_t)n_seq * n_tok * H),
                     span_of(beta, 1, 0, 1, 0, (int64_t)n_seq * n_tok * H),
                     span_of(dt, 1, 0, 1, 0, H),
                     span_of(a, 1, 0, 1, 0, H),
                     span_of(w, 1, 0, 1, 0, S),
                     span_of(z, n_seq, z_seq, n_tok, z_tok, row)};
  const Span outs[] = {span_of(state, n_seq, st_seq, 1, 0, st_len),
                       span_of(out, n_seq, o_seq, n_tok, o_tok, row),
                       g ? span_of(g, 1, 0, 1, 0, (int64_t)n_seq * n_tok * H) : Span{},
                       y ? span_of(y, n_seq, y_seq, n_tok, y_tok, row) : Span{},
                       snap && n_snap > 0 ? span_of(snap, n_seq, sn_seq, n_snap, st_len, st_len)
                                          : Span{}};
  for (const Span &o : outs) {
    for (const Span &i : in)
      if (overlap(o, i)) return GDN_ERR_ALIAS;
  }
  for (int i = 0; i < 5; ++i)
    for (int j = i + 1; j < 5; ++j)
      if (overlap(outs[i], outs[j])) return GDN_ERR_ALIAS;
  return GDN_OK;
}

size_t step_workspace_bytes(int n_seq, int Hk) {
  if (n_seq < 1 || Hk < 1) return 0;
  return (size_t)n_seq * (size_t)Hk * 2 * sizeof(int32_t);
}

int check_prefill(const float *state, int64_t st_seq, const float *x, int64_t x_tok,
                  int64_t x_seq, const float *cw, const float *hist, int64_t h_seq,
                  const float *alpha, const float *dt, const float *a, const float *beta,
                  const float *y, int64_t y_tok, int64_t y_seq, int n_seq, int n_tok, int H,
                  int Hk, int S, int D, int chunk, const void *ws, size_t ws_bytes,
                  size_t ws_needed) {
  if (n_seq < 1 || n_tok < 1 || H < 1 || Hk < 1 || H % Hk != 0) return GDN_ERR_SHAPE;
  if (S < 32 || S % 32 != 0 || S > 256) return GDN_ERR_SHAPE;
  if (D < 2 || D > 8) return GDN_ERR_SHAPE;
  if (S != 128 || D != 4 || chunk != 64) return GDN_ERR_UNSUPPORTED;
  if (st_seq < 0 || x_tok < 0 || x_seq < 0 || h_seq < 0 || y_tok < 0 || y_seq < 0)
    return GDN_ERR_SHAPE;
  if (!state || !x || !cw || !hist || !alpha || !dt || !a || !beta || !y) return GDN_ERR_NULL;
  const int64_t C = (2 * (int64_t)Hk + H) * S;
  if (C > INT32_MAX / 8) return GDN_ERR_SHAPE;
  if (n_tok > 1 && x_tok < C) return GDN_ERR_SHAPE;
  const int64_t hlen = C * (D - 1), row = (int64_t)H * S, st_len = (int64_t)S * S * H;
  if (!rows_disjoint(n_seq, st_seq, 1, 0, st_len)) return GDN_ERR_SHAPE;
  if (!rows_disjoint(n_seq, h_seq, 1, 0, hlen)) return GDN_ERR_SHAPE;
  if (!rows_disjoint(n_seq, y_seq, n_tok, y_tok, row)) return GDN_ERR_SHAPE;
  // 16-byte accesses of the state, x, the taps, the history and y
  if (!aligned(state, 16) || !aligned(x, 16) || !aligned(cw, 16) || !aligned(hist, 16) ||
      !aligned(y, 16) || st_seq % 4 || x_tok % 4 || x_seq % 4 || h_seq % 4 || y_tok % 4 ||
      y_seq % 4)
    return GDN_ERR_SHAPE;
  if (!ws || ws_bytes < ws_needed || !aligned(ws, 256)) return GDN_ERR_WORKSPACE;
  const int64_t rows = (int64_t)n_seq * n_tok * H;
  const Span in[] = {span_of(x, n_seq, x_seq, n_tok, x_tok, C),
                     span_of(cw, 1, 0, 1, 0, C * D),
                     span_of(alpha, 1, 0, 1, 0, rows),
                     span_of(beta, 1, 0, 1, 0, rows),
                     span_of(dt, 1, 0, 1, 0, H),
                     span_of(a, 1, 0, 1, 0, H)};
  const Span outs[] = {span_of(state, n_seq, st_seq, 1, 0, st_len),
                       span_of(hist, n_seq, h_seq, 1, 0, hlen),
                       span_of(y, n_seq, y_seq, n_tok, y_tok, row),
                       Span{(uintptr_t)ws, (uintptr_t)ws + ws_bytes}};
  for (const Span &o : outs) {
    for (const Span &i : in)
      if (overlap(o, i)) return GDN_ERR_ALIAS;
    for (const Span &o2 : outs)
      if (&o2 != &o && overlap(o, o2)) return GDN_ERR_ALIAS;
  }
  return GDN_OK;
}

int check_step(const float *state, int64_t st_seq, const float *x, int64_t x_tok, int64_t x_seq,
               const float *cw, const float *hist, int64_t h_seq, const float *csnap,
               int64_t cs_tok, int64_t cs_seq, const float *alpha, const float *dt,
               const float *a, const float *beta, const float *w, const float *z, int64_t z_tok,
               int64_t z_seq, const float *out, int64_t o_tok, int64_t o_seq, const float *g,
               const float *y, int64_t y_tok, int64_t y_seq, const float *snap, int64_t sn_seq,
               int n_seq, int n_tok, int H, int Hk, int S, int D, const void *ws,
               size_t ws_bytes, bool lib_scratch) {
  if (n_seq < 1 || n_tok < 1 || H < 1 || Hk < 1 || H % Hk != 0) return GDN_ERR_SHAPE;
  if (n_tok > (S <= 128 ? 32 : 16)) return GDN_ERR_SHAPE;   // positions staged in LDS
  if (D < 2 || D > 8) return GDN_ERR_SHAPE;
  if (x_tok < 0 || x_seq < 0 || h_seq < 0 || cs_tok < 0 || cs_seq < 0) return GDN_ERR_SHAPE;
  if (!x || !cw || !hist) return GDN_ERR_NULL;
  // the recurrence, gate and norm rules, with q, k, v the channel ranges of x
  const int64_t qk = (int64_t)Hk * S;
  const int rc = check_fused(state, st_seq, x, x + qk, x_tok, x_seq, x + 2 * qk, x_tok, x_seq,
                             alpha, dt, a, beta, w, z, z_tok, z_seq, out, o_tok, o_seq, g, y,
                             y_tok, y_seq, snap, sn_seq, n_seq, n_tok, H, Hk, S);
  if (rc != GDN_OK) return rc;
  // the conv rules for this channel layout (q and k L2-normalised per S-wide
  // head, which check_fused has already limited to the supported widths)
  const int64_t C = (2 * (int64_t)Hk + H) * S;
  if (C > INT32_MAX / 8) return GDN_ERR_SHAPE;
  if (n_tok > 1 && x_tok < C) return GDN_ERR_SHAPE;
  const int64_t hlen = C * (D - 1);
  if (!rows_disjoint(n_seq, h_seq, 1, 0, hlen)) return GDN_ERR_SHAPE;
  const int n_snap = n_tok - 1;
  if (csnap && n_snap > 0 && !rows_disjoint(n_seq, cs_seq, n_snap, cs_tok, hlen))
    return GDN_ERR_SHAPE;
  // 16-byte conv accesses
  if (!aligned(x, 16) || !aligned(cw, 16) || !aligned(hist, 16) || (csnap && !aligned(csnap, 16)) ||
      x_tok % 4 || x_seq % 4 || h_seq % 4 || cs_tok % 4 || cs_seq % 4)
    return GDN_ERR_SHAPE;
  // the library's own scratch array is checked by its caller and cannot
  // overlap caller memory
  if (!lib_scratch && (!ws || ws_bytes < step_workspace_bytes(n_seq, Hk) || !aligned(ws, 4)))
    return GDN_ERR_WORKSPACE;
  const int64_t row = (int64_t)H * S, st_len = (int64_t)S * S * H;
  const Span in[] = {span_of(x, n_seq, x_seq, n_tok, x_tok, C),
                     span_of(cw, 1, 0, 1, 0, (int64_t)C * D),
                     span_of(alpha, 1, 0, 1, 0, (int64_t)n_seq * n_tok * H),
                     span_of(beta, 1, 0, 1, 0, (int64_t)n_seq * n_tok * H),
                     span_of(dt, 1, 0, 1, 0, H),
                     span_of(a, 1, 0, 1, 0, H),
                     span_of(w, 1, 0, 1, 0, S),
                     span_of(z, n_seq, z_seq, n_tok, z_tok, row)};
  const Span outs[] = {span_of(state, n_seq, st_seq, 1, 0, st_len),
                       span_of(out, n_seq, o_seq, n_tok, o_tok, row),
                       g ? span_of(g, 1, 0, 1, 0, (int64_t)n_seq * n_tok * H) : Span{},
                       y ? span_of(y, n_seq, y_seq, n_tok, y_tok, row) : Span{},
                       snap && n_snap > 0 ? span_of(snap, n_seq, sn_seq, n_snap, st_len, st_len)
                                          : Span{},
                       span_of(hist, n_seq, h_seq, 1, 0, hlen),
                       csnap && n_snap > 0 ? span_of(csnap, n_seq, cs_seq, n_snap, cs_tok, hlen)
                                           : Span{},
                       lib_scratch ? Span{} : Span{(uintptr_t)ws, (uintptr_t)ws + ws_bytes}};
  constexpr int NO = sizeof(outs) / sizeof(outs[0]);
  for (const Span &o : outs)
    for (const Span &i : in)
      if (overlap(o, i)) return GDN_ERR_ALIAS;
  for (int i = 0; i < NO; ++i)
    for (int j = i + 1; j < NO; ++j)
      if (overlap(outs[i], outs[j])) return GDN_ERR_ALIAS;
  if (D > 4) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

}  // namespace gdn
