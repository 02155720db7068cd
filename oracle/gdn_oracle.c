/*
 * gdn_oracle.c -- plain, slow, obviously-correct CPU oracle for the gated-delta
 * SSM layer core, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  The parity tests, the smoke check and the CPU
 * baseline leg of the benchmark call this file; the HIP library never does, and
 * this file includes no header of it and shares no code with it.
 *
 * Every input arrives as fp64 (the callers widen fp32 arrays exactly), every
 * output is fp64.  Loops are written in the order the pages state the method;
 * OpenMP only splits independent units (rows, sequences x heads, channels).
 *
 * Sources (page title, then the part of the page):
 *   [FM]  fm_kernel_ssm.h, Foundry Metal kernels (git.teamide.dev)
 *   [AT]  ssm_mamba.rs, spark_model layers/ops (atlas-docs)
 *   [SCR] scr_state.hpp, regolith Metal engine scripts (tangled.org)
 *
 * Parity status of each function (what pins it is in tests/test_oracle_pins.py):
 *   oracle_decay_gate          pinned (closed forms, library softplus, identities)
 *   oracle_conv1d_silu_l2norm  pinned (brute-force correlation, tap special cases)
 *   oracle_recurrence_seq      pinned (closed forms, P3 matrix closed form, recall,
 *                              staleness bound)
 *   oracle_recurrence_chunked  pinned against oracle_recurrence_seq (fp64, 1e-12)
 *   oracle_gated_rmsnorm       pinned (constant-input closed form, library rms_norm)
 *   oracle_mamba2_dt           pinned (library softplus, clamp limits)
 *   oracle_mamba2_ssd_seq      pinned (one-token closed form, pure decay, D skip,
 *                              brute-force quadratic form on tiny inputs)
 *   oracle_mamba2_ssd_chunked  pinned against oracle_mamba2_ssd_seq (fp64, 1e-12)
 *
 * The Mamba-2 functions follow [AT]'s mamba2_ssm_prefill wrapper (its
 * arguments: state h, x, B and C projections, raw dt with a per-head bias and
 * dt_min / dt_max limits, A_log, the D skip, n_groups; "same algorithm as
 * decode", one thread per state index) and its "Mamba-2 SSD chunked prefill
 * scan" comment (the chunked state-space-duality form of the same scan).  The
 * page prints no formula; the recurrence written here is the published
 * Mamba-2 selective scan those arguments name:
 *   dt = clamp(softplus(dt_raw + dt_bias), dt_min, dt_max),  A = -exp(A_log)
 *   h  <- exp(dt A) h + dt x B^T          (h [head_dim][state], per head)
 *   y  =  h C + D x
 * with value head h reading B, C of group h / (H / n_groups).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus with the guard at 20: [FM] "Decay gate" section (fm_ssm_decay_gate_at
 * doc: above the guard softplus(v) is v, below it log1p(exp(v))); the same
 * strict comparison in double is [SCR] "GDN staleness", log_gate. */
static double softplus_guarded(double v) { return v > 20.0 ? v : log1p(exp(v)); }

/* g[r][h] = a[h] * softplus(alpha[r][h] + dt[h]); a = -exp(A_log) pre-baked,
 * g is returned pre-exp.  [FM] "Decay gate" section, fm_ssm_decay_gate_at. */
void oracle_decay_gate(const double *alpha, const double *dt, const double *a, double *g,
                       long rows, int n_heads) {
  long r;
#pragma omp parallel for schedule(static)
  for (r = 0; r < rows; ++r)
    for (int h = 0; h < n_heads; ++h) {
      const double v = alpha[r * n_heads + h] + dt[h];
      g[r * n_heads + h] = a[h] * softplus_guarded(v);
    }
}

static double silu(double x) { return x / (1.0 + exp(-x)); }

/*
 * Depthwise causal conv1d + SiLU with per-head L2 norm on the Q/K channels.
 *   [FM] "Causal depthwise conv1d + SiLU" section, fm_ssm_conv1d_silu_at and
 *        fm_ssm_conv1d_silu_seq_at: window = [history oldest..newest, x];
 *        out = silu(sum_t w[c][t] * window[t]); then the history shifts by one
 *        place: its oldest value leaves and the input x itself (not the
 *        activated output) becomes its newest value.
 *   [AT] conv1d_update_l2norm: channels [0, qk_channels) are L2-normalised per
 *        head_dim block after SiLU, the rest get SiLU only;
 *        gdn_verify_fused_conv_k2: the window after position 0 is the rollback
 *        snapshot, the committed window stays in place.
 *   [SCR] "GDN staleness": the L2 form is x / sqrt(sum x^2 + eps).
 *
 * Layouts (dense, fp64):
 *   x    [n_seq][n_tok][C]         out  [n_seq][n_tok][C]
 *   w    [C][d]                    hist [n_seq][C][d-1], oldest first, in/out
 *   snap [n_seq][n_tok-1][C][d-1]  or NULL: the history after token t < n_tok-1
 */
void oracle_conv1d_silu_l2norm(const double *x, const double *w, double *hist, double *out,
                               double *snap, int n_seq, int n_tok, int C, int d,
                               int qk_channels, int head_dim, double eps) {
  const int dh = d - 1;
  int s;
#pragma omp parallel for schedule(static)
  for (s = 0; s < n_seq; ++s) {
    double *win = (double *)malloc(sizeof(double) * (size_t)d);
    for (int t = 0; t < n_tok; ++t) {
      const double *xt = x + ((size_t)s * n_tok + t) * C;
      double *ot = out + ((size_t)s * n_tok + t) * C;
      for (int c = 0; c < C; ++c) {
        double *hc = hist + ((size_t)s * C + c) * dh;
        for (int j = 0; j < dh; ++j) win[j] = hc[j];
        win[dh] = xt[c];
        double acc = 0.0;
        for (int j = 0; j < d; ++j) acc += w[(size_t)c * d + j] * win[j];
        ot[c] = silu(acc);
        for (int j = 0; j < dh; ++j) hc[j] = win[j + 1]; /* roll with the raw input */
      }
      if (snap && t < n_tok - 1)
        memcpy(snap + (((size_t)s * (n_tok - 1) + t) * C) * dh, hist + (size_t)s * C * dh,
               sizeof(double) * (size_t)C * dh);
      for (int c0 = 0; c0 + head_dim <= qk_channels; c0 += head_dim) {
        double ss = 0.0;
        for (int c = c0; c < c0 + head_dim; ++c) ss += ot[c] * ot[c];
        const double inv = 1.0 / sqrt(ss + eps);
        for (int c = c0; c < c0 + head_dim; ++c) ot[c] *= inv;
      }
    }
    free(win);
  }
}

/*
 * Sequential gated delta-rule scan, the plain definition.
 *   [FM] "Delta-rule recurrence" section, fm_ssm_recurrence_at and
 *        fm_ssm_recurrence_seq_at.  Per head and token, in this order:
 *        S <- exp(g) S;  p = S^T k;  delta = beta (v - p);  S <- S + k delta^T;
 *        y = scale * S^T q   (the readout uses the updated state).
 *   [SCR] "GDN staleness" restates it as S' = g (I - b k k^T) S + b k v^T.
 *
 * The state is held here as S[i][j], i over the key dimension, j over the value
 * dimension (the GPU stores its transpose; the Python wrapper converts).
 * Grouped heads: value head h reads q/k head h / (H / Hk).
 *
 * Layouts (dense, fp64):
 *   S    [n_seq][H][dk][dv] in/out
 *   q, k [n_seq][n_tok][Hk][dk]    v, y [n_seq][n_tok][H][dv]
 *   g, beta [n_seq][n_tok][H]      (g pre-exp, beta already sigmoid'd)
 *   snap [n_seq][n_tok-1][H][dk][dv] or NULL: the state after token t < n_tok-1
 */
void oracle_recurrence_seq(double *S, const double *q, const double *k, const double *v,
                           const double *g, const double *beta, double *y, double *snap,
                           int n_seq, int n_tok, int H, int Hk, int dk, int dv, double scale) {
  const int group = H / Hk;
  long u;
#pragma omp parallel for schedule(dynamic)
  for (u = 0; u < (long)n_seq * H; ++u) {
    const int s = (int)(u / H), h = (int)(u % H), hk = h / group;
    double *St = S + (size_t)u * dk * dv;
    double *p = (double *)malloc(sizeof(double) * (size_t)dv);
    for (int t = 0; t < n_tok; ++t) {
      const size_t row = (size_t)s * n_tok + t;
      const double *kt = k + (row * Hk + hk) * dk;
      const double *qt = q + (row * Hk + hk) * dk;
      const double *vt = v + (row * H + h) * dv;
      double *yt = y + (row * H + h) * dv;
      const double gamma = exp(g[row * H + h]);
      const double b = beta[row * H + h];
      for (int i = 0; i < dk * dv; ++i) St[i] *= gamma; /* decay */
      for (int j = 0; j < dv; ++j) {                    /* p = S^T k */
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += St[(size_t)i * dv + j] * kt[i];
        p[j] = acc;
      }
      for (int j = 0; j < dv; ++j) p[j] = b * (vt[j] - p[j]); /* delta */
      for (int i = 0; i < dk; ++i)                            /* S += k delta^T */
        for (int j = 0; j < dv; ++j) St[(size_t)i * dv + j] += kt[i] * p[j];
      for (int j = 0; j < dv; ++j) { /* y = scale S^T q */
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += St[(size_t)i * dv + j] * qt[i];
        yt[j] = scale * acc;
      }
      if (snap && t < n_tok - 1)
        memcpy(snap + ((((size_t)s * (n_tok - 1) + t) * H + h) * dk) * dv, St,
               sizeof(double) * (size_t)dk * dv);
    }
    free(p);
  }
}

/*
 * Chunked (WY / UT-transform) form of the same scan.
 *
 * The pages only state that a chunked path needs one dependent step per
 * 64-position chunk instead of one per position ([AT] "Mamba-2 SSD chunked
 * prefill scan" comment) and that the
 * sequential scan is its permanent correctness reference ([FM]
 * fm_ssm_recurrence_seq_at doc).  The algebra below is derived from the
 * sequential definition by unrolling it over a chunk of n tokens that starts
 * from state S0, with G_t = sum_{s<=t} g_s (inclusive, within the chunk):
 *
 *   S_t = e^{G_t} S0 + sum_{s<=t} e^{G_t-G_s} k_s u_s^T,   u_t = delta_t
 *   u_t = beta_t (v_t - e^{G_t} S0^T k_t - sum_{s<t} e^{G_t-G_s} (k_t.k_s) u_s)
 *   => (I + A) U = diag(beta) V - diag(beta e^G) K S0,
 *      A[t][s] = beta_t e^{G_t-G_s} (k_t.k_s) for s < t, else 0
 *   T  = (I + A)^{-1}            (unit lower triangular; forward substitution)
 *   W  = T diag(beta e^G) K,     Ut = T diag(beta) V,     U = Ut - W S0
 *   O  = scale [diag(e^G) Q S0 + (L o Q K^T) U],  L[t][s] = e^{G_t-G_s}, s <= t
 *   S_n = e^{G_n} S0 + (diag(e^{G_n - G}) K)^T U
 *
 * Every exponential is of a non-positive argument (G is non-increasing since
 * g < 0), taken only where the mask keeps it.  Same layouts as
 * oracle_recurrence_seq; the last chunk may be partial.
 */
void oracle_recurrence_chunked(double *S, const double *q, const double *k, const double *v,
                               const double *g, const double *beta, double *y, int n_seq,
                               int n_tok, int H, int Hk, int dk, int dv, int chunk,
                               double scale) {
  const int group = H / Hk;
  const int C = chunk;
  long u;
#pragma omp parallel for schedule(dynamic)
  for (u = 0; u < (long)n_seq * H; ++u) {
    const int s = (int)(u / H), h = (int)(u % H), hk = h / group;
    double *S0 = S + (size_t)u * dk * dv;
    double *G = malloc(sizeof(double) * C);
    double *Ti = malloc(sizeof(double) * C * C); /* (I + A)^{-1} */
    double *A = malloc(sizeof(double) * C * C);
    double *Wm = malloc(sizeof(double) * C * dk);
    double *Um = malloc(sizeof(double) * C * dv);
    double *Ut = malloc(sizeof(double) * C * dv);
    double *QK = malloc(sizeof(double) * C * C);
    double *Sn = malloc(sizeof(double) * dk * dv);
    for (int c0 = 0; c0 < n_tok; c0 += C) {
      const int n = (n_tok - c0 < C) ? (n_tok - c0) : C;
#define ROW(t) ((size_t)s * n_tok + (size_t)(c0 + (t)))
#define KV(t) (k + (ROW(t) * Hk + hk) * dk)
#define QV(t) (q + (ROW(t) * Hk + hk) * dk)
#define VV(t) (v + (ROW(t) * H + h) * dv)
#define YV(t) (y + (ROW(t) * H + h) * dv)
#define GB(arr, t) (arr[ROW(t) * H + h])
      double acc = 0.0;
      for (int t = 0; t < n; ++t) { acc += GB(g, t); G[t] = acc; }
      /* A = strictly-lower(beta_t e^{G_t - G_s} k_t . k_s) */
      for (int t = 0; t < n; ++t)
        for (int j = 0; j < n; ++j) {
          double a = 0.0;
          if (j < t) {
            double kk = 0.0;
            for (int i = 0; i < dk; ++i) kk += KV(t)[i] * KV(j)[i];
            a = GB(beta, t) * exp(G[t] - G[j]) * kk;
          }
          A[t * C + j] = a;
        }
      /* Ti = (I + A)^{-1} by forward substitution, column by column */
      for (int col = 0; col < n; ++col)
        for (int t = 0; t < n; ++t) {
          double x = (t == col) ? 1.0 : 0.0;
          for (int j = col; j < t; ++j) x -= A[t * C + j] * Ti[j * C + col];
          Ti[t * C + col] = (t < col) ? 0.0 : x;
        }
      /* W = Ti diag(beta e^G) K ;  Ut = Ti diag(beta) V */
      for (int t = 0; t < n; ++t) {
        for (int i = 0; i < dk; ++i) {
          double a = 0.0;
          for (int j = 0; j <= t; ++j) a += Ti[t * C + j] * GB(beta, j) * exp(G[j]) * KV(j)[i];
          Wm[t * dk + i] = a;
        }
        for (int jv = 0; jv < dv; ++jv) {
          double a = 0.0;
          for (int j = 0; j <= t; ++j) a += Ti[t * C + j] * GB(beta, j) * VV(j)[jv];
          Ut[t * dv + jv] = a;
        }
      }
      /* U = Ut - W S0 */
      for (int t = 0; t < n; ++t)
        for (int jv = 0; jv < dv; ++jv) {
          double a = 0.0;
          for (int i = 0; i < dk; ++i) a += Wm[t * dk + i] * S0[(size_t)i * dv + jv];
          Um[t * dv + jv] = Ut[t * dv + jv] - a;
        }
      /* (L o Q K^T), L including the diagonal */
      for (int t = 0; t < n; ++t)
        for (int j = 0; j < n; ++j) {
          double a = 0.0;
          if (j <= t) {
            double qk = 0.0;
            for (int i = 0; i < dk; ++i) qk += QV(t)[i] * KV(j)[i];
            a = exp(G[t] - G[j]) * qk;
          }
          QK[t * C + j] = a;
        }
      /* O = scale [diag(e^G) Q S0 + (L o QK^T) U] */
      for (int t = 0; t < n; ++t)
        for (int jv = 0; jv < dv; ++jv) {
          double inter = 0.0, intra = 0.0;
          for (int i = 0; i < dk; ++i) inter += QV(t)[i] * S0[(size_t)i * dv + jv];
          for (int j = 0; j <= t; ++j) intra += QK[t * C + j] * Um[j * dv + jv];
          YV(t)[jv] = scale * (exp(G[t]) * inter + intra);
        }
      /* S_n = e^{G_n} S0 + (diag(e^{G_n - G}) K)^T U */
      const double Gn = G[n - 1];
      for (int i = 0; i < dk; ++i)
        for (int jv = 0; jv < dv; ++jv) {
          double a = 0.0;
          for (int t = 0; t < n; ++t) a += exp(Gn - G[t]) * KV(t)[i] * Um[t * dv + jv];
          Sn[(size_t)i * dv + jv] = exp(Gn) * S0[(size_t)i * dv + jv] + a;
        }
      memcpy(S0, Sn, sizeof(double) * (size_t)dk * dv);
#undef ROW
#undef KV
#undef QV
#undef VV
#undef YV
#undef GB
    }
    free(G); free(Ti); free(A); free(Wm); free(Um); free(Ut); free(QK); free(Sn);
  }
}

/*
 * Gated RMSNorm, per (row, head):
 *   out = ((y * (1 / sqrt(mean(y^2) + eps))) * w) * silu(z)
 * with w[head_dim] shared by every head.  [FM] "Gated RMSNorm" section,
 * fm_ssm_gated_norm_at (multiply order and shared weight); [AT]
 * gdn_verify_fused_norm_k2 reads z from a wider row at an offset, which the
 * caller resolves before this dense form.
 *
 * Layouts (dense, fp64): y, z, out [rows][H][head_dim]; w [head_dim].
 */
void oracle_gated_rmsnorm(const double *y, const double *w, const double *z, double *out,
                          long rows, int H, int head_dim, double eps) {
  long u;
#pragma omp parallel for schedule(static)
  for (u = 0; u < rows * H; ++u) {
    const double *yu = y + (size_t)u * head_dim;
    const double *zu = z + (size_t)u * head_dim;
    double *ou = out + (size_t)u * head_dim;
    double ss = 0.0;
    for (int e = 0; e < head_dim; ++e) ss += yu[e] * yu[e];
    const double inv = 1.0 / sqrt(ss / head_dim + eps);
    for (int e = 0; e < head_dim; ++e) ou[e] = ((yu[e] * inv) * w[e]) * silu(zu[e]);
  }
}

/*
 * Mamba-2 step size per (row, head): dt = softplus(dt_raw + dt_bias) with the
 * guard at 20 (as the decay gate's), then clamped to [dt_min, dt_max]: [AT]
 * mamba2_ssm_prefill passes the raw projection, a per-head bias and the two
 * limits.  Layouts: dt_raw, dt [rows][H]; dt_bias [H].
 */
void oracle_mamba2_dt(const double *dt_raw, const double *dt_bias, double *dt, long rows, int H,
                      double dt_min, double dt_max) {
  long r;
#pragma omp parallel for schedule(static)
  for (r = 0; r < rows; ++r)
    for (int h = 0; h < H; ++h) {
      double d = softplus_guarded(dt_raw[r * H + h] + dt_bias[h]);
      if (d < dt_min) d = dt_min;
      if (d > dt_max) d = dt_max;
      dt[r * H + h] = d;
    }
}

/*
 * Mamba-2 selective scan, token by token (the definition; [AT]
 * mamba2_ssm_prefill: "same algorithm as decode", looped over the tokens).
 * Per sequence b, head h (group gi = h / (H / G)), token t:
 *   a = exp(dt[t][h] * A[h])
 *   h[p][n] = a * h[p][n] + dt[t][h] * x[t][h][p] * B[t][gi][n]
 *   y[t][h][p] = sum_n h[p][n] * C[t][gi][n] + D[h] * x[t][h][p]
 * Layouts (dense, fp64): state [B][H][P][N] in/out; x, y [B][T][H][P];
 * Bm, Cm [B][T][G][N]; dt [B][T][H] (already through oracle_mamba2_dt);
 * A [H] (= -exp(A_log)), D [H].
 */
void oracle_mamba2_ssd_seq(double *state, const double *x, const double *Bm, const double *Cm,
                           const double *dt, const double *A, const double *D, double *y,
                           int n_seq, int T, int H, int G, int P, int N) {
  int u;
#pragma omp parallel for schedule(dynamic)
  for (u = 0; u < n_seq * H; ++u) {
    const int b = u / H, h = u % H, gi = h / (H / G);
    double *st = state + (size_t)u * P * N;
    for (int t = 0; t < T; ++t) {
      const size_t row = (size_t)b * T + t;
      const double d = dt[row * H + h];
      const double a = exp(d * A[h]);
      const double *xt = x + (row * H + h) * P;
      const double *bt = Bm + (row * G + gi) * N;
      const double *ct = Cm + (row * G + gi) * N;
      double *yt = y + (row * H + h) * P;
      for (int p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int n = 0; n < N; ++n) {
          st[p * N + n] = a * st[p * N + n] + d * xt[p] * bt[n];
          acc += st[p * N + n] * ct[n];
        }
        yt[p] = acc + D[h] * xt[p];
      }
    }
  }
}

/*
 * The same scan in chunked (state-space-duality) form: [AT] "Mamba-2 SSD
 * chunked prefill scan" comment (one dependent step per chunk, everything
 * else as dense matrix products).  Derived from the sequential definition: with
 * c_t = sum_{s<=t} dt_s A (inclusive, within the chunk) and h0 the state
 * entering the chunk,
 *   y_t  = sum_{s<=t} e^{c_t - c_s} (C_t . B_s) dt_s x_s + e^{c_t} C_t h0^T + D x_t
 *   h_n  = e^{c_n} h0 + sum_s e^{c_n - c_s} dt_s x_s B_s^T
 * (h0^T C_t meaning sum_n h0[p][n] C_t[n]).  Same layouts as the sequential form.
 */
void oracle_mamba2_ssd_chunked(double *state, const double *x, const double *Bm,
                               const double *Cm, const double *dt, const double *A,
                               const double *D, double *y, int n_seq, int T, int H, int G, int P,
                               int N, int chunk) {
  int u;
#pragma omp parallel for schedule(dynamic)
  for (u = 0; u < n_seq * H; ++u) {
    const int b = u / H, h = u % H, gi = h / (H / G);
    double *st = state + (size_t)u * P * N;
    double *c = malloc(sizeof(double) * chunk);
    double *hn = malloc(sizeof(double) * P * N);
    for (int t0 = 0; t0 < T; t0 += chunk) {
      const int n = T - t0 < chunk ? T - t0 : chunk;
      double run = 0.0;
      for (int t = 0; t < n; ++t) {
        run += dt[((size_t)b * T + t0 + t) * H + h] * A[h];
        c[t] = run;
      }
      for (int t = 0; t < n; ++t) {
        const size_t rt = (size_t)b * T + t0 + t;
        const double *ct = Cm + (rt * G + gi) * N;
        const double *xt = x + (rt * H + h) * P;
        double *yt = y + (rt * H + h) * P;
        for (int p = 0; p < P; ++p) {
          double inter = 0.0;
          for (int k = 0; k < N; ++k) inter += st[p * N + k] * ct[k];
          double intra = 0.0;
          for (int s = 0; s <= t; ++s) {
            const size_t rs = (size_t)b * T + t0 + s;
            const double *bs = Bm + (rs * G + gi) * N;
            double cb = 0.0;
            for (int k = 0; k < N; ++k) cb += ct[k] * bs[k];
            intra += exp(c[t] - c[s]) * cb * dt[rs * H + h] * x[(rs * H + h) * P + p];
          }
          yt[p] = intra + exp(c[t]) * inter + D[h] * xt[p];
        }
      }
      for (int p = 0; p < P; ++p)
        for (int k = 0; k < N; ++k) {
          double acc = exp(c[n - 1]) * st[p * N + k];
          for (int s = 0; s < n; ++s) {
            const size_t rs = (size_t)b * T + t0 + s;
            acc += exp(c[n - 1] - c[s]) * dt[rs * H + h] * x[(rs * H + h) * P + p] *
                   Bm[(rs * G + gi) * N + k];
          }
          hn[p * N + k] = acc;
        }
      memcpy(st, hn, sizeof(double) * P * N);
    }
    free(c);
    free(hn);
  }
}

/* Thread count the OpenMP runtime will use (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
