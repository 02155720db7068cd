// k_chunk_small.hip -- the chunked (WY / UT) form of the gated delta-rule
// recurrence for state sizes 32 and 64, in fp32 on the vector ALUs.
//
// ssm_mamba.rs (spark_model), "Mamba-2 SSD chunked prefill scan" comment: the
// idea of running a long prompt with one dependent step per 64-position chunk.  The
// algebra per chunk of n <= 64 positions from state S0, with G the inclusive
// cumulative sum of g over the chunk (fm_kernel_ssm.h, "Delta-rule
// recurrence" section, is the sequential definition it reproduces):
//   A  = strictly_lower(beta_t e^{G_t - G_s} k_t . k_s),  T = (I + A)^{-1}
//   W  = T diag(beta e^G) K,  U = T diag(beta) V - W S0
//   y  = scale [diag(e^G) Q S0 + (L o Q K^T) U],  L[t][s] = e^{G_t - G_s} (s <= t)
//   S  = e^{G_n} S0 + (diag(e^{G_n - G}) K)^T U
// At these widths a chunk's contractions (64 x 64 x S) are too small to fill
// MFMA tiles, so one 256-thread workgroup per (sequence, head) keeps the state
// and every chunk tile in LDS and forms each product element as an fp32 dot
// product; it needs no workspace.  Positions past the end of the last chunk
// enter with k = q = v = 0, g = 0 and beta = 0, which leaves A, W, U, y and
// the state update untouched (G is flat past the end, so G_n is the last
// real position's).
#include <hip/hip_runtime.h>

#include "gdn.h"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int SC = 64;   // positions per chunk

// First token row and length of sequence s: a fixed-length batch addresses
// sequences through their strides (row 0, n_tok positions; g and beta rows
// s * n_tok + t), a packed one through its row table (seq strides are 0).
struct SeqRows {
  int64_t row0, grow0;
  int len;
};
__device__ __forceinline__ SeqRows seq_rows(const NoTab &, int s, int n_tok) {
  return SeqRows{0, (int64_t)s * n_tok, n_tok};
}
__device__ __forceinline__ SeqRows seq_rows(const VarTab &tab, int s, int) {
  return SeqRows{tab.tok0[s], tab.tok0[s], tab.tok0[s + 1] - tab.tok0[s]};
}

// q, k, v elements: fp32, or bf16 bit patterns widened exactly to fp32
__device__ __forceinline__ float in_f32(float x) { return x; }
__device__ __forceinline__ float in_f32(unsigned short b) {
  return __builtin_bit_cast(float, (unsigned)b << 16);
}

template <int S, class TAB, class TIN>
__global__ __launch_bounds__(256) void k_chunk_small(
    float *__restrict__ state, int64_t st_seq, const TIN *__restrict__ q,
    const TIN *__restrict__ k, int64_t qk_tok, int64_t qk_seq, const TIN *__restrict__ v,
    int64_t v_tok, int64_t v_seq, const float *__restrict__ g, const float *__restrict__ beta,
    float *__restrict__ y, int64_t y_tok, int64_t y_seq, int n_tok_arg, int H, int Hk,
    float scale, const TAB tab) {
  constexpr int P = S + 1;        // row pitch of the [64][S] and [S][S] tiles
  constexpr int PC = SC + 1;      // row pitch of the [64][64] tiles
  static_assert(SC * PC >= SC * P, "U reuses the A tile");
  __shared__ float sS[S * P];     // state S0[i][j] (key i, value j)
  __shared__ float sK[SC * P], sQ[SC * P], sV[SC * P], sW[SC * P];
  __shared__ float sA[SC * PC];   // A, then U (pitch P)
  __shared__ float sL[SC * PC];   // L o Q K^T
  __shared__ float sT[SC * PC];   // T = (I + A)^{-1}
  __shared__ float sG[SC], sB[SC], sEG[SC], sEGn[SC];
  float *sU = sA;

  const int tid = threadIdx.x;
  const int h = blockIdx.x, s = blockIdx.y, hk = h / (H / Hk);
  const SeqRows sr = seq_rows(tab, s, n_tok_arg);
  const int n_tok = sr.len;
  float *st = state + s * st_seq + (int64_t)h * S * S;   // st[j * S + i] = S0[i][j]
  for (int e = tid; e < S * S; e += 256) sS[(e % S) * P + e / S] = st[e];

  const int n_chunks = (n_tok + SC - 1) / SC;
  for (int c = 0; c < n_chunks; ++c) {
    const int t0 = c * SC, n = min(SC, n_tok - t0);
    __syncthreads();   // the previous chunk is done with every tile
    for (int e = tid; e < SC * S; e += 256) {
      const int t = e / S, i = e - t * S;
      const bool ok = t < n;
      const int64_t tt = sr.row0 + (ok ? t0 + t : t0);
      const float kv = in_f32(k[s * qk_seq + tt * qk_tok + (int64_t)hk * S + i]);
      const float qv = in_f32(q[s * qk_seq + tt * qk_tok + (int64_t)hk * S + i]);
      const float vv = in_f32(v[s * v_seq + tt * v_tok + (int64_t)h * S + i]);
      sK[t * P + i] = ok ? kv : 0.0f;
      sQ[t * P + i] = ok ? qv : 0.0f;
      sV[t * P + i] = ok ? vv : 0.0f;
    }
    if (tid < SC) {   // wave 0: G (inclusive cumsum), beta
      const int t = tid;
      const int64_t gi = (sr.grow0 + t0 + (t < n ? t : 0)) * H + h;
      float gv = t < n ? g[gi] : 0.0f;
      const float bv = t < n ? beta[gi] : 0.0f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(gv, off, 64);
        if (t >= off) gv += o;
      }
      const float gn = __shfl(gv, 63, 64);
      sG[t] = gv;
      sB[t] = bv;
      sEG[t] = expf(gv);
      sEGn[t] = expf(gn - gv);
    }
    __syncthreads();

    // A (strictly lower) and L o Q K^T (lower, diagonal included)
    for (int e = tid; e < SC * SC; e += 256) {
      const int t = e / SC, u = e - t * SC;
      float a = 0.0f, l = 0.0f;
      if (u <= t) {
        float dk = 0.0f, dq = 0.0f;
#pragma unroll 8
        for (int i = 0; i < S; ++i) {
          dk = __builtin_fmaf(sK[t * P + i], sK[u * P + i], dk);
          dq = __builtin_fmaf(sQ[t * P + i], sK[u * P + i], dq);
        }
        const float dec = expf(sG[t] - sG[u]);
        if (u < t) a = sB[t] * dec * dk;
        l = dec * dq;
      }
      sA[t * PC + u] = a;
      sL[t * PC + u] = l;
    }
    __syncthreads();

    // T = (I + A)^{-1}: thread c forward-substitutes column c (rows >= c)
    if (tid < SC) {
      const int cc = tid;
      for (int r = 0; r < SC; ++r) {
        float acc = r == cc ? 1.0f : 0.0f;
        for (int j = cc; j < r; ++j) acc = __builtin_fmaf(-sA[r * PC + j], sT[j * PC + cc], acc);
        sT[r * PC + cc] = r >= cc ? acc : 0.0f;
      }
    }
    __syncthreads();

    // W = T diag(beta e^G) K and Ut = T diag(beta) V (into the A tile)
    for (int e = tid; e < SC * S; e += 256) {
      const int t = e / S, i = e - t * S;
      float w = 0.0f, u = 0.0f;
      for (int r = 0; r <= t; ++r) {
        const float tb = sT[t * PC + r] * sB[r];
        w = __builtin_fmaf(tb * sEG[r], sK[r * P + i], w);
        u = __builtin_fmaf(tb, sV[r * P + i], u);
      }
      sW[t * P + i] = w;
      sU[t * P + i] = u;
    }
    __syncthreads();

    // U = Ut - W S0 (each thread updates its own elements)
    for (int e = tid; e < SC * S; e += 256) {
      const int t = e / S, j = e - t * S;
      float acc = sU[t * P + j];
#pragma unroll 8
      for (int i = 0; i < S; ++i) acc = __builtin_fmaf(-sW[t * P + i], sS[i * P + j], acc);
      sU[t * P + j] = acc;
    }
    __syncthreads();

    // y = scale (e^{G_t} (Q S0)[t] + sum_{u <= t} L[t][u] U[u])
    for (int e = tid; e < SC * S; e += 256) {
      const int t = e / S, j = e - t * S;
      if (t < n) {
        float qs = 0.0f, lu = 0.0f;
#pragma unroll 8
        for (int i = 0; i < S; ++i) qs = __builtin_fmaf(sQ[t * P + i], sS[i * P + j], qs);
        for (int u = 0; u <= t; ++u) lu = __builtin_fmaf(sL[t * PC + u], sU[u * P + j], lu);
        y[s * y_seq + (sr.row0 + t0 + t) * y_tok + (int64_t)h * S + j] =
            scale * (sEG[t] * qs + lu);
      }
    }
    __syncthreads();   // every read of S0 is done

    // S = e^{G_n} S0 + sum_t e^{G_n - G_t} k_t u_t^T
    const float egn = sEG[SC - 1];
    for (int e = tid; e < S * S; e += 256) {
      const int i = e / S, j = e - i * S;
      float acc = 0.0f;
#pragma unroll 8
      for (int t = 0; t < SC; ++t) acc = __builtin_fmaf(sEGn[t] * sK[t * P + i], sU[t * P + j], acc);
      sS[i * P + j] = __builtin_fmaf(egn, sS[i * P + j], acc);
    }
  }
  __syncthreads();
  for (int e = tid; e < S * S; e += 256) st[e] = sS[(e % S) * P + e / S];
}

template <int S, class TAB, class TIN>
int run_small(const RecurArgs &a, const TAB &tab, const TIN *q, const TIN *k, const TIN *v,
              hipStream_t stream) {
  return launch_kernel(k_chunk_small<S, TAB, TIN>, dim3((unsigned)a.H, (unsigned)a.n_seq),
                       dim3(256), 0, stream, a.state, a.st_seq, q, k, a.qk_tok, a.qk_seq, v,
                       a.v_tok, a.v_seq, a.g, a.beta, a.y, a.y_tok, a.y_seq, a.n_tok, a.H, a.Hk,
                       a.scale, tab);
}

template <class TAB, class TIN>
int run_small_s(const RecurArgs &a, const TAB &tab, const TIN *q, const TIN *k, const TIN *v,
                hipStream_t stream) {
  switch (a.S) {
    case 32: return run_small<32>(a, tab, q, k, v, stream);
    case 64: return run_small<64>(a, tab, q, k, v, stream);
    default: return GDN_ERR_UNSUPPORTED;
  }
}

}  // namespace

int launch_chunk_small(const RecurArgs &a, hipStream_t stream) {
  return run_small_s(a, NoTab{}, a.q, a.k, a.v, stream);
}

int launch_chunk_small_varlen(const RecurArgs &a, const VarTab &tab, bool bf16_in,
                              hipStream_t stream) {
  if (bf16_in) {
    typedef unsigned short b16;
    return run_small_s(a, tab, reinterpret_cast<const b16 *>(a.q),
                       reinterpret_cast<const b16 *>(a.k), reinterpret_cast<const b16 *>(a.v),
                       stream);
  }
  return run_small_s(a, tab, a.q, a.k, a.v, stream);
}

}  // namespace gdn
