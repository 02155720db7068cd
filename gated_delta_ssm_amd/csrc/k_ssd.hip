// k_ssd.hip -- the Mamba-2 selective scan in chunked (state-space-duality)
// form.  ssm_mamba.rs (spark_model layers/ops), mamba2_ssm_prefill: its
// arguments (state h, x, B and C projections, raw dt with a per-head bias and
// dt_min / dt_max limits, A_log, the D skip, n_groups) and the "Mamba-2 SSD
// chunked prefill scan" comment (dense matrix products inside each chunk, one
// dependent step per chunk).  Per head (group gi = h / (H / G)), token t:
//   dt = clamp(softplus(dt_raw + dt_bias), dt_min, dt_max),  A = -exp(A_log)
//   h  <- exp(dt A) h + dt x B^T        (h [P][N])
//   y  =  h C + D x
// For a chunk of n <= 64 positions entering with state h0, with c_t the
// inclusive within-chunk sum of dt A (so every exponential below takes a
// non-positive argument):
//   y_t = sum_{s<=t} e^{c_t - c_s} (C_t . B_s) dt_s x_s + e^{c_t} h0 C_t + D x_t
//   h_n = e^{c_n} h0 + sum_s e^{c_n - c_s} dt_s x_s B_s^T
// Three launches:
//   k_ssd_chunk  every (sequence, head, chunk) at once: the intra-chunk output
//                (first sum, plus D x) into y, and the chunk's own state
//                contribution (second sum) and decay e^{c_n} into a workspace
//   k_ssd_state  the sequential link, elementwise over h: for each chunk, the
//                state entering it is written over its contribution, then
//                h <- e^{c_n} h + contribution; the last h is the new state
//   k_ssd_out    every chunk again: y_t += e^{c_t} h0 C_t
// At head_dim 64 / state 128 the chunk and output kernels run their products
// as 16x16x32 bf16 MFMA tiles with each fp32 operand split into hi + lo
// (k_ssd_chunk_mma, k_ssd_out_mma); other shapes use fp32 on the vector ALUs,
// 4 x 4 (or 4 x 8) register tiles over LDS rows read as float4.
#include <hip/hip_runtime.h>

#include "bf16_frag.hpp"
#include "gdn.h"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int SC = 64;     // positions per chunk
constexpr int NT = 256;    // threads per workgroup

__device__ __forceinline__ float softplus20(float v) { return v > 20.0f ? v : log1pf(expf(v)); }

// Per-position dt and inclusive cumsum of dt A for the chunk, in LDS (wave 0;
// positions past n get dt = 0, so the cumsum stays flat there), and if asked
// the state weights w_t = e^{c_n - c_t} dt_t.  Both kernels that need c_t call
// this, so they agree bit for bit.
__device__ __forceinline__ void chunk_dt(const float *dt_raw, int64_t dt_row0, int64_t dt_tok,
                                         int h, int n, float bias, float A, float dt_min,
                                         float dt_max, float *sDt, float *sCs,
                                         float *sW = nullptr) {
  const int t = threadIdx.x;
  if (t < SC) {
    float d = 0.0f;
    if (t < n) {
      d = softplus20(dt_raw[dt_row0 + (int64_t)t * dt_tok + h] + bias);
      d = fminf(fmaxf(d, dt_min), dt_max);
    }
    float c = d * A;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(c, off, 64);
      if (t >= off) c += o;
    }
    sDt[t] = d;
    sCs[t] = c;
    const float cn = __shfl(c, SC - 1, 64);
    if (sW != nullptr) sW[t] = expf(cn - c) * d;
  }
}

// Rows [0, n) of a [ROWS][W] tile with row stride `tok` (elements) into LDS
// (pitch W + 4); rows n .. ROWS-1 are zero.  16-byte accesses.
template <int W, int ROWS = SC>
__device__ __forceinline__ void load_rows(float *dst, const float *src, int64_t tok, int n) {
  constexpr int PW = W + 4, V = W / 4;
  for (int e = threadIdx.x; e < ROWS * V; e += NT) {
    const int r = e / V, c4 = (e - r * V) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < n) v = *reinterpret_cast<const float4 *>(src + (int64_t)r * tok + c4);
    *reinterpret_cast<float4 *>(dst + r * PW + c4) = v;
  }
}

struct SsdArgs {
  const float *x, *Bm, *Cm, *dt_raw, *A_log, *D, *dt_bias;
  int64_t x_tok, x_seq, bc_tok, bc_seq, dt_tok, dt_seq, y_tok, y_seq;
  float *y;
  int n_tok, H, G, n_chunks;
  float dt_min, dt_max;
};

// Workspace: per (sequence, head, chunk) a [P][N] fp32 block (the chunk's
// state contribution, then the state entering the chunk), and after all of
// them one float per (sequence, head, chunk): e^{c_n}.
template <int P, int N>
__device__ __forceinline__ float *ws_block(float *ws, int s, int h, int c, int H, int nc) {
  return ws + (((size_t)s * H + h) * nc + c) * (size_t)(P * N);
}
__device__ __forceinline__ float *ws_decay(float *ws, size_t blocks_floats, int s, int h, int c,
                                           int H, int nc) {
  return ws + blocks_floats + ((size_t)s * H + h) * nc + c;
}

template <int P, int N>
__global__ __launch_bounds__(NT) void k_ssd_chunk(SsdArgs a, float *__restrict__ ws) {
  constexpr int PX = P + 4, PB = N + 4, PM = SC + 4;
  __shared__ __attribute__((aligned(16))) float sX[SC * PX];
  __shared__ __attribute__((aligned(16))) float sB[SC * PB];
  __shared__ __attribute__((aligned(16))) float sC[SC * PB];
  __shared__ __attribute__((aligned(16))) float sM[SC * PM];
  __shared__ float sDt[SC], sCs[SC];
  const int c = blockIdx.x, h = blockIdx.y, s = blockIdx.z, tid = threadIdx.x;
  const int gi = h / (a.H / a.G);
  const int t0 = c * SC, n = min(SC, a.n_tok - t0);
  const float A = -expf(a.A_log[h]);

  chunk_dt(a.dt_raw, s * a.dt_seq + (int64_t)t0 * a.dt_tok, a.dt_tok, h, n, a.dt_bias[h], A,
           a.dt_min, a.dt_max, sDt, sCs);
  const float *xc = a.x + s * a.x_seq + (int64_t)t0 * a.x_tok + (int64_t)h * P;
  const float *bc = a.Bm + s * a.bc_seq + (int64_t)t0 * a.bc_tok + (int64_t)gi * N;
  const float *cc = a.Cm + s * a.bc_seq + (int64_t)t0 * a.bc_tok + (int64_t)gi * N;
  load_rows<P>(sX, xc, a.x_tok, n);
  load_rows<N>(sB, bc, a.bc_tok, n);
  load_rows<N>(sC, cc, a.bc_tok, n);
  __syncthreads();

  // M[t][s] = e^{c_t - c_s} (C_t . B_s) dt_s for s <= t, else 0: 4 x 4 entries
  // per thread, rows 4 tr .. +3 and columns sc + 16 j (the 16 lanes of a row
  // group read 16 consecutive B rows, which fall in distinct LDS banks)
  {
    const int tr = tid >> 4, sc = tid & 15;
    float acc[4][4] = {};
    for (int k = 0; k < N; k += 4) {
      float4 cv[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        cv[i] = *reinterpret_cast<const float4 *>(sC + (4 * tr + i) * PB + k);
        bv[i] = *reinterpret_cast<const float4 *>(sB + (sc + 16 * i) * PB + k);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = fmaf(cv[i].w, bv[j].w, fmaf(cv[i].z, bv[j].z,
                      fmaf(cv[i].y, bv[j].y, fmaf(cv[i].x, bv[j].x, acc[i][j]))));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * tr + i;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int u = sc + 16 * j;
        const float arg = u <= t ? sCs[t] - sCs[u] : 0.0f;
        sM[t * PM + u] = u <= t ? expf(arg) * acc[i][j] * sDt[u] : 0.0f;
      }
    }
  }
  __syncthreads();

  // y_t (intra-chunk part) = sum_s M[t][s] x_s + D x_t: a 4 x (P/16) block per
  // thread (rows 4 tr .. +3, columns 4 pc .. +3 for P = 64)
  {
    constexpr int PCOLS = P / 4;              // float4 columns of a row
    constexpr int TROWS = NT / PCOLS;         // row groups
    constexpr int RPT = SC / TROWS;           // rows per thread
    const int pc = tid % PCOLS, tr = tid / PCOLS;
    float4 acc[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int u = 0; u < SC; u += 4) {
      float4 xv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[j] = *reinterpret_cast<const float4 *>(sX + (u + j) * PX + 4 * pc);
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float4 m = *reinterpret_cast<const float4 *>(sM + (RPT * tr + i) * PM + u);
        acc[i].x = fmaf(m.w, xv[3].x, fmaf(m.z, xv[2].x, fmaf(m.y, xv[1].x, fmaf(m.x, xv[0].x, acc[i].x))));
        acc[i].y = fmaf(m.w, xv[3].y, fmaf(m.z, xv[2].y, fmaf(m.y, xv[1].y, fmaf(m.x, xv[0].y, acc[i].y))));
        acc[i].z = fmaf(m.w, xv[3].z, fmaf(m.z, xv[2].z, fmaf(m.y, xv[1].z, fmaf(m.x, xv[0].z, acc[i].z))));
        acc[i].w = fmaf(m.w, xv[3].w, fmaf(m.z, xv[2].w, fmaf(m.y, xv[1].w, fmaf(m.x, xv[0].w, acc[i].w))));
      }
    }
    const float Dh = a.D[h];
    float *yc = a.y + s * a.y_seq + (int64_t)t0 * a.y_tok + (int64_t)h * P;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int t = RPT * tr + i;
      if (t < n) {
        const float4 xv = *reinterpret_cast<const float4 *>(sX + t * PX + 4 * pc);
        *reinterpret_cast<float4 *>(yc + (int64_t)t * a.y_tok + 4 * pc) =
            make_float4(acc[i].x + Dh * xv.x, acc[i].y + Dh * xv.y, acc[i].z + Dh * xv.z,
                        acc[i].w + Dh * xv.w);
      }
    }
  }

  // chunk contribution Hc[p][k] = sum_s w_s x_s[p] B_s[k], w_s = e^{c_n - c_s} dt_s:
  // P x N outputs; a thread holds RPT rows x 8 columns, the columns 4 kc .. +3
  // and N/2 + 4 kc .. +3 (consecutive lanes read consecutive 16 bytes)
  {
    constexpr int KC = N / 8;                 // 8-column groups
    constexpr int PR = NT / KC;               // row groups
    constexpr int RPT = P / PR;               // rows per thread
    static_assert(RPT >= 1 && P % PR == 0, "thread map");
    const int kc = tid % KC, pr = tid / KC;
    const float cn = sCs[SC - 1];
    float acc[RPT][8] = {};
    for (int u = 0; u < SC; ++u) {
      const float w = expf(cn - sCs[u]) * sDt[u];
      const float4 b0 = *reinterpret_cast<const float4 *>(sB + u * PB + 4 * kc);
      const float4 b1 = *reinterpret_cast<const float4 *>(sB + u * PB + N / 2 + 4 * kc);
      const float bw[8] = {w * b0.x, w * b0.y, w * b0.z, w * b0.w,
                           w * b1.x, w * b1.y, w * b1.z, w * b1.w};
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float xv = sX[u * PX + RPT * pr + i];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(xv, bw[j], acc[i][j]);
      }
    }
    float *blk = ws_block<P, N>(ws, s, h, c, a.H, a.n_chunks);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      float *row = blk + (RPT * pr + i) * N + 4 * kc;
      *reinterpret_cast<float4 *>(row) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
      *reinterpret_cast<float4 *>(row + N / 2) =
          make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
    }
    if (tid == 0) {
      const size_t blocks = (size_t)gridDim.z * a.H * a.n_chunks * (P * N);
      *ws_decay(ws, blocks, s, h, c, a.H, a.n_chunks) = expf(cn);
    }
  }
}

// The sequential link: thread e of (sequence, head) owns elements 4e .. 4e+3
// of the [P][N] state.
template <int P, int N>
__global__ __launch_bounds__(NT) void k_ssd_state(float *__restrict__ state, int64_t st_seq,
                                                  float *__restrict__ ws, int n_seq, int H,
                                                  int nc) {
  const int h = blockIdx.y, s = blockIdx.z;
  const int e = blockIdx.x * NT + threadIdx.x;   // float4 index, < P N / 4 by the grid
  float4 *sp = reinterpret_cast<float4 *>(state + s * st_seq + (size_t)h * P * N) + e;
  float4 st = *sp;
  const size_t blocks = (size_t)n_seq * H * nc * (P * N);
  const float *dec = ws_decay(ws, blocks, s, h, 0, H, nc);
  // U chunks' contributions are loaded before the first is used: the grid has
  // only P N / 4 threads per head, so each needs many bytes in flight
  constexpr int U = 16;
  float4 *bp = reinterpret_cast<float4 *>(ws_block<P, N>(ws, s, h, 0, H, nc)) + e;
  for (int c0 = 0; c0 < nc; c0 += U) {
    float4 contrib[U];
    float gam[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u < nc) {
        contrib[u] = bp[(size_t)(c0 + u) * (P * N / 4)];
        gam[u] = dec[c0 + u];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u < nc) {
        bp[(size_t)(c0 + u) * (P * N / 4)] = st;   // the state entering chunk c0 + u
        st = make_float4(gam[u] * st.x + contrib[u].x, gam[u] * st.y + contrib[u].y,
                         gam[u] * st.z + contrib[u].z, gam[u] * st.w + contrib[u].w);
      }
    }
  }
  *sp = st;
}

// y_t += e^{c_t} sum_k h0[p][k] C_t[k] with h0 the state entering the chunk.
template <int P, int N>
__global__ __launch_bounds__(NT) void k_ssd_out(SsdArgs a, const float *__restrict__ ws) {
  constexpr int PB = N + 4;
  __shared__ __attribute__((aligned(16))) float sC[SC * PB];
  __shared__ __attribute__((aligned(16))) float sH[P * PB];
  __shared__ float sDt[SC], sCs[SC];
  const int c = blockIdx.x, h = blockIdx.y, s = blockIdx.z, tid = threadIdx.x;
  const int gi = h / (a.H / a.G);
  const int t0 = c * SC, n = min(SC, a.n_tok - t0);
  const float A = -expf(a.A_log[h]);
  chunk_dt(a.dt_raw, s * a.dt_seq + (int64_t)t0 * a.dt_tok, a.dt_tok, h, n, a.dt_bias[h], A,
           a.dt_min, a.dt_max, sDt, sCs);
  load_rows<N>(sC, a.Cm + s * a.bc_seq + (int64_t)t0 * a.bc_tok + (int64_t)gi * N, a.bc_tok, n);
  const float *blk = ws_block<P, N>(const_cast<float *>(ws), s, h, c, a.H, a.n_chunks);
  load_rows<N, P>(sH, blk, N, P);   // the P rows of the entering state, row stride N
  __syncthreads();

  constexpr int PCOLS = P / 4;
  constexpr int TROWS = NT / PCOLS;
  constexpr int RPT = SC / TROWS;
  const int pc = tid % PCOLS, tr = tid / PCOLS;
  float4 acc[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < N; k += 4) {
    float4 hv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) hv[j] = *reinterpret_cast<const float4 *>(sH + (pc + PCOLS * j) * PB + k);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float4 cv = *reinterpret_cast<const float4 *>(sC + (RPT * tr + i) * PB + k);
      acc[i].x = fmaf(cv.w, hv[0].w, fmaf(cv.z, hv[0].z, fmaf(cv.y, hv[0].y, fmaf(cv.x, hv[0].x, acc[i].x))));
      acc[i].y = fmaf(cv.w, hv[1].w, fmaf(cv.z, hv[1].z, fmaf(cv.y, hv[1].y, fmaf(cv.x, hv[1].x, acc[i].y))));
      acc[i].z = fmaf(cv.w, hv[2].w, fmaf(cv.z, hv[2].z, fmaf(cv.y, hv[2].y, fmaf(cv.x, hv[2].x, acc[i].z))));
      acc[i].w = fmaf(cv.w, hv[3].w, fmaf(cv.z, hv[3].z, fmaf(cv.y, hv[3].y, fmaf(cv.x, hv[3].x, acc[i].w))));
    }
  }
  float *yc = a.y + s * a.y_seq + (int64_t)t0 * a.y_tok + (int64_t)h * P;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int t = RPT * tr + i;
    if (t < n) {
      // columns pc + PCOLS j: consecutive lanes hit consecutive elements
      const float e = expf(sCs[t]);
      float *yr = yc + (int64_t)t * a.y_tok + pc;
      yr[0] += e * acc[i].x;
      yr[PCOLS] += e * acc[i].y;
      yr[2 * PCOLS] += e * acc[i].z;
      yr[3 * PCOLS] += e * acc[i].w;
    }
  }
}

// ----------------------------------------------------------------------------- MFMA form
// The same three launches for head_dim 64 and state 128 with the dense
// products on v_mfma_f32_16x16x32_bf16, each fp32 operand split into bf16
// hi + lo (hi*hi + hi*lo + lo*hi, fp32 accumulation; ~2^-16 relative per
// product).  8 waves; LDS tiles are row-major bf16 hi/lo planes.
constexpr int MP = 64, MN = 128;          // head_dim, state
constexpr int MNT = 512;                  // threads
constexpr int PXb = MP + 8, PBb = MN + 8, PMb = SC + 8;   // pitches (bf16 elements)

// A [ROWS][W] fp32 tile (row stride `tok`) moves to LDS in two steps, so a
// thread's loads are all in flight before the first is used: rows [0, n) into
// registers (zeros past n), then split into bf16 hi/lo planes of pitch PW.
template <int W, int ROWS>
constexpr int rows_per_thread() { return ROWS * (W / 4) / MNT; }
template <int W, int ROWS>
__device__ __forceinline__ void fetch_rows(const float *src, int64_t tok, int n,
                                           float4 (&v)[rows_per_thread<W, ROWS>()]) {
  constexpr int V = W / 4;
  static_assert(ROWS * V % MNT == 0, "whole passes");
#pragma unroll
  for (int i = 0; i < rows_per_thread<W, ROWS>(); ++i) {
    const int e = threadIdx.x + i * MNT, r = e / V, c4 = (e - r * V) * 4;
    v[i] = r < n ? *reinterpret_cast<const float4 *>(src + (int64_t)r * tok + c4)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}
template <int W, int ROWS, int PW>
__device__ __forceinline__ void put_rows(u16 *hi, u16 *lo,
                                         const float4 (&v)[rows_per_thread<W, ROWS>()]) {
  constexpr int V = W / 4;
#pragma unroll
  for (int i = 0; i < rows_per_thread<W, ROWS>(); ++i) {
    const int e = threadIdx.x + i * MNT, r = e / V, c4 = (e - r * V) * 4;
    store4_split(hi + r * PW + c4, lo + r * PW + c4, v[i].x, v[i].y, v[i].z, v[i].w);
  }
}

// The MN / 32 k-step fragments of row `row` of a [SC][MN] fp32 tile in global
// memory (zero past row n): lane (kg, l16) holds k = 32 ks + 8 kg .. +7, split
// in registers exactly as store4_split splits the LDS planes.
struct RowFrags {
  float4 v[MN / 32][2];
};
__device__ __forceinline__ void fetch_row_frags(const float *src, int64_t tok, int row, int n,
                                                int kg, RowFrags &f) {
#pragma unroll
  for (int ks = 0; ks < MN / 32; ++ks) {
    const float *p = src + (int64_t)row * tok + 32 * ks + 8 * kg;
    f.v[ks][0] = row < n ? *reinterpret_cast<const float4 *>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
    f.v[ks][1] =
        row < n ? *reinterpret_cast<const float4 *>(p + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}
__device__ __forceinline__ Frag split_frag(const float4 &a, const float4 &b) {
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  return split8(x);
}

__global__ __launch_bounds__(MNT) void k_ssd_chunk_mma(SsdArgs a, float *__restrict__ ws) {
  // Only x and B pass through LDS: each wave splits its row tile of C in
  // registers, w B overwrites B once M is formed, and M (held in registers
  // meanwhile) overwrites w B once the state contribution is formed, so three
  // workgroups fit in one CU's LDS
  __shared__ __attribute__((aligned(16))) u16 sXh[SC * PXb], sXl[SC * PXb];
  __shared__ __attribute__((aligned(16))) u16 sBh[SC * PBb], sBl[SC * PBb];   // B, w B, M
  static_assert(SC * PMb <= SC * PBb, "M fits in B's planes");
  u16 *const sMh = sBh, *const sMl = sBl;
  __shared__ float sDt[SC], sCs[SC], sW[SC];
  const int c = blockIdx.x, h = blockIdx.y, s = blockIdx.z, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
  const int gi = h / (a.H / a.G);
  const int t0 = c * SC, n = min(SC, a.n_tok - t0);
  const float A = -expf(a.A_log[h]);
  chunk_dt(a.dt_raw, s * a.dt_seq + (int64_t)t0 * a.dt_tok, a.dt_tok, h, n, a.dt_bias[h], A,
           a.dt_min, a.dt_max, sDt, sCs, sW);
  const float *xc = a.x + s * a.x_seq + (int64_t)t0 * a.x_tok + (int64_t)h * MP;
  const float *bc = a.Bm + s * a.bc_seq + (int64_t)t0 * a.bc_tok + (int64_t)gi * MN;
  const float *cc = a.Cm + s * a.bc_seq + (int64_t)t0 * a.bc_tok + (int64_t)gi * MN;
  // M's 10 lower 16x16 tiles (ti >= tj) go to waves 0..5 by token tile, so a
  // wave needs one row tile of C: w0 (3; 0,1), w1 (3; 2,3), w2 (2; 0,1),
  // w3 (2; 2), w4 (1; 0,1), w5 (0; 0); waves 6 and 7 have none
  const int mti = w < 2 ? 3 : w < 4 ? 2 : w == 4 ? 1 : 0;
  const int mtj = (w == 1 || w == 3) ? 2 : 0;
  const int mnt = w < 6 ? ((w == 3 || w == 5) ? 1 : 2) : 0;
  // the y tiles of this lane: token tile w & 3, value tiles 2 (w >> 2), +1
  const int yti = w & 3;
  RowFrags fcr;
  float xv[2][4];   // x at this lane's y slots, for D x
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * yti + 4 * kg + r, p = 16 * (2 * (w >> 2) + j) + l16;
      xv[j][r] = t < n ? xc[(int64_t)t * a.x_tok + p] : 0.0f;
    }
  float4 vb[rows_per_thread<MN, SC>()];   // B, kept for w B
  {
    float4 vx[rows_per_thread<MP, SC>()];
    fetch_rows<MP, SC>(xc, a.x_tok, n, vx);
    fetch_rows<MN, SC>(bc, a.bc_tok, n, vb);
    if (mnt > 0) fetch_row_frags(cc, a.bc_tok, 16 * mti + l16, n, kg, fcr);
    put_rows<MP, SC, PXb>(sXh, sXl, vx);
    put_rows<MN, SC, PBb>(sBh, sBl, vb);
  }
  __syncthreads();

  // M[t][s] = e^{c_t - c_s} (C_t . B_s) dt_s, lower 16x16 tiles (ti >= tj)
  float mv[2][4];   // this wave's M tiles, kept in registers until B's planes are free
  if (mnt > 0) {
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < MN / 32; ++ks) {
      const Frag fc = split_frag(fcr.v[ks][0], fcr.v[ks][1]);
      acc[0] = mfma3(fc, frag(sBh, sBl, PBb, 16 * mtj + l16, 32 * ks + 8 * kg), acc[0]);
      if (mnt > 1)
        acc[1] = mfma3(fc, frag(sBh, sBl, PBb, 16 * (mtj + 1) + l16, 32 * ks + 8 * kg), acc[1]);
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int u = 16 * (mtj + jj) + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * mti + 4 * kg + r;
        const float arg = u <= t ? sCs[t] - sCs[u] : 0.0f;
        mv[jj][r] = u <= t ? expf(arg) * acc[jj][r] * sDt[u] : 0.0f;
      }
    }
  }
  __syncthreads();   // M formed; B no longer read as B
  // w_s B_s over B's planes, for the state contribution: each thread scales
  // the fp32 B elements it stored there (rows past n are zero)
#pragma unroll
  for (int i = 0; i < rows_per_thread<MN, SC>(); ++i) {
    const int e = tid + i * MNT, r = e / (MN / 4), c4 = (e - r * (MN / 4)) * 4;
    const float f = sW[r];
    store4_split(sBh + r * PBb + c4, sBl + r * PBb + c4, f * vb[i].x, f * vb[i].y, f * vb[i].z,
                 f * vb[i].w);
  }

  __syncthreads();   // w B complete

  // state contribution Hc[p][k] = sum_s x_s[p] w_s B_s[k]: 4 x 8 tiles (p, k),
  // wave w takes value tile w & 3 and state tiles 4 (w >> 2) .. +3
  {
    const int tp = w & 3;
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < SC / 32; ++ks) {
      const Frag fx = frag_tr(sXh, sXl, PXb, 32 * ks, 16 * tp, kg, l16);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = mfma3(fx, frag_tr(sBh, sBl, PBb, 32 * ks, 16 * (4 * (w >> 2) + j), kg, l16),
                       acc[j]);
    }
    float *blk = ws_block<MP, MN>(ws, s, h, c, a.H, a.n_chunks);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = 16 * (4 * (w >> 2) + j) + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) blk[(16 * tp + 4 * kg + r) * MN + k] = acc[j][r];
    }
    if (tid == 0) {
      const size_t blocks = (size_t)gridDim.z * a.H * a.n_chunks * (MP * MN);
      *ws_decay(ws, blocks, s, h, c, a.H, a.n_chunks) = expf(sCs[SC - 1]);
    }
  }
  __syncthreads();   // w B no longer read

  // M over B's planes: waves 0..5 their lower tiles; waves 6 and 7 zero the
  // upper tiles (0, 1) and (2, 3), the only ones the products below read
  if (w < 6) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      if (jj >= mnt) break;
      const int u = 16 * (mtj + jj) + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * mti + 4 * kg + r;
        u16 hh, ll;
        split(mv[jj][r], hh, ll);
        sMh[t * PMb + u] = hh;
        sMl[t * PMb + u] = ll;
      }
    }
  } else {
    const int zt = w == 6 ? 0 : 2;   // tile (zt, zt + 1)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * zt + 4 * kg + r, u = 16 * (zt + 1) + l16;
      sMh[t * PMb + u] = 0;
      sMl[t * PMb + u] = 0;
    }
  }
  __syncthreads();

  // y_t (intra-chunk part) = sum_s M[t][s] x_s + D x_t: 16 tiles (t, p), wave w
  // takes token tile w & 3 and value tiles 2 (w >> 2), +1; token tiles 0 and 1
  // need only positions s < 32
  {
    const int ti = yti;
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    for (int ks = 0; ks < (ti < 2 ? 1 : 2); ++ks) {
      const Frag fm = frag_pi(sMh, sMl, PMb, 16 * ti + l16, 32 * ks, kg);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[j] = mfma3(fm, frag_tr(sXh, sXl, PXb, 32 * ks, 16 * (2 * (w >> 2) + j), kg, l16),
                       acc[j]);
    }
    const float Dh = a.D[h];
    float *yc = a.y + s * a.y_seq + (int64_t)t0 * a.y_tok + (int64_t)h * MP;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int p = 16 * (2 * (w >> 2) + j) + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * ti + 4 * kg + r;
        if (t < n) yc[(int64_t)t * a.y_tok + p] = acc[j][r] + Dh * xv[j][r];
      }
    }
  }
}

// y_t += e^{c_t} sum_k C_t[k] h0[p][k]: 16 tiles (t, p), wave w takes token
// tile w & 3 and value tiles 2 (w >> 2), +1.  Only h0 goes through LDS; each
// wave splits its row tile of C in registers.
__global__ __launch_bounds__(MNT) void k_ssd_out_mma(SsdArgs a, const float *__restrict__ ws) {
  __shared__ __attribute__((aligned(16))) u16 sHh[MP * PBb], sHl[MP * PBb];
  __shared__ float sDt[SC], sCs[SC];
  const int c = blockIdx.x, h = blockIdx.y, s = blockIdx.z, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
  const int gi = h / (a.H / a.G);
  const int t0 = c * SC, n = min(SC, a.n_tok - t0);
  const float A = -expf(a.A_log[h]);
  chunk_dt(a.dt_raw, s * a.dt_seq + (int64_t)t0 * a.dt_tok, a.dt_tok, h, n, a.dt_bias[h], A,
           a.dt_min, a.dt_max, sDt, sCs);
  const int ti = w & 3;
  float *yc = a.y + s * a.y_seq + (int64_t)t0 * a.y_tok + (int64_t)h * MP;
  float yv[2][4];   // the intra-chunk y this lane completes, read with the other loads
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = 16 * (2 * (w >> 2) + j) + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * ti + 4 * kg + r;
      yv[j][r] = t < n ? yc[(int64_t)t * a.y_tok + p] : 0.0f;
    }
  }
  RowFrags fcr;
  {
    float4 vh[rows_per_thread<MN, MP>()];
    fetch_rows<MN, MP>(ws_block<MP, MN>(const_cast<float *>(ws), s, h, c, a.H, a.n_chunks), MN,
                       MP, vh);
    fetch_row_frags(a.Cm + s * a.bc_seq + (int64_t)t0 * a.bc_tok + (int64_t)gi * MN, a.bc_tok,
                    16 * ti + l16, n, kg, fcr);
    put_rows<MN, MP, PBb>(sHh, sHl, vh);
  }
  __syncthreads();
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ks = 0; ks < MN / 32; ++ks) {
    const Frag fc = split_frag(fcr.v[ks][0], fcr.v[ks][1]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[j] = mfma3(fc, frag(sHh, sHl, PBb, 16 * (2 * (w >> 2) + j) + l16, 32 * ks + 8 * kg),
                     acc[j]);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = 16 * (2 * (w >> 2) + j) + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * ti + 4 * kg + r;
      if (t < n) yc[(int64_t)t * a.y_tok + p] = yv[j][r] + expf(sCs[t]) * acc[j][r];
    }
  }
}

template <int P, int N>
int run_ssd(const SsdLaunch &l, hipStream_t stream) {
  const int nc = (l.n_tok + SC - 1) / SC;
  SsdArgs a{l.x,     l.Bm,     l.Cm,     l.dt_raw, l.A_log,  l.D,    l.dt_bias,
            l.x_tok, l.x_seq,  l.bc_tok, l.bc_seq, l.dt_tok, l.dt_seq, l.y_tok,
            l.y_seq, l.y,      l.n_tok,  l.H,      l.G,      nc,     l.dt_min,
            l.dt_max};
  float *ws = static_cast<float *>(l.ws);
  const dim3 grid_c((unsigned)nc, (unsigned)l.H, (unsigned)l.n_seq);
  int rc = launch_kernel(k_ssd_chunk<P, N>, grid_c, dim3(NT), 0, stream, a, ws);
  if (rc != GDN_OK) return rc;
  static_assert((P * N / 4) % NT == 0, "state grid");
  rc = launch_kernel(k_ssd_state<P, N>, dim3(P * N / 4 / NT, (unsigned)l.H, (unsigned)l.n_seq),
                     dim3(NT), 0, stream, l.state, l.st_seq, ws, l.n_seq, l.H, nc);
  if (rc != GDN_OK) return rc;
  return launch_kernel(k_ssd_out<P, N>, grid_c, dim3(NT), 0, stream, a,
                       static_cast<const float *>(ws));
}

int run_ssd_mma(const SsdLaunch &l, hipStream_t stream) {
  const int nc = (l.n_tok + SC - 1) / SC;
  SsdArgs a{l.x,     l.Bm,     l.Cm,     l.dt_raw, l.A_log,  l.D,    l.dt_bias,
            l.x_tok, l.x_seq,  l.bc_tok, l.bc_seq, l.dt_tok, l.dt_seq, l.y_tok,
            l.y_seq, l.y,      l.n_tok,  l.H,      l.G,      nc,     l.dt_min,
            l.dt_max};
  float *ws = static_cast<float *>(l.ws);
  const dim3 grid_c((unsigned)nc, (unsigned)l.H, (unsigned)l.n_seq);
  int rc = launch_kernel(k_ssd_chunk_mma, grid_c, dim3(MNT), 0, stream, a, ws);
  if (rc != GDN_OK) return rc;
  rc = launch_kernel(k_ssd_state<MP, MN>, dim3(MP * MN / 4 / NT, (unsigned)l.H, (unsigned)l.n_seq),
                     dim3(NT), 0, stream, l.state, l.st_seq, ws, l.n_seq, l.H, nc);
  if (rc != GDN_OK) return rc;
  return launch_kernel(k_ssd_out_mma, grid_c, dim3(MNT), 0, stream, a,
                       static_cast<const float *>(ws));
}

}  // namespace

size_t ssd_workspace_bytes(int n_seq, int n_tok, int H, int P, int N) {
  const size_t nc = (size_t)((n_tok + SC - 1) / SC);
  const size_t units = (size_t)n_seq * H * nc;
  return units * (size_t)P * N * sizeof(float) + ((units * sizeof(float) + 255) & ~(size_t)255);
}

int launch_ssd(const SsdLaunch &l, hipStream_t stream) {
  if (l.P == 64 && l.N == 128) return run_ssd_mma(l, stream);
  if (l.P == 64 && l.N == 64) return run_ssd<64, 64>(l, stream);
  if (l.P == 32 && l.N == 128) return run_ssd<32, 128>(l, stream);
  if (l.P == 32 && l.N == 64) return run_ssd<32, 64>(l, stream);
  return GDN_ERR_UNSUPPORTED;
}

}  // namespace gdn
