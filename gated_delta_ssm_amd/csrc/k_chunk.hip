// k_chunk.hip -- chunked (WY / UT-transform) prefill form of the gated
// delta-rule recurrence, for S = 128 and chunks of 64 positions.
//
// The pages state the chunked idea (ssm_mamba.rs, spark_model, "Mamba-2 SSD
// chunked prefill scan" comment: ceil(T/64) sequential links instead of T) and
// that the sequential scan is its correctness reference (fm_kernel_ssm.h,
// Foundry, fm_ssm_recurrence_seq_at).  The algebra is derived from the
// sequential definition.  For a chunk of n <= 64 positions starting from
// state S0 (S[i][j], i key, j value), with G_t the inclusive cumulative sum of
// g inside the chunk:
//   A  = strictly_lower(beta_t e^{G_t-G_s} k_t.k_s),  T = (I + A)^{-1}
//   W  = T diag(beta e^G) K           Ut = T diag(beta) V
//   L  = lower(e^{G_t-G_s})  (diagonal included)
//   Q' = diag(e^G) Q - (L o Q K^T) W  Oi = (L o Q K^T) Ut
//   U  = Ut - W S0,   y = scale (Q' S0 + Oi),   S = e^{G_n} S0 + K'^T U,
//   K' = diag(e^{G_n-G}) K.
// Only the last three lines depend on S0, so the work splits in two kernels:
//
//   k_chunk_prep (phase A) -- one workgroup per (sequence, head, chunk), all
//     in parallel: everything that does not depend on S0, written to the
//     workspace (W, Q', K'^T as bf16 hi/lo planes; Ut^T, Oi^T in fp32; e^{G_n}).
//   k_chunk_scan (phase B) -- one workgroup per (sequence, head, block of 16
//     value columns), walking the chunks in order: the value columns of S are
//     independent, so 8 workgroups share a head.  Each of its 4 waves owns 32
//     key rows of the state block as MFMA accumulators; per chunk it computes
//     16 rows of U and y and its 32 state rows.
//
// Precision: every contraction runs on MFMA v_mfma_f32_16x16x32_bf16 with each
// fp32 operand split into bf16 hi + lo, accumulating hi*hi + hi*lo + lo*hi in
// fp32 (relative error ~2^-16 per product instead of bf16's 2^-8).  The
// triangular inverse, the gate cumsum, every exponential and the state carry
// are fp32.  Exponentials are only taken of non-positive arguments (masked
// before the exp), so g must be <= 0, which the decay gate guarantees.
//
// MFMA operand layout (16x16x32 bf16, wave64): lane l holds row (l % 16) of
// A / column (l % 16) of B, with k = 8*(l / 16) + e, e = 0..7, so every
// operand is stored k-contiguous ([row][k]) and one fragment is one 16-byte
// load per plane.  The accumulator holds D[4*(l/16) + r][l % 16], r = 0..3.
#include <hip/hip_runtime.h>

#include "gdn.h"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int CH = 64;           // positions per chunk
constexpr int DK = 128;          // key dimension (state rows)
constexpr int DV = 128;          // value dimension (state columns)
constexpr int NBLK = 16;         // value columns per scan workgroup
constexpr int NVB = DV / NBLK;   // scan workgroups per head

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

struct Frag {
  bf16x8 hi, lo;
};

__device__ __forceinline__ u16 bf16_bits(float x) {
  return __builtin_bit_cast(u16, (__bf16)x);  // round to nearest even (v_cvt_pk_bf16_f32)
}
__device__ __forceinline__ float bf16_value(u16 b) {
  return __builtin_bit_cast(float, (unsigned)b << 16);
}
// x = hi + lo + O(2^-16 |x|); x - hi is exact in fp32.
__device__ __forceinline__ void split(float x, u16 &hi, u16 &lo) {
  hi = bf16_bits(x);
  lo = bf16_bits(x - bf16_value(hi));
}

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// c += a*b with both operands split: hi*hi + hi*lo + lo*hi.
__device__ __forceinline__ f32x4 mfma3(const Frag &a, const Frag &b, f32x4 c) {
  c = mfma(a.lo, b.hi, c);
  c = mfma(a.hi, b.lo, c);
  c = mfma(a.hi, b.hi, c);
  return c;
}

// Fragment rows [row][k..k+7] of a pair of k-contiguous bf16 planes.
__device__ __forceinline__ Frag frag(const u16 *hi, const u16 *lo, int pitch, int row, int k) {
  Frag f;
  f.hi = *reinterpret_cast<const bf16x8 *>(hi + row * pitch + k);
  f.lo = *reinterpret_cast<const bf16x8 *>(lo + row * pitch + k);
  return f;
}

// Split 4 floats and store them as 4 consecutive bf16 in each plane.
__device__ __forceinline__ void store4_split(u16 *hi, u16 *lo, float a, float b, float c, float d) {
  u16 h[4], l[4];
  split(a, h[0], l[0]);
  split(b, h[1], l[1]);
  split(c, h[2], l[2]);
  split(d, h[3], l[3]);
  *reinterpret_cast<uint2 *>(hi) =
      make_uint2(h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16));
  *reinterpret_cast<uint2 *>(lo) =
      make_uint2(l[0] | ((unsigned)l[1] << 16), l[2] | ((unsigned)l[3] << 16));
}

// Split 8 floats into one 16-byte store per plane.
__device__ __forceinline__ void store8_split(u16 *hi, u16 *lo, const float (&x)[8]) {
  unsigned h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    u16 h0, l0, h1, l1;
    split(x[2 * e], h0, l0);
    split(x[2 * e + 1], h1, l1);
    h[e] = h0 | ((unsigned)h1 << 16);
    l[e] = l0 | ((unsigned)l1 << 16);
  }
  *reinterpret_cast<uint4 *>(hi) = make_uint4(h[0], h[1], h[2], h[3]);
  *reinterpret_cast<uint4 *>(lo) = make_uint4(l[0], l[1], l[2], l[3]);
}

// ----------------------------------------------------------------------------- workspace
// Per (sequence, head, chunk), all offsets in bytes, each region 256-aligned.
constexpr size_t WS_PLANE = (size_t)CH * DK * 2;        // one bf16 plane of a 64x128 matrix
constexpr size_t WS_W = 0;                              // W  [t][i]  hi, lo
constexpr size_t WS_Q = 2 * WS_PLANE;                   // Q' [t][i]  hi, lo
constexpr size_t WS_K = 4 * WS_PLANE;                   // K'^T [i][t] hi, lo
constexpr size_t WS_U = 6 * WS_PLANE;                   // Ut^T [j][t] fp32
constexpr size_t WS_O = WS_U + (size_t)DV * CH * 4;     // Oi^T [j][t] fp32
constexpr size_t WS_G = WS_O + (size_t)DV * CH * 4;     // e^{G_n}
constexpr size_t WS_CHUNK = WS_G + 256;

// ----------------------------------------------------------------------------- phase A
// LDS plan (bytes).  R1/R2 hold, in turn: K/Q rows; X^T = (beta e^G K)^T and
// (beta V)^T; W^T and Ut^T.  R3 holds A (fp32) then T (bf16 hi/lo); R4 holds T
// in fp32 while it is built; R3+R4 then stage W and Q' for coalesced stores.
constexpr int P136 = 136;  // pitch (bf16) of a [64][128] matrix
constexpr int P72 = 72;    // pitch (bf16) of a [..][64] matrix
constexpr int PF = 65;     // pitch (fp32) of a [64][64] matrix
constexpr int L_R1 = 0;
constexpr int L_R2 = L_R1 + 2 * DK * P72 * 2;           // 36864
constexpr int L_R3 = L_R2 + 2 * DK * P72 * 2;           // 73728
constexpr int L_R4 = L_R3 + 2 * CH * P72 * 2;           // +18432
constexpr int L_R5 = L_R4 + CH * PF * 4;                // +16640
constexpr int L_R6 = L_R5 + 2 * CH * P72 * 2;           // +18432
constexpr int L_R7 = L_R6 + 3 * 16 * 16 * 4;            // +3072
constexpr int L_TOTAL = L_R7 + 4 * CH * 4;              // +1024
static_assert(2 * CH * P136 * 2 <= L_R2 - L_R1, "K/Q rows fit in R1/R2");
static_assert(2 * CH * P136 * 2 <= L_R5 - L_R3, "staging fits in R3+R4");
static_assert(CH * PF * 4 <= L_R4 - L_R3, "fp32 A fits in R3");

__global__ __launch_bounds__(256) void k_chunk_prep(
    const float *__restrict__ q, const float *__restrict__ k, int64_t qk_tok, int64_t qk_seq,
    const float *__restrict__ v, int64_t v_tok, int64_t v_seq, const float *__restrict__ g,
    const float *__restrict__ beta, unsigned char *__restrict__ ws, int n_tok, int n_chunks,
    int H, int Hk) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[L_TOTAL];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
  const int c = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int hk = h / (H / Hk);
  const int t0 = c * CH;
  const int n = min(CH, n_tok - t0);

  u16 *r1h = reinterpret_cast<u16 *>(smem + L_R1), *r1l = r1h + DK * P72;
  u16 *r2h = reinterpret_cast<u16 *>(smem + L_R2), *r2l = r2h + DK * P72;
  float *sA = reinterpret_cast<float *>(smem + L_R3);
  u16 *r3h = reinterpret_cast<u16 *>(smem + L_R3), *r3l = r3h + CH * P72;
  float *sT = reinterpret_cast<float *>(smem + L_R4);
  u16 *sth = reinterpret_cast<u16 *>(smem + L_R3), *stl = sth + CH * P136;  // staging
  u16 *r5h = reinterpret_cast<u16 *>(smem + L_R5), *r5l = r5h + CH * P72;
  float *scratch = reinterpret_cast<float *>(smem + L_R6);
  float *sG = reinterpret_cast<float *>(smem + L_R7);
  float *sBeta = sG + CH, *sEG = sG + 2 * CH, *sEGn = sG + 3 * CH;

  const float *kc = k + s * qk_seq + (int64_t)t0 * qk_tok + hk * DK;
  const float *qc = q + s * qk_seq + (int64_t)t0 * qk_tok + hk * DK;
  const float *vc = v + s * v_seq + (int64_t)t0 * v_tok + h * DV;
  unsigned char *wc = ws + (((size_t)s * H + h) * n_chunks + c) * WS_CHUNK;

  // 1. gate cumsum (wave 0), beta
  // Loads past the last position read a valid position and are zeroed by a
  // select, so no load sits behind a branch (a branch would force the compiler
  // to wait for every outstanding load at the join).
  if (w == 0) {
    const int64_t gi = ((int64_t)s * n_tok + t0 + min(lane, n - 1)) * H + h;
    const float gv = g[gi], bv = beta[gi];
    float x = lane < n ? gv : 0.0f;
    const float b = lane < n ? bv : 0.0f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    const float gn = __shfl(x, 63, 64);
    sG[lane] = x;
    sBeta[lane] = b;
    sEG[lane] = expf(x);
    sEGn[lane] = expf(gn - x);
  }
  // 2. K, Q rows -> R1, R2 (bf16 hi/lo, [t][i])
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int idx = it * 256 + tid, row = idx >> 5, col = (idx & 31) * 4;
    const int rr = min(row, n - 1);
    float4 kv = *reinterpret_cast<const float4 *>(kc + (int64_t)rr * qk_tok + col);
    float4 qv = *reinterpret_cast<const float4 *>(qc + (int64_t)rr * qk_tok + col);
    if (row >= n) kv = qv = make_float4(0.f, 0.f, 0.f, 0.f);
    store4_split(r1h + row * P136 + col, r1l + row * P136 + col, kv.x, kv.y, kv.z, kv.w);
    store4_split(r2h + row * P136 + col, r2l + row * P136 + col, qv.x, qv.y, qv.z, qv.w);
  }
  __syncthreads();

  // 3. K K^T and Q K^T, lower tiles; wave w owns tile row w
  for (int j = 0; j < 4; ++j) {
    if (j <= w) {
      f32x4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = akk;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const Frag fk = frag(r1h, r1l, P136, 16 * w + l16, 32 * ks + 8 * kg);
        const Frag fq = frag(r2h, r2l, P136, 16 * w + l16, 32 * ks + 8 * kg);
        const Frag fb = frag(r1h, r1l, P136, 16 * j + l16, 32 * ks + 8 * kg);
        akk = mfma3(fk, fb, akk);
        aqk = mfma3(fq, fb, aqk);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * w + 4 * kg + r, sidx = 16 * j + l16;
        const float e = sidx <= t ? expf(sG[t] - sG[sidx]) : 0.0f;
        sA[t * PF + sidx] = sidx < t ? sBeta[t] * e * akk[r] : 0.0f;
        u16 hh, ll;
        split(e * aqk[r], hh, ll);
        r5h[t * P72 + sidx] = hh;
        r5l[t * P72 + sidx] = ll;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * w + 4 * kg + r, sidx = 16 * j + l16;
        sA[t * PF + sidx] = 0.0f;
        r5h[t * P72 + sidx] = 0;
        r5l[t * P72 + sidx] = 0;
      }
    }
  }
  // zero the fp32 inverse buffer
  for (int e = tid; e < CH * PF; e += 256) sT[e] = 0.0f;
  __syncthreads();

  // 4. R1 <- X^T = (beta e^G K)^T, R2 <- (beta V)^T, K'^T -> workspace;
  //    meanwhile threads 0..63 invert the four 16x16 diagonal blocks of I + A.
  if (tid < 64) {
    const int b = tid >> 4, cc = tid & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = r == cc ? 1.0f : 0.0f;
#pragma unroll
      for (int j = 0; j < r; ++j) acc -= sA[(16 * b + r) * PF + 16 * b + j] * x[j];
      x[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sT[(16 * b + r) * PF + 16 * b + cc] = x[r];
  }
  {
    u16 *kth = reinterpret_cast<u16 *>(wc + WS_K), *ktl = kth + DK * CH;
    for (int it = tid; it < DK * 8; it += 256) {
      const int i = it & (DK - 1), tg = it >> 7;
      float xk[8], xv[8], xkp[8], kl[8], vl[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = min(8 * tg + e, n - 1);
        kl[e] = kc[(int64_t)t * qk_tok + i];
        vl[e] = vc[(int64_t)t * v_tok + i];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = 8 * tg + e;
        const float kk = t < n ? kl[e] : 0.0f;
        const float vv = t < n ? vl[e] : 0.0f;
        xk[e] = sBeta[t] * sEG[t] * kk;
        xv[e] = sBeta[t] * vv;
        xkp[e] = sEGn[t] * kk;
      }
      store8_split(r1h + i * P72 + 8 * tg, r1l + i * P72 + 8 * tg, xk);
      store8_split(r2h + i * P72 + 8 * tg, r2l + i * P72 + 8 * tg, xv);
      store8_split(kth + i * CH + 8 * tg, ktl + i * CH + 8 * tg, xkp);
    }
  }
  __syncthreads();
  // off-diagonal blocks: T_ib,jb = -T_ib,ib * sum_{kb=jb}^{ib-1} A_ib,kb T_kb,jb
  for (int ib = 1; ib < 4; ++ib) {
    for (int e = tid; e < ib * 256; e += 256) {
      const int jb = e >> 8, r = (e >> 4) & 15, cc = e & 15;
      float acc = 0.0f;
      for (int kb = jb; kb < ib; ++kb)
#pragma unroll
        for (int m = 0; m < 16; ++m)
          acc += sA[(16 * ib + r) * PF + 16 * kb + m] * sT[(16 * kb + m) * PF + 16 * jb + cc];
      scratch[e] = acc;
    }
    __syncthreads();
    for (int e = tid; e < ib * 256; e += 256) {
      const int jb = e >> 8, r = (e >> 4) & 15, cc = e & 15;
      float acc = 0.0f;
#pragma unroll
      for (int m = 0; m < 16; ++m)
        acc += sT[(16 * ib + r) * PF + 16 * ib + m] * scratch[(jb << 8) + (m << 4) + cc];
      sT[(16 * ib + r) * PF + 16 * jb + cc] = -acc;
    }
    __syncthreads();
  }
  // T (fp32) -> R3 as bf16 hi/lo [t][s]
  for (int it = tid; it < CH * 8; it += 256) {
    const int row = it >> 3, cg = (it & 7) * 8;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = sT[row * PF + cg + e];
    store8_split(r3h + row * P72 + cg, r3l + row * P72 + cg, x);
  }
  __syncthreads();

  // 5. W = T X and Ut = T (beta V): wave w -> rows 16w..16w+15, all 128 columns
  f32x4 accW[8], accU[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    accW[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    accU[nt] = accW[nt];
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const Frag ft = frag(r3h, r3l, P72, 16 * w + l16, 32 * ks + 8 * kg);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      accW[nt] = mfma3(ft, frag(r1h, r1l, P72, 16 * nt + l16, 32 * ks + 8 * kg), accW[nt]);
      accU[nt] = mfma3(ft, frag(r2h, r2l, P72, 16 * nt + l16, 32 * ks + 8 * kg), accU[nt]);
    }
  }
  __syncthreads();  // R1, R2, R3 are rewritten below
  {
    float *utg = reinterpret_cast<float *>(wc + WS_U);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int col = 16 * nt + l16, t = 16 * w + 4 * kg;
      store4_split(r1h + col * P72 + t, r1l + col * P72 + t, accW[nt][0], accW[nt][1],
                   accW[nt][2], accW[nt][3]);
      store4_split(r2h + col * P72 + t, r2l + col * P72 + t, accU[nt][0], accU[nt][1],
                   accU[nt][2], accU[nt][3]);
      *reinterpret_cast<float4 *>(utg + col * CH + t) =
          make_float4(accU[nt][0], accU[nt][1], accU[nt][2], accU[nt][3]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u16 hh, ll;
        split(accW[nt][r], hh, ll);
        sth[(t + r) * P136 + col] = hh;
        stl[(t + r) * P136 + col] = ll;
      }
    }
  }
  __syncthreads();
  {  // staged W -> workspace, 16 bytes per thread per step
    u16 *wg = reinterpret_cast<u16 *>(wc + WS_W);
    for (int it = tid; it < 2 * CH * 16; it += 256) {
      const int plane = it >> 10, row = (it >> 4) & 63, c16 = (it & 15) * 8;
      const u16 *src = (plane ? stl : sth) + row * P136 + c16;
      *reinterpret_cast<uint4 *>(wg + plane * CH * DK + row * DK + c16) =
          *reinterpret_cast<const uint4 *>(src);
    }
  }

  // 6. Q' = e^G Q - (L o QK^T) W and Oi = (L o QK^T) Ut
  f32x4 accQ[8], accO[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    accQ[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    accO[nt] = accQ[nt];
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const Frag fl = frag(r5h, r5l, P72, 16 * w + l16, 32 * ks + 8 * kg);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      accQ[nt] = mfma3(fl, frag(r1h, r1l, P72, 16 * nt + l16, 32 * ks + 8 * kg), accQ[nt]);
      accO[nt] = mfma3(fl, frag(r2h, r2l, P72, 16 * nt + l16, 32 * ks + 8 * kg), accO[nt]);
    }
  }
  __syncthreads();  // staging reads of W are done before Q' overwrites it
  {
    float *oig = reinterpret_cast<float *>(wc + WS_O);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int col = 16 * nt + l16, t = 16 * w + 4 * kg;
      *reinterpret_cast<float4 *>(oig + col * CH + t) =
          make_float4(accO[nt][0], accO[nt][1], accO[nt][2], accO[nt][3]);
      float ql[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ql[r] = qc[(int64_t)min(t + r, n - 1) * qk_tok + col];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float qv = (t + r) < n ? ql[r] : 0.0f;
        u16 hh, ll;
        split(sEG[t + r] * qv - accQ[nt][r], hh, ll);
        sth[(t + r) * P136 + col] = hh;
        stl[(t + r) * P136 + col] = ll;
      }
    }
  }
  __syncthreads();
  {
    u16 *qg = reinterpret_cast<u16 *>(wc + WS_Q);
    for (int it = tid; it < 2 * CH * 16; it += 256) {
      const int plane = it >> 10, row = (it >> 4) & 63, c16 = (it & 15) * 8;
      const u16 *src = (plane ? stl : sth) + row * P136 + c16;
      *reinterpret_cast<uint4 *>(qg + plane * CH * DK + row * DK + c16) =
          *reinterpret_cast<const uint4 *>(src);
    }
  }
  if (tid == 0) *reinterpret_cast<float *>(wc + WS_G) = sEG[CH - 1];
}

// ----------------------------------------------------------------------------- phase B
struct ChunkOps {
  Frag w[4], q[4], k[2][2];
  float4 ut, oi;
  float gam;
};

__device__ __forceinline__ void load_chunk(ChunkOps &o, const unsigned char *wc, int w, int l16,
                                           int kg, int blk) {
  const u16 *wh = reinterpret_cast<const u16 *>(wc + WS_W), *wl = wh + CH * DK;
  const u16 *qh = reinterpret_cast<const u16 *>(wc + WS_Q), *ql = qh + CH * DK;
  const u16 *kh = reinterpret_cast<const u16 *>(wc + WS_K), *kl = kh + DK * CH;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    o.w[ks] = frag(wh, wl, DK, 16 * w + l16, 32 * ks + 8 * kg);
    o.q[ks] = frag(qh, ql, DK, 16 * w + l16, 32 * ks + 8 * kg);
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      o.k[mt][ks] = frag(kh, kl, CH, 32 * w + 16 * mt + l16, 32 * ks + 8 * kg);
  const int j = blk * NBLK + l16, t = 16 * w + 4 * kg;
  o.ut = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(wc + WS_U) + j * CH + t);
  o.oi = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(wc + WS_O) + j * CH + t);
  o.gam = *reinterpret_cast<const float *>(wc + WS_G);
}

constexpr int SP = DK + 8;     // pitch of the S^T block in LDS (bf16)
constexpr int UP = CH + 8;     // pitch of the U^T block in LDS (bf16)

// One chunk of the scan for this wave: state rows 32w..32w+31 (two 16-row
// tiles) of the 16-column block in `st`; U and y rows 16w..16w+15.
__device__ __forceinline__ void scan_chunk(const ChunkOps &o, f32x4 (&st)[2], u16 *ssh,
                                           u16 *ssl, u16 *suh, u16 *sul, float *yc,
                                           int64_t y_tok, int n, float scale, int w, int l16,
                                           int kg) {
  // state block -> LDS as S^T [j][i] hi/lo (the B operand of W S and Q' S)
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int i = 32 * w + 16 * mt + 4 * kg;
    store4_split(ssh + l16 * SP + i, ssl + l16 * SP + i, st[mt][0], st[mt][1], st[mt][2],
                 st[mt][3]);
  }
  __syncthreads();
  f32x4 p = {0.f, 0.f, 0.f, 0.f}, rr = p;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const Frag b = frag(ssh, ssl, SP, l16, 32 * ks + 8 * kg);
    p = mfma3(o.w[ks], b, p);
    rr = mfma3(o.q[ks], b, rr);
  }
  // U = Ut - W S;  y = scale (Q' S + Oi)
  const float u0 = o.ut.x - p[0], u1 = o.ut.y - p[1], u2 = o.ut.z - p[2], u3 = o.ut.w - p[3];
  const int t = 16 * w + 4 * kg;
  const float yo[4] = {scale * (rr[0] + o.oi.x), scale * (rr[1] + o.oi.y),
                       scale * (rr[2] + o.oi.z), scale * (rr[3] + o.oi.w)};
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (t + r < n) yc[(int64_t)(t + r) * y_tok] = yo[r];
  store4_split(suh + l16 * UP + t, sul + l16 * UP + t, u0, u1, u2, u3);
  __syncthreads();
  // S = e^{G_n} S + K'^T U
  Frag bu[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) bu[ks] = frag(suh, sul, UP, l16, 32 * ks + 8 * kg);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    st[mt] = st[mt] * o.gam;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) st[mt] = mfma3(o.k[mt][ks], bu[ks], st[mt]);
  }
}

__global__ __launch_bounds__(256) void k_chunk_scan(
    float *__restrict__ state, int64_t st_seq, const unsigned char *__restrict__ ws,
    float *__restrict__ y, int64_t y_tok, int64_t y_seq, int n_tok, int n_chunks, int H,
    float scale) {
  __shared__ __attribute__((aligned(16))) u16 ssh[NBLK * SP], ssl[NBLK * SP];
  __shared__ __attribute__((aligned(16))) u16 suh[NBLK * UP], sul[NBLK * UP];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
  // XCD-aware order: consecutive workgroup ids go to different XCDs, so map
  // them so that the 8 blocks of one head land on the same XCD (shared L2).
  const int nwg = gridDim.x, per_xcd = nwg / 8;
  const int unit = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const int blk = unit % NVB, sh = unit / NVB, h = sh % H, s = sh / H;

  float *sp = state + s * st_seq + (int64_t)h * DK * DV + (int64_t)(blk * NBLK + l16) * DK;
  f32x4 st[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const float4 t4 = *reinterpret_cast<const float4 *>(sp + 32 * w + 16 * mt + 4 * kg);
    st[mt] = f32x4{t4.x, t4.y, t4.z, t4.w};
  }
  const unsigned char *wh = ws + ((size_t)s * H + h) * n_chunks * WS_CHUNK;
  float *yh = y + s * y_seq + (int64_t)h * DV + blk * NBLK + l16;

  ChunkOps a, b;
  load_chunk(a, wh, w, l16, kg, blk);
  int c = 0;
  for (; c + 1 < n_chunks; c += 2) {
    load_chunk(b, wh + (size_t)(c + 1) * WS_CHUNK, w, l16, kg, blk);
    scan_chunk(a, st, ssh, ssl, suh, sul, yh + (int64_t)c * CH * y_tok, y_tok,
               min(CH, n_tok - c * CH), scale, w, l16, kg);
    // always issue the prefetch (the last one re-reads a valid chunk): a
    // conditional load would make the compiler wait for every load in flight
    load_chunk(a, wh + (size_t)min(c + 2, n_chunks - 1) * WS_CHUNK, w, l16, kg, blk);
    scan_chunk(b, st, ssh, ssl, suh, sul, yh + (int64_t)(c + 1) * CH * y_tok, y_tok,
               min(CH, n_tok - (c + 1) * CH), scale, w, l16, kg);
  }
  if (c < n_chunks)
    scan_chunk(a, st, ssh, ssl, suh, sul, yh + (int64_t)c * CH * y_tok, y_tok,
               min(CH, n_tok - c * CH), scale, w, l16, kg);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
    *reinterpret_cast<float4 *>(sp + 32 * w + 16 * mt + 4 * kg) =
        make_float4(st[mt][0], st[mt][1], st[mt][2], st[mt][3]);
}

}  // namespace

size_t chunked_workspace_bytes(int n_seq, int n_tok, int H, int, int, int) {
  const size_t n_chunks = ((size_t)n_tok + CH - 1) / CH;
  return (size_t)n_seq * H * n_chunks * WS_CHUNK;
}

int launch_recur_chunked(const RecurArgs &a, int chunk, void *ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (chunk != CH || a.S != DK) return GDN_ERR_UNSUPPORTED;
  const int n_chunks = (a.n_tok + CH - 1) / CH;
  if (ws_bytes < chunked_workspace_bytes(a.n_seq, a.n_tok, a.H, a.Hk, a.S, chunk))
    return GDN_ERR_WORKSPACE;
  unsigned char *wsb = static_cast<unsigned char *>(ws);
  int rc = launch_kernel(k_chunk_prep, dim3(n_chunks, a.H, a.n_seq), dim3(256), 0, stream, a.q,
                         a.k, a.qk_tok, a.qk_seq, a.v, a.v_tok, a.v_seq, a.g, a.beta, wsb,
                         a.n_tok, n_chunks, a.H, a.Hk);
  if (rc != GDN_OK) return rc;
  const int nwg = a.n_seq * a.H * NVB;  // a multiple of 8 (NVB == 8)
  return launch_kernel(k_chunk_scan, dim3(nwg), dim3(256), 0, stream, a.state, a.st_seq,
                       (const unsigned char *)wsb, a.y, a.y_tok, a.y_seq, a.n_tok, n_chunks, a.H,
                       a.scale);
}

}  // namespace gdn
