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
//     independent, so 8 workgroups share a head.  Each of its 8 waves owns 16
//     key rows of the state block as an MFMA accumulator and one 16-token tile
//     of either U or y; operands are prefetched two chunks ahead.
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
// The three MFMA A operands of the scan are stored fragment-major: fragment
// (row tile m, k-step ks, plane) is 64 lanes x 16 bytes, lane (kg, l16)
// holding row 16m + l16, columns 32ks + 8kg .. +7, so each wave load in the
// scan is 1 KiB of consecutive bytes.  Ut and Oi are stored in the
// accumulator layout [column tile][token tile][lane][4], which is the same lane
// map on the writing and the reading side.
constexpr size_t WS_PLANE = (size_t)CH * DK * 2;        // one bf16 plane of a 64x128 matrix
constexpr size_t WS_W = 0;                              // W   (4 row tiles x 4 k-steps) hi, lo
constexpr size_t WS_Q = 2 * WS_PLANE;                   // Q'  (4 x 4) hi, lo
constexpr size_t WS_K = 4 * WS_PLANE;                   // K'^T (8 row tiles x 2 k-steps) hi, lo
constexpr size_t WS_U = 6 * WS_PLANE;                   // Ut  fp32, accumulator layout
constexpr size_t WS_O = WS_U + (size_t)DV * CH * 4;     // Oi  fp32, accumulator layout
constexpr size_t WS_G = WS_O + (size_t)DV * CH * 4;     // e^{G_n}
constexpr size_t WS_CHUNK = WS_G + 256;

// u16 offset of a fragment's 8 elements for lane `lane`
__device__ __forceinline__ int frag_off(int m, int ks, int n_ks, int plane, int lane) {
  return (((m * n_ks + ks) * 2 + plane) * 64 + lane) * 8;
}
__device__ __forceinline__ Frag frag_ws(const u16 *base, int m, int ks, int n_ks, int lane) {
  Frag f;
  f.hi = *reinterpret_cast<const bf16x8 *>(base + frag_off(m, ks, n_ks, 0, lane));
  f.lo = *reinterpret_cast<const bf16x8 *>(base + frag_off(m, ks, n_ks, 1, lane));
  return f;
}
// float offset of the 4 accumulator values of (column tile nt, token tile mt, lane)
__device__ __forceinline__ int acc_off(int nt, int mt, int lane) {
  return ((nt * 4 + mt) * 64 + lane) * 4;
}

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
  // n == 0 for a padding chunk (an even chunk count keeps the scan's
  // two-deep operand pipeline free of a tail): it yields e^{G_n} = 1 and
  // all-zero operands, which leaves the state unchanged.
  const int n = max(0, min(CH, n_tok - t0));
  const int nl = max(n - 1, 0);  // last valid position, clamped for the loads

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

  const int tb = min(t0, n_tok - 1);  // base position of the loads (valid for padding)
  const float *kc = k + s * qk_seq + (int64_t)tb * qk_tok + hk * DK;
  const float *qc = q + s * qk_seq + (int64_t)tb * qk_tok + hk * DK;
  const float *vc = v + s * v_seq + (int64_t)tb * v_tok + h * DV;
  unsigned char *wc = ws + (((size_t)s * H + h) * n_chunks + c) * WS_CHUNK;

  // 1. gate cumsum (wave 0), beta
  // Loads past the last position read a valid position and are zeroed by a
  // select, so no load sits behind a branch (a branch would force the compiler
  // to wait for every outstanding load at the join).
  if (w == 0) {
    const int64_t gi = ((int64_t)s * n_tok + min(t0 + min(lane, nl), n_tok - 1)) * H + h;
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
    const int rr = min(row, nl);
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
    u16 *ktg = reinterpret_cast<u16 *>(wc + WS_K);
    for (int it = tid; it < DK * 8; it += 256) {
      const int i = it & (DK - 1), tg = it >> 7;
      float xk[8], xv[8], xkp[8], kl[8], vl[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = min(8 * tg + e, nl);
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
      const int kl_lane = (tg & 3) * 16 + (i & 15);
      store8_split(ktg + frag_off(i >> 4, tg >> 2, 2, 0, kl_lane),
                   ktg + frag_off(i >> 4, tg >> 2, 2, 1, kl_lane), xkp);
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
      *reinterpret_cast<float4 *>(utg + acc_off(nt, w, lane)) =
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
  {  // staged W -> workspace in fragment order, 16 bytes per thread per step
    u16 *wg = reinterpret_cast<u16 *>(wc + WS_W);
    for (int it = tid; it < 4 * 4 * 2 * 64; it += 256) {
      const int ln = it & 63, plane = (it >> 6) & 1, ks = (it >> 7) & 3, m = it >> 9;
      const u16 *src = (plane ? stl : sth) + (16 * m + (ln & 15)) * P136 + 32 * ks + 8 * (ln >> 4);
      *reinterpret_cast<uint4 *>(wg + frag_off(m, ks, 4, plane, ln)) =
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
      *reinterpret_cast<float4 *>(oig + acc_off(nt, w, lane)) =
          make_float4(accO[nt][0], accO[nt][1], accO[nt][2], accO[nt][3]);
      float ql[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ql[r] = qc[(int64_t)min(t + r, nl) * qk_tok + col];
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
  {  // staged Q' -> workspace in fragment order, 16 bytes per thread per step
    u16 *qg = reinterpret_cast<u16 *>(wc + WS_Q);
    for (int it = tid; it < 4 * 4 * 2 * 64; it += 256) {
      const int ln = it & 63, plane = (it >> 6) & 1, ks = (it >> 7) & 3, m = it >> 9;
      const u16 *src = (plane ? stl : sth) + (16 * m + (ln & 15)) * P136 + 32 * ks + 8 * (ln >> 4);
      *reinterpret_cast<uint4 *>(qg + frag_off(m, ks, 4, plane, ln)) =
          *reinterpret_cast<const uint4 *>(src);
    }
  }
  if (tid == 0) *reinterpret_cast<float *>(wc + WS_G) = sEG[CH - 1];
}

// ----------------------------------------------------------------------------- phase B
// Eight waves per workgroup.  Wave w computes, per chunk:
//   w < 4 : P = W S for token rows 16(w&3)..+15, then U = Ut - P  (shared via LDS)
//   w >= 4: R = Q' S for token rows 16(w&3)..+15, then y = scale (R + Oi)
//   all   : state rows 16w..16w+15 of the block, S <- e^{G_n} S + K'^T U.
// Each wave's operands for one chunk are ~52 VGPRs; two chunks are kept in
// flight (prefetch distance 2).
struct ChunkOps {
  Frag a[4];      // W or Q' rows of this wave; slot j = k-step (j + blk) mod 4 over keys
  Frag k[2];      // K'^T rows 16w..; slot j = k-step (j + blk) mod 2 over tokens
  float4 add;     // Ut (P waves) or Oi (R waves) for this lane's 4 tokens
  float gam;      // e^{G_n}
};

__device__ __forceinline__ void load_chunk(ChunkOps &o, const unsigned char *wc, int w, int l16,
                                           int kg, int blk) {
  const bool pw = w < 4;
  const int lane = kg * 16 + l16;
  const u16 *ag = reinterpret_cast<const u16 *>(wc + (pw ? WS_W : WS_Q));
  const u16 *kgp = reinterpret_cast<const u16 *>(wc + WS_K);
  // The 8 workgroups of a head read the same lines at about the same time;
  // slot j holds k-step (j + blk) mod n, so their requests start on different
  // lines.  The scan pairs each slot with the matching B fragment.
#pragma unroll
  for (int j = 0; j < 4; ++j) o.a[j] = frag_ws(ag, w & 3, (j + blk) & 3, 4, lane);
#pragma unroll
  for (int j = 0; j < 2; ++j) o.k[j] = frag_ws(kgp, w, (j + blk) & 1, 2, lane);
  const float *addp = reinterpret_cast<const float *>(wc + (pw ? WS_U : WS_O));
  o.add = *reinterpret_cast<const float4 *>(addp + acc_off(blk, w & 3, lane));
  o.gam = *reinterpret_cast<const float *>(wc + WS_G);
}

constexpr int SP = DK + 8;     // pitch of the S^T block in LDS (bf16)
constexpr int UP = CH + 8;     // pitch of the U^T block in LDS (bf16)

__device__ __forceinline__ void scan_chunk(const ChunkOps &o, f32x4 &st, u16 *ssh, u16 *ssl,
                                           u16 *suh, u16 *sul, float *yc, int64_t y_tok, int n,
                                           float scale, int w, int l16, int kg, int rot) {
  // state tile -> LDS as S^T [j][i] (the B operand of W S and Q' S)
  store4_split(ssh + l16 * SP + 16 * w + 4 * kg, ssl + l16 * SP + 16 * w + 4 * kg, st[0], st[1],
               st[2], st[3]);
  __syncthreads();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = mfma3(o.a[j], frag(ssh, ssl, SP, l16, 32 * ((j + rot) & 3) + 8 * kg), acc);
  const int t = 16 * (w & 3) + 4 * kg;
  if (w < 4) {
    store4_split(suh + l16 * UP + t, sul + l16 * UP + t, o.add.x - acc[0], o.add.y - acc[1],
                 o.add.z - acc[2], o.add.w - acc[3]);
  } else {
    const float yo[4] = {scale * (acc[0] + o.add.x), scale * (acc[1] + o.add.y),
                         scale * (acc[2] + o.add.z), scale * (acc[3] + o.add.w)};
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (t + r < n) yc[(int64_t)(t + r) * y_tok] = yo[r];
  }
  __syncthreads();
  st = st * o.gam;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    st = mfma3(o.k[j], frag(suh, sul, UP, l16, 32 * ((j + rot) & 1) + 8 * kg), st);
}

__global__ __launch_bounds__(512) void k_chunk_scan(
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

  // state rows 16w + 4kg + r, column blk*16 + l16 (value-major storage)
  float *sp = state + s * st_seq + (int64_t)h * DK * DV + (int64_t)(blk * NBLK + l16) * DK +
              16 * w + 4 * kg;
  const float4 s4 = *reinterpret_cast<const float4 *>(sp);
  f32x4 st = {s4.x, s4.y, s4.z, s4.w};
  const unsigned char *wh = ws + ((size_t)s * H + h) * n_chunks * WS_CHUNK;
  float *yh = y + s * y_seq + (int64_t)h * DV + blk * NBLK + l16;
  auto chunk_ptr = [&](int c) { return wh + (size_t)min(c, n_chunks - 1) * WS_CHUNK; };
  auto run = [&](const ChunkOps &o, int c) {
    scan_chunk(o, st, ssh, ssl, suh, sul, yh + (int64_t)c * CH * y_tok, y_tok,
               min(CH, n_tok - c * CH), scale, w, l16, kg, blk);
  };

  // Two chunks in flight: a chunk's operands are requested two chunks ahead.
  // n_chunks is even (the workspace is padded with an identity chunk), so the
  // loop has no tail; a tail would make the compiler copy the operand
  // registers at the loop head, which waits for every load in flight.
  ChunkOps a, b;
  load_chunk(a, chunk_ptr(0), w, l16, kg, blk);
  load_chunk(b, chunk_ptr(1), w, l16, kg, blk);
  for (int c = 0; c < n_chunks; c += 2) {
    run(a, c);
    load_chunk(a, chunk_ptr(c + 2), w, l16, kg, blk);
    run(b, c + 1);
    load_chunk(b, chunk_ptr(c + 3), w, l16, kg, blk);
  }
  *reinterpret_cast<float4 *>(sp) = make_float4(st[0], st[1], st[2], st[3]);
}

}  // namespace

// chunks per sequence in the workspace: ceil(n_tok / 64) rounded up to even
static int padded_chunks(int n_tok) { return ((n_tok + CH - 1) / CH + 1) & ~1; }

size_t chunked_workspace_bytes(int n_seq, int n_tok, int H, int, int, int) {
  return (size_t)n_seq * H * padded_chunks(n_tok) * WS_CHUNK;
}

int launch_recur_chunked(const RecurArgs &a, int chunk, void *ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (chunk != CH || a.S != DK) return GDN_ERR_UNSUPPORTED;
  const int n_chunks = padded_chunks(a.n_tok);
  if (ws_bytes < chunked_workspace_bytes(a.n_seq, a.n_tok, a.H, a.Hk, a.S, chunk))
    return GDN_ERR_WORKSPACE;
  unsigned char *wsb = static_cast<unsigned char *>(ws);
  int rc = launch_kernel(k_chunk_prep, dim3(n_chunks, a.H, a.n_seq), dim3(256), 0, stream, a.q,
                         a.k, a.qk_tok, a.qk_seq, a.v, a.v_tok, a.v_seq, a.g, a.beta, wsb,
                         a.n_tok, n_chunks, a.H, a.Hk);
  if (rc != GDN_OK) return rc;
  const int nwg = a.n_seq * a.H * NVB;  // a multiple of 8 (NVB == 8)
  return launch_kernel(k_chunk_scan, dim3(nwg), dim3(512), 0, stream, a.state, a.st_seq,
                       (const unsigned char *)wsb, a.y, a.y_tok, a.y_seq, a.n_tok, n_chunks, a.H,
                       a.scale);
}

}  // namespace gdn
