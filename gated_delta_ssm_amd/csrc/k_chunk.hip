// k_chunk.hip -- chunked (WY / UT-transform) prefill form of the gated
// delta-rule recurrence, for S = 128 and chunks of 64 positions (S = 32 and 64:
// k_chunk_small.hip).
//
// The pages state the chunked idea (ssm_mamba.rs, spark_model, "Mamba-2 SSD
// chunked prefill scan" comment: one dependent step per 64-position chunk
// rather than one per position) and
// that the sequential scan is its correctness reference (fm_kernel_ssm.h,
// Foundry, fm_ssm_recurrence_seq_at).  The algebra is derived from the
// sequential definition.  For a chunk of n <= 64 positions starting from
// state S0 (S[i][j], i key, j value), with G_t the inclusive cumulative sum of
// g inside the chunk:
//   A  = strictly_lower(beta_t e^{G_t-G_s} k_t.k_s),  T = (I + A)^{-1}
//   W  = T diag(beta e^G) K           Ut = T diag(beta) V
//   M  = lower(e^{G_t-G_s}) o Q K^T  (diagonal included)
//   U  = Ut - W S0
//   y  = scale (diag(e^G) Q S0 + M U)
//   S  = e^{G_n} S0 + K^T diag(e^{G_n-G}) U.
// (U is the chunk's block of sequential deltas beta_t (v_t - S_{t-1}^T k_t);
// y_t reads the state after position t, whose part from inside the chunk is
// the sum over s <= t of e^{G_t-G_s} k_s U_s^T.)  Only the last three lines
// depend on S0, so the work splits in two kernels:
//
//   k_chunk_prep (phase A) -- every (sequence, head, chunk) independently:
//     everything that does not depend on S0, written to a workspace in the
//     exact register layout the scan loads: W, M, Ut per value head; Q and K
//     per query/key head, written once and read by every value head of the
//     group.  Persistent: one workgroup per CU
//     walks its chunks, loading the next chunk while computing this one.  Its
//     K, Q, V and g come either as given (gdn_recurrence_chunked) or from the
//     layer's conv input and gate inputs (gdn_prefill_chunked: the decay gate
//     and the conv1d + SiLU + L2 of ssm_mamba.rs conv1d_update_prefill are
//     computed here, bit for bit as the gate and conv kernels compute them,
//     and never stored); the scan then also writes the conv history.
//   k_chunk_scan (phase B) -- one workgroup per (sequence, head, block of 16
//     value columns), walking the chunks in order: the value columns of S are
//     independent, so 8 workgroups share a head, and they are mapped to one
//     XCD so they share its L2.  A chunk's operands are requested while the
//     chunk before it runs.
//
// Precision: phase A's contractions run on MFMA v_mfma_f32_16x16x32_bf16 with
// each fp32 operand split into bf16 hi + lo, accumulating hi*hi + hi*lo +
// lo*hi in fp32 (relative error ~2^-16 per product instead of bf16's 2^-8).
// Phase B's operands W, Q, M and K are stored as fp16 (their entries are
// bounded by 1, see the workspace notes; K as hi + lo); its products take them
// as they are on v_mfma_f32_16x16x32_f16 against the fp32 state or U tile
// split into fp16 hi + lo (hi*W + lo*W: the split keeps 22 significant bits), each tile first
// scaled by a power of two chosen from a running bound on its norm so that
// the split cannot overflow fp16.  The triangular inverse, the gate cumsum,
// every exponential and the state carry are fp32.  Exponentials are only
// taken of non-positive arguments (masked before the exp), so g must be <= 0,
// which the decay gate guarantees.
//
// MFMA operand layout (16x16x32 bf16, wave64): lane l holds row (l % 16) of
// A / column (l % 16) of B, and 8 k values chosen by l / 16; the accumulator
// holds D[4*(l/16) + r][l % 16], r = 0..3.  Operands that are the transpose of
// a row-major LDS tile are read with ds_read_b64_tr_b16 (gfx950).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "bf16_frag.hpp"
#include "conv.hpp"
#include "gate.hpp"
#include "wave.hpp"
#include "gdn.h"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int CH = 64;           // positions per chunk
constexpr int DK = 128;          // key dimension (state rows)
constexpr int DV = 128;          // value dimension (state columns)
constexpr int NBLK = 16;         // value columns per value tile of the scan
constexpr int NVB = DV / NBLK;   // value tiles per head

// ----------------------------------------------------------------------------- workspace
// Two regions.  Value slots, one per (sequence, value head, chunk), all
// offsets in bytes, each region 256-aligned:
//   W      : fragment (token tile m, key k-step ks) = 64 lanes x 16 B (8 fp16),
//            lane (kg, l16) holding row 16m + l16, keys pi(32ks, kg)
//   M^T    : fragment (token tile m, token k-step ks), lane holding row
//            16m + l16 of M, positions pi(32ks, kg); hi and lo planes
//   Ut     : fp32 accumulator tiles [value tile][token tile][lane][4], lane
//            (kg, l16) holding values 16d + 4kg + r of token 16m + l16
//   header : e^{G_n}, b, a, 0; e^{G_t} (64 floats); e^{G_n - G_t} (64 floats)
// Key slots, one per (sequence, query/key head, chunk), after all value slots:
//   Q      : fragment (token tile m, key k-step ks) as W
//   K^T    : fragment (key tile m, token k-step ks), lane holding key row
//            16m + l16, tokens pi(32ks, kg); hi and lo planes
// These are the exact register images the scan loads, so each of its wave
// loads is 1 KiB (or 1 KiB of float4) of consecutive bytes.  Q and K depend on
// the query/key head only: the first value head of each group writes them and
// every value head of the group reads them.
//
// W, Q, M and K are stored as fp16 (relative rounding 2^-11): the scan is
// bound by the operand bytes each CU pulls from L2 per chunk.  They are small:
// with beta_t |k_t|^2 <= 2 every factor I - beta_t k_t k_t^T has spectral
// norm <= 1, and with g <= 0 row t of W is beta_t e^{G_t} P^T k_t for a
// product P of such factors, so |W[t][i]| <= beta_t |k_t|; |Q[t][i]| <= |q_t|,
// |K[t][i]| <= |k_t| and |M[t][s]| <= |q_t| |k_s|.  For unit-length keys and
// queries every entry is at most 2 in magnitude.
// K and M are kept as two fp16 planes, hi and lo = fp16(x - hi) (22
// significant bits): the state update K^T diag(e^{G_n-G}) U and y's M U sum
// 64 terms that can cancel (repeated or low-rank keys with beta near 1 and no
// decay make the terms of size |v| while their sum stays of size |v|), so
// single fp16 rounding of K or M would show in the state or in y at
// ~2^-11 * sqrt(64) relative; W and Q meet no such cancellation (they multiply
// the state, whose rows do not cancel this way) and stay single fp16.
// The header's b = sum_t beta_t |k_t| |v_t| and a = max_t beta_t |k_t| over
// the chunk's positions: a chunk raises the state's spectral norm by at most
// b (each position adds at most beta_t |k_t| |v_t|), and every entry of U
// (row t is the sequential delta beta_t (v_t - (decayed S_{t-1})^T k_t)) is
// at most b + a * (the state's bound), which is how the scan picks its fp16
// scaling without a reduction.
constexpr size_t WS_PLANE = (size_t)CH * DK * 2;        // one fp16 64x128 matrix
constexpr size_t WV_W = 0;                              // W   (4 token tiles x 4 k-steps)
constexpr size_t WV_M = WS_PLANE;                       // M^T (4 token tiles x 2 k-steps), hi
constexpr size_t WV_ML = WV_M + (size_t)CH * CH * 2;    // M^T lo: M - hi, in fp16
constexpr size_t WV_U = WV_ML + (size_t)CH * CH * 2;    // Ut  fp32 accumulator tiles
constexpr size_t WV_G = WV_U + (size_t)DV * CH * 4;     // e^{G_n}, b, a (float4)
constexpr size_t WV_EG = WV_G + 16;                     // e^{G_t}
constexpr size_t WV_D = WV_EG + (size_t)CH * 4;         // e^{G_n - G_t}
constexpr size_t WV_CHUNK = WV_G + 768;
constexpr size_t WK_Q = 0;                              // Q   (4 token tiles x 4 k-steps)
constexpr size_t WK_K = WS_PLANE;                       // K^T (8 key tiles x 2 k-steps), hi
constexpr size_t WK_KL = 2 * WS_PLANE;                  // K^T lo: K - hi, in fp16
constexpr size_t WK_CHUNK = 3 * WS_PLANE;
static_assert(WV_D + CH * 4 <= WV_CHUNK && WV_CHUNK % 256 == 0 && WK_CHUNK % 256 == 0,
              "workspace slots");

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));

// u16 offset of a fragment's 8 fp16 values for lane `lane`
__device__ __forceinline__ int frag_off(int m, int ks, int n_ks, int lane) {
  return ((m * n_ks + ks) * 64 + lane) * 8;
}
__device__ __forceinline__ h16x8 frag_ws(const u16 *base, int m, int ks, int n_ks, int lane) {
  return *reinterpret_cast<const h16x8 *>(base + frag_off(m, ks, n_ks, lane));
}
// 8 floats -> one 16-byte store of fp16 (round to nearest even)
__device__ __forceinline__ void store8_h(u16 *p, const float (&x)[8]) {
  h16x8 h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (_Float16)x[e];
  *reinterpret_cast<h16x8 *>(p) = h;
}
// DPP move with CTRL on the rows in ROW_MASK; lanes whose source is out of
// range, and lanes of masked rows, read 0
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_zero(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xF, true));
}

// |x|^2 of a 128-wide row held as channel quads l and 16 + l by the 16 lanes
// l of a DPP row: each quad's sum left to right, the lane's two quads added,
// then the 16-lane butterfly (every lane gets the same bits)
__device__ __forceinline__ float row_sumsq(const float4 &a, const float4 &b) {
  const float sa = a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
  const float sb = b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
  return group_sum<16>(sa + sb);
}
// maximum over the wave (exact in any order)
__device__ __forceinline__ float group_max64(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// 8 floats -> 16-byte stores of fp16 hi and lo = fp16(x - hi)
__device__ __forceinline__ void store8_h2(u16 *ph, u16 *pl, const float (&x)[8]) {
  h16x8 h, l;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = (_Float16)x[e];
    l[e] = (_Float16)(x[e] - (float)h[e]);
  }
  *reinterpret_cast<h16x8 *>(ph) = h;
  *reinterpret_cast<h16x8 *>(pl) = l;
}

// float offset of the accumulator tile (value tile d, token tile m) for lane
__device__ __forceinline__ int acc_off(int d, int m, int lane) {
  return ((d * 4 + m) * 64 + lane) * 4;
}

// ----------------------------------------------------------------------------- phase A
// One workgroup (8 waves) per CU, one (sequence, head, chunk) at a time.  All
// row-major LDS tiles are bf16 hi/lo planes.  Plan (bytes):
//   L_K : K rows [t][i]
//   L_Q : Q rows [t][i]
//   L_V : V rows [t][j]
//   L_L : M = L o Q K^T             [t][s]
//   L_A : A, then T in place (fp32 [64][68]);  L_S: four 16x16 blocks (pitch XP) of the inverse
//         (T1 = T diag(beta e^G) and T2 = T diag(beta) are formed from it as
//         fragments, in registers)
//   L_G : G, beta, e^G, e^{G_n - G};  L_N: |k_t|^2, |v_t|^2
//   L_T : the 4 conv taps of each of the item's 3 x 128 K, Q, V channels
// The products are computed transposed (feature index as the MFMA row):
//   W^T = K^T T1^T,  Ut^T = V^T T2^T
// with K^T, V^T read from row-major tiles by transpose reads, so a wave's
// accumulators are already the scan's fragments.
constexpr int PR = 136;   // pitch (bf16) of a [64][128] row-major tile
constexpr int PS = 72;    // pitch (bf16) of a [64][64] tile
constexpr int PA = 68;    // pitch (fp32) of the [64][64] inverse
constexpr int TILE128 = 2 * CH * PR * 2;
constexpr int TILE64 = 2 * CH * PS * 2;
constexpr int L_K = 0;
constexpr int L_Q = L_K + TILE128;
constexpr int L_V = L_Q + TILE128;
constexpr int L_L = L_V + TILE128;
constexpr int L_A = L_L + TILE64;
constexpr int L_S = L_A + CH * PA * 4;
constexpr int XP = 17;   // pitch (fp32) of the inverse's scratch blocks
constexpr int L_G = L_S + 4 * 16 * XP * 4;
constexpr int L_N = L_G + 4 * CH * 4;   // |k_t|^2, |v_t|^2
constexpr int L_T = L_N + 2 * CH * 4;   // conv taps of the item's K, Q, V channels (ConvSrc)
constexpr int L_TOTAL = L_T + 3 * DK * 16;
static_assert(L_TOTAL <= 160 * 1024, "phase A LDS fits one CU");

// Lower 16x16 tiles of K K^T (A = beta_t e^{G_t - G_s} k_t.k_s, strictly lower)
// and of Q K^T (e^{G_t - G_s} q_t.k_s, diagonal included, stored as bf16 hi/lo):
// a wave takes one or two tile positions (ti, tj) and both products at each,
// so each k-step reads the K fragment of column tile tj once for two tiles
// (and the row fragments once when a wave's two positions share ti).
template <int NJ>
__device__ __forceinline__ void lower_tiles(int w, const u16 *kh, const u16 *klo, const u16 *qh,
                                            const u16 *qlo, float *sA, u16 *lqh, u16 *lql,
                                            const float *sG, const float *sBeta, int l16, int kg) {
  // positions: waves 0, 1 take (3,0),(3,1) and (3,2),(3,3); waves 2..7 one of
  // (0,0),(1,0),(1,1),(2,0),(2,1),(2,2); each position gives a K K^T and a Q K^T
  // tile, which share the K fragment of column tile tj and the row tile ti
  bool qk[NJ];
  int ti[NJ], tj[NJ];
  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int pos = w < 2 ? 2 * w + (j >> 1) : w - 2;
    const int pti = w < 2 ? 3 : (pos < 1 ? 0 : pos < 3 ? 1 : 2);
    const int ptj = w < 2 ? pos : pos - pti * (pti + 1) / 2;
    qk[j] = (j & 1) != 0;
    ti[j] = pti;
    tj[j] = ptj;
    acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    Frag fk[NJ / 2], fq[NJ / 2], fb[NJ / 2];
#pragma unroll
    for (int p = 0; p < NJ / 2; ++p) {
      fb[p] = frag(kh, klo, PR, 16 * tj[2 * p] + l16, 32 * ks + 8 * kg);
      if (ti[2 * p] == tj[2 * p]) fk[p] = fb[p];
      else fk[p] = frag(kh, klo, PR, 16 * ti[2 * p] + l16, 32 * ks + 8 * kg);
      fq[p] = frag(qh, qlo, PR, 16 * ti[2 * p] + l16, 32 * ks + 8 * kg);
    }
#pragma unroll
    for (int p = 0; p < NJ / 2; ++p) {
      acc[2 * p] = mfma3(fk[p], fb[p], acc[2 * p]);
      acc[2 * p + 1] = mfma3(fq[p], fb[p], acc[2 * p + 1]);
    }
  }
  // e^{G_t - G_s} is the hardware base-2 exponential of (G_t - G_s) log2(e),
  // with the argument masked to 0 above the diagonal before it is taken; every
  // entry of the tile is stored (zeros above the diagonal), so no lane branches
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int sx = 16 * tj[j] + l16;
    const float gs = sG[sx];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * ti[j] + 4 * kg + r;
      const float d = sx <= t ? sG[t] - gs : 0.0f;
      const float e = __builtin_amdgcn_exp2f(d * 1.4426950408889634f);
      if (!qk[j]) {
        sA[t * PA + sx] = sx < t ? sBeta[t] * e * acc[j][r] : 0.0f;
      } else {
        u16 hh, ll;
        split(sx <= t ? e * acc[j][r] : 0.0f, hh, ll);
        lqh[t * PS + sx] = hh;
        lql[t * PS + sx] = ll;
      }
    }
  }
}


// Fragments of T1 = T diag(beta e^G) and T2 = T diag(beta), row `row`, k in
// pi(k0, kg), formed from the fp32 inverse in LDS and split into bf16 hi + lo.
__device__ __forceinline__ void t_frags(const float *sA, const float *sBeta, const float *sEG,
                                        int row, int k0, int kg, Frag &f1, Frag &f2) {
  const int c = k0 + 4 * kg;
  const float4 a0 = *reinterpret_cast<const float4 *>(sA + row * PA + c);
  const float4 a1 = *reinterpret_cast<const float4 *>(sA + row * PA + c + 16);
  const float4 b0 = *reinterpret_cast<const float4 *>(sBeta + c);
  const float4 b1 = *reinterpret_cast<const float4 *>(sBeta + c + 16);
  const float4 e0 = *reinterpret_cast<const float4 *>(sEG + c);
  const float4 e1 = *reinterpret_cast<const float4 *>(sEG + c + 16);
  const float tv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
  float v1[8], v2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v1[e] = tv[e] * (bv[e] * ev[e]);
    v2[e] = tv[e] * bv[e];
  }
  f1 = split8(v1);
  f2 = split8(v2);
}

// ---- fp32 16x16 block products for the triangular inverse
// v_mfma_f32_16x16x4f32: lane l supplies A[l%16][k], B[k][l%16] with
// k = l/16 of the step, and holds D[4(l/16) + r][l%16].  Step s of a 16-long
// sum uses k = 4(l/16) + s, so an accumulator block (which holds rows
// 4(l/16) + r) is already the B operand of the next product, with r = s.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// c += A B, A and B 16x16 blocks of row-major fp32 LDS arrays (pitches PA_, PB_)
template <int PA_, int PB_>
__device__ __forceinline__ f32x4 blk_mm(const float *A, const float *B, f32x4 c, int l16, int kg) {
#pragma unroll
  for (int st = 0; st < 4; ++st)
    c = mfma_f32(A[l16 * PA_ + 4 * kg + st], B[(4 * kg + st) * PB_ + l16], c);
  return c;
}
// c += A Bacc, Bacc an accumulator block held by this wave
template <int PA_>
__device__ __forceinline__ f32x4 blk_mm_acc(const float *A, const f32x4 &b, f32x4 c, int l16,
                                            int kg) {
#pragma unroll
  for (int st = 0; st < 4; ++st) c = mfma_f32(A[l16 * PA_ + 4 * kg + st], b[st], c);
  return c;
}
// store an accumulator block times `sign` to a row-major block with pitch PD_
template <int PD_>
__device__ __forceinline__ void blk_store(float *D, const f32x4 &c, float sign, int l16, int kg) {
#pragma unroll
  for (int r = 0; r < 4; ++r) D[(4 * kg + r) * PD_ + l16] = sign * c[r];
}

// One phase A work item: chunk c of value head h of sequence s.
struct PrepItem {
  int h, s, hk;
  int n;      // positions in the chunk; 0 for a padding chunk (each sequence's
              // chunk count is rounded up to even so the scan's two-deep operand
              // pipeline has no tail): it yields e^{G_n} = 1 and all-zero
              // operands, which leaves the state unchanged
  int nl;     // last valid row, for clamped loads
  int t0;     // the chunk's first position within its sequence
  int tb;     // row of the chunk's first load (clamped to the sequence's last
              // row for padding chunks); within the sequence for a fixed-length
              // batch, within the packed token rows for a variable-length one
  int64_t grow;   // g / beta row of tb
  size_t slot;    // value slot
  size_t kslot;   // key slot of the chunk's query/key head
  bool kown;      // the first value head of its group: writes the key slot
};
// Fixed-length batch: item u = (chunk, sequence, head), heads fastest, the
// chunks from the last to the first.  Phase B reads chunk 0 of every head
// first and the last chunk last; the workspace outgrows the last-level cache
// (MALL) at long prompts, and written in the reverse of its read order, what
// the cache still holds when phase B starts is what phase B reads first.
// Within a chunk, when the (sequence, query/key head) groups come in
// multiples of 8, the G value heads of a group are items 8 apart: the
// persistent grid (a multiple of 8 workgroups, workgroup b on XCD b % 8) then
// runs them at the same time on one XCD, which reads the group's q and k rows
// from HBM once.
__device__ __forceinline__ PrepItem prep_item(int u, int n_chunks, int H, int Hk, int n_tok,
                                              const NoTab &, int n_items) {
  PrepItem it;
  const int nsh = n_items / n_chunks;   // sequences x heads
  const int c = n_chunks - 1 - u / nsh;
  const int G = H / Hk, idx = u % nsh;
  if (nsh % (8 * G) == 0) {
    const int gi = (idx / (8 * G)) * 8 + idx % 8, mem = (idx / 8) % G;
    it.s = gi / Hk;
    it.h = (gi % Hk) * G + mem;
  } else {
    it.h = idx % H;
    it.s = idx / H;
  }
  it.hk = it.h / (H / Hk);
  const int t0 = c * CH;
  it.n = max(0, min(CH, n_tok - t0));
  it.nl = max(it.n - 1, 0);
  it.t0 = t0;
  it.tb = min(t0, n_tok - 1);
  it.grow = (int64_t)it.s * n_tok + it.tb;
  it.slot = ((size_t)it.s * H + it.h) * n_chunks + c;
  it.kslot = ((size_t)it.s * Hk + it.hk) * n_chunks + c;
  it.kown = it.h % (H / Hk) == 0;
  return it;
}
// Variable-length batch: item u = (packed chunk gc, head), heads fastest, the
// packed chunks from the last to the first, and the G value heads of a group
// 8 items apart when H is a multiple of 8 G, as for a fixed-length batch: the
// group's q and k rows then come from HBM once, and the chunks at the front
// of the packing, which phase B's first workgroups read, are the last written.
// The sequence holding gc is found by binary search over the chunk offsets.
__device__ __forceinline__ PrepItem prep_item(int u, int n_chunks, int H, int Hk, int,
                                              const VarTab &tab, int) {
  PrepItem it;
  const int G = H / Hk, gc = n_chunks - 1 - u / H, idx = u % H;
  if (H % (8 * G) == 0)
    it.h = ((idx / (8 * G)) * 8 + idx % 8) * G + (idx / 8) % G;
  else
    it.h = idx;
  it.hk = it.h / G;
  int lo = 0, hi = tab.n_seq - 1;   // last s with ch0[s] <= gc: a nonempty sequence
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tab.ch0[mid] <= gc) lo = mid; else hi = mid - 1;
  }
  it.s = lo;
  const int len = tab.tok0[lo + 1] - tab.tok0[lo];
  const int t0 = (gc - tab.ch0[lo]) * CH;
  it.n = max(0, min(CH, len - t0));
  it.nl = max(it.n - 1, 0);
  it.t0 = t0;
  it.tb = tab.tok0[lo] + min(t0, len - 1);
  it.grow = it.tb;
  it.slot = (size_t)it.h * n_chunks + gc;
  it.kslot = (size_t)it.hk * n_chunks + gc;
  it.kown = it.h % (H / Hk) == 0;
  return it;
}

// ---- phase A inputs
// An item's gate values and K, Q, V rows come from one of two sources with one
// interface:
//   Regs         the next item's loads, in flight while the current item runs
//   load_gate    g (or what g is computed from) and beta of the chunk's 64
//                positions, one position per lane
//   gate         the lane's g
//   load_rows    the K, Q, V rows (or what they are computed from)
//   rows_to_lds  K, Q, V rows into their LDS tiles as bf16 hi/lo (rows past n
//                as zeros) and the row norms |k_t|^2, |v_t|^2 (0 past n)
//   taps_to_lds  what rows_to_lds reads from LDS besides the rows (after the
//                last read of the current item's, before the next item)
// Only wave 7, which forms the gate cumsum, loads the gate values.
// Rows past n read a valid row and are zeroed where they are used: a load
// behind a branch would make the compiler wait for every load in flight at
// the join.
struct Tiles {
  u16 *kh, *kl, *qh, *ql, *vh, *vl;
  float *sNK, *sNV;
  float4 *taps;   // [3][128]
};
__device__ __forceinline__ float bf16_to_f32(unsigned b) { return __builtin_bit_cast(float, b << 16); }
// Rows of 128 features are moved by the 16 lanes l of a DPP row, lane l
// holding the feature quads l and 16 + l (features 4l .. 4l+3 and
// 64 + 4l .. 64 + 4l+3): each load instruction then reads 256 contiguous
// bytes per row, and the quads are the 4-channel groups of the conv
// kernels' lanes.
// 4 consecutive elements as a float4.  fp32 inputs read once are loaded
// non-temporally, so that they do not displace the workspace from the
// last-level cache.
__device__ __forceinline__ float4 load4f(const float *p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float4 load4f(const u16 *p) {
  const uint2 u = *reinterpret_cast<const uint2 *>(p);
  return make_float4(bf16_to_f32(u.x & 0xffffu), bf16_to_f32(u.x >> 16),
                     bf16_to_f32(u.y & 0xffffu), bf16_to_f32(u.y >> 16));
}
// q and k rows, read by every value head of their group (whose items run side
// by side on one XCD): ordinary loads, so the group's later heads find them
// in the XCD's L2 (measured: 1 to 2 % off the call against non-temporal ones)
__device__ __forceinline__ void load_quads_shared(const float *p, int l, float4 &a, float4 &b) {
  a = *reinterpret_cast<const float4 *>(p + 4 * l);
  b = *reinterpret_cast<const float4 *>(p + 64 + 4 * l);
}
__device__ __forceinline__ void load_quads_shared(const u16 *p, int l, float4 &a, float4 &b) {
  a = load4f(p + 4 * l);
  b = load4f(p + 64 + 4 * l);
}
// the lane's two quads of the row at p
template <class T>
__device__ __forceinline__ void load_quads(const T *p, int l, float4 &a, float4 &b) {
  a = load4f(p + 4 * l);
  b = load4f(p + 64 + 4 * l);
}
// Thread tid moves row (i * 512 + tid) / 16 in pass i (i = 0, 1) as lane
// l = tid % 16 of its row.
__device__ __forceinline__ int row_of(int i, int tid) { return (i * 512 + tid) >> 4; }
// the lane's two quads into the bf16 hi/lo planes of row `row` of a tile;
// rows past n are written as zeros
__device__ __forceinline__ void store_quads(u16 *hi, u16 *lo, int row, int l, const float4 &a,
                                            const float4 &b, bool valid) {
  const int o = row * PR + 4 * l;
  if (valid) {
    store4_split(hi + o, lo + o, a.x, a.y, a.z, a.w);
    store4_split(hi + o + 64, lo + o + 64, b.x, b.y, b.z, b.w);
  } else {
    store4_split(hi + o, lo + o, 0.f, 0.f, 0.f, 0.f);
    store4_split(hi + o + 64, lo + o + 64, 0.f, 0.f, 0.f, 0.f);
  }
}

// q, k, v, g as given; q, k, v elements fp32 or bf16 (TIN = u16, the bit
// pattern), widened to fp32 on load, exactly, so a bf16 call equals an fp32
// call on the same values bit for bit.
template <class TIN>
struct DirectSrc {
  const TIN *q, *k, *v;
  const float *g, *beta;
  int64_t qk_tok, qk_seq, v_tok, v_seq;
  int n_tok, H;
  struct Regs {
    float4 kr[4], qr[4], vr[4];
    float gv, bv;
  };
  __device__ __forceinline__ void load_gate(const PrepItem &it, int lane, Regs &r) const {
    const int64_t gi = (it.grow + min(lane, it.nl)) * H + it.h;
    r.gv = g[gi];
    r.bv = beta[gi];
  }
  __device__ __forceinline__ float gate(const Regs &r) const { return r.gv; }
  // part 0: K rows, 1: Q rows, 2: V rows
  template <int PART>
  __device__ __forceinline__ void load_rows(const PrepItem &it, int tid, Regs &r) const {
    const int64_t kb = it.s * qk_seq + (int64_t)it.tb * qk_tok + it.hk * DK;
    const int64_t vb = it.s * v_seq + (int64_t)it.tb * v_tok + it.h * DV;
    const int l = tid & 15;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rr = min(row_of(i, tid), it.nl);
      if constexpr (PART == 0)
        load_quads_shared(k + kb + (int64_t)rr * qk_tok, l, r.kr[2 * i], r.kr[2 * i + 1]);
      if constexpr (PART == 1)
        load_quads_shared(q + kb + (int64_t)rr * qk_tok, l, r.qr[2 * i], r.qr[2 * i + 1]);
      if constexpr (PART == 2)
        load_quads(v + vb + (int64_t)rr * v_tok, l, r.vr[2 * i], r.vr[2 * i + 1]);
    }
  }
  __device__ __forceinline__ void rows_to_lds(const PrepItem &it, int tid, const Regs &r,
                                              const Tiles &t) const {
    const int l = tid & 15;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = row_of(i, tid);
      const bool valid = row < it.n;
      store_quads(t.kh, t.kl, row, l, r.kr[2 * i], r.kr[2 * i + 1], valid);
      store_quads(t.qh, t.ql, row, l, r.qr[2 * i], r.qr[2 * i + 1], valid);
      store_quads(t.vh, t.vl, row, l, r.vr[2 * i], r.vr[2 * i + 1], valid);
      const float nk = row_sumsq(r.kr[2 * i], r.kr[2 * i + 1]);
      const float nv = row_sumsq(r.vr[2 * i], r.vr[2 * i + 1]);
      if (l == 0) {
        t.sNK[row] = valid ? nk : 0.0f;
        t.sNV[row] = valid ? nv : 0.0f;
      }
    }
  }
  __device__ __forceinline__ void taps_to_lds(int, const Regs &, const Tiles &) const {}
};

__device__ __forceinline__ float f4_at(const float4 &v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

// The layer's own inputs: the conv input rows x (channels: q heads, k heads,
// v heads, S = 128 wide), the 4-tap conv weights and history, alpha (g is
// decay_gate_value(alpha, dt[h], a[h]), as the gate kernel computes it) and
// beta.  K, Q, V are the conv1d + SiLU outputs (K and Q then L2-normalised
// per head) with the conv kernels' arithmetic: conv_position() per channel,
// and the L2 sum of squares in the same tree as their 32-lane butterfly over
// 4-channel lanes (that butterfly sums channel quads 0..15 and 16..31 of the
// head in two 16-lane trees, then adds the two: here a lane holds quads l
// and 16 + l, and runs the two 16-lane trees itself), so K, Q, V are bit for
// bit the rows gdn_conv1d_silu_l2norm writes.
// Lanes: waves 0, 1 hold K, waves 2, 3 Q (8 rows each: rows 8rg .. 8rg+7,
// rg = tid / 16 % 8), waves 4..7 V (4 rows each: rows 4rg .. 4rg+3,
// rg = tid / 16 % 16), so every SIMD (waves w and w + 4) computes 12 rows:
// the conv is VALU work, about 20 instructions per output.  A lane holds
// quads l, 16 + l (l = tid % 16) of its rows, the 16 lanes of a DPP row
// sharing their rows, and keeps the input rows of its rows' windows (11
// rows for K and Q, 7 for V).  The taps go through LDS (L_T), one 16-byte
// record per channel, read by every lane that needs them.
struct ConvSrc {
  const float *x;
  int64_t x_tok, x_seq;
  const float *w;       // [conv channel][4 taps], oldest tap first
  const float *hist;    // [sequence][conv channel][3], oldest first
  int64_t h_seq;
  const float *alpha, *dt, *a, *beta;
  float eps;
  int n_tok, H, Hk;
  struct Regs {
    float4 raw[11][2];   // [input row][quad l, quad 16 + l]
    float4 tw;           // lane tid < 384: the taps of channel tid % 128 of matrix tid / 128
    float gv, bv, dtv, av;
  };
  __device__ __forceinline__ int64_t chan0(const PrepItem &it, int m) const {
    return m == 0 ? (int64_t)(Hk + it.hk) * DK
                  : m == 1 ? (int64_t)it.hk * DK : (int64_t)2 * Hk * DK + (int64_t)it.h * DV;
  }
  __device__ __forceinline__ void load_gate(const PrepItem &it, int lane, Regs &r) const {
    const int64_t gi = (it.grow + min(lane, it.nl)) * H + it.h;
    r.gv = alpha[gi];
    r.bv = beta[gi];
    r.dtv = dt[it.h];
    r.av = a[it.h];
  }
  __device__ __forceinline__ float gate(const Regs &r) const {
    return decay_gate_value(r.gv, r.dtv, r.av);
  }
  // the lane's matrix (0 K, 1 Q, 2 V), first row and row count
  __device__ __forceinline__ static void lane_rows(int tid, int &m, int &row0, int &nrow) {
    const int w = tid >> 6;
    m = w < 4 ? w >> 1 : 2;
    nrow = w < 4 ? 8 : 4;
    row0 = w < 4 ? 8 * ((tid >> 4) & 7) : 4 * ((tid >> 4) & 15);
  }
  // part 0: input rows 0..3, 1: rows 4..7, 2: rows 8..10 and the taps.
  // In a sequence's first chunk, rows 0..2 of the lanes whose first row is 0
  // are positions before 0, read from the history ([channel][tap]) instead
  // of x: that item (a uniform branch) reads rows 0..2 element by element,
  // each lane from its own source.  Either way only loads into the same
  // registers are issued, so the later wait for them counts these loads
  // alone (a wait after a branch whose loads are newer than the item's
  // stores would also wait for the stores).
  template <int PART>
  __device__ __forceinline__ void load_rows(const PrepItem &it, int tid, Regs &r) const {
    const int l = tid & 15;
    int m, row0, nrow;
    lane_rows(tid, m, row0, nrow);
    const int64_t ch = chan0(it, m) + 4 * l;
    const float *xs = x + it.s * x_seq + ch;
    // input row j is position t0 + row0 - 3 + j (a V lane needs rows 0..6)
    auto pos = [&](int j) { return min(max(it.t0 + row0 - 3 + j, 0), n_tok - 1); };
    auto row = [&](int j) __attribute__((always_inline)) {
      const float *xr = xs + (int64_t)pos(j) * x_tok;
      r.raw[j][0] = load4f(xr);
      r.raw[j][1] = load4f(xr + 64);
    };
    if constexpr (PART == 0) {
      if (it.t0 == 0) {
        const float *hp = hist + it.s * h_seq + ch * 3;
        const bool from_hist = row0 == 0;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const float *xr = xs + (int64_t)pos(j) * x_tok;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int c = (e & 3) + (e >> 2) * 64;   // channel offset from ch
            v[e] = from_hist ? hp[c * 3 + j] : xr[c];
          }
          r.raw[j][0] = make_float4(v[0], v[1], v[2], v[3]);
          r.raw[j][1] = make_float4(v[4], v[5], v[6], v[7]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 3; ++j) row(j);
      }
      row(3);
    }
    if constexpr (PART == 1) {
#pragma unroll
      for (int j = 4; j < 7; ++j) row(j);
      if (nrow == 8) row(7);   // uniform per wave
    }
    if constexpr (PART == 2) {
      if (nrow == 8) {         // uniform per wave
#pragma unroll
        for (int j = 8; j < 11; ++j) row(j);
      }
      // the item's taps, 16 contiguous bytes per lane (lanes 384..511 read
      // the first record again and store nothing)
      const int tm = min(tid >> 7, 2), tc = tid < 384 ? tid & 127 : 0;
      r.tw = *reinterpret_cast<const float4 *>(w + (chan0(it, tm) + tc) * 4);
    }
  }
  __device__ __forceinline__ void taps_to_lds(int tid, const Regs &r, const Tiles &t) const {
    if (tid < 384) t.taps[tid] = r.tw;
  }
  __device__ __forceinline__ void rows_to_lds(const PrepItem &it, int tid, const Regs &r,
                                              const Tiles &t) const {
    const int l = tid & 15;
    int m, row0, nrow;
    lane_rows(tid, m, row0, nrow);
    // the K, Q, V tiles are evenly spaced, |v|^2 follows |k|^2 (an offset,
    // not a choice among pointers, which the compiler would keep in memory)
    static_assert(L_Q - L_K == TILE128 && L_V - L_Q == TILE128, "tile spacing");
    u16 *hi = t.kh + m * (TILE128 / 2);
    u16 *lo = hi + CH * PR;
    float *sn = t.sNK + (m == 0 ? 0 : CH);
    float wv[8][4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float4 tv = t.taps[m * DK + 4 * l + (e & 3) + (e >> 2) * 64];
      wv[e][0] = tv.x;
      wv[e][1] = tv.y;
      wv[e][2] = tv.z;
      wv[e][3] = tv.w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < nrow) {   // uniform per wave
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float win[4] = {f4_at(r.raw[i][e >> 2], e & 3), f4_at(r.raw[i + 1][e >> 2], e & 3),
                                f4_at(r.raw[i + 2][e >> 2], e & 3),
                                f4_at(r.raw[i + 3][e >> 2], e & 3)};
          o[e] = conv_position<4>(wv[e], win);
        }
        if (m < 2) {
          float sa = o[0] * o[0], sb = o[4] * o[4];
#pragma unroll
          for (int e = 1; e < 4; ++e) {
            sa = __builtin_fmaf(o[e], o[e], sa);
            sb = __builtin_fmaf(o[4 + e], o[4 + e], sb);
          }
          const float inv = l2_rsqrt(group_sum<16>(sa) + group_sum<16>(sb) + eps);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] *= inv;
        }
        const int row = row0 + i;
        const bool valid = row < it.n;
        const float4 a0 = make_float4(o[0], o[1], o[2], o[3]);
        const float4 a1 = make_float4(o[4], o[5], o[6], o[7]);
        store_quads(hi, lo, row, l, a0, a1, valid);
        if (m != 1) {
          const float nr = row_sumsq(a0, a1);
          if (l == 0) sn[row] = valid ? nr : 0.0f;
        }
      }
    }
  }
};

// Persistent: workgroup b handles items b, b + G, b + 2G, ... (G = grid size,
// at most one workgroup per CU given the LDS it takes).  The next item's
// gate values and rows are loaded into registers as soon as the current item
// has consumed them, so a workgroup's loads and stores overlap its own compute
// instead of every CU loading, then computing, then storing in lockstep.
template <class TAB, class SRC>
__global__ __launch_bounds__(512) void k_chunk_prep(const SRC src, unsigned char *__restrict__ ws,
                                                    unsigned char *__restrict__ wsk, int n_tok,
                                                    int n_chunks, int H, int Hk, int n_items,
                                                    const TAB tab) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[L_TOTAL];

  u16 *kh = reinterpret_cast<u16 *>(smem + L_K), *klo = kh + CH * PR;
  u16 *qh = reinterpret_cast<u16 *>(smem + L_Q), *qlo = qh + CH * PR;
  u16 *vh = reinterpret_cast<u16 *>(smem + L_V), *vlo = vh + CH * PR;
  u16 *lqh = reinterpret_cast<u16 *>(smem + L_L), *lql = lqh + CH * PS;
  float *sA = reinterpret_cast<float *>(smem + L_A);
  float *scratch = reinterpret_cast<float *>(smem + L_S);
  float *sG = reinterpret_cast<float *>(smem + L_G);
  float *sBeta = sG + CH, *sEG = sG + 2 * CH, *sEGn = sG + 3 * CH;
  float *sNK = reinterpret_cast<float *>(smem + L_N), *sNV = sNK + CH;
  const Tiles tiles{kh, klo, qh, qlo, vh, vlo, sNK, sNV, reinterpret_cast<float4 *>(smem + L_T)};

  // (L o QK^T) and A, which lie back to back, are cleared once: every item
  // writes every entry of their lower 16x16 tiles (zeros above the diagonal
  // included) and nothing writes their upper tiles, which must stay zero (the
  // first item's first barrier orders this before any use).  16-byte stores.
  {
    static_assert(L_A == L_L + TILE64 && (TILE64 + CH * PA * 4) % 16 == 0 && L_L % 16 == 0,
                  "one contiguous region");
    uint4 *zp = reinterpret_cast<uint4 *>(smem + L_L);
    for (int e = threadIdx.x; e < (TILE64 + CH * PA * 4) / 16; e += 512)
      zp[e] = make_uint4(0, 0, 0, 0);
  }
  // the grid never exceeds n_items, so every workgroup has a first item
  PrepItem it = prep_item(blockIdx.x, n_chunks, H, Hk, n_tok, tab, n_items);
  typename SRC::Regs pre;
  if ((threadIdx.x >> 6) == 7) src.load_gate(it, threadIdx.x & 63, pre);
  src.template load_rows<0>(it, threadIdx.x, pre);
  src.template load_rows<1>(it, threadIdx.x, pre);
  src.template load_rows<2>(it, threadIdx.x, pre);
  src.taps_to_lds(threadIdx.x, pre, tiles);
  __syncthreads();

  // One item; the first is peeled off the loop below so that the loop head is
  // reached from one place only and the compiler's load/store counts there
  // are exact (a merged count forces waits for every store still in flight).
  auto run_item = [&](int u) {
  // The thread index is re-read opaquely on every pass: otherwise the
  // compiler hoists every per-lane LDS and workspace offset of the item out of
  // the loop and keeps them all live, which spills.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
  // the item after this one (this one again on the last pass: its loads are
  // then redundant but in bounds, and no load sits behind a branch)
  const PrepItem nx = prep_item(u + gridDim.x < n_items ? u + gridDim.x : u, n_chunks, H, Hk,
                                n_tok, tab, n_items);
  const int n = it.n;
  unsigned char *wc = ws + it.slot * WV_CHUNK;
  unsigned char *wk = wsk + it.kslot * WK_CHUNK;

  // S0. gate cumsum (wave 7): an inclusive scan over the 64 lanes on DPP
  // (row shifts within each 16-lane row, then the row totals broadcast across
  // rows), and the exponentials as the hardware base-2 exponential of
  // x log2(e) (all arguments are <= 0)
  if (w == 7) {
    float x = lane < n ? src.gate(pre) : 0.0f;
    const float b = lane < n ? pre.bv : 0.0f;
    x += dpp_zero<0x111, 0xF>(x);   // row_shr:1
    x += dpp_zero<0x112, 0xF>(x);   // row_shr:2
    x += dpp_zero<0x114, 0xF>(x);   // row_shr:4
    x += dpp_zero<0x118, 0xF>(x);   // row_shr:8
    x += dpp_zero<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp_zero<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
    const float gn = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
    constexpr float LOG2E = 1.4426950408889634f;
    sG[lane] = x;
    sBeta[lane] = b;
    sEG[lane] = __builtin_amdgcn_exp2f(x * LOG2E);
    sEGn[lane] = __builtin_amdgcn_exp2f((gn - x) * LOG2E);
  }
  if (w == 7) src.load_gate(nx, lane, pre);
  // S1. K, Q, V rows -> LDS (bf16 hi/lo); |k_t|^2, |v_t|^2 of each row
  src.rows_to_lds(it, tid, pre, tiles);
  // the next item's rows in three parts, spread over the item so that no
  // section issues them all at once
  src.template load_rows<0>(nx, tid, pre);
  __syncthreads();

  // S2a. K K^T and Q K^T on the 10 lower tile positions each: 20 tiles; waves
  // 0 and 1 take two positions of row tile 3 (four tiles), waves 2..7 one of
  // the other six positions (two tiles), each wave's tiles all at once so their
  // MFMA chains interleave
  if (w < 2) {
    lower_tiles<4>(w, kh, klo, qh, qlo, sA, lqh, lql, sG, sBeta, l16, kg);
  } else {
    lower_tiles<2>(w, kh, klo, qh, qlo, sA, lqh, lql, sG, sBeta, l16, kg);
  }
  src.template load_rows<1>(nx, tid, pre);
  // the chunk's header, formed and stored by wave 7 (its Gram share is one of
  // the lighter ones; every lane stores the same bits): e^{G_n}, b, a, then
  // e^{G_t} and e^{G_n - G_t}
  if (w == 7) {
    const float bk = sBeta[lane] * sqrtf(sNK[lane]);
    const float b = group_sum<64>(bk * sqrtf(sNV[lane]));
    const float am = group_max64(bk);
    *reinterpret_cast<float4 *>(wc + WV_G) = make_float4(sEG[CH - 1], b, am, 0.0f);
    reinterpret_cast<float *>(wc + WV_EG)[lane] = sEG[lane];
    reinterpret_cast<float *>(wc + WV_D)[lane] = sEGn[lane];
  }
  __syncthreads();

  src.template load_rows<2>(nx, tid, pre);
  // S3a. T = (I + A)^{-1} in place: threads 0..63 invert the four 16x16
  // diagonal blocks (one column each, forward substitution in fp32).
  float x[16];
  if (tid < 64) {
    const int b = tid >> 4, cc = tid & 15;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = r == cc ? 1.0f : 0.0f;
#pragma unroll
      for (int j = 0; j < r; ++j) acc -= sA[(16 * b + r) * PA + 16 * b + j] * x[j];
      x[r] = acc;
    }
  }
  // While wave 0 inverts, the waves store the fragments that need only the
  // K, Q and M tiles (wave 0 its share after the inverse).
  // S2b. K^T fragments straight from the K tile, as fp16 hi and lo planes
  // (the first value head of a group only): wave w writes key tile w, both
  // token k-steps
  if (it.kown) {
    u16 *ktg = reinterpret_cast<u16 *>(wk + WK_K);
    u16 *ktl = reinterpret_cast<u16 *>(wk + WK_KL);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const Frag f = frag_tr(kh, klo, PR, 32 * ks, 16 * w, kg, l16);
      float xf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xf[e] = bf16_value((u16)f.hi[e]) + bf16_value((u16)f.lo[e]);
      store8_h2(ktg + frag_off(w, ks, 2, lane), ktl + frag_off(w, ks, 2, lane), xf);
    }
  }
  // S6. M^T fragments from the M tile (wave w: token tile w >> 1, position
  // k-step w & 1) as fp16 hi and lo planes and, in the first value head of a
  // group, Q fragments from the Q tile (wave w: token tile w & 3, key k-steps
  // 2 (w >> 2) and 2 (w >> 2) + 1) as fp16, both of the tiles' bf16 hi + lo
  {
    const int mt = w >> 1, ks = w & 1;
    const Frag f = frag_pi(lqh, lql, PS, 16 * mt + l16, 32 * ks, kg);
    float xf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) xf[e] = bf16_value((u16)f.hi[e]) + bf16_value((u16)f.lo[e]);
    store8_h2(reinterpret_cast<u16 *>(wc + WV_M) + frag_off(mt, ks, 2, lane),
              reinterpret_cast<u16 *>(wc + WV_ML) + frag_off(mt, ks, 2, lane), xf);
  }
  if (it.kown) {
    const int mt = w & 3;
    u16 *qg = reinterpret_cast<u16 *>(wk + WK_Q);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int ks = 2 * (w >> 2) + j;
      const Frag f = frag_pi(qh, qlo, PR, 16 * mt + l16, 32 * ks, kg);
      float xf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xf[e] = bf16_value((u16)f.hi[e]) + bf16_value((u16)f.lo[e]);
      store8_h(qg + frag_off(mt, ks, 4, lane), xf);
    }
  }
  __syncthreads();  // every diagonal block read before any is overwritten
  if (tid < 64) {
    const int b = tid >> 4, cc = tid & 15;
#pragma unroll
    for (int r = 0; r < 16; ++r) sA[(16 * b + r) * PA + 16 * b + cc] = x[r];
  }
  __syncthreads();
  // S3b. off-diagonal blocks of T, with D_b = T_bb and A_ij the blocks of A:
  //   T10 = -D1 A10 D0,  T32 = -D3 A32 D2,
  //   X20 = A20 D0 + A21 T10, X21 = A21 D1, X30 = A30 D0 + A31 T10, X31 = A31 D1,
  //   T20 = -D2 X20, T21 = -D2 X21, T30 = -(T32 X20 + D3 X30), T31 = -(T32 X21 + D3 X31)
  // (the 2x2 block-triangular inverse applied twice).  Three stages; each
  // product is four fp32 MFMAs; a block of T overwrites the block of A that
  // only its own wave reads.
  {
    auto B_ = [&](int bi, int bj) { return sA + (16 * bi) * PA + 16 * bj; };
    auto X_ = [&](int i) { return scratch + i * 16 * XP; };    // X20, X21, X30, X31
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 xa = z;
    if (w == 0 || w == 1) {                // stage 1: T10, T32
      const int b0 = 2 * w;                // 0 or 2
      const f32x4 p = blk_mm<PA, PA>(B_(b0 + 1, b0), B_(b0, b0), z, l16, kg);
      const f32x4 t = blk_mm_acc<PA>(B_(b0 + 1, b0 + 1), p, z, l16, kg);
      blk_store<PA>(B_(b0 + 1, b0), t, -1.0f, l16, kg);
    } else if (w == 2 || w == 3) {         // X21 = A21 D1, X31 = A31 D1
      const f32x4 x = blk_mm<PA, PA>(B_(w, 1), B_(1, 1), z, l16, kg);
      blk_store<XP>(X_(w == 2 ? 1 : 3), x, 1.0f, l16, kg);
    } else if (w == 4 || w == 5) {         // A20 D0, A30 D0 (kept for stage 2)
      xa = blk_mm<PA, PA>(B_(w - 2, 0), B_(0, 0), z, l16, kg);
    }
    __syncthreads();
    if (w == 4 || w == 5) {                // stage 2: X20 = A20 D0 + A21 T10, X30 likewise
      xa = blk_mm<PA, PA>(B_(w - 2, 1), B_(1, 0), xa, l16, kg);
      blk_store<XP>(X_(w == 4 ? 0 : 2), xa, 1.0f, l16, kg);
    }
    __syncthreads();
    if (w < 4) {                           // stage 3: T20, T21, T30, T31
      const int bi = 2 + (w >> 1), bj = w & 1;
      f32x4 t = z;
      if (bi == 3) t = blk_mm<PA, XP>(B_(3, 2), X_(bj), t, l16, kg);          // T32 X2bj
      t = blk_mm<PA, XP>(B_(bi, bi), X_(2 * (bi - 2) + bj), t, l16, kg);      // D_bi X_bi,bj
      blk_store<PA>(B_(bi, bj), t, -1.0f, l16, kg);
    }
    __syncthreads();
  }
  // S5. W^T = K^T T1^T and Ut^T = V^T T2^T.  Wave w owns token tile
  // mt = w >> 1 and key/value tiles 4hf .. 4hf + 3 (hf = w & 1), so the T
  // fragments it forms (one token tile, two k-steps) serve four tiles each.
  const int mt = w >> 1, hf = w & 1;
  f32x4 accW[4], accU[4];   // key / value tile 4hf + d
#pragma unroll
  for (int d = 0; d < 4; ++d) accW[d] = accU[d] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    Frag bt1, bt2;
    t_frags(sA, sBeta, sEG, 16 * mt + l16, 32 * ks, kg, bt1, bt2);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const Frag ak = frag_tr(kh, klo, PR, 32 * ks, 16 * (4 * hf + d), kg, l16);
      const Frag av = frag_tr(vh, vlo, PR, 32 * ks, 16 * (4 * hf + d), kg, l16);
      accW[d] = mfma3(ak, bt1, accW[d]);
      accU[d] = mfma3(av, bt2, accU[d]);
    }
  }
  {  // W fragments (token tile mt, key k-steps 2hf, 2hf + 1) and Ut tiles -> workspace
    u16 *wg = reinterpret_cast<u16 *>(wc + WV_W);
    float *ug = reinterpret_cast<float *>(wc + WV_U);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const f32x4 a0 = accW[2 * p], a1 = accW[2 * p + 1];
      const float xw[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      store8_h(wg + frag_off(mt, 2 * hf + p, 4, lane), xw);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d)
      *reinterpret_cast<float4 *>(ug + acc_off(4 * hf + d, mt, lane)) =
          make_float4(accU[d][0], accU[d][1], accU[d][2], accU[d][3]);
  }
  src.taps_to_lds(tid, pre, tiles);
  __syncthreads();   // the next item rewrites every LDS tile
  it = nx;
  };
  run_item(blockIdx.x);
  for (int u = blockIdx.x + gridDim.x; u < n_items; u += gridDim.x) run_item(u);
}

// ----------------------------------------------------------------------------- phase B
// One workgroup (8 waves) per (sequence, head, block b of 16 value columns),
// computing the transposed recurrence on the state block S^T[j][i] (j in the
// block, i over all 128 keys):
//   P^T = S^T W^T,  U^T = Ut^T - P^T,  Y^T = S^T Q^T,
//   S^T <- e^{G_n} S^T + (diag(e^{G_n-G}) U)^T K,
//   y^T = scale (Y^T diag(e^G) + U^T M^T)
// Wave w owns key tile w of the state (one accumulator) and token tile w & 3
// of P^T (w < 4) or of Y^T and y^T (w >= 4).  S, U and diag(e^{G_n-G}) U
// travel through LDS as row-major [key][j] / [token][j] tiles and are read
// back by transpose reads.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// A wave's role in the chunk step: P waves (w < 4) form P and U; y waves of
// token tiles 0 and 1 need one position k-step of M (M is lower triangular),
// those of token tiles 2 and 3 two.  Each role runs its own copy of the chunk
// loop, so a wave loads exactly its operands, with no branch in the loop.
enum : int { ROLE_P = 0, ROLE_Y1 = 1, ROLE_Y2 = 2 };
template <int VT, int ROLE>
struct ChunkOps {
  static constexpr int NX = ROLE == ROLE_P ? VT : ROLE == ROLE_Y1 ? 2 : 4;
  float hdr;     // header word lane & 3: e^{G_n}, b, a, 0
  float tk;      // the lane's token t: e^{G_n - G_t} (P waves) or e^{G_t} (y waves)
  h16x8 b[4];    // W (P waves) or Q (y waves) fragments of token tile w & 3, 4 key k-steps
  h16x8 k[2];    // K^T fragments of key tile w, 2 token k-steps (hi)
  h16x8 kl[2];   // and their lo parts
  // P waves: the Ut accumulator tiles (value tile, w & 3); y waves: the M^T
  // fragments of the chunk before, token tile w & 3, hi and lo of position
  // k-step 0 (and of k-step 1)
  u32x4 x[NX];
};

// The header is read as one word per lane (lane l: word l & 3), a vector
// load: a scalar load of it would share the LDS wait counter, so every LDS
// wait behind it would also wait for the scalar cache.  hdr_word() hands every
// lane word i.
__device__ __forceinline__ float load_hdr(const unsigned char *wc, int lane) {
  return reinterpret_cast<const float *>(wc + WV_G)[lane & 3];
}
__device__ __forceinline__ float hdr_word(float hdr, int i) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hdr), i));
}

// The operands of one chunk, by the part of the chunk step that consumes
// them: wv, wk are the chunk's value and key slots, wvm the value slot of the
// chunk before (y waves read its M), blk the workgroup's first value tile.
// The scan requests each part of chunk c + 2 right after chunk c's step has
// read that part, so the requests of the 8 waves spread over the step rather
// than queueing at the texture addresser all at once.
struct ChunkSrc {
  const unsigned char *wv, *wk, *wvm;
};
// W or Q (and the P waves' Ut tiles: read where W is)
template <int VT, int ROLE>
__device__ __forceinline__ void load_b(ChunkOps<VT, ROLE> &o, const ChunkSrc &p, int w, int lane,
                                       int blk) {
  const u16 *bg = reinterpret_cast<const u16 *>(ROLE == ROLE_P ? p.wv + WV_W : p.wk + WK_Q);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) o.b[ks] = frag_ws(bg, w & 3, ks, 4, lane);
  if constexpr (ROLE == ROLE_P) {
#pragma unroll
    for (int i = 0; i < VT; ++i)
      o.x[i] = *reinterpret_cast<const u32x4 *>(p.wv + WV_U + 4 * acc_off(blk + i, w & 3, lane));
  }
}
// y waves: the M^T fragments of the chunk before
template <int VT, int ROLE>
__device__ __forceinline__ void load_m(ChunkOps<VT, ROLE> &o, const ChunkSrc &p, int w,
                                       int lane) {
  if constexpr (ROLE != ROLE_P) {
#pragma unroll
    for (int i = 0; i < ChunkOps<VT, ROLE>::NX; ++i)
      o.x[i] = *reinterpret_cast<const u32x4 *>(p.wvm + ((i & 1) ? WV_ML : WV_M) +
                                                 2 * frag_off(w & 3, i >> 1, 2, lane));
  }
}
// K^T hi and lo, and the header words
template <int VT, int ROLE>
__device__ __forceinline__ void load_k(ChunkOps<VT, ROLE> &o, const ChunkSrc &p, int w,
                                       int lane) {
  const u16 *kgp = reinterpret_cast<const u16 *>(p.wk + WK_K);
  const u16 *klp = reinterpret_cast<const u16 *>(p.wk + WK_KL);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    o.k[ks] = frag_ws(kgp, w, ks, 2, lane);
    o.kl[ks] = frag_ws(klp, w, ks, 2, lane);
  }
  o.hdr = load_hdr(p.wv, lane);
  o.tk = reinterpret_cast<const float *>(p.wv + (ROLE == ROLE_P ? WV_D : WV_EG))[16 * (w & 3) +
                                                                                 lane % 16];
}
template <int VT, int ROLE>
__device__ __forceinline__ void load_chunk(ChunkOps<VT, ROLE> &o, const ChunkSrc &p, int w,
                                           int lane, int blk) {
  load_k(o, p, w, lane);
  load_b(o, p, w, lane, blk);
  load_m(o, p, w, lane);
}

// ---- fp16 operands of the scan
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
struct FragH {
  h16x8 hi, lo;
};
// two floats -> fp16 hi and lo halves (x = hi + lo + O(2^-22 |x|) for x in
// fp16's normal range; x - hi is exact in fp32)
__device__ __forceinline__ void split2_h(float a, float b, unsigned &hi, unsigned &lo) {
  const h16x2 h = __builtin_convertvector(f32x2{a, b}, h16x2);
  const h16x2 l = __builtin_convertvector(f32x2{a - (float)h[0], b - (float)h[1]}, h16x2);
  hi = __builtin_bit_cast(unsigned, h);
  lo = __builtin_bit_cast(unsigned, l);
}
// 4 floats times `sc` (a power of two) split into 4 consecutive fp16 per plane
__device__ __forceinline__ void store4_split_h(u16 *hi, u16 *lo, const f32x4 &x, float sc) {
  unsigned h0, l0, h1, l1;
  split2_h(x[0] * sc, x[1] * sc, h0, l0);
  split2_h(x[2] * sc, x[3] * sc, h1, l1);
  *reinterpret_cast<uint2 *>(hi) = make_uint2(h0, h1);
  *reinterpret_cast<uint2 *>(lo) = make_uint2(l0, l1);
}
__device__ __forceinline__ h16x8 cat_h(v4s a, v4s b) {
  return __builtin_bit_cast(h16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
// frag_tr for fp16 planes (the transpose read moves 16-bit values of any type)
__device__ __forceinline__ FragH frag_tr_h(const u16 *hi, const u16 *lo, int pitch, int k0,
                                           int nb, int kg, int l16) {
  const int o = (k0 + 4 * kg + (l16 >> 2)) * pitch + nb + 4 * (l16 & 3);
  FragH f;
  f.hi = cat_h(tr4(hi + o), tr4(hi + o + 16 * pitch));
  f.lo = cat_h(tr4(lo + o), tr4(lo + o + 16 * pitch));
  return f;
}
// c += (a.hi + a.lo) b on fp16 MFMA (b exact in fp16)
__device__ __forceinline__ f32x4 mfma2_h(const FragH &a, const h16x8 &b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.lo, b, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.hi, b, c, 0, 0, 0);
  return c;
}
// c += (a.hi + a.lo)(bh + bl), dropping a.lo * bl (2^-22 relative)
__device__ __forceinline__ f32x4 mfma3_h(const FragH &a, const h16x8 &bh, const h16x8 &bl,
                                         f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.lo, bh, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.hi, bl, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.hi, bh, c, 0, 0, 0);
  return c;
}

// Power-of-two scales of one chunk, identical in every wave (they follow from
// the running bound and the chunk header only): the state tile is multiplied
// by sS = 2^-eS and U by sU = 2^-eU before the fp16 split, with e chosen so
// that the bound times the scale is below 2^14 (fp16 reaches 65504).
struct Scales {
  float sS, iS, sU, iU;   // 2^-eS, 2^eS, 2^-eU, 2^eU
};
__device__ __forceinline__ float pow2i(int e) { return __builtin_bit_cast(float, (e + 127) << 23); }
__device__ __forceinline__ Scales chunk_scales(float &bound, float hdr) {
  const float hb = hdr_word(hdr, 1), ha = hdr_word(hdr, 2);
  const float bs = bound;                   // the state entering the chunk
  const float nb = bound + hb;              // every state inside it
  const float bu = hb + ha * nb;            // every entry of U
  bound = nb;
  int es, eu;
  (void)frexpf(bs, &es);                    // bs = m 2^es, m in [0.5, 1)
  (void)frexpf(bu, &eu);
  es = min(max(es - 14, -100), 100);
  eu = min(max(eu - 14, -100), 100);
  return Scales{pow2i(-es), pow2i(es), pow2i(-eu), pow2i(eu)};
}

// The Frobenius norm (a bound on the spectral norm) of the state's columns in
// each value tile, over the 8 waves that hold its key tiles: each wave's
// butterfly sum, then the 8 partial sums in a fixed order, so every wave gets
// the same bits.  `red` is VT x 8 floats of LDS owned by the 8 waves.  Each
// value tile carries its own bound (and so its own scales), which makes a
// tile's arithmetic independent of how many tiles a workgroup holds.
template <int VT>
__device__ __forceinline__ void tile_norms(const f32x4 (&st)[VT], float *red, int w, int lane,
                                           float (&bound)[VT]) {
#pragma unroll
  for (int d = 0; d < VT; ++d) {
    const float ss = group_sum<64>(st[d][0] * st[d][0] + st[d][1] * st[d][1] +
                                   st[d][2] * st[d][2] + st[d][3] * st[d][3]);
    if (lane == 0) red[8 * d + w] = ss;
  }
  __syncthreads();
#pragma unroll
  for (int d = 0; d < VT; ++d) {
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) t += red[8 * d + i];
    bound[d] = sqrtf(t);
  }
}

// The chunks one (sequence, head) walks in phase B: its first workspace slot,
// chunk count (even), positions and first token row.  An empty sequence has
// no chunks; its first slot is then slot 0, so the operand loads issued before
// the (empty) chunk loop stay inside the workspace, and the state is written
// back as it was read.  (The scan kernels have no early exit: on the 16-wave
// form one changed its results even where it was never taken.)
struct HeadChunks {
  size_t first, kfirst;   // value and key slots of the first chunk
  int nch, len;
  int64_t row0;
};
__device__ __forceinline__ HeadChunks head_chunks(const NoTab &, int s, int h, int H, int Hk,
                                                  int n_tok, int n_chunks) {
  const int hk = h / (H / Hk);
  return HeadChunks{((size_t)s * H + h) * n_chunks, ((size_t)s * Hk + hk) * n_chunks, n_chunks,
                    n_tok, 0};
}
__device__ __forceinline__ HeadChunks head_chunks(const VarTab &tab, int s, int h, int H, int Hk,
                                                  int, int n_chunks) {
  const int nch = tab.ch0[s + 1] - tab.ch0[s], hk = h / (H / Hk);
  return HeadChunks{nch > 0 ? (size_t)h * n_chunks + tab.ch0[s] : 0,
                    nch > 0 ? (size_t)hk * n_chunks + tab.ch0[s] : 0, nch,
                    tab.tok0[s + 1] - tab.tok0[s], tab.tok0[s]};
}

// XCD-aware order of the scan's workgroups.  Consecutive workgroup ids go to
// different XCDs (id % 8).  The `per` workgroups of one unit (a sequence and
// query/key group) get ids on one XCD, so they share its L2.  When the unit
// count is a multiple of 8, consecutive units are interleaved over the 8
// XCDs, so every XCD holds an even share of every sequence: dealing each XCD
// a contiguous run of units would give it whole sequences, and with sequences
// of different lengths the XCD holding the longest would run long after the
// others are idle.  Otherwise units are dealt in contiguous runs (XCD x < r
// of nwg = 8q + r taking q + 1 workgroups, the others q).
__device__ __forceinline__ void xcd_order(int b, int nwg, int per, int &sh, int &sub) {
  const int xcd = b % 8, idx = b / 8;
  if ((nwg / per) % 8 == 0) {
    sh = (idx / per) * 8 + xcd;
    sub = idx % per;
  } else {
    const int q8 = nwg / 8, r8 = nwg % 8;
    const int unit = (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + idx;
    sh = unit / per;
    sub = unit % per;
  }
}

// The conv history after a sequence's last position, when phase A took its
// K, Q, V from the conv (ConvSrc): phase B writes it, since phase A's first
// chunks read the old history and no phase A workgroup can know when the
// others are done with it.  Each scan workgroup takes the channels of its
// value columns [c0, c0 + nc): the v channels of head h and, in the first
// value head of each query/key group, the q and k channels of the group's
// head.  Thread t < 3 nc takes one channel (part t / nc: v, q, k) and
// its 3 taps, new tap j = input position n_tok - 3 + j, or old tap
// n_tok + j when that position is before 0; the taps are read in the
// prologue and written after the scan, by the same thread, so no tap is
// overwritten before it is read.  hist == nullptr: no history (x is then any
// valid address and the reads are discarded).
struct HistOut {
  const float *x;
  int64_t x_tok, x_seq;
  float *hist;
  int64_t h_seq;
  int n_tok, Hk, G;   // G value heads per query/key head
};
struct HistTaps {
  float v[3];
  float *dst;        // the channel's 3 taps, or nullptr
};
__device__ __forceinline__ HistTaps hist_read(const HistOut &ho, int s, int h, int c0, int nc,
                                              int tid) {
  const int part = tid / nc, i = tid % nc, hk = h / ho.G;
  const bool on = ho.hist != nullptr && part < (h % ho.G == 0 ? 3 : 1);
  const int64_t ch = part == 0 ? (int64_t)2 * ho.Hk * DK + (int64_t)h * DV + c0 + i
                   : part == 1 ? (int64_t)hk * DK + c0 + i
                               : (int64_t)(ho.Hk + hk) * DK + c0 + i;
  HistTaps r;
  float *hp = on ? ho.hist + s * ho.h_seq + ch * 3 : nullptr;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int p = ho.n_tok - 3 + j;
    const float *src = !on ? ho.x : p >= 0 ? ho.x + s * ho.x_seq + (int64_t)p * ho.x_tok + ch
                                           : hp + (p + 3);
    r.v[j] = *src;
  }
  r.dst = hp;
  return r;
}
__device__ __forceinline__ void hist_write(const HistTaps &r) {
  if (r.dst != nullptr) {
#pragma unroll
    for (int j = 0; j < 3; ++j) r.dst[j] = r.v[j];
  }
}

constexpr int SPB = 24;   // pitch (bf16) of the [128][16] S tile and the [64][16] U tile

// y waves: what the y of a chunk still needs when the chunk step has run
// (its U tile is formed only then; M U is added in the next chunk's step)
template <int VT>
struct YCarry {
  f32x4 q[VT];    // (S^T Q^T) iS of the chunk, per value tile
  float iU[VT];   // the chunk's U scales
  float tk;       // e^{G_t} of the lane's token
};

// y^T of chunk c (its U tile in LDS at uh/ul): (Y^T diag(e^G) + U^T M^T) scale,
// with M^T fragments m (hi, lo of position k-step 0, then of k-step 1)
template <int VT, int ROLE>
__device__ __forceinline__ void y_out(const YCarry<VT> &yc, const u32x4 (&m)[ROLE == ROLE_Y1 ? 2 : 4],
                                      const u16 *uh, const u16 *ul, float *yp, int64_t y_tok,
                                      int n, float scale, int t, int l16, int kg) {
  constexpr int SP = NBLK * VT + 8;
#pragma unroll
  for (int d = 0; d < VT; ++d) {
    f32x4 ym = mfma3_h(frag_tr_h(uh, ul, SP, 0, 16 * d, kg, l16),
                       __builtin_bit_cast(h16x8, m[0]), __builtin_bit_cast(h16x8, m[1]),
                       f32x4{0.f, 0.f, 0.f, 0.f});
    if constexpr (ROLE == ROLE_Y2)
      ym = mfma3_h(frag_tr_h(uh, ul, SP, 32, 16 * d, kg, l16),
                   __builtin_bit_cast(h16x8, m[2]), __builtin_bit_cast(h16x8, m[3]), ym);
    if (t < n) {   // y is not read again here: a non-temporal store
      const f32x4 yv = (yc.q[d] * yc.tk + ym * yc.iU[d]) * scale;
      __builtin_nontemporal_store(
          yv, reinterpret_cast<f32x4 *>(yp + (int64_t)t * y_tok + 16 * d + 4 * kg));
    }
  }
}

// Chunk c of the scan on a workgroup's VT value tiles.  The state tile of
// value tile d (values 16d + 4kg + r of key 16w + l16) goes to LDS as rows
// [i][j] of the S tile (pitch SP); P waves (w < 4) form U^T = Ut^T - S^T W^T
// for token tile w and write U and diag(e^{G_n-G}) U as rows [t][j] of the U
// tile (buffer c % 2) and of the D tile; y waves form Y^T = S^T Q^T and, in the
// same stretch, finish y of chunk c - 1 with U^T M^T from the other U buffer
// (y feeds nothing, so it stays off the chain from state to state); then
// every wave updates its state tiles with the D tile times K.  The B operands
// (W or Q, K, M) are loaded once and serve all VT tiles.  yp: y rows of the
// sequence's first position; len: its positions.
template <int VT, int ROLE>
__device__ __forceinline__ void scan_chunk(ChunkOps<VT, ROLE> &o, const ChunkSrc &nx,
                                           YCarry<VT> &yc, float (&bound)[VT], f32x4 (&st)[VT],
                                           u16 *ssh, u16 *ssl, u16 *suh, u16 *sul, u16 *sdh,
                                           u16 *sdl, float *yp, int64_t y_tok, int c, int len,
                                           float scale, int w, int l16, int kg, int blk) {
  constexpr int SP = NBLK * VT + 8;
  constexpr int UB = CH * SP;   // one U buffer
  // nothing of this chunk's work is scheduled above this point: its header
  // words were loaded a chunk ago, and reading them earlier would wait for
  // the operand loads still in flight
  __builtin_amdgcn_sched_barrier(0);
  Scales sc[VT];
#pragma unroll
  for (int d = 0; d < VT; ++d) {
    sc[d] = chunk_scales(bound[d], o.hdr);
    store4_split_h(ssh + (16 * w + l16) * SP + 16 * d + 4 * kg,
                   ssl + (16 * w + l16) * SP + 16 * d + 4 * kg, st[d], sc[d].sS);
  }
  __syncthreads();
  f32x4 acc[VT];
#pragma unroll
  for (int d = 0; d < VT; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int d = 0; d < VT; ++d)
      acc[d] = mfma2_h(frag_tr_h(ssh, ssl, SP, 32 * ks, 16 * d, kg, l16), o.b[ks], acc[d]);
  const int t = 16 * (w & 3) + l16;   // this lane's token; values 4kg + r
#pragma unroll
  for (int d = 0; d < VT; ++d) acc[d] = acc[d] * sc[d].iS;
  if constexpr (ROLE == ROLE_P) {
#pragma unroll
    for (int d = 0; d < VT; ++d) {
      const f32x4 u = __builtin_bit_cast(f32x4, o.x[d]) - acc[d];
      const int off = t * SP + 16 * d + 4 * kg;
      store4_split_h(suh + (c & 1) * UB + off, sul + (c & 1) * UB + off, u, sc[d].sU);
      store4_split_h(sdh + off, sdl + off, u * o.tk, sc[d].sU);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_b(o, nx, w, l16 + 16 * kg, blk);   // W and Ut of chunk c + 2
  } else {
    __builtin_amdgcn_sched_barrier(0);
    load_b(o, nx, w, l16 + 16 * kg, blk);   // Q of chunk c + 2
    if (c > 0)
      y_out<VT, ROLE>(yc, o.x, suh + ((c - 1) & 1) * UB, sul + ((c - 1) & 1) * UB,
                      yp + (int64_t)(c - 1) * CH * y_tok, y_tok, len - (c - 1) * CH, scale, t,
                      l16, kg);
#pragma unroll
    for (int d = 0; d < VT; ++d) {
      yc.q[d] = acc[d];
      yc.iU[d] = sc[d].iU;
    }
    yc.tk = o.tk;
    __builtin_amdgcn_sched_barrier(0);
    load_m(o, nx, w, l16 + 16 * kg);        // M of chunk c + 1
  }
  __syncthreads();
  f32x4 du[VT];
#pragma unroll
  for (int d = 0; d < VT; ++d) du[d] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int d = 0; d < VT; ++d)
      du[d] = mfma3_h(frag_tr_h(sdh, sdl, SP, 32 * ks, 16 * d, kg, l16), o.k[ks], o.kl[ks],
                      du[d]);
  const float gam = hdr_word(o.hdr, 0);
#pragma unroll
  for (int d = 0; d < VT; ++d) st[d] = st[d] * gam + du[d] * sc[d].iU;
  __builtin_amdgcn_sched_barrier(0);
  load_k(o, nx, w, l16 + 16 * kg);          // K and header of chunk c + 2
}

template <class TAB, int VT>
__global__ __launch_bounds__(512) void k_chunk_scan(
    float *__restrict__ state, int64_t st_seq, const unsigned char *__restrict__ ws,
    const unsigned char *__restrict__ wsk, float *__restrict__ y, int64_t y_tok, int64_t y_seq,
    int n_tok, int n_chunks, int H, int Hk, float scale, const TAB tab, const HistOut ho) {
  constexpr int SP = NBLK * VT + 8;
  __shared__ __attribute__((aligned(16))) u16 ssh[DK * SP], ssl[DK * SP];
  __shared__ __attribute__((aligned(16))) u16 suh[2 * CH * SP], sul[2 * CH * SP];
  __shared__ __attribute__((aligned(16))) u16 sdh[CH * SP], sdl[CH * SP];
  __shared__ float red[8 * VT];
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  // the G NVB / VT workgroups of one (sequence, query/key head) group on one
  // XCD (xcd_order), so the group's Q and K cross from the MALL into its L2
  // once
  int gu, sub;
  const int G = H / Hk;
  xcd_order(blockIdx.x, gridDim.x, G * (NVB / VT), gu, sub);
  const int s = gu / Hk, h = (gu % Hk) * G + sub / (NVB / VT);
  const int blk = (sub % (NVB / VT)) * VT;   // first value tile
  const HeadChunks hc = head_chunks(tab, s, h, H, Hk, n_tok, n_chunks);
  const HistTaps taps = hist_read(ho, s, h, blk * NBLK, VT * NBLK, tid);

  // state element (value j = 16 (blk + d) + 4kg + r, key i = 16w + l16), value-major
  float *sp = state + s * st_seq + (int64_t)h * DK * DV +
              (int64_t)(blk * NBLK + 4 * kg) * DK + 16 * w + l16;
  f32x4 st[VT];
#pragma unroll
  for (int d = 0; d < VT; ++d) {
    const float *p = sp + (int64_t)16 * d * DK;
    st[d] = f32x4{p[0], p[DK], p[2 * DK], p[3 * DK]};
  }
  float bound[VT];
  tile_norms(st, red, w, lane, bound);
  const unsigned char *wh = ws + hc.first * WV_CHUNK, *wkh = wsk + hc.kfirst * WK_CHUNK;
  float *yh = y + s * y_seq + hc.row0 * y_tok + (int64_t)h * DV + blk * NBLK;
  auto cidx = [&](int c) { return (size_t)max(min(c, hc.nch - 1), 0); };
  // Two operand sets: chunk c + 2's are requested as soon as chunk c has run
  // (into the registers chunk c used), so each request has the whole of
  // chunk c + 1 to arrive.  n_chunks is even (the workspace is padded with an
  // identity chunk), so the loop has no tail; a tail would make the compiler
  // copy the operand registers at the loop head, which waits for every load
  // in flight.  One copy of the loop per wave role (a uniform branch).
  auto walk = [&](auto role) {
    constexpr int ROLE = decltype(role)::value;
    // the sources of chunk c (y waves: with the M of chunk c - 1)
    auto src = [&](int c) {
      return ChunkSrc{wh + cidx(c) * WV_CHUNK, wkh + cidx(c) * WK_CHUNK,
                      wh + cidx(c - 1) * WV_CHUNK};
    };
    YCarry<VT> yc;
    auto run = [&](ChunkOps<VT, ROLE> &o, int c) {
      scan_chunk<VT, ROLE>(o, src(c + 2), yc, bound, st, ssh, ssl, suh, sul, sdh, sdl, yh, y_tok,
                           c, hc.len, scale, w, l16, kg, blk);
    };
    ChunkOps<VT, ROLE> a, b;
    load_chunk(a, src(0), w, lane, blk);
    load_chunk(b, src(1), w, lane, blk);
    for (int c = 0; c < hc.nch; c += 2) {
      run(a, c);
      run(b, c + 1);
    }
    // y of the last chunk: set a was loaded for chunk nch, so it holds the M
    // of chunk nch - 1, whose U tile is the last one written
    if constexpr (ROLE != ROLE_P) {
      const int c = hc.nch;
      if (c > 0)
        y_out<VT, ROLE>(yc, a.x, suh + ((c - 1) & 1) * CH * SP, sul + ((c - 1) & 1) * CH * SP,
                        yh + (int64_t)(c - 1) * CH * y_tok, y_tok, hc.len - (c - 1) * CH, scale,
                        16 * (w & 3) + l16, l16, kg);
    }
  };
  if (w < 4)
    walk(std::integral_constant<int, ROLE_P>{});
  else if ((w & 3) < 2)
    walk(std::integral_constant<int, ROLE_Y1>{});
  else
    walk(std::integral_constant<int, ROLE_Y2>{});
#pragma unroll
  for (int d = 0; d < VT; ++d) {
    float *p = sp + (int64_t)16 * d * DK;
    p[0] = st[d][0];
    p[DK] = st[d][1];
    p[2 * DK] = st[d][2];
    p[3 * DK] = st[d][3];
  }
  hist_write(taps);
}

// ---- phase B for grids that exceed one pass of the chip
// One 16-wave workgroup per (sequence, head, pair of value blocks): waves
// 8g .. 8g+7 run exactly the per-wave arithmetic of k_chunk_scan on value
// block 2p + g, so the results are bit-identical to it.  The two groups share
// one LDS copy of each chunk's W, Q, K hi and lo, and M hi and lo (80 KiB,
// copied byte for byte), which halves the head's operand reads from L2; the price is that
// every wave now reads its fragments from LDS, so this form only pays once
// the 8-wave grid would need a second pass.
// The copy is staged through registers one chunk ahead: each thread holds 32
// bytes of W and Q, 32 bytes of K and 16 bytes of M.  W and Q are rewritten in
// LDS right after the barrier that ends their last reads (the U barrier), K
// and M right after the barrier that ends the state update's and y's reads of
// them (the S barrier).
constexpr int OPS_WQ = (int)(2 * WS_PLANE);   // W (value slot), Q (key slot)
constexpr int OPS_K = (int)(2 * WS_PLANE);    // K^T hi and lo (key slot)
constexpr int OPS_M = 2 * CH * CH * 2;        // M^T hi and lo (value slot)
constexpr int PAIR_THREADS = 1024;
static_assert(WS_PLANE == 16 * PAIR_THREADS && WK_KL == WK_K + WS_PLANE &&
              OPS_M == 16 * PAIR_THREADS && WV_ML == WV_M + OPS_M / 2, "copy split");

template <class TAB>
__global__ __launch_bounds__(PAIR_THREADS) void k_chunk_scan_pair(
    float *__restrict__ state, int64_t st_seq, const unsigned char *__restrict__ ws,
    const unsigned char *__restrict__ wsk, float *__restrict__ y, int64_t y_tok, int64_t y_seq,
    int n_tok, int n_chunks, int H, int Hk, float scale, const TAB tab, const HistOut ho) {
  __shared__ __attribute__((aligned(16))) u16 ssh[2][DK * SPB], ssl[2][DK * SPB];
  __shared__ __attribute__((aligned(16))) u16 suh[2][CH * SPB], sul[2][CH * SPB];
  __shared__ __attribute__((aligned(16))) u16 sdh[2][CH * SPB], sdl[2][CH * SPB];
  __shared__ __attribute__((aligned(16))) unsigned char ops[OPS_WQ + OPS_K + OPS_M];
  __shared__ float red[2][8];
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
  const int grp = tid >> 9, w = (tid >> 6) & 7;
  // the 4 G workgroups of one (sequence, query/key head) group on one XCD
  // (xcd_order; the grid need not be a multiple of 8)
  int gu, sub;
  const int G = H / Hk;
  xcd_order(blockIdx.x, gridDim.x, G * (NVB / 2), gu, sub);
  const int s = gu / Hk, h = (gu % Hk) * G + sub / (NVB / 2), pair = sub % (NVB / 2);
  const int blk = 2 * pair + grp;
  const HeadChunks hc = head_chunks(tab, s, h, H, Hk, n_tok, n_chunks);
  const HistTaps taps = hist_read(ho, s, h, 2 * pair * NBLK, 2 * NBLK, tid);

  float *sp = state + s * st_seq + (int64_t)h * DK * DV +
              (int64_t)(blk * NBLK + 4 * kg) * DK + 16 * w + l16;
  f32x4 st = {sp[0], sp[DK], sp[2 * DK], sp[3 * DK]};
  float bound;
  {
    const f32x4 st1[1] = {st};
    float b1[1];
    tile_norms<1>(st1, red[grp], w, lane, b1);
    bound = b1[0];
  }
  const unsigned char *wh = ws + hc.first * WV_CHUNK, *wkh = wsk + hc.kfirst * WK_CHUNK;
  float *yh = y + s * y_seq + hc.row0 * y_tok + (int64_t)h * DV + blk * NBLK;
  auto cidx = [&](int c) { return (size_t)max(min(c, hc.nch - 1), 0); };
  auto vptr = [&](int c) { return wh + cidx(c) * WV_CHUNK; };
  auto kptr = [&](int c) { return wkh + cidx(c) * WK_CHUNK; };
  u16 *s_hi = ssh[grp], *s_lo = ssl[grp], *u_hi = suh[grp], *u_lo = sul[grp];
  u16 *d_hi = sdh[grp], *d_lo = sdl[grp];
  const u16 *b_lds = reinterpret_cast<const u16 *>(ops + (w < 4 ? 0 : OPS_WQ / 2));
  const u16 *k_lds = reinterpret_cast<const u16 *>(ops + OPS_WQ);
  const u16 *m_lds = reinterpret_cast<const u16 *>(ops + OPS_WQ + OPS_K);
  const int add_off = 4 * acc_off(blk, w & 3, lane);
  const int t = 16 * (w & 3) + l16;   // this lane's token; values 4kg + r

  u32x4 rwq[2], rk[2], rm;
  auto load_wq = [&](int c) __attribute__((always_inline)) {
    rwq[0] = *reinterpret_cast<const u32x4 *>(vptr(c) + WV_W + 16 * tid);
    rwq[1] = *reinterpret_cast<const u32x4 *>(kptr(c) + WK_Q + 16 * tid);
  };
  auto load_k = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      rk[i] = *reinterpret_cast<const u32x4 *>(kptr(c) + WK_K + 16 * (tid + PAIR_THREADS * i));
    rm = *reinterpret_cast<const u32x4 *>(vptr(c) + WV_M + 16 * tid);
  };
  auto put_wq = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4 *>(ops + 16 * (tid + PAIR_THREADS * i)) = rwq[i];
  };
  auto put_k = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4 *>(ops + OPS_WQ + 16 * (tid + PAIR_THREADS * i)) = rk[i];
    *reinterpret_cast<u32x4 *>(ops + OPS_WQ + OPS_K + 16 * tid) = rm;
  };
  // P waves: the Ut tile and e^{G_n - G_t}; y waves: e^{G_t} (their add slot
  // reads the header, one line for the whole wave)
  auto load_add = [&](int c, float4 &add, float &hdr, float &tk)
      __attribute__((always_inline)) {
    const unsigned char *wv = vptr(c);
    add = *reinterpret_cast<const float4 *>(w < 4 ? wv + WV_U + add_off : wv + WV_G);
    hdr = load_hdr(wv, lane);
    tk = reinterpret_cast<const float *>(wv + (w < 4 ? WV_D : WV_EG))[t];
  };
  auto run = [&](int c, const float4 &add, float hdr, float tk) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);   // as in scan_chunk
    const Scales sc = chunk_scales(bound, hdr);
    store4_split_h(s_hi + (16 * w + l16) * SPB + 4 * kg, s_lo + (16 * w + l16) * SPB + 4 * kg,
                   st, sc.sS);
    __syncthreads();   // S barrier: W, Q of chunk c and the S tiles are in LDS
    put_k();           // K, M of chunk c, first read after the U barrier
    load_k(c + 1);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const h16x8 b = *reinterpret_cast<const h16x8 *>(b_lds + frag_off(w & 3, ks, 4, lane));
      acc = mfma2_h(frag_tr_h(s_hi, s_lo, SPB, 32 * ks, 0, kg, l16), b, acc);
    }
    acc = acc * sc.iS;
    if (w < 4) {
      const f32x4 u = __builtin_bit_cast(f32x4, add) - acc;
      store4_split_h(u_hi + t * SPB + 4 * kg, u_lo + t * SPB + 4 * kg, u, sc.sU);
      store4_split_h(d_hi + t * SPB + 4 * kg, d_lo + t * SPB + 4 * kg, u * tk, sc.sU);
    }
    __syncthreads();   // U barrier: K, M and the U, D tiles are in LDS, W and Q are read
    put_wq();          // W, Q of chunk c + 1
    load_wq(c + 2);
    f32x4 du = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const h16x8 kh = *reinterpret_cast<const h16x8 *>(k_lds + frag_off(w, ks, 2, lane));
      const h16x8 kl =
          *reinterpret_cast<const h16x8 *>(k_lds + CH * DK + frag_off(w, ks, 2, lane));
      du = mfma3_h(frag_tr_h(d_hi, d_lo, SPB, 32 * ks, 0, kg, l16), kh, kl, du);
    }
    if (w >= 4) {
      auto mfr = [&](int ks, int plane) {
        return *reinterpret_cast<const h16x8 *>(m_lds + plane * CH * CH +
                                                frag_off(w & 3, ks, 2, lane));
      };
      f32x4 ym = mfma3_h(frag_tr_h(u_hi, u_lo, SPB, 0, 0, kg, l16), mfr(0, 0), mfr(0, 1),
                         f32x4{0.f, 0.f, 0.f, 0.f});
      if ((w & 3) >= 2)
        ym = mfma3_h(frag_tr_h(u_hi, u_lo, SPB, 32, 0, kg, l16), mfr(1, 0), mfr(1, 1), ym);
      if (t < min(CH, hc.len - c * CH))
        __builtin_nontemporal_store((acc * tk + ym * sc.iU) * scale,
                                    reinterpret_cast<f32x4 *>(yh + (int64_t)(c * CH + t) * y_tok +
                                                              4 * kg));
    }
    st = st * hdr_word(hdr, 0) + du * sc.iU;
  };

  load_wq(0);
  put_wq();   // visible after the first S barrier
  load_wq(1);
  load_k(0);
  float4 add0, add1;
  float hdr0, hdr1, tk0, tk1;
  load_add(0, add0, hdr0, tk0);
  load_add(1, add1, hdr1, tk1);
  // the chunk count is even, as for k_chunk_scan
  for (int c = 0; c < hc.nch; c += 2) {
    run(c, add0, hdr0, tk0);
    load_add(c + 2, add0, hdr0, tk0);
    run(c + 1, add1, hdr1, tk1);
    load_add(c + 3, add1, hdr1, tk1);
  }
  sp[0] = st[0];
  sp[DK] = st[1];
  sp[2 * DK] = st[2];
  sp[3 * DK] = st[3];
  hist_write(taps);
}

}  // namespace

static_assert(CH == 64, "padded_chunks counts 64-position chunks");

// bytes of the value and key slots of one chunk position over all heads
static size_t slots_bytes(int H, int Hk) { return (size_t)H * WV_CHUNK + (size_t)Hk * WK_CHUNK; }

size_t chunked_workspace_bytes(int n_seq, int n_tok, int H, int Hk, int S, int) {
  if (S != DK) return 0;   // the S = 32 / 64 form keeps everything on chip
  return (size_t)n_seq * padded_chunks(n_tok) * slots_bytes(H, Hk);
}

// Sum over sequences of padded_chunks(len) <= sum(ceil(len / 64)) + n_seq
// <= (total_tok + 63 n_seq) / 64 + n_seq, for any split of total_tok.
size_t chunked_varlen_workspace_bytes(int n_seq, int total_tok, int H, int Hk, int S) {
  if (S != DK) return 0;
  const int64_t slots = ((int64_t)total_tok + 63 * (int64_t)n_seq) / CH + n_seq;
  return (size_t)slots * slots_bytes(H, Hk);
}

// Compute units of the current device, queried once per device.
static int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      return -1;
    cached[dev] = n;
  }
  return cached[dev];
}

// Phase A then phase B of one call; n_chunks is the per-sequence chunk count
// (fixed-length batch) or the packed total (variable-length batch).  The
// n_items value slots come first in the workspace, then the key slots.
template <class TAB, class SRC>
static int launch_two_phase(const RecurArgs &a, const TAB &tab, const SRC &src, const HistOut &ho,
                            int n_chunks, int n_items, unsigned char *wsb, hipStream_t stream) {
  // phase A: one persistent workgroup per CU (its LDS allows no more), or one
  // per item when there are fewer items than CUs
  const int cus = device_cu_count();
  if (cus <= 0) return GDN_ERR_LAUNCH;
  const int grid_a = n_items < cus ? n_items : cus;
  unsigned char *wsk = wsb + (size_t)n_items * WV_CHUNK;
  int rc = launch_kernel(k_chunk_prep<TAB, SRC>, dim3(grid_a), dim3(512), 0, stream, src, wsb,
                         wsk, a.n_tok, n_chunks, a.H, a.Hk, n_items, tab);
  if (rc != GDN_OK) return rc;
  // phase B: 8-wave workgroups of one value tile each while they fit in one
  // pass of the chip (measured: two or four tiles per workgroup lengthen the
  // chain more than they save in operand traffic, 168 and 241 against 133 us
  // at 32 heads); past that, the 16-wave form whose pairs of value tiles share
  // operand copies in LDS.  All forms give the same bits.
  const int units = a.n_seq * a.H;
  if (units * NVB > cus)
    return launch_kernel(k_chunk_scan_pair<TAB>, dim3(units * (NVB / 2)), dim3(PAIR_THREADS), 0,
                         stream, a.state, a.st_seq, (const unsigned char *)wsb,
                         (const unsigned char *)wsk, a.y, a.y_tok, a.y_seq, a.n_tok, n_chunks,
                         a.H, a.Hk, a.scale, tab, ho);
  return launch_kernel(k_chunk_scan<TAB, 1>, dim3(units * NVB), dim3(512), 0, stream, a.state,
                       a.st_seq, (const unsigned char *)wsb, (const unsigned char *)wsk, a.y,
                       a.y_tok, a.y_seq, a.n_tok, n_chunks, a.H, a.Hk, a.scale, tab, ho);
}

// No conv history to write: any valid address for the discarded reads.
static HistOut no_hist(const RecurArgs &a) {
  return HistOut{a.state, 0, 0, nullptr, 0, 3, a.Hk, a.H / a.Hk};
}

template <class TIN>
static DirectSrc<TIN> direct_src(const RecurArgs &a, const TIN *q, const TIN *k, const TIN *v) {
  return DirectSrc<TIN>{q, k, v, a.g, a.beta, a.qk_tok, a.qk_seq, a.v_tok, a.v_seq, a.n_tok, a.H};
}

int launch_recur_chunked(const RecurArgs &a, int chunk, void *ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (chunk != CH) return GDN_ERR_UNSUPPORTED;
  if (a.S != DK) return launch_chunk_small(a, stream);
  const int n_chunks = padded_chunks(a.n_tok);
  if (ws_bytes < chunked_workspace_bytes(a.n_seq, a.n_tok, a.H, a.Hk, a.S, chunk))
    return GDN_ERR_WORKSPACE;
  return launch_two_phase(a, NoTab{}, direct_src(a, a.q, a.k, a.v), no_hist(a), n_chunks,
                          n_chunks * a.H * a.n_seq, static_cast<unsigned char *>(ws), stream);
}

int launch_recur_chunked_varlen(const RecurArgs &a, const VarTab &tab, bool bf16_in, int chunk,
                                void *ws, size_t ws_bytes, hipStream_t stream) {
  if (chunk != CH) return GDN_ERR_UNSUPPORTED;
  if (a.S != DK) return launch_chunk_small_varlen(a, tab, bf16_in, stream);
  const int n_chunks = tab.ch0[tab.n_seq];   // packed total, even per sequence
  if (n_chunks == 0) return GDN_OK;           // every sequence is empty
  if (ws_bytes < (size_t)n_chunks * slots_bytes(a.H, a.Hk)) return GDN_ERR_WORKSPACE;
  unsigned char *wsb = static_cast<unsigned char *>(ws);
  if (bf16_in)
    return launch_two_phase(a, tab,
                            direct_src(a, reinterpret_cast<const u16 *>(a.q),
                                       reinterpret_cast<const u16 *>(a.k),
                                       reinterpret_cast<const u16 *>(a.v)),
                            no_hist(a), n_chunks, n_chunks * a.H, wsb, stream);
  return launch_two_phase(a, tab, direct_src(a, a.q, a.k, a.v), no_hist(a), n_chunks,
                          n_chunks * a.H, wsb, stream);
}

int launch_prefill_chunked(const RecurArgs &a, const PrefillConv &pc, int chunk, void *ws,
                           size_t ws_bytes, hipStream_t stream) {
  if (chunk != CH || a.S != DK || pc.D != 4) return GDN_ERR_UNSUPPORTED;
  const int n_chunks = padded_chunks(a.n_tok);
  if (ws_bytes < chunked_workspace_bytes(a.n_seq, a.n_tok, a.H, a.Hk, a.S, chunk))
    return GDN_ERR_WORKSPACE;
  const ConvSrc src{pc.x,     pc.x_tok, pc.x_seq, pc.w,    pc.hist, pc.h_seq, pc.alpha,
                    pc.dt,    pc.a,     a.beta,   pc.eps,  a.n_tok, a.H,      a.Hk};
  const HistOut ho{pc.x, pc.x_tok, pc.x_seq, pc.hist, pc.h_seq, a.n_tok, a.Hk, a.H / a.Hk};
  return launch_two_phase(a, NoTab{}, src, ho, n_chunks, n_chunks * a.H * a.n_seq,
                          static_cast<unsigned char *>(ws), stream);
}

}  // namespace gdn
