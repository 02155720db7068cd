// bf16_frag.hpp -- bf16 hi/lo split operands and their LDS fragment loads for
// v_mfma_f32_16x16x32_bf16 (gfx950, wave64), shared by the MFMA kernels.
//
// MFMA operand layout (16x16x32 bf16, wave64): lane l holds row (l % 16) of
// A / column (l % 16) of B, and 8 k values chosen by l / 16; the accumulator
// holds D[4*(l/16) + r][l % 16], r = 0..3.  Operands that are the transpose of
// a row-major LDS tile are read with ds_read_b64_tr_b16 (gfx950).  An fp32
// operand is carried as bf16 hi + lo and a product as hi*hi + hi*lo + lo*hi
// (relative error ~2^-16 per product instead of bf16's 2^-8).
#pragma once
#include <hip/hip_runtime.h>

namespace gdn {
namespace {

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

// split() of two values at once, packed as stored: element 0 in the low half.
// One v_cvt_pk_bf16_f32 per plane; the same roundings as split(), so the
// same bits.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split2(float a, float b, unsigned &hi, unsigned &lo) {
  const unsigned h = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2v));
  const float ha = __builtin_bit_cast(float, h << 16);
  const float hb = __builtin_bit_cast(float, h & 0xffff0000u);
  lo = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a - ha, b - hb}, bf16x2v));
  hi = h;
}

// Eight values split into one fragment (slot e holds x[e]).
__device__ __forceinline__ Frag split8(const float (&x)[8]) {
  unsigned h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) split2(x[2 * e], x[2 * e + 1], h[e], l[e]);
  Frag f;
  f.hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  f.lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
  return f;
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

// ----------------------------------------------------------------------------- fragments
// Standard fragment of a k-contiguous tile: row `row`, k = k + 8*kg + 0..7.
__device__ __forceinline__ Frag frag(const u16 *hi, const u16 *lo, int pitch, int row, int k) {
  Frag f;
  f.hi = *reinterpret_cast<const bf16x8 *>(hi + row * pitch + k);
  f.lo = *reinterpret_cast<const bf16x8 *>(lo + row * pitch + k);
  return f;
}

// The permuted k order used wherever a fragment meets an accumulator tile:
// slot e of lane (kg, l16) in k-step ks holds k = 32ks + 4kg + e (e < 4) and
// k = 32ks + 16 + 4kg + (e - 4) (e >= 4).  Both operands of a product use it
// (the sum over k does not depend on the order), and it is exactly the set of
// rows an accumulator tile pair gives one lane, so accumulators turn into
// fragments without any transpose.
__device__ __forceinline__ int pi_k(int k0, int kg, int e) {
  return k0 + 4 * kg + (e & 3) + ((e >> 2) << 4);
}

typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 cat(v4s a, v4s b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Permuted fragment of a k-contiguous tile: row `row`, k in pi(k0, kg).
__device__ __forceinline__ Frag frag_pi(const u16 *hi, const u16 *lo, int pitch, int row, int k0,
                                        int kg) {
  const int o = row * pitch + k0 + 4 * kg;
  Frag f;
  f.hi = cat(*reinterpret_cast<const v4s *>(hi + o), *reinterpret_cast<const v4s *>(hi + o + 16));
  f.lo = cat(*reinterpret_cast<const v4s *>(lo + o), *reinterpret_cast<const v4s *>(lo + o + 16));
  return f;
}

// Transposed permuted fragment of a row-major [k][n] LDS tile: column
// nb + l16, rows pi(k0, kg), read with ds_read_b64_tr_b16.  In each 16-lane
// group, lane j points at row k0 + 4kg + j/4 (then + 16), columns
// nb + 4(j%4) .. +3; the transpose hands lane i column nb + i of those 4 rows.
__device__ __forceinline__ v4s tr4(const u16 *p) {
  typedef short v4s_lds __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s_lds *)(p));
}
__device__ __forceinline__ Frag frag_tr(const u16 *hi, const u16 *lo, int pitch, int k0, int nb,
                                        int kg, int l16) {
  const int o = (k0 + 4 * kg + (l16 >> 2)) * pitch + nb + 4 * (l16 & 3);
  Frag f;
  f.hi = cat(tr4(hi + o), tr4(hi + o + 16 * pitch));
  f.lo = cat(tr4(lo + o), tr4(lo + o + 16 * pitch));
  return f;
}

// Split 4 floats and store them as 4 consecutive bf16 in each plane.
__device__ __forceinline__ void store4_split(u16 *hi, u16 *lo, float a, float b, float c, float d) {
  unsigned h0, l0, h1, l1;
  split2(a, b, h0, l0);
  split2(c, d, h1, l1);
  *reinterpret_cast<uint2 *>(hi) = make_uint2(h0, h1);
  *reinterpret_cast<uint2 *>(lo) = make_uint2(l0, l1);
}

// Split 8 floats into one 16-byte store per plane.
__device__ __forceinline__ void store8_split(u16 *hi, u16 *lo, const float (&x)[8]) {
  unsigned h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) split2(x[2 * e], x[2 * e + 1], h[e], l[e]);
  *reinterpret_cast<uint4 *>(hi) = make_uint4(h[0], h[1], h[2], h[3]);
  *reinterpret_cast<uint4 *>(lo) = make_uint4(l[0], l[1], l[2], l[3]);
}

}  // namespace
}  // namespace gdn
