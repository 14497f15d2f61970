// Device-side helpers shared by the libpkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;

// ---- bf16 -------------------------------------------------------------------

// A 32-bit word holds two bf16 values; bf16 is the top half of a binary32, so
// widening is a shift or a mask.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// binary32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

__device__ __forceinline__ void unpack8(const uint4 v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// ---- OCP e4m3fn -------------------------------------------------------------

// Eight e4m3fn bytes -> eight floats with the gfx950 converter, which reads
// the OCP encoding (exact: every e4m3fn value is a binary32 value).
__device__ __forceinline__ void unpack8(const uint2 v, float (&f)[8]) {
  auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, false);
  auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, true);
  auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, false);
  auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, true);
  f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
  f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
}

// binary32 -> e4m3fn, round to nearest (ties to even), saturating at +-448.
// Bit-level: below 2^-6 the format is fixed point with step 2^-9, so the
// code is rint(|y| * 2^9) (8 lands exactly on the smallest normal, 0x08);
// above, the binary32 significand is rounded to 3 bits at bit 20 and the
// exponent is re-biased from 127 to 7 (a carry out of the significand bumps
// the exponent, which the addition does by itself).  The sign bit is
// copied, so negative values that round to zero give 0x80.  NaN gives 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3fn_rne_sat(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __builtin_fabsf(y);
  if (a != a) return 0x7Fu;
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {                              // 2^-6
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  uint32_t ua = __float_as_uint(a);
  ua += 0x7ffffu + ((ua >> 20) & 1u);
  const uint32_t exp8 = (ua >> 23) - 127u + 7u;     // 1..15
  const uint32_t man3 = (ua >> 20) & 7u;
  return sign | (exp8 << 3) | man3;
}

// Scale of a block that a new token opens: amax / 448 in fp32 (correctly
// rounded division), or 1 when the token is all zeros.  Elements are then
// stored as e4m3fn(x / scale).  Both append paths use exactly this.
__device__ __forceinline__ float fp8_block_scale(float amax) {
  return amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
}
__device__ __forceinline__ uint32_t fp8_encode_scaled(float x, float scale) {
  return f32_to_e4m3fn_rne_sat(__fdiv_rn(x, scale));
}

// ---- INT8 --------------------------------------------------------------------

// Eight int8 codes -> eight floats (exact).
__device__ __forceinline__ void unpack8_i8(const uint2 v, float (&f)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[k] = (float)(int8_t)(v.x >> (8 * k));
    f[4 + k] = (float)(int8_t)(v.y >> (8 * k));
  }
}

// Scale of a block that a new token opens: amax / 127 in fp32 (correctly
// rounded division), or 1 when the token is all zeros; elements are stored
// as clamp(rint(x / scale), -127, 127), rint rounding halves to even.
// Both append paths use exactly this.
__device__ __forceinline__ float int8_block_scale(float amax) {
  return amax == 0.0f ? 1.0f : __fdiv_rn(amax, 127.0f);
}
__device__ __forceinline__ uint32_t int8_encode_scaled(float x, float scale) {
  const float y = __fdiv_rn(x, scale);
  if (y != y) return 0u;
  const float r = fminf(fmaxf(__builtin_rintf(y), -127.0f), 127.0f);
  return (uint32_t)(int32_t)r & 0xffu;
}

// ---- cross-lane reductions (DPP within a 16-lane row) -----------------------

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over aligned groups of N lanes (N in 1, 2, 4, 8, 16); every lane of the
// group gets the group's total.  After the two quad steps each quad holds its
// sum; the half-row mirror pairs quad 0 with quad 1 (lane i with 7 - i) and
// the row mirror pairs the two halves (lane i with 15 - i).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group size");
  if constexpr (N >= 2) x += dpp_mov<kDppQuadXor1>(x);
  if constexpr (N >= 4) x += dpp_mov<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp_mov<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_mov<kDppRowMirror>(x);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_mov<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_mov<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_mov<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_mov<kDppRowMirror>(x));
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- rotary embedding --------------------------------------------------------

// Nearest-even rounding of a double straight to bf16 (8 significant bits):
// round the double's 52-bit significand at bit 45, then the value is exact
// in binary32 and its top 16 bits are the bf16.  (Finite values in the
// normal range; rotated activations are.)
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const unsigned long long lsb = (u >> 45) & 1ull;
  u += (1ull << 44) - 1ull + lsb;
  u &= ~((1ull << 45) - 1ull);
  const float f = (float)__longlong_as_double((long long)u);   // exact
  return (uint16_t)(__float_as_uint(f) >> 16);
}

// Cosine and sine of an fp64 angle, for RoPE angles (a position times a
// frequency <= 1, so |x| < 2^31).  Cody-Waite reduction x = k pi/2 + r,
// |r| <= pi/4, with pi/2 split in three parts (the first two with 33
// significant bits), each subtracted with a fused multiply-add: the product
// k * part is exact inside the fma, so each step rounds once, on a result
// that shrinks by 2^-33 per step, and r is accurate to far below an ulp of
// sin for any such k.  Then the Taylor series of sin r to the r^19 term and
// of cos r to the r^18 term (the first omitted terms are below 2^-70 for
// |r| <= pi/4), evaluated with correctly rounded fused multiply-adds; the
// quadrant k mod 4 swaps and negates.  Every operation is spelled out (no
// contraction left to the compiler), so the two kernels that use it get
// identical bits; and it calls no library routine, whose registers would
// weigh on the kernels that inline it.
__device__ __forceinline__ void rope_sincos(double x, double* s, double* c) {
  constexpr double kTwoOverPi = 0.6366197723675814;
  constexpr double kP1 = 1.5707963267341256;        // 0x1.921fb544p+0
  constexpr double kP2 = 6.077100506303966e-11;     // 0x1.0b4611a6p-34
  constexpr double kP3 = 2.0222662487959506e-21;    // 0x1.3198a2e037073p-69
  const double k = __builtin_rint(__dmul_rn(x, kTwoOverPi));
  double r = __fma_rn(-k, kP1, x);
  r = __fma_rn(-k, kP2, r);
  r = __fma_rn(-k, kP3, r);
  const double z = __dmul_rn(r, r);
  // sin r = r (1 - z/3! + z^2/5! - ... - z^9/19!), cos r = 1 - z/2! + ... + z^9/18!
  double ps = -8.22063524662433e-18;                 // -1/19!
  ps = __fma_rn(ps, z, 2.8114572543455206e-15);      //  1/17!
  ps = __fma_rn(ps, z, -7.647163731819816e-13);      // -1/15!
  ps = __fma_rn(ps, z, 1.6059043836821613e-10);      //  1/13!
  ps = __fma_rn(ps, z, -2.505210838544172e-08);      // -1/11!
  ps = __fma_rn(ps, z, 2.7557319223985893e-06);      //  1/9!
  ps = __fma_rn(ps, z, -0.0001984126984126984);      // -1/7!
  ps = __fma_rn(ps, z, 0.008333333333333333);        //  1/5!
  ps = __fma_rn(ps, z, -0.16666666666666666);        // -1/3!
  const double sr = __fma_rn(__dmul_rn(ps, z), r, r);
  double pc = 1.5619206968586225e-16;                //  1/18!
  pc = __fma_rn(pc, z, -4.779477332387385e-14);      // -1/16!
  pc = __fma_rn(pc, z, 1.1470745597729725e-11);      //  1/14!
  pc = __fma_rn(pc, z, -2.08767569878681e-09);       // -1/12!
  pc = __fma_rn(pc, z, 2.755731922398589e-07);       //  1/10!
  pc = __fma_rn(pc, z, -2.48015873015873e-05);       // -1/8!
  pc = __fma_rn(pc, z, 0.001388888888888889);        //  1/6!
  pc = __fma_rn(pc, z, -0.041666666666666664);       // -1/4!
  pc = __fma_rn(pc, z, 0.5);                         //  1/2!  (subtracted below)
  const double cr = __fma_rn(-pc, z, 1.0);
  const int q = (int)((long long)k & 3);
  const double sv = (q & 1) ? cr : sr;
  const double cv = (q & 1) ? sr : cr;
  *s = (q & 2) ? -sv : sv;
  *c = ((q + 1) & 2) ? -cv : cv;
}

// Rotate one pair (x[2i], x[2i+1]), two bf16 in a word, by the angle whose
// cosine and sine are c, s: two separately rounded fp64 products and a
// rounded sum or difference each, no fused multiply-add, then one rounding
// to bf16.  Returns the rotated pair in the same packing.
__device__ __forceinline__ uint32_t rotate_pair(uint32_t pair, double c, double s) {
  const double x0 = (double)bf16_lo(pair), x1 = (double)bf16_hi(pair);
  const uint32_t r0 = f64_to_bf16_rne(__dsub_rn(__dmul_rn(x0, c), __dmul_rn(x1, s)));
  const uint32_t r1 = f64_to_bf16_rne(__dadd_rn(__dmul_rn(x0, s), __dmul_rn(x1, c)));
  return r0 | (r1 << 16);
}

}  // namespace pkv
