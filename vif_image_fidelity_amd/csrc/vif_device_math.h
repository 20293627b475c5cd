// vif_device_math.h -- per-pixel arithmetic of the float VIF kernels (gfx950).
//
// Every function here is plain fp32/fp64 code whose roundings are fixed by
// the build: -ffp-contract=off (no fused multiply-add), correctly rounded
// fp32 division, IEEE denormals, no fast-math (ADR-1444 "float_vif_hip runs
// the arithmetic of the CUDA twin ...", Context: HIP spells each rounding
// step as a plain operator under those flags).  Each operation below is one
// IEEE rounding, in the order written.  The scoring kernels and the
// self-test kernels include this header, so the gates test the very code
// the pipeline runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vif_internal.h"

namespace vifk {

// Floor of the variance terms: the fp32 value nearest 1e-10.
constexpr float kEps = 1e-10f;

// Mirror an index into [0, n): reflect about the edge sample once, then
// clamp.  Every index an output consumes lies within one reflection of the
// plane, so the clamp only moves loads that no output uses (ADR-1444,
// Decision: reflected tile indices pass through a clamp so a frame under
// 72 px never reads outside its plane).
__device__ __forceinline__ int mirror_clamp(int i, int n) {
  int m = i < 0 ? -i : i;
  m = m > n - 1 ? 2 * (n - 1) - m : m;
  m = m < 0 ? 0 : m;
  return m > n - 1 ? n - 1 : m;
}

// log2 polynomial (ADR-1422, Context: the CPU evaluates log2 with a
// polynomial in fp32, not a library log2).  This method's coefficients:
// Chebyshev interpolation of log2(1+t)/t on [0,1], degree 9, rounded to
// fp32; c1 first.  x = 2^e * (1 + t); returns (float)e + t * P(t), Horner
// from the highest coefficient.  Meant for finite x >= 1; an infinite or NaN
// x (a zero noise variance can produce them) is read the same way: its
// exponent field 255 gives e = 128.
__device__ __forceinline__ float bits_f32(uint32_t u) {
  return __builtin_bit_cast(float, u);
}

__device__ __forceinline__ float log2_poly(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const int e = static_cast<int>((u >> 23) & 0xffu) - 127;
  const float m = bits_f32((u & 0x007fffffu) | 0x3f800000u);
  const float t = m - 1.0f;
  float p = bits_f32(0xbb96254au);   // c10
  p = p * t + bits_f32(0x3ce6f6e9u); // c9
  p = p * t + bits_f32(0xbda6904fu); // c8
  p = p * t + bits_f32(0x3e1bc356u); // c7
  p = p * t + bits_f32(0xbe6194f1u); // c6
  p = p * t + bits_f32(0x3e913ea6u); // c5
  p = p * t + bits_f32(0xbeb84ebdu); // c4
  p = p * t + bits_f32(0x3ef63175u); // c3
  p = p * t + bits_f32(0xbf38aa21u); // c2
  p = p * t + bits_f32(0x3fb8aa3bu); // c1
  const float q = p * t;
  return static_cast<float>(e) + q;
}

// The correctly rounded fp64 quotient a / d for operands whose quotient needs
// no scaling: a == +0 or 2^-700 <= a <= 2^600, and 2^-100 <= d <= 2^200 (so
// the quotient lies in [2^-900, 2^700] and the exponents of a and d differ
// by at most 700).  These are the steps of the compiler's IEEE fp64
// division on gfx950 -- a hardware reciprocal, two Newton-Raphson
// refinements, the product with a, the remainder and the corrected quotient
// (six fused multiply-adds, the last of which the expansion issues as
// v_div_fmas with its scale flag clear) -- without the
// two operand-scaling steps and the special-case fix-up around them.  In this
// domain those are identities (the scaling acts only on zero, denormal or
// extreme-exponent operands and quotients, and the fix-up only on zero,
// infinite or NaN operands and on overflowing or underflowing quotients; for
// a == +0 every step gives +0, as the fix-up does), so the result has the
// same bits.  The fused multiply-adds below are the division's own, exactly
// as the expansion has them; nowhere else does the library fuse.
__device__ __forceinline__ double div_in_range(double a, double d) {
  double r = __builtin_amdgcn_rcp(d);
  double e = __builtin_fma(-d, r, 1.0);
  r = __builtin_fma(r, e, r);
  e = __builtin_fma(-d, r, 1.0);
  r = __builtin_fma(r, e, r);
  const double q = a * r;
  const double rem = __builtin_fma(-d, q, a);
  return __builtin_fma(rem, r, q);
}

// The correctly rounded fp32 quotient a / d for operands that need no
// scaling: a == +0 or 2^-100 <= |a| <= 2^17, and 2^-20 <= d <= 2^17.  These
// are the compiler's IEEE fp32 division steps on gfx950 (a hardware
// reciprocal, one Newton-Raphson refinement, the product with a, and two
// rounds of remainder and correction, the last of which the expansion issues
// as v_div_fmas with its scale flag clear) without the two v_div_scale steps
// and the closing v_div_fixup.  In this domain those are identities:
// v_div_scale changes an operand only for a zero, denormal or near-overflow
// one, an exponent gap of 96 or more, a denormal reciprocal or quotient, or
// a numerator below 2^-103, none of which occurs (|a / d| lies in
// [2^-117, 2^37]); v_div_fixup changes the result only for zero, infinite or
// NaN operands and quotients that overflow or underflow, and for a == +0
// every step gives +0, as the fix-up does.  So the bits are the division's.
// The statistic's sigma12 / sigma1_sq stays in this domain in the kPow2
// branch: sigma1_sq >= nsq >= 2^-20 there, every filtered value is below
// 2^16, and a non-zero sigma12 is at least 2^-100 (a non-zero filtered value
// of a plane whose samples are multiples of 2^-8 is at least 2^-77 at every
// scale, and sigma12 is a difference of two such values or zero).
__device__ __forceinline__ float div_in_range_f32(float a, float d) {
  float r = __builtin_amdgcn_rcpf(d);
  const float e = __builtin_fmaf(-d, r, 1.0f);
  r = __builtin_fmaf(e, r, r);
  float q = a * r;
  float rem = __builtin_fmaf(-d, q, a);
  q = __builtin_fmaf(rem, r, q);
  rem = __builtin_fmaf(-d, q, a);
  return __builtin_fmaf(rem, r, q);
}

// fl32(1 + a / (sv + nsq)) with the sum, quotient and sum with one in fp64
// and a single conversion to fp32 at the end; nsq is the noise variance,
// kept in binary64 (ADR-1422 "float_vif_sycl computes the CPU's arithmetic
// ...", Context and Decision).  kPow2 marks the kernels for a power-of-two
// nsq in [2^-20, 2^20] (see den_ratio): there a is a finite fp32 value
// (0 or at least 2^-149, below 2^128) and d = sv + nsq lies in
// [2^-20, 2^129], inside div_in_range's domain, so the quotient takes the
// shorter sequence; any other nsq divides with the compiler's expansion.
template <bool kPow2>
__device__ __forceinline__ float num_ratio(float a, float sv, double nsq) {
  const double d = static_cast<double>(sv) + nsq;
  double q;
  if constexpr (kPow2)
    q = div_in_range(static_cast<double>(a), d);
  else
    q = static_cast<double>(a) / d;
  return static_cast<float>(1.0 + q);
}

// fl32(1 + sigma1_sq / nsq), fp64 quotient and sum, one conversion.  kPow2
// is a compile-time choice: the kernels come in both forms and the host
// launches the one that matches nsq, so neither carries the other's
// arithmetic (a run-time branch on it was turned into both computations and
// a select).
//
// For a power-of-two nsq in [2^-20, 2^20] (kPow2: sa.inv_nsq = 1 / nsq, not
// 0) the same value comes from two fp32 operations, 1.0f + s1 * (1 / nsq).
// Let q = s1 * 2^k exactly; fp64 holds it exactly.  When |q| >= 2^-28, 1 + q
// is exact in fp64 too (q's 24 significant bits and the leading 1 span at
// most 53 bits; beyond 2^53 the fp64 sum is q rounded, as fp32 rounds it),
// so the conversion is the one rounding of 1 + q to fp32, which is what
// 1.0f + q gives: the fp32 product is q itself unless it overflows, and
// then both paths give an infinity.  When |q| < 2^-28 both give 1.0f: fp32
// rounds 1 + q to 1 (whether or not a tiny product underflows), and fp64
// rounds it to within 2^-28 of 1, which converts to 1.  NaN stays NaN.
template <bool kPow2>
__device__ __forceinline__ float den_ratio(float s1, const StatArgs &sa) {
  if constexpr (kPow2) {
    return 1.0f + s1 * sa.inv_nsq_f;
  } else {
    const double q = static_cast<double>(s1) / sa.nsq;
    return static_cast<float>(1.0 + q);
  }
}

// Per-pixel statistic from the five filtered values.
//   sigma1_sq = xx - mu1*mu1, sigma2_sq = yy - mu2*mu2 (each clamped at 0),
//   sigma12 = xy - mu1*mu2.  Below the noise variance (compared in fp64,
//   ADR-1422, Decision) both terms are 1.  Above it: g = sigma12 /
//   sigma1_sq, sv_sq = sigma2_sq - g * sigma12; sigma2_sq < eps sets g and
//   sv_sq to 0; g < 0 sets sv_sq = sigma2_sq and g = 0; sv_sq is floored at
//   eps; the enhancement gain limit then bounds g where it enters the
//   numerator (C's MIN(g, limit), see StatArgs); then the two ratios and
//   their log2.  With nsq = 0 nothing is special-cased: IEEE arithmetic
//   throughout, as in the plain definition.
//
//   Some of these selects are written as one maximum or minimum instruction
//   where that gives the same terms:
//   - the clamps of s1 and s2 at 0, always: xx and yy are >= +0 and never
//     -0 (sums of products of values >= +0), and so are m11 and m22; their
//     difference is then never NaN and never -0 (a difference is -0 only
//     when the left operand is -0), and for such a value max(s, +0) is
//     exactly s < 0 ? 0 : s;
//   - the floor of sv at eps and the gain limit, in the kPow2 form only:
//     there s1 >= nsq >= 2^-20 in this branch, so g = s12 / s1, g * s12 and
//     sv are finite, never NaN, and max(sv, eps) is the select.  The limit
//     is >= +0 and never NaN and g >= +0 here, so min(g, gain) is the select
//     except when g and gain are zeros of opposite sign, where g * g is +0
//     either way and the terms are the same.  (With nsq = 0, a zero s1 makes
//     g NaN, and the selects must keep C's handling of it.)
template <bool kPow2>
__device__ __forceinline__ void pixel_terms(float mu1, float mu2, float xx,
                                            float yy, float xy,
                                            const StatArgs &sa, float &num,
                                            float &den) {
  const float m11 = mu1 * mu1;
  const float m22 = mu2 * mu2;
  const float m12 = mu1 * mu2;
  float s1 = xx - m11;
  float s2 = yy - m22;
  const float s12 = xy - m12;
  s1 = __builtin_fmaxf(s1, 0.0f);
  s2 = __builtin_fmaxf(s2, 0.0f);
  // the comparison in fp64; for a power-of-two nsq (kPow2) its fp32 value
  // is exact, and comparing s1 with it is the same test
  if (kPow2 ? s1 < sa.nsq_f : static_cast<double>(s1) < sa.nsq) {
    num = 1.0f;
    den = 1.0f;
    return;
  }
  // kPow2: s1 >= nsq >= 2^-20 here, inside div_in_range_f32's domain
  float g = kPow2 ? div_in_range_f32(s12, s1) : s12 / s1;
  const float gs = g * s12;
  float sv = s2 - gs;
  if (s2 < kEps) {
    g = 0.0f;
    sv = 0.0f;
  }
  if (g < 0.0f) {
    sv = s2;
    g = 0.0f;
  }
  if constexpr (kPow2) {
    sv = __builtin_fmaxf(sv, kEps);
    g = __builtin_fminf(g, sa.gain);
  } else {
    sv = sv < kEps ? kEps : sv;
    g = g < sa.gain ? g : sa.gain;
  }
  const float gg = g * g;
  const float a = gg * s1;
  num = log2_poly(num_ratio<kPow2>(a, sv, sa.nsq));
  den = log2_poly(den_ratio<kPow2>(s1, sa));
}

}  // namespace vifk
