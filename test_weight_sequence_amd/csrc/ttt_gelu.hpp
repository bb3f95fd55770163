// Branch-free GELU (exact erf form) and its derivatives for the MFMA kernels.
//
// Phi(x) = 1/2 erfc(-x / sqrt 2) is evaluated with the rational-exponential form of
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26:
//   erfc(z) = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),  t = 1 / (1 + p z),  z >= 0,
// with |error| <= 1.5e-7 in erf. The exponential exp(-x^2/2) is shared with the normal
// density phi(x) that GELU' = Phi + x phi and GELU'' = phi (2 - x^2) need, so one exp2 and
// one reciprocal give GELU and its derivatives without data-dependent branches.
//
// Plain C++ with two hooks (TTT_EXP2, TTT_RCP) so that the same formula compiles for the
// device (hardware exp2 / reciprocal) and for host-side accuracy tests.
#pragma once

#ifndef TTT_HD
#define TTT_HD inline
#endif
#ifndef TTT_EXP2
#define TTT_EXP2(x) exp2f(x)
#endif
#ifndef TTT_RCP
#define TTT_RCP(x) (1.0f / (x))
#endif
#ifndef TTT_RELU
#define TTT_RELU(x) ((x) > 0.0f ? (x) : 0.0f)
#endif

namespace ttt_gelu {

// A&S 7.1.26 coefficients, pre-multiplied by 1/2 (the kernel needs erfc / 2).
constexpr float kP = 0.3275911f * 0.70710678118654752440f;  // p / sqrt(2): t = 1 / (1 + p |x| / sqrt 2)
constexpr float kA1 = 0.5f * 0.254829592f;
constexpr float kA2 = 0.5f * -0.284496736f;
constexpr float kA3 = 0.5f * 1.421413741f;
constexpr float kA4 = 0.5f * -1.453152027f;
constexpr float kA5 = 0.5f * 1.061405429f;
constexpr float kNegHalfLog2e = -0.72134752044448170368f;   // exp(-x^2/2) = 2^(x^2 * this)
constexpr float kInvSqrt2Pi = 0.39894228040143267794f;

struct PhiPhi {
  float cdf;  // Phi(x)
  float e;    // exp(-x^2 / 2)
};

TTT_HD PhiPhi phi_pair(float x) {
  const float ax = x < 0.f ? -x : x;
  const float t = TTT_RCP(ax * kP + 1.0f);
  const float poly = t * (kA1 + t * (kA2 + t * (kA3 + t * (kA4 + t * kA5))));
  const float e = TTT_EXP2((x * x) * kNegHalfLog2e);
  const float half_erfc = poly * e;                // Phi(-|x|)
  PhiPhi r;
  r.cdf = x < 0.f ? half_erfc : 1.0f - half_erfc;
  r.e = e;
  return r;
}

// GELU(x) = x Phi(x)
TTT_HD float gelu(float x) { return x * phi_pair(x).cdf; }

// value and first derivative: GELU' = Phi + x phi
TTT_HD void gelu_d(float x, float& v, float& d1) {
  const PhiPhi p = phi_pair(x);
  v = x * p.cdf;
  d1 = p.cdf + x * (p.e * kInvSqrt2Pi);
}

// value, first and second derivative: GELU'' = phi (2 - x^2)
TTT_HD void gelu_d2(float x, float& v, float& d1, float& d2) {
  const PhiPhi p = phi_pair(x);
  const float pdf = p.e * kInvSqrt2Pi;
  v = x * p.cdf;
  d1 = p.cdf + x * pdf;
  d2 = pdf * (2.0f - x * x);
}

// Lower-order variant for the forward kernels, whose activations are rounded to bf16
// (relative step 2^-8) right after: A&S 7.1.25,
//   erfc(z) = (b1 t + b2 t^2 + b3 t^3) exp(-z^2),  t = 1 / (1 + q z),  z >= 0,
// with |error| <= 2.5e-5 in erf, i.e. <= 1.25e-5 in Phi. Two fewer multiply-adds per value
// than 7.1.26, and the constants are folded further:
//  - GELU alone: x Phi(x) = max(x, 0) - |x| Phi(-|x|), with no select on the sign;
//  - with GELU': the exponential is taken as the density phi(x) = 2^(-x^2/2 log2 e -
//    log2 sqrt(2 pi)) directly (the sqrt(2 pi) moves into the coefficients), so that
//    GELU' = Phi + x phi is one multiply-add.
namespace fast {
constexpr float kQ = 0.47047f * 0.70710678118654752440f;  // q / sqrt(2)
constexpr float kB1 = 0.5f * 0.3480242f;
constexpr float kB2 = 0.5f * -0.0958798f;
constexpr float kB3 = 0.5f * 0.7478556f;
constexpr float kSqrt2Pi = 2.50662827463100050242f;
constexpr float kC1 = kB1 * kSqrt2Pi;
constexpr float kC2 = kB2 * kSqrt2Pi;
constexpr float kC3 = kB3 * kSqrt2Pi;
constexpr float kLog2InvSqrt2Pi = -1.32574806473616f;  // log2(1 / sqrt(2 pi))
}  // namespace fast

TTT_HD float gelu_fast(float x) {
  const float ax = __builtin_fabsf(x);
  const float t = TTT_RCP(ax * fast::kQ + 1.0f);
  const float e = TTT_EXP2((x * x) * kNegHalfLog2e);
  const float h = t * (fast::kB1 + t * (fast::kB2 + t * fast::kB3)) * e;  // Phi(-|x|)
  return TTT_RELU(x) - ax * h;
}

TTT_HD void gelu_d_fast(float x, float& v, float& d1) {
  const float ax = __builtin_fabsf(x);
  const float t = TTT_RCP(ax * fast::kQ + 1.0f);
  const float pdf = TTT_EXP2((x * x) * kNegHalfLog2e + fast::kLog2InvSqrt2Pi);
  const float h = t * (fast::kC1 + t * (fast::kC2 + t * fast::kC3)) * pdf;  // Phi(-|x|)
  const float cdf = x < 0.f ? h : 1.0f - h;
  v = x * cdf;
  d1 = x * pdf + cdf;
}

}  // namespace ttt_gelu
