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

}  // namespace ttt_gelu
