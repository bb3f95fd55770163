// Device helpers shared by the gfx950 TTT kernels: I/O dtype conversion, GELU and
// its derivatives, wave64 reductions and the status word.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttt_internal.h"
#include "ttt_poison.hpp"  // test-build instrumentation (TTT_POISON)

#define TTT_HD __device__ __forceinline__
#define TTT_EXP2(x) __builtin_amdgcn_exp2f(x)
#define TTT_RCP(x) __builtin_amdgcn_rcpf(x)
#define TTT_RELU(x) __builtin_amdgcn_fmed3f((x), 0.0f, __builtin_inff())
#include "ttt_gelu.hpp"

namespace ttt {

// ---------------------------------------------------------------------------
// I/O element types. bf16 is carried as raw uint16 bits; conversion to fp32 is
// exact, conversion from fp32 rounds to nearest even (NaN stays NaN).
// ---------------------------------------------------------------------------
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  uint32_t u = __float_as_uint(x);
  bf16_t r;
  if ((u & 0x7fffffffu) > 0x7f800000u) {
    r.bits = static_cast<uint16_t>((u >> 16) | 0x40u);  // quiet NaN
  } else {
    u += 0x7fffu + ((u >> 16) & 1u);
    r.bits = static_cast<uint16_t>(u >> 16);
  }
  return r;
}

// ---------------------------------------------------------------------------
// GELU (exact erf form, or the tanh form) and its first/second derivatives.
// erf form: GELU = x Phi(x); GELU' = Phi + x phi; GELU'' = phi (2 - x^2).
// ---------------------------------------------------------------------------
constexpr float kInvSqrt2 = 0.70710678118654752440f;
constexpr float kInvSqrt2Pi = 0.39894228040143267794f;
constexpr float kTanhC = 0.79788456080286535588f;  // sqrt(2/pi)
constexpr float kTanhA = 0.044715f;

struct Gelu3 {
  float v, d1, d2;
};

__device__ __forceinline__ float gelu(float x, int kind) {
  if (kind == TTT_GELU_TANH) {
    float u = kTanhC * (x + kTanhA * x * x * x);
    return 0.5f * x * (1.0f + tanhf(u));
  }
  return 0.5f * x * (1.0f + erff(x * kInvSqrt2));
}

// value and first derivative
__device__ __forceinline__ void gelu_d(float x, int kind, float& v, float& d1) {
  if (kind == TTT_GELU_TANH) {
    float x2 = x * x;
    float u = kTanhC * (x + kTanhA * x2 * x);
    float th = tanhf(u);
    float du = kTanhC * (1.0f + 3.0f * kTanhA * x2);
    v = 0.5f * x * (1.0f + th);
    d1 = 0.5f * (1.0f + th) + 0.5f * x * (1.0f - th * th) * du;
    return;
  }
  float cdf = 0.5f * (1.0f + erff(x * kInvSqrt2));
  float pdf = __expf(-0.5f * x * x) * kInvSqrt2Pi;
  v = x * cdf;
  d1 = cdf + x * pdf;
}

__device__ __forceinline__ Gelu3 gelu_d2(float x, int kind) {
  Gelu3 r;
  if (kind == TTT_GELU_TANH) {
    float x2 = x * x;
    float u = kTanhC * (x + kTanhA * x2 * x);
    float th = tanhf(u);
    float s = 1.0f - th * th;                       // sech^2
    float du = kTanhC * (1.0f + 3.0f * kTanhA * x2);
    float ddu = kTanhC * 6.0f * kTanhA * x;
    r.v = 0.5f * x * (1.0f + th);
    r.d1 = 0.5f * (1.0f + th) + 0.5f * x * s * du;
    // d/dx [0.5(1+th)] = 0.5 s du ; d/dx [0.5 x s du] = 0.5 s du + 0.5 x (-2 th s du) du + 0.5 x s ddu
    r.d2 = s * du - x * th * s * du * du + 0.5f * x * s * ddu;
    return r;
  }
  float cdf = 0.5f * (1.0f + erff(x * kInvSqrt2));
  float pdf = __expf(-0.5f * x * x) * kInvSqrt2Pi;
  r.v = x * cdf;
  r.d1 = cdf + x * pdf;
  r.d2 = pdf * (2.0f - x * x);
  return r;
}

// ---------------------------------------------------------------------------
// wave64 reductions (butterfly over all 64 lanes)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ void flag_nonfinite(unsigned* status, float x) {
  if (!isfinite(x)) atomicOr(status, kStatusNonFinite);
}

}  // namespace ttt
