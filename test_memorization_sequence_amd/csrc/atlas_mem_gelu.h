// atlas_mem_gelu.h -- GELU of the MLP memory and its derivative (device code).
//
// gelu(z) = z Phi(z) = z (1 + erf(z / sqrt 2)) / 2,  gelu'(z) = Phi(z) + z phi(z).
// erf from Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: for x >= 0, erfc x = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^{-x^2}
// with t = 1 / (1 + p x), |error| <= 1.5e-7.  With x = |z| / sqrt 2 the factor
// e^{-x^2} = e^{-z^2/2} is also the one phi(z) needs, so both values cost one
// reciprocal, one exponential and a dozen FMAs, with no branch.  The values
// feed bf16 MFMA operands, whose rounding (2^-9 relative) is far larger.
#pragma once

#include <hip/hip_runtime.h>

namespace atlas {

// 2 Phi(z) = 1 + erf(z / sqrt 2), and e^{-z^2/2}
__device__ __forceinline__ float two_phi(float z, float& e) {
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  e = __builtin_amdgcn_exp2f(-(x * x) * 1.44269504088896341f);
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f), -0.284496736f),
                              0.254829592f);
  const float tail = poly * e;                 // erfc(x)
  return z >= 0.f ? 2.f - tail : tail;
}
__device__ __forceinline__ float gelu(float z) {
  float e;
  return 0.5f * z * two_phi(z, e);
}
__device__ __forceinline__ float gelu_prime(float z) {
  float e;
  const float c2 = two_phi(z, e);
  return fmaf(z * e, 0.39894228040143268f, 0.5f * c2);
}
// both at once
__device__ __forceinline__ void gelu_and_prime(float z, float& a, float& da) {
  float e;
  const float c2 = two_phi(z, e);
  a = 0.5f * z * c2;
  da = fmaf(z * e, 0.39894228040143268f, 0.5f * c2);
}

}  // namespace atlas
