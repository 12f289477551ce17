// atlas_mem_bias.h -- derivatives of the attentional biases that reshape the
// error (device code).  Miras review, "Alternative Attentional Biases":
//   l_p loss |e|_p^p / p       -> sign(e) |e|^(p-1), elementwise (p >= 1)
//   Huber, threshold delta      -> e while |e|_2 <= delta, else delta sign(e)
//                                  (one choice for the whole token)
// sign(e) is exact, or tanh(alpha e) for alpha > 0 (the review's Remark 5).
#pragma once

#include <hip/hip_runtime.h>

namespace atlas {

__device__ __forceinline__ float sign_of(float x, float alpha) {
  return alpha > 0.f ? tanhf(alpha * x) : x > 0.f ? 1.f : x < 0.f ? -1.f : 0.f;
}

// sign(e) |e|^(p-1), zero at e = 0 (for p = 1 the plain sign)
__device__ __forceinline__ float lp_slope(float e, float p, float alpha) {
  const float a = fabsf(e);
  return a > 0.f ? sign_of(e, alpha) * exp2f((p - 1.f) * log2f(a)) : 0.f;
}

// Huber slope given the token's choice (small: |e|_2 <= delta)
__device__ __forceinline__ float huber_slope(float e, bool small, float delta, float alpha) {
  return small ? e : delta * sign_of(e, alpha);
}

}  // namespace atlas
