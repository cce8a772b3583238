// Epilogue pieces shared by the tiled and the small-M linear kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

// Per-launch epilogue operands.  int8 mode: Y = A sa[m] sb[n] + bias[n];
// gated: the up weight (B2, its scales sb2 and bias bias2) shares the packed
// activation.
struct EpiArgs {
  const float* sa;
  const float* sb;
  const float* bias;
  const uint8_t* B2;
  int64_t ldb2;
  const float* sb2;
  const float* bias2;
};

// Standard normal CDF, branch-free.  For z = |y| / sqrt 2, erfc(z) is taken
// from the five-term form t (a1 + a2 t + ... + a5 t^4) e^{-z^2} with
// t = 1 / (1 + p z) of Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26 (absolute error at most 1.5e-7).  Phi(y) is
// erfc(z) / 2 for y < 0 and 1 - erfc(z) / 2 otherwise, so the lower tail is
// never formed by cancellation.  One reciprocal and one exp2 per value.
__device__ __forceinline__ float std_normal_cdf(float y) {
  const float z = fabsf(y) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.f));
  float q = fmaf(t, 1.061405429f, -1.453152027f);
  q = fmaf(t, q, 1.421413741f);
  q = fmaf(t, q, -0.284496736f);
  q = fmaf(t, q, 0.254829592f);
  // e^{-z^2} = 2^{-z^2 log2 e}
  const float half_erfc = 0.5f * t * q * __builtin_amdgcn_exp2f(-1.44269504088896341f * z * z);
  return y < 0.f ? half_erfc : 1.f - half_erfc;
}

// Activations of the fused epilogue: 0 none, 1 GELU in its erf form
// y Phi(y), 2 GELU in its tanh form y (1 + tanh u) / 2 with
// u = sqrt(2/pi) (y + 0.044715 y^3), evaluated as y / (1 + e^{-2u}) (the same
// quantity: (1 + tanh u) / 2 is the logistic function of 2u).  Both are
// branch-free so that the epilogue of a wide tile stays a straight run of
// vector instructions.
template <int ACT>
__device__ __forceinline__ float activation(float y) {
  if constexpr (ACT == 1) {
    return y * std_normal_cdf(y);
  } else if constexpr (ACT == 2) {
    const float u = 0.79788456080286536f * fmaf(0.044715f * y, y * y, y);
    // e^{-2u} = 2^{-2u log2 e}; at e^{-2u} = inf the reciprocal is 0
    return y * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-2.88539008177792681f * u));
  } else {
    return y;
  }
}


}  // namespace convrot
