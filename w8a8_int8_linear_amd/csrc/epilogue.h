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

// Producer fusion of the next layer's pack: per-group maxima of the rotated
// output.  out [M, ld] fp32 receives, for every row and every contiguous
// group of G = 2^log2g output features, the largest magnitude of that group
// of the output (as stored) multiplied by the regular rotation R_G.
struct RowmaxArgs {
  float* out;
  int64_t ld;
  int log2g;
};

// GELU in its erf form, y Phi(y), branch-free.  With a = |y| and
// h = erfc(a / sqrt 2) / 2 (the normal tail beyond a), y Phi(y) equals
// max(y, 0) - a h for either sign of y, one fused multiply-add that never
// forms the lower tail by cancellation.  erfc(z) is taken from the
// five-term form t (a1 + a2 t + ... + a5 t^4) e^{-z^2} with t = 1 / (1 + p z)
// of Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26
// (absolute error at most 1.5e-7); the coefficients below are those halved
// (exactly, so h is the same value), p is folded with 1 / sqrt 2, and
// e^{-z^2} = 2^{-y^2 log2(e) / 2}.  One reciprocal and one exp2 per value.
__device__ __forceinline__ float gelu_erf(float y) {
  const float a = fabsf(y);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.23164189f, a, 1.f));  // p / sqrt 2
  float q = fmaf(t, 0.5307027145f, -0.7265760135f);
  q = fmaf(t, q, 0.7107068705f);
  q = fmaf(t, q, -0.142248368f);
  q = fmaf(t, q, 0.127414796f);
  const float h = t * q * __builtin_amdgcn_exp2f(y * (y * -0.72134752044448170f));
  return fmaf(-a, h, fmaxf(y, 0.f));
}

// Activations of the fused epilogue: 0 none, 1 GELU in its erf form
// (gelu_erf above), 2 GELU in its tanh form y (1 + tanh u) / 2 with
// u = sqrt(2/pi) (y + 0.044715 y^3), evaluated as y / (1 + e^{-2u}) (the same
// quantity: (1 + tanh u) / 2 is the logistic function of 2u), where
// -2u log2(e) = y (c1 + c2 y^2) with the constants folded.  Both are
// branch-free so that the epilogue of a wide tile stays a straight run of
// vector instructions.
template <int ACT>
__device__ __forceinline__ float activation(float y) {
  if constexpr (ACT == 1) {
    return gelu_erf(y);
  } else if constexpr (ACT == 2) {
    // c1 = -2 log2(e) sqrt(2/pi), c2 = 0.044715 c1
    const float e = y * fmaf(y * y, -0.10294324f, -2.3022082f);
    // 2^e = e^{-2u}; at 2^e = inf the reciprocal is 0
    return y * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(e));
  } else {
    return y;
  }
}


}  // namespace convrot
